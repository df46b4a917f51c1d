"""torch's own sub-byte float conversions (E2M1 and friends), for pinning the
4-bit oracle against a library routine.

The routines live in torch.testing._internal.common_quantized, whose import
pulls in torch's test harness (it needs the `expecttest` package and turns off
torch's global backend flags as a side effect).  This helper instead takes
just the conversion functions and their constants from that module's source
file and runs them in a namespace of their own: the code is torch's, unchanged.
"""
import ast
import pathlib

import torch

_NAMES = {"_n_ones", "EBITS_F32", "MBITS_F32", "F32_EXP_BIAS", "_f32_to_floatx_unpacked",
          "_floatx_unpacked_to_f32", "down_size", "pack_uint4"}


def _load():
    import torch.testing._internal as pkg
    src = (pathlib.Path(pkg.__file__).parent / "common_quantized.py").read_text()
    keep = []
    for node in ast.parse(src).body:
        if isinstance(node, ast.FunctionDef) and node.name in _NAMES:
            keep.append(node)
        elif isinstance(node, ast.Assign) and any(
                isinstance(t, ast.Name) and t.id in _NAMES for tt in node.targets
                for t in (tt.elts if isinstance(tt, ast.Tuple) else [tt])):
            keep.append(node)
    ns = {"torch": torch, "Tensor": torch.Tensor}
    exec(compile(ast.Module(body=keep, type_ignores=[]), "common_quantized.py", "exec"), ns)
    missing = _NAMES - set(ns)
    if missing:
        raise ImportError(f"torch's floatx helpers not found: {sorted(missing)}")
    return ns


_NS = _load()


def f32_to_e2m1(x):
    """float32 tensor -> E2M1 codes (uint8, low 4 bits), round to nearest even,
    values beyond 6 clamped to 6."""
    return _NS["_f32_to_floatx_unpacked"](x, 2, 1)


def e2m1_to_f32(codes):
    """E2M1 codes (uint8) -> float32 values."""
    return _NS["_floatx_unpacked_to_f32"](codes, 2, 1)


def pack_uint4(codes):
    """Pairs of 4-bit codes -> bytes as torch packs float4_e2m1fn_x2."""
    return _NS["pack_uint4"](codes)
