"""Python binding of the MSA HIP library (libmsa.so).

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI of ``include/msa.h``.  PyTorch supplies device
memory and the current stream.  There is no fallback: if the library is
missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

__all__ = [
    "MSAError", "Dims", "OP_INDEX_SELECT", "OP_BUILD_LISTS", "OP_ATTEND", "OP_INDEX_PROJECT",
    "load_library",
    "make_dims", "workspace_size", "index_select", "build_block_query_lists", "attend",
    "msa_forward", "exported_symbols", "LIB_PATH", "HEADER_PATH", "index_quantize_fp8",
    "index_select_fp8", "Fp8Index", "index_project", "attend_with_mass", "index_kl",
    "attend_reads_lists", "Fp8Main", "main_quantize_fp8", "attend_fp8", "Q8K4Index",
    "index_quantize_q8k4", "index_select_q8k4", "Q8KV4Main", "main_quantize_q8kv4", "attend_q8kv4",
    "attend_noalloc", "NOALLOC_SCRATCH_BYTES", "attend_pass_rows", "FLAG_COMPACT_PARTIALS",
    "hbm_stream",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "msa.h")

OP_INDEX_SELECT, OP_BUILD_LISTS, OP_ATTEND, OP_INDEX_PROJECT = 0, 1, 2, 3
BLOCK = 128
FLAG_COMPACT_PARTIALS = 1          # MSA_FLAG_COMPACT_PARTIALS
NOALLOC_SCRATCH_BYTES = 64 << 20   # MSA_NOALLOC_SCRATCH_BYTES


class MSAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: status {status} ({_status_string(status)}) {detail}".strip())


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("max_q_len", ctypes.c_int32), ("max_k_len", ctypes.c_int32),
        ("q_chunk", ctypes.c_int32), ("kv_pages", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmsa.so once; raises OSError/RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"MSA HIP library not built: {path} (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(Dims)
    lib.msa_abi_version.restype = I32
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_status_string.argtypes = [I32]
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_workspace_size.restype = I32
    lib.msa_workspace_size.argtypes = [DP, I32, ctypes.POINTER(SZ)]
    lib.msa_index_select.restype = I32
    lib.msa_index_select.argtypes = [DP, P, P, P, P, P, P, P, SZ, P]
    lib.msa_attend_with_mass.restype = I32
    lib.msa_attend_with_mass.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_index_kl.restype = I32
    lib.msa_index_kl.argtypes = [DP, P, P, P, P, P, P, P, P, P, P]
    lib.msa_index_project.restype = I32
    lib.msa_index_project.argtypes = [DP, I32, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_index_quantize_fp8.restype = I32
    lib.msa_index_quantize_fp8.argtypes = [DP, P, P, P, P, P, P, P, P]
    lib.msa_index_select_fp8.restype = I32
    lib.msa_index_select_fp8.argtypes = [DP, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_index_quantize_q8k4.restype = I32
    lib.msa_index_quantize_q8k4.argtypes = [DP, P, P, P, P, P, P, P, P]
    lib.msa_index_select_q8k4.restype = I32
    lib.msa_index_select_q8k4.argtypes = [DP, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_build_block_query_lists.restype = I32
    lib.msa_build_block_query_lists.argtypes = [DP, P, P, P, P, P, P, SZ, P]
    lib.msa_attend.restype = I32
    lib.msa_attend.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_main_quantize_fp8.restype = I32
    lib.msa_main_quantize_fp8.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P]
    lib.msa_attend_fp8.restype = I32
    lib.msa_attend_fp8.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_main_quantize_q8kv4.restype = I32
    lib.msa_main_quantize_q8kv4.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P]
    lib.msa_attend_q8kv4.restype = I32
    lib.msa_attend_q8kv4.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_attend_noalloc.restype = I32
    lib.msa_attend_noalloc.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P]
    lib.msa_hbm_stream.restype = I32
    lib.msa_hbm_stream.argtypes = [P, SZ, I32, P, P, P]
    lib.msa_attend_pass_rows.restype = ctypes.c_int64
    lib.msa_attend_pass_rows.argtypes = [DP]
    lib.msa_attend_reads_lists.restype = I32
    lib.msa_attend_reads_lists.argtypes = [DP]
    lib.msa_profile_enable.restype = I32
    lib.msa_profile_enable.argtypes = [I32]
    lib.msa_profile_collect.restype = I32
    lib.msa_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I32)]
    lib.msa_profile_kernel_name.restype = ctypes.c_char_p
    lib.msa_profile_kernel_name.argtypes = [I32]
    _lib = lib
    return lib


def _status_string(s: int) -> str:
    try:
        return load_library().msa_status_string(int(s)).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(status: int, where: str):
    if status != 0:
        raise MSAError(status, where, load_library().msa_last_error().decode())


def exported_symbols(header: str = HEADER_PATH) -> list:
    """Function names declared in include/msa.h."""
    txt = open(header).read()
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", txt)))


def make_dims(*, batch, num_q_heads, num_kv_heads, head_dim, index_dim, top_k, total_q, total_k,
              max_q_len, max_k_len, softmax_scale=0.0, q_chunk=0, block_size=BLOCK,
              block_table=None, flags=0) -> Dims:
    """Problem sizes.  ``block_table`` (device int32 [batch, max_blocks_per_seq]) selects a
    paged key cache: ``total_k`` is then the cache's row count, 128 per page.  The
    returned dims keep a reference to the table (they hold its device address).
    ``flags``: 0 or FLAG_COMPACT_PARTIALS (the Main Branch's partials in 2 * head_dim + 8
    bytes instead of 4 * head_dim + 8 on prefill-shaped steps)."""
    pages, table, mbs = 0, None, 0
    if block_table is not None:
        _ptr(block_table, "block_table", torch.int32)
        if block_table.dim() != 2 or block_table.shape[0] != int(batch):
            raise ValueError("block_table must be [batch, max_blocks_per_seq]")
        pages, table, mbs = int(total_k) // BLOCK, block_table.data_ptr(), int(block_table.shape[1])
    d = Dims(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(index_dim),
             int(block_size), int(top_k), float(softmax_scale), int(total_q), int(total_k),
             int(max_q_len), int(max_k_len), int(q_chunk), pages, table, mbs, int(flags))
    # the struct holds the table's device address: keep the tensor alive with it
    d._block_table = block_table
    return d


def workspace_size(dims: Dims, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_workspace_size(ctypes.byref(dims), int(op), ctypes.byref(n)),
           "msa_workspace_size")
    return int(n.value)


def _ptr(t, name, dtype=None, device=True):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(dims, op, workspace, device, stream=None):
    """The caller's workspace, or a temporary one from torch's caching
    allocator.  A temporary is tied to the launch stream (record_stream), so
    the allocator does not hand it to other work before the library's
    kernels on that stream are done with it."""
    need = workspace_size(dims, op)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
    return workspace


def nb_max(dims: Dims) -> int:
    return (dims.max_k_len + BLOCK - 1) // BLOCK


def index_select(dims, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, sel, sel_score=None,
                 workspace=None, stream=None):
    G, T = dims.num_kv_heads, dims.total_q
    _shape(q_idx, (T, G, dims.index_dim), "q_idx")
    _shape(k_idx, (dims.total_k, dims.index_dim), "k_idx")
    _shape(sel, (T, G, dims.top_k), "sel")
    if sel_score is not None:
        _shape(sel_score, (T, G, dims.top_k), "sel_score")
    ws = _workspace(dims, OP_INDEX_SELECT, workspace, q_idx.device, stream)
    st = load_library().msa_index_select(
        ctypes.byref(dims), _ptr(q_idx, "q_idx", torch.bfloat16), _ptr(k_idx, "k_idx", torch.bfloat16),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(sel, "sel", torch.int32), _ptr(sel_score, "sel_score", torch.float32),
        _ptr(ws, "workspace"), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_index_select")
    return sel


def index_project(dims, x, w_q, w_k, cu_seqlens_q, cu_seqlens_k, q_idx, k_idx, workspace=None,
                  stream=None):
    """q_idx = x W_q^T, and the new tokens' rows of k_idx = x W_k^T (bf16)."""
    G, T, DI = dims.num_kv_heads, dims.total_q, dims.index_dim
    D = int(x.shape[1]) if x.dim() == 2 else -1
    _shape(x, (T, D), "x")
    _shape(w_q, (G * DI, D), "w_q")
    _shape(w_k, (DI, D), "w_k")
    _shape(q_idx, (T, G, DI), "q_idx")
    _shape(k_idx, (dims.total_k, DI), "k_idx")
    ws = _workspace(dims, OP_INDEX_PROJECT, workspace, q_idx.device, stream)
    st = load_library().msa_index_project(
        ctypes.byref(dims), D, _ptr(x, "x", torch.bfloat16), _ptr(w_q, "w_q", torch.bfloat16),
        _ptr(w_k, "w_k", torch.bfloat16), _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32), _ptr(q_idx, "q_idx", torch.bfloat16),
        _ptr(k_idx, "k_idx", torch.bfloat16), _ptr(ws, "workspace"), ws.numel(), _stream(stream))
    _check(st, "msa_index_project")
    return q_idx, k_idx


def _k_exp_shape(dims):
    """Per-block exponents of the quantised index keys: [batch, nb_max], or one per page."""
    return (dims.kv_pages,) if dims.kv_pages else (dims.batch, nb_max(dims))


class Fp8Index:
    """E4M3 codes and E8M0 exponents of the index projections for fixed dims."""

    def __init__(self, dims: Dims, device):
        T, G, DI = dims.total_q, dims.num_kv_heads, dims.index_dim
        dev = torch.device(device)
        self.q_idx8 = torch.empty((T, G, DI), dtype=torch.uint8, device=dev)
        self.q_exp = torch.empty((T, G), dtype=torch.uint8, device=dev)
        self.k_idx8 = torch.empty((dims.total_k, DI), dtype=torch.uint8, device=dev)
        self.k_exp = torch.empty(_k_exp_shape(dims), dtype=torch.uint8, device=dev)


def index_quantize_fp8(dims, q_idx, k_idx, cu_seqlens_k, fp8: Fp8Index, stream=None):
    """bf16 index projections -> E4M3 codes with power-of-two scales (into `fp8`).

    Either q_idx or k_idx may be None: that side is left as it is in `fp8`.
    """
    G, T, DI = dims.num_kv_heads, dims.total_q, dims.index_dim
    if q_idx is not None:
        _shape(q_idx, (T, G, DI), "q_idx")
    if k_idx is not None:
        _shape(k_idx, (dims.total_k, DI), "k_idx")
    _shape(fp8.q_idx8, (T, G, DI), "q_idx8")
    _shape(fp8.q_exp, (T, G), "q_exp")
    _shape(fp8.k_idx8, (dims.total_k, DI), "k_idx8")
    _shape(fp8.k_exp, _k_exp_shape(dims), "k_exp")
    st = load_library().msa_index_quantize_fp8(
        ctypes.byref(dims), _ptr(q_idx, "q_idx", torch.bfloat16), _ptr(k_idx, "k_idx", torch.bfloat16),
        _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32), _ptr(fp8.q_idx8, "q_idx8", torch.uint8),
        _ptr(fp8.q_exp, "q_exp", torch.uint8), _ptr(fp8.k_idx8, "k_idx8", torch.uint8),
        _ptr(fp8.k_exp, "k_exp", torch.uint8), _stream(stream))
    _check(st, "msa_index_quantize_fp8")
    return fp8


def _kv_exp_shape(dims):
    """Per-block exponents of quantised keys/values: [batch, nb_max, G], or [pages, G]."""
    G = dims.num_kv_heads
    return (dims.kv_pages, G) if dims.kv_pages else (dims.batch, nb_max(dims), G)


class Fp8Main:
    """E4M3 codes and E8M0 exponents of the Main Branch's q, k and v for fixed dims."""

    def __init__(self, dims: Dims, device):
        T, Hq, G, D = dims.total_q, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
        dev = torch.device(device)
        self.q8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=dev)
        self.q_exp = torch.empty((T, Hq), dtype=torch.uint8, device=dev)
        self.k8 = torch.empty((dims.total_k, G, D), dtype=torch.uint8, device=dev)
        self.v8 = torch.empty((dims.total_k, G, D), dtype=torch.uint8, device=dev)
        self.k_exp = torch.empty(_kv_exp_shape(dims), dtype=torch.uint8, device=dev)
        self.v_exp = torch.empty(_kv_exp_shape(dims), dtype=torch.uint8, device=dev)


def _check_fp8_main(dims, f8):
    T, Hq, G, D = dims.total_q, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
    _shape(f8.q8, (T, Hq, D), "q8")
    _shape(f8.q_exp, (T, Hq), "q_exp")
    _shape(f8.k8, (dims.total_k, G, D), "k8")
    _shape(f8.v8, (dims.total_k, G, D), "v8")
    _shape(f8.k_exp, _kv_exp_shape(dims), "k_exp")
    _shape(f8.v_exp, _kv_exp_shape(dims), "v_exp")


def main_quantize_fp8(dims, q, k, v, cu_seqlens_k, f8: Fp8Main, stream=None):
    """bf16 q / k / v -> E4M3 codes with power-of-two scales (into `f8`).

    Any of q, k, v may be None: that part of `f8` is left as it is.
    """
    T, Hq, G, D = dims.total_q, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
    if q is not None:
        _shape(q, (T, Hq, D), "q")
    for name, x in (("k", k), ("v", v)):
        if x is not None:
            _shape(x, (dims.total_k, G, D), name)
    _check_fp8_main(dims, f8)
    st = load_library().msa_main_quantize_fp8(
        ctypes.byref(dims), _ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
        _ptr(v, "v", torch.bfloat16), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(f8.q8, "q8", torch.uint8), _ptr(f8.q_exp, "q_exp", torch.uint8),
        _ptr(f8.k8, "k8", torch.uint8), _ptr(f8.k_exp, "k_exp", torch.uint8),
        _ptr(f8.v8, "v8", torch.uint8), _ptr(f8.v_exp, "v_exp", torch.uint8), _stream(stream))
    _check(st, "msa_main_quantize_fp8")
    return f8


def attend_fp8(dims, f8: Fp8Main, cu_seqlens_q, cu_seqlens_k, sel, block_offsets, block_entries, out,
               lse=None, workspace=None, stream=None):
    """The Main Branch on quantised q, k, v (msa_attend_fp8)."""
    T, Hq, D = dims.total_q, dims.num_q_heads, dims.head_dim
    _check_fp8_main(dims, f8)
    _shape(out, (T, Hq, D), "out")
    if lse is not None:
        _shape(lse, (T, Hq), "lse")
    ws = _workspace(dims, OP_ATTEND, workspace, out.device, stream)
    st = load_library().msa_attend_fp8(
        ctypes.byref(dims), _ptr(f8.q8, "q8", torch.uint8), _ptr(f8.q_exp, "q_exp", torch.uint8),
        _ptr(f8.k8, "k8", torch.uint8), _ptr(f8.k_exp, "k_exp", torch.uint8),
        _ptr(f8.v8, "v8", torch.uint8), _ptr(f8.v_exp, "v_exp", torch.uint8),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(sel, "sel", torch.int32), _ptr(block_offsets, "block_offsets", torch.int32),
        _ptr(block_entries, "block_entries", torch.int32), _ptr(out, "out", torch.bfloat16),
        _ptr(lse, "lse", torch.float32), _ptr(ws, "workspace"),
        ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_attend_fp8")
    return out


class Q8KV4Main:
    """The Main Branch's 8-bit q codes and 4-bit k, v codes for fixed dims:
    E4M3 q with one E8M0 exponent per (row, head); E2M1 k and v packed two per
    byte with one E8M0 exponent per 32 elements of every (key, KV head) row."""

    def __init__(self, dims: Dims, device):
        T, Hq, G, D = dims.total_q, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
        dev = torch.device(device)
        self.q8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=dev)
        self.q_exp = torch.empty((T, Hq), dtype=torch.uint8, device=dev)
        self.k4 = torch.empty((dims.total_k, G, D // 2), dtype=torch.uint8, device=dev)
        self.v4 = torch.empty((dims.total_k, G, D // 2), dtype=torch.uint8, device=dev)
        self.k_exp4 = torch.empty((dims.total_k, G, D // 32), dtype=torch.uint8, device=dev)
        self.v_exp4 = torch.empty((dims.total_k, G, D // 32), dtype=torch.uint8, device=dev)


def _check_q8kv4(dims, m: Q8KV4Main):
    T, Hq, G, D = dims.total_q, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
    _shape(m.q8, (T, Hq, D), "q8")
    _shape(m.q_exp, (T, Hq), "q_exp")
    for name in ("k4", "v4"):
        _shape(getattr(m, name), (dims.total_k, G, D // 2), name)
    for name in ("k_exp4", "v_exp4"):
        _shape(getattr(m, name), (dims.total_k, G, D // 32), name)


def main_quantize_q8kv4(dims, q, k, v, cu_seqlens_k, m: Q8KV4Main, stream=None):
    """bf16 q / k / v -> 8-bit q codes and 4-bit k, v codes (into `m`).

    Any of q, k, v may be None: that part of `m` is left as it is.
    """
    T, Hq, G, D = dims.total_q, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
    if q is not None:
        _shape(q, (T, Hq, D), "q")
    for name, x in (("k", k), ("v", v)):
        if x is not None:
            _shape(x, (dims.total_k, G, D), name)
    _check_q8kv4(dims, m)
    st = load_library().msa_main_quantize_q8kv4(
        ctypes.byref(dims), _ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
        _ptr(v, "v", torch.bfloat16), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(m.q8, "q8", torch.uint8), _ptr(m.q_exp, "q_exp", torch.uint8),
        _ptr(m.k4, "k4", torch.uint8), _ptr(m.k_exp4, "k_exp4", torch.uint8),
        _ptr(m.v4, "v4", torch.uint8), _ptr(m.v_exp4, "v_exp4", torch.uint8), _stream(stream))
    _check(st, "msa_main_quantize_q8kv4")
    return m


def attend_q8kv4(dims, m: Q8KV4Main, cu_seqlens_q, cu_seqlens_k, sel, block_offsets, block_entries,
                 out, lse=None, workspace=None, stream=None):
    """The Main Branch on 8-bit q and 4-bit k, v (msa_attend_q8kv4)."""
    T, Hq, D = dims.total_q, dims.num_q_heads, dims.head_dim
    _check_q8kv4(dims, m)
    _shape(out, (T, Hq, D), "out")
    if lse is not None:
        _shape(lse, (T, Hq), "lse")
    ws = _workspace(dims, OP_ATTEND, workspace, out.device, stream)
    st = load_library().msa_attend_q8kv4(
        ctypes.byref(dims), _ptr(m.q8, "q8", torch.uint8), _ptr(m.q_exp, "q_exp", torch.uint8),
        _ptr(m.k4, "k4", torch.uint8), _ptr(m.k_exp4, "k_exp4", torch.uint8),
        _ptr(m.v4, "v4", torch.uint8), _ptr(m.v_exp4, "v_exp4", torch.uint8),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(sel, "sel", torch.int32), _ptr(block_offsets, "block_offsets", torch.int32),
        _ptr(block_entries, "block_entries", torch.int32), _ptr(out, "out", torch.bfloat16),
        _ptr(lse, "lse", torch.float32), _ptr(ws, "workspace"),
        ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_attend_q8kv4")
    return out


class Q8K4Index:
    """8-bit index-query codes and 4-bit index-key codes for fixed dims: E4M3
    queries with one E8M0 exponent per (row, group); E2M1 keys packed two per
    byte with one E8M0 exponent per 32 elements of a key row."""

    def __init__(self, dims: Dims, device):
        T, G, DI = dims.total_q, dims.num_kv_heads, dims.index_dim
        dev = torch.device(device)
        self.q_idx8 = torch.empty((T, G, DI), dtype=torch.uint8, device=dev)
        self.q_exp = torch.empty((T, G), dtype=torch.uint8, device=dev)
        self.k_idx4 = torch.empty((dims.total_k, DI // 2), dtype=torch.uint8, device=dev)
        self.k_exp4 = torch.empty((dims.total_k, DI // 32), dtype=torch.uint8, device=dev)


def _check_q8k4(dims, qk: Q8K4Index):
    G, T, DI = dims.num_kv_heads, dims.total_q, dims.index_dim
    _shape(qk.q_idx8, (T, G, DI), "q_idx8")
    _shape(qk.q_exp, (T, G), "q_exp")
    _shape(qk.k_idx4, (dims.total_k, DI // 2), "k_idx4")
    _shape(qk.k_exp4, (dims.total_k, DI // 32), "k_exp4")


def index_quantize_q8k4(dims, q_idx, k_idx, cu_seqlens_k, qk: Q8K4Index, stream=None):
    """bf16 index projections -> 8-bit query codes and 4-bit key codes (into `qk`).

    Either q_idx or k_idx may be None: that side is left as it is in `qk`.
    """
    G, T, DI = dims.num_kv_heads, dims.total_q, dims.index_dim
    if q_idx is not None:
        _shape(q_idx, (T, G, DI), "q_idx")
    if k_idx is not None:
        _shape(k_idx, (dims.total_k, DI), "k_idx")
    _check_q8k4(dims, qk)
    st = load_library().msa_index_quantize_q8k4(
        ctypes.byref(dims), _ptr(q_idx, "q_idx", torch.bfloat16), _ptr(k_idx, "k_idx", torch.bfloat16),
        _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32), _ptr(qk.q_idx8, "q_idx8", torch.uint8),
        _ptr(qk.q_exp, "q_exp", torch.uint8), _ptr(qk.k_idx4, "k_idx4", torch.uint8),
        _ptr(qk.k_exp4, "k_exp4", torch.uint8), _stream(stream))
    _check(st, "msa_index_quantize_q8k4")
    return qk


def index_select_q8k4(dims, qk: Q8K4Index, cu_seqlens_q, cu_seqlens_k, sel, sel_score=None,
                      workspace=None, stream=None):
    """Index Branch on 8-bit queries and 4-bit keys (see msa_index_select_q8k4)."""
    G, T = dims.num_kv_heads, dims.total_q
    _check_q8k4(dims, qk)
    _shape(sel, (T, G, dims.top_k), "sel")
    if sel_score is not None:
        _shape(sel_score, (T, G, dims.top_k), "sel_score")
    ws = _workspace(dims, OP_INDEX_SELECT, workspace, sel.device, stream)
    st = load_library().msa_index_select_q8k4(
        ctypes.byref(dims), _ptr(qk.q_idx8, "q_idx8", torch.uint8), _ptr(qk.q_exp, "q_exp", torch.uint8),
        _ptr(qk.k_idx4, "k_idx4", torch.uint8), _ptr(qk.k_exp4, "k_exp4", torch.uint8),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(sel, "sel", torch.int32), _ptr(sel_score, "sel_score", torch.float32),
        _ptr(ws, "workspace"), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_index_select_q8k4")
    return sel


def index_select_fp8(dims, fp8: Fp8Index, cu_seqlens_q, cu_seqlens_k, sel, sel_score=None,
                     workspace=None, stream=None):
    """Index Branch on the quantised projections (see msa_index_select_fp8)."""
    G, T = dims.num_kv_heads, dims.total_q
    _shape(fp8.q_idx8, (T, G, dims.index_dim), "q_idx8")
    _shape(fp8.k_idx8, (dims.total_k, dims.index_dim), "k_idx8")
    _shape(fp8.q_exp, (T, G), "q_exp")
    _shape(fp8.k_exp, _k_exp_shape(dims), "k_exp")
    _shape(sel, (T, G, dims.top_k), "sel")
    if sel_score is not None:
        _shape(sel_score, (T, G, dims.top_k), "sel_score")
    ws = _workspace(dims, OP_INDEX_SELECT, workspace, sel.device, stream)
    st = load_library().msa_index_select_fp8(
        ctypes.byref(dims), _ptr(fp8.q_idx8, "q_idx8", torch.uint8), _ptr(fp8.q_exp, "q_exp", torch.uint8),
        _ptr(fp8.k_idx8, "k_idx8", torch.uint8), _ptr(fp8.k_exp, "k_exp", torch.uint8),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(sel, "sel", torch.int32), _ptr(sel_score, "sel_score", torch.float32),
        _ptr(ws, "workspace"), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_index_select_fp8")
    return sel


def build_block_query_lists(dims, sel, cu_seqlens_q, cu_seqlens_k, block_offsets, block_entries,
                            workspace=None, stream=None):
    U = dims.batch * dims.num_kv_heads * nb_max(dims)
    _shape(block_offsets, (U + 1,), "block_offsets")
    if block_entries.numel() < dims.total_q * dims.num_kv_heads * dims.top_k:
        raise ValueError("block_entries too small")
    ws = _workspace(dims, OP_BUILD_LISTS, workspace, sel.device, stream)
    st = load_library().msa_build_block_query_lists(
        ctypes.byref(dims), _ptr(sel, "sel", torch.int32),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(block_offsets, "block_offsets", torch.int32), _ptr(block_entries, "block_entries", torch.int32),
        _ptr(ws, "workspace"), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_build_block_query_lists")
    return block_offsets, block_entries


def attend(dims, q, k, v, cu_seqlens_q, cu_seqlens_k, sel, block_offsets, block_entries, out,
           lse=None, workspace=None, stream=None):
    T, Hq, D, G = dims.total_q, dims.num_q_heads, dims.head_dim, dims.num_kv_heads
    _shape(q, (T, Hq, D), "q")
    _shape(k, (dims.total_k, G, D), "k")
    _shape(v, (dims.total_k, G, D), "v")
    _shape(out, (T, Hq, D), "out")
    if lse is not None:
        _shape(lse, (T, Hq), "lse")
    ws = _workspace(dims, OP_ATTEND, workspace, q.device, stream)
    st = load_library().msa_attend(
        ctypes.byref(dims), _ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
        _ptr(v, "v", torch.bfloat16), _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32), _ptr(sel, "sel", torch.int32),
        _ptr(block_offsets, "block_offsets", torch.int32), _ptr(block_entries, "block_entries", torch.int32),
        _ptr(out, "out", torch.bfloat16), _ptr(lse, "lse", torch.float32), _ptr(ws, "workspace"),
        ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_attend")
    return out


def attend_noalloc(dims, q, k, v, cu_seqlens_q, cu_seqlens_k, sel, block_offsets, block_entries, out,
                   lse=None, stream=None):
    """msa_attend_noalloc: msa_attend with its partials in the library's own
    per-GPU scratch; no workspace is allocated or passed."""
    T, Hq, D, G = dims.total_q, dims.num_q_heads, dims.head_dim, dims.num_kv_heads
    _shape(q, (T, Hq, D), "q")
    _shape(k, (dims.total_k, G, D), "k")
    _shape(v, (dims.total_k, G, D), "v")
    _shape(out, (T, Hq, D), "out")
    if lse is not None:
        _shape(lse, (T, Hq), "lse")
    st = load_library().msa_attend_noalloc(
        ctypes.byref(dims), _ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
        _ptr(v, "v", torch.bfloat16), _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32), _ptr(sel, "sel", torch.int32),
        _ptr(block_offsets, "block_offsets", torch.int32), _ptr(block_entries, "block_entries", torch.int32),
        _ptr(out, "out", torch.bfloat16), _ptr(lse, "lse", torch.float32), _stream(stream))
    _check(st, "msa_attend_noalloc")
    return out


def attend_with_mass(dims, q, k, v, cu_seqlens_q, cu_seqlens_k, sel, block_offsets, block_entries,
                     out, block_mass, lse=None, workspace=None, stream=None):
    """msa_attend plus the Main Branch's attention mass per selected block
    (averaged over the group's heads) into block_mass [T, G, top_k] fp32."""
    T, Hq, D, G = dims.total_q, dims.num_q_heads, dims.head_dim, dims.num_kv_heads
    _shape(q, (T, Hq, D), "q")
    _shape(k, (dims.total_k, G, D), "k")
    _shape(v, (dims.total_k, G, D), "v")
    _shape(out, (T, Hq, D), "out")
    _shape(block_mass, (T, G, dims.top_k), "block_mass")
    if lse is not None:
        _shape(lse, (T, Hq), "lse")
    ws = _workspace(dims, OP_ATTEND, workspace, q.device, stream)
    st = load_library().msa_attend_with_mass(
        ctypes.byref(dims), _ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
        _ptr(v, "v", torch.bfloat16), _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32), _ptr(sel, "sel", torch.int32),
        _ptr(block_offsets, "block_offsets", torch.int32), _ptr(block_entries, "block_entries", torch.int32),
        _ptr(out, "out", torch.bfloat16), _ptr(lse, "lse", torch.float32),
        _ptr(block_mass, "block_mass", torch.float32), _ptr(ws, "workspace"),
        ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream))
    _check(st, "msa_attend_with_mass")
    return out, block_mass


def index_kl(dims, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, sel, sel_score, block_mass, kl,
             log_q=None, stream=None):
    """KL(P || Q) per (query, group) of the Main-Branch masses P and the index
    distribution Q over the selection; log Q optionally."""
    T, G, k = dims.total_q, dims.num_kv_heads, dims.top_k
    _shape(q_idx, (T, G, dims.index_dim), "q_idx")
    _shape(k_idx, (dims.total_k, dims.index_dim), "k_idx")
    for t_, n_ in ((sel, "sel"), (sel_score, "sel_score"), (block_mass, "block_mass")):
        _shape(t_, (T, G, k), n_)
    _shape(kl, (T, G), "kl")
    if log_q is not None:
        _shape(log_q, (T, G, k), "log_q")
    st = load_library().msa_index_kl(
        ctypes.byref(dims), _ptr(q_idx, "q_idx", torch.bfloat16), _ptr(k_idx, "k_idx", torch.bfloat16),
        _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32), _ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _ptr(sel, "sel", torch.int32), _ptr(sel_score, "sel_score", torch.float32),
        _ptr(block_mass, "block_mass", torch.float32), _ptr(log_q, "log_q", torch.float32),
        _ptr(kl, "kl", torch.float32), _stream(stream))
    _check(st, "msa_index_kl")
    return kl


class Buffers:
    """Output and workspace buffers of one MSA forward for fixed dims."""

    def __init__(self, dims: Dims, device, want_scores=False, want_lse=True):
        T, G, k = dims.total_q, dims.num_kv_heads, dims.top_k
        dev = torch.device(device)
        self.sel = torch.empty((T, G, k), dtype=torch.int32, device=dev)
        self.sel_score = torch.empty((T, G, k), dtype=torch.float32, device=dev) if want_scores else None
        U = dims.batch * G * nb_max(dims)
        self.offsets = torch.empty((U + 1,), dtype=torch.int32, device=dev)
        self.entries = torch.empty((max(1, T * G * k),), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, dims.num_q_heads, dims.head_dim), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=dev) if want_lse else None
        need = max(workspace_size(dims, op)
                   for op in (OP_INDEX_SELECT, OP_BUILD_LISTS, OP_ATTEND, OP_INDEX_PROJECT))
        self.workspace = torch.empty((need,), dtype=torch.uint8, device=dev)


def attend_pass_rows(dims: Dims) -> int:
    """Query rows per internal pass of msa_attend for these dims."""
    n = int(load_library().msa_attend_pass_rows(ctypes.byref(dims)))
    if n < 0:
        _check(-n, "msa_attend_pass_rows")
    return n


def attend_reads_lists(dims: Dims) -> bool:
    """Whether attend reads the per-block query lists for these dims (False for
    decode-shaped steps, which attend per (query, slot) from the selection)."""
    r = int(load_library().msa_attend_reads_lists(ctypes.byref(dims)))
    if r < 0:
        _check(-r, "msa_attend_reads_lists")
    return r == 1


def msa_forward(dims: Dims, q, k, v, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, bufs: Buffers = None,
                stream=None, fp8: Fp8Index = None, fp8_main: Fp8Main = None,
                q8k4: Q8K4Index = None) -> Buffers:
    """The whole hot path: index_select -> build_block_query_lists -> attend.

    One workspace serves the three calls (they run in order on one stream).
    Decode-shaped steps skip the lists, which their attend does not read.
    With `fp8` given, the Index Branch quantises q_idx and k_idx into it and
    selects on the codes (index_quantize_fp8 -> index_select_fp8); k_idx=None
    keeps the key codes already in `fp8` (a quantised index-key cache).
    With `q8k4` given instead, the same with 4-bit index keys
    (index_quantize_q8k4 -> index_select_q8k4).
    With `fp8_main` given (Fp8Main: 8-bit q, k, v; Q8KV4Main: 8-bit q, 4-bit
    k, v), the Main Branch quantises q (and k, v unless they are
    None: a quantised key/value cache already in `fp8_main`) and attends on the
    codes (main_quantize_fp8 -> attend_fp8).
    """
    bufs = bufs or Buffers(dims, q.device)
    if fp8 is not None and q8k4 is not None:
        raise ValueError("pass at most one of fp8 and q8k4")
    if q8k4 is not None:
        index_quantize_q8k4(dims, q_idx, k_idx, cu_seqlens_k, q8k4, stream)
        index_select_q8k4(dims, q8k4, cu_seqlens_q, cu_seqlens_k, bufs.sel, bufs.sel_score,
                          bufs.workspace, stream)
    elif fp8 is None:
        index_select(dims, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, bufs.sel, bufs.sel_score,
                     bufs.workspace, stream)
    else:
        index_quantize_fp8(dims, q_idx, k_idx, cu_seqlens_k, fp8, stream)
        index_select_fp8(dims, fp8, cu_seqlens_q, cu_seqlens_k, bufs.sel, bufs.sel_score,
                         bufs.workspace, stream)
    if attend_reads_lists(dims):
        build_block_query_lists(dims, bufs.sel, cu_seqlens_q, cu_seqlens_k, bufs.offsets,
                                bufs.entries, bufs.workspace, stream)
    if fp8_main is None:
        attend(dims, q, k, v, cu_seqlens_q, cu_seqlens_k, bufs.sel, bufs.offsets, bufs.entries,
               bufs.out, bufs.lse, bufs.workspace, stream)
    elif isinstance(fp8_main, Q8KV4Main):
        main_quantize_q8kv4(dims, q, k, v, cu_seqlens_k, fp8_main, stream)
        attend_q8kv4(dims, fp8_main, cu_seqlens_q, cu_seqlens_k, bufs.sel, bufs.offsets, bufs.entries,
                     bufs.out, bufs.lse, bufs.workspace, stream)
    else:
        main_quantize_fp8(dims, q, k, v, cu_seqlens_k, fp8_main, stream)
        attend_fp8(dims, fp8_main, cu_seqlens_q, cu_seqlens_k, bufs.sel, bufs.offsets, bufs.entries,
                   bufs.out, bufs.lse, bufs.workspace, stream)
    return bufs


def hbm_stream(src, ratio, dst, sink, stream=None):
    """Measuring aid (msa_hbm_stream): stream all of `src` (uint8, a multiple of 16
    bytes) and write ratio * its size into `dst`; `sink`: >= 8 KiB scratch."""
    nbytes = src.numel() * src.element_size()
    if ratio > 0 and dst.numel() * dst.element_size() < ratio * nbytes:
        raise ValueError("dst too small")
    if sink.numel() * sink.element_size() < 4 * 2048:
        raise ValueError("sink too small")
    _check(load_library().msa_hbm_stream(_ptr(src, "src"), ctypes.c_size_t(nbytes), int(ratio),
                                         _ptr(dst, "dst") if ratio > 0 else None, _ptr(sink, "sink"),
                                         _stream(stream)), "msa_hbm_stream")


PROFILE_KERNELS = 17


def profile_enable(on: bool = True):
    """Bracket every kernel stage with hipEvents on its launch stream."""
    _check(load_library().msa_profile_enable(1 if on else 0), "msa_profile_enable")


def profile_collect() -> dict:
    """{stage name: (total ms, launches)} of the stages recorded since the last
    collect; waits for the recorded events."""
    lib = load_library()
    ms = (ctypes.c_float * PROFILE_KERNELS)()
    n = (ctypes.c_int32 * PROFILE_KERNELS)()
    _check(lib.msa_profile_collect(ms, n), "msa_profile_collect")
    return {lib.msa_profile_kernel_name(i).decode(): (float(ms[i]), int(n[i]))
            for i in range(PROFILE_KERNELS)}


def dims_for(workload_like, q_chunk=0, softmax_scale=0.0, flags=0) -> Dims:
    """Dims of a problem described by per-sequence lengths and head sizes."""
    w = workload_like
    return make_dims(batch=len(w.seq_k_lens), num_q_heads=w.num_q_heads,
                     num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, index_dim=w.index_dim,
                     top_k=w.top_k, total_q=sum(w.seq_q_lens), total_k=sum(w.seq_k_lens),
                     max_q_len=max(w.seq_q_lens), max_k_len=max(w.seq_k_lens),
                     softmax_scale=softmax_scale, q_chunk=q_chunk, flags=flags)
