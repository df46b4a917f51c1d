"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function include/msa.h declares, and
reject bad arguments on the host before any launch.  Pointers passed here
are fake; every call below fails validation, so none reaches the device.
"""
import ctypes

import pytest

import block_sparse_long_index_amd as msa

lib = None


def setup_module(_):
    global lib
    lib = msa.load_library()


def _dims(**kw):
    base = dict(batch=1, num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128, top_k=16,
                total_q=32768, total_k=32768, max_q_len=32768, max_k_len=32768)
    base.update(kw)
    return msa.make_dims(**base)


def test_exports_every_declared_symbol():
    names = msa.exported_symbols()
    assert set(names) >= {"msa_index_select", "msa_build_block_query_lists", "msa_attend",
                          "msa_workspace_size", "msa_status_string", "msa_abi_version",
                          "msa_last_error"}
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_struct_layout():
    assert lib.msa_abi_version() == 3
    assert ctypes.sizeof(msa.Dims) == 80
    assert msa.Dims.block_table.offset == 64 and msa.Dims.flags.offset == 76


def test_status_strings():
    for s in range(7):
        assert lib.msa_status_string(s).decode().startswith("MSA_")


def test_workspace_sizes_scale_with_chunk():
    d = _dims()
    # prefill selects inside its scoring kernel: no block-score buffer
    assert msa.workspace_size(d, msa.OP_INDEX_SELECT) <= 4096
    # decode (<= 32 rows per sequence) keeps a block-score buffer per pass
    dec = _dims(batch=32, total_q=32, total_k=32 * 65536, max_q_len=1, max_k_len=65536)
    full = msa.workspace_size(dec, msa.OP_INDEX_SELECT)
    assert full >= 32 * 8 * 512 * 4
    dec2 = _dims(batch=32, total_q=32, total_k=32 * 65536, max_q_len=1, max_k_len=65536, q_chunk=8)
    assert msa.workspace_size(dec2, msa.OP_INDEX_SELECT) < full
    a_full = msa.workspace_size(_dims(), msa.OP_ATTEND)
    a_small = msa.workspace_size(_dims(q_chunk=256), msa.OP_ATTEND)
    assert a_small < a_full
    assert a_small >= 256 * 64 * 16 * (128 * 4 + 8)
    assert msa.workspace_size(d, msa.OP_BUILD_LISTS) >= 256 * 8 * 256 * 4


def test_1m_context_default_workspace_is_bounded():
    d = _dims(total_q=1 << 20, total_k=1 << 20, max_q_len=1 << 20, max_k_len=1 << 20)
    for op in (msa.OP_INDEX_SELECT, msa.OP_ATTEND):
        assert msa.workspace_size(d, op) <= (73 << 30)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 2), (dict(num_q_heads=60), 2), (dict(num_q_heads=48, num_kv_heads=8), 3),
    (dict(head_dim=96), 3), (dict(index_dim=48), 3), (dict(block_size=64), 3),
    (dict(top_k=0), 2), (dict(top_k=33), 2), (dict(softmax_scale=-1.0), 2),
    (dict(total_q=40000), 2), (dict(max_q_len=40000), 2), (dict(q_chunk=-1), 2),
    (dict(total_q=1 << 26, total_k=1 << 27, max_q_len=1, max_k_len=1), 3),
    (dict(total_k=1 << 22, max_k_len=1 << 22), 3),
    (dict(batch=65536, total_q=65536, total_k=1 << 20, max_q_len=1, max_k_len=16), 3),
    # a KV head count beyond a grid dimension's 65535
    (dict(num_q_heads=131072, num_kv_heads=65536), 3),
    # (sequence, group) pairs beyond what the list builder's grid holds
    (dict(batch=65535, num_q_heads=512, num_kv_heads=512, total_q=65535, total_k=1 << 20,
          max_q_len=1, max_k_len=16), 3),
])
def test_bad_dims_rejected(kw, status):
    d = _dims(**kw)
    n = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == status


def test_unknown_flag_bits_rejected():
    n = ctypes.c_size_t(0)
    for bits in (2, 4, 1 << 30, -1):
        d = _dims()
        d.flags = bits
        assert lib.msa_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == 2


def test_compact_partials_workspace_and_scope():
    """Compact partials take 2 * head_dim + 8 bytes per row on the lists path;
    decode-shaped steps keep fp32 partials; the block-mass call refuses them."""
    full = msa.workspace_size(_dims(q_chunk=256), msa.OP_ATTEND)
    comp = msa.workspace_size(_dims(q_chunk=256, flags=msa.FLAG_COMPACT_PARTIALS), msa.OP_ATTEND)
    rows = 256 * 64 * 16
    assert full >= rows * (128 * 4 + 8) and comp >= rows * (128 * 2 + 8)
    assert comp < full and comp <= rows * (128 * 2 + 8) + 4096
    # 72 GiB default cap: a compact pass holds nearly twice the rows
    p_full = msa.attend_pass_rows(_dims(total_q=1 << 20, total_k=1 << 20, max_q_len=1 << 20,
                                        max_k_len=1 << 20))
    p_comp = msa.attend_pass_rows(_dims(total_q=1 << 20, total_k=1 << 20, max_q_len=1 << 20,
                                        max_k_len=1 << 20, flags=msa.FLAG_COMPACT_PARTIALS))
    assert p_comp > 1.7 * p_full          # passes are rounded to equal sizes
    dec = dict(batch=32, total_q=32, total_k=32 * 65536, max_q_len=1, max_k_len=65536)
    assert msa.workspace_size(_dims(**dec), msa.OP_ATTEND) == \
        msa.workspace_size(_dims(**dec, flags=msa.FLAG_COMPACT_PARTIALS), msa.OP_ATTEND)
    d = _dims(flags=msa.FLAG_COMPACT_PARTIALS)
    st = lib.msa_attend_with_mass(ctypes.byref(d), *([None] * 12), ctypes.c_size_t(0), None)
    assert st == 3


def test_null_and_alignment_and_workspace_checks_launch_nothing():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    big = ctypes.c_size_t(1 << 40)
    sel = lib.msa_index_select
    assert sel(ctypes.byref(d), None, ok, ok, ok, ok, None, ok, big, None) == 1
    assert sel(ctypes.byref(d), odd, ok, ok, ok, ok, None, ok, big, None) == 4
    assert sel(ctypes.byref(d), ok, ok, ok, ok, ok, None, ok, ctypes.c_size_t(16), None) == 5
    assert "small" in lib.msa_last_error().decode()
    bl = lib.msa_build_block_query_lists
    assert bl(ctypes.byref(d), ok, ok, ok, None, ok, ok, big, None) == 1
    assert bl(ctypes.byref(d), ok, ok, ok, ok, odd, ok, big, None) == 4
    assert bl(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ctypes.c_size_t(0), None) == 5
    at = lib.msa_attend
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, None, None, ok, big, None) == 1
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, odd, ok, big, None) == 4
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, ctypes.c_size_t(1), None) == 5
    assert sel(None, ok, ok, ok, ok, ok, None, ok, big, None) == 1


def test_python_binding_rejects_cpu_tensors():
    import torch
    d = msa.make_dims(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, index_dim=32, top_k=4,
                      total_q=256, total_k=256, max_q_len=256, max_k_len=256)
    q_idx = torch.zeros((256, 1, 32), dtype=torch.bfloat16)
    k_idx = torch.zeros((256, 32), dtype=torch.bfloat16)
    cu = torch.tensor([0, 256], dtype=torch.int32)
    sel = torch.zeros((256, 1, 4), dtype=torch.int32)
    ws = torch.zeros(msa.workspace_size(d, msa.OP_INDEX_SELECT), dtype=torch.uint8)
    with pytest.raises(ValueError):
        msa.index_select(d, q_idx, k_idx, cu, cu, sel, workspace=ws, stream=object())


def test_product_path_does_not_import_oracle():
    import ast
    import glob
    import os
    pkg = os.path.dirname(msa.__file__)
    for f in glob.glob(os.path.join(pkg, "**", "*.py"), recursive=True):
        tree = ast.parse(open(f).read())
        for node in ast.walk(tree):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                assert not any(m.split(".")[0] == "oracle" for m in mods), f


def test_fp8_entry_points_validate_on_host():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    big = ctypes.c_size_t(1 << 40)
    qz = lib.msa_index_quantize_fp8
    # a side with an input needs its outputs
    assert qz(ctypes.byref(d), ok, None, None, None, ok, None, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, ok, None, None, ok, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, None, None, None, ok, ok, None) == 1
    assert qz(ctypes.byref(d), ok, ok, ok, odd, ok, ok, ok, None) == 4
    assert qz(ctypes.byref(d), None, ok, ok, None, None, odd, ok, None) == 4
    # exponent arrays are bytes: no alignment asked of them (fails later on NULL k_exp)
    assert qz(ctypes.byref(d), ok, ok, ok, ok, odd, ok, None, None) == 1
    s8 = lib.msa_index_select_fp8
    assert s8(ctypes.byref(d), ok, None, ok, ok, ok, ok, ok, None, ok, big, None) == 1
    assert s8(ctypes.byref(d), ok, ok, odd, ok, ok, ok, ok, None, ok, big, None) == 4
    assert s8(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, None, ok, ctypes.c_size_t(8), None) == 5
    # more key blocks per sequence than the kernels hold on chip
    long = _dims(total_q=1, total_k=16385 * 128, max_q_len=1, max_k_len=16385 * 128)
    assert s8(ctypes.byref(long), ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == 3
    # no queries and no keys: nothing to do, success without touching pointers
    empty = _dims(total_q=0, total_k=0, max_q_len=0, max_k_len=0)
    assert qz(ctypes.byref(empty), None, None, None, None, None, None, None, None) == 0
    # no inputs at all: nothing to quantise
    assert qz(ctypes.byref(d), None, None, None, None, None, None, None, None) == 0
    assert s8(ctypes.byref(empty), None, None, None, None, None, None, None, None, None, big, None) == 0


def test_q8k4_entry_points_validate_on_host():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    big = ctypes.c_size_t(1 << 40)
    qz = lib.msa_index_quantize_q8k4
    # a side with an input needs its outputs
    assert qz(ctypes.byref(d), ok, None, None, None, ok, None, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, ok, None, None, ok, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, None, None, None, ok, ok, None) == 1
    assert qz(ctypes.byref(d), ok, ok, ok, odd, ok, ok, None, None) == 1     # k_exp4 NULL
    assert qz(ctypes.byref(d), ok, ok, ok, odd, ok, ok, ok, None) == 4
    # key codes and their exponents are read in 16-byte pieces
    assert qz(ctypes.byref(d), None, odd, ok, None, None, ok, ok, None) == 4
    assert qz(ctypes.byref(d), None, ok, ok, None, None, odd, ok, None) == 4
    assert qz(ctypes.byref(d), None, ok, ok, None, None, ok, odd, None) == 4
    s4 = lib.msa_index_select_q8k4
    assert s4(ctypes.byref(d), ok, None, ok, ok, ok, ok, ok, None, ok, big, None) == 1
    assert s4(ctypes.byref(d), ok, ok, odd, ok, ok, ok, ok, None, ok, big, None) == 4
    assert s4(ctypes.byref(d), ok, ok, ok, odd, ok, ok, ok, None, ok, big, None) == 4
    assert s4(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, None, ok, ctypes.c_size_t(8), None) == 5
    empty = _dims(total_q=0, total_k=0, max_q_len=0, max_k_len=0)
    assert qz(ctypes.byref(empty), None, None, None, None, None, None, None, None) == 0
    assert qz(ctypes.byref(d), None, None, None, None, None, None, None, None) == 0
    assert s4(ctypes.byref(empty), None, None, None, None, None, None, None, None, None, big, None) == 0


def test_q8kv4_main_entry_points_validate_on_host():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    big = ctypes.c_size_t(1 << 40)
    qz = lib.msa_main_quantize_q8kv4
    # (dims, q, k, v, cu_k, q8, q_exp, k4, k_exp4, v4, v_exp4, stream)
    assert qz(ctypes.byref(d), ok, None, None, None, None, ok, None, None, None, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, None, ok, None, None, ok, None, None, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, None, None, None, None, ok, ok, None, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, None, ok, None, None, ok, odd, None, None, None) == 4
    assert qz(ctypes.byref(d), None, None, ok, ok, None, None, None, None, odd, ok, None) == 4
    assert qz(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, None) == 0
    at = lib.msa_attend_q8kv4
    # (dims, q8, q_exp, k4, k_exp4, v4, v_exp4, cu_q, cu_k, sel, offs, ents, out, lse, ws, bytes, stream)
    assert at(ctypes.byref(d), ok, ok, ok, None, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == 1
    assert at(ctypes.byref(d), ok, ok, ok, odd, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == 4
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok,
              ctypes.c_size_t(8), None) == 5


def test_projection_entry_point_validates_on_host():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    pj = lib.msa_index_project
    assert pj(ctypes.byref(d), 96, ok, ok, ok, ok, ok, ok, ok, None, 0, None) == 3   # not a multiple of 64
    assert pj(ctypes.byref(d), 0, ok, ok, ok, ok, ok, ok, ok, None, 0, None) == 3
    assert pj(ctypes.byref(d), 8192, None, ok, ok, ok, ok, ok, ok, None, 0, None) == 1
    assert pj(ctypes.byref(d), 8192, ok, ok, odd, ok, ok, ok, ok, None, 0, None) == 4
    empty = _dims(total_q=0, max_q_len=0)
    assert pj(ctypes.byref(empty), 8192, None, None, None, None, None, None, None, None, 0, None) == 0
    # steps of up to 512 tokens split the sum over model_dim: they need a workspace
    assert msa.workspace_size(d, msa.OP_INDEX_PROJECT) == 0
    for T in (1, 32, 100, 512):
        dd = _dims(batch=T, total_q=T, max_q_len=1, max_k_len=1024, total_k=T * 1024)
        need = msa.workspace_size(dd, msa.OP_INDEX_PROJECT)
        assert need == 32 * ((T + 31) // 32 * 32) * (9 * 128) * 4    # up to 32 fp32 slices
        assert pj(ctypes.byref(dd), 8192, ok, ok, ok, ok, ok, ok, ok, None, need, None) == 1
        assert pj(ctypes.byref(dd), 8192, ok, ok, ok, ok, ok, ok, ok, odd, need, None) == 4
        assert pj(ctypes.byref(dd), 8192, ok, ok, ok, ok, ok, ok, ok, ok, need - 1, None) == 5
    # larger steps: the large-tile kernel (512 tokens x 128 features per workgroup, one per CU)
    # splits K only while its tiles would leave half the 256 CUs idle, into 256 // tiles slices
    # (at most 16) of fp32 T x F tiles; the workspace is then optional
    F = 9 * 128
    for T, slices in ((513, 14), (2048, 7), (7168, 2), (7680, 0), (32768, 0)):
        tiles = 9 * ((T + 511) // 512)
        assert slices == (min(16, 256 // tiles) if 2 * tiles <= 256 else 0)
        dd = _dims(total_q=T, max_q_len=T, total_k=T, max_k_len=T)
        assert msa.workspace_size(dd, msa.OP_INDEX_PROJECT) == slices * T * F * 4
        # an optional workspace is still used, so it must be aligned too
        assert pj(ctypes.byref(dd), 8192, ok, ok, ok, ok, ok, ok, ok, odd, 1 << 30, None) == 4
    for T in range(513, 20000, 97):
        dd = _dims(total_q=T, max_q_len=T, total_k=T, max_k_len=T)
        assert msa.workspace_size(dd, msa.OP_INDEX_PROJECT) <= 64 << 20


def test_kl_entry_points_validate_on_host():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    big = ctypes.c_size_t(1 << 40)
    aw = lib.msa_attend_with_mass
    assert aw(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, None, None, ok, big, None) == 1
    assert aw(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, None, odd, ok, big, None) == 4
    assert aw(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, ok, ctypes.c_size_t(8), None) == 5
    kl = lib.msa_index_kl
    assert kl(ctypes.byref(d), ok, ok, ok, ok, ok, None, ok, None, ok, None) == 1
    assert kl(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, None, odd, None) == 4
    empty = _dims(total_q=0, max_q_len=0)
    assert kl(ctypes.byref(empty), None, None, None, None, None, None, None, None, None, None) == 0


def test_paged_cache_fields_validated():
    n = ctypes.c_size_t(0)
    ws = lib.msa_workspace_size
    d = _dims(total_k=32768)
    d.kv_pages = 256
    assert ws(ctypes.byref(d), 0, ctypes.byref(n)) == 1          # no block table
    d.block_table = 0x10000
    d.max_blocks_per_seq = 255                                   # below ceil(32768 / 128)
    assert ws(ctypes.byref(d), 0, ctypes.byref(n)) == 2
    d.max_blocks_per_seq = 256
    assert ws(ctypes.byref(d), 0, ctypes.byref(n)) == 0
    d.kv_pages = 300                                             # total_k != 128 * pages
    assert ws(ctypes.byref(d), 0, ctypes.byref(n)) == 2
    d.kv_pages = -1
    assert ws(ctypes.byref(d), 0, ctypes.byref(n)) == 2
    c = _dims()
    c.max_blocks_per_seq = 4                                     # table fields without pages
    assert ws(ctypes.byref(c), 0, ctypes.byref(n)) == 2



def test_attend_reads_lists_only_beyond_decode_shapes():
    P = ctypes.c_void_p
    ok = P(0x10000)
    big = ctypes.c_size_t(1 << 40)
    at = lib.msa_attend
    assert lib.msa_attend_reads_lists(ctypes.byref(_dims())) == 1
    assert not msa.attend_reads_lists(_dims(batch=32, total_q=32 * 8, max_q_len=8,
                                            total_k=32 * 4096, max_k_len=4096))
    assert msa.attend_reads_lists(_dims(batch=32, total_q=32 * 9, max_q_len=9,
                                        total_k=32 * 4096, max_k_len=4096))
    assert lib.msa_attend_reads_lists(ctypes.byref(_dims(top_k=0))) < 0
    # lists required where they are read, optional where they are not
    d = _dims()
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, None, ok, ok, None, ok, big, None) == 1
    dd = _dims(batch=32, total_q=32, max_q_len=1, total_k=32 * 4096, max_k_len=4096)
    assert at(ctypes.byref(dd), ok, ok, ok, ok, ok, ok, None, None, P(0x10004), None, ok, big, None) == 4


def test_fp8_main_entry_points_validate_on_host():
    d = _dims()
    P = ctypes.c_void_p
    ok = P(0x10000)
    odd = P(0x10004)
    big = ctypes.c_size_t(1 << 40)
    qz = lib.msa_main_quantize_fp8
    # q given without its outputs; k without cu_seqlens_k
    assert qz(ctypes.byref(d), ok, None, None, None, None, None, None, None, None, None, None) == 1
    assert qz(ctypes.byref(d), None, ok, None, None, None, None, ok, ok, None, None, None) == 1
    assert qz(ctypes.byref(d), None, None, ok, ok, None, None, None, None, odd, ok, None) == 4
    assert qz(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, None) == 0
    at = lib.msa_attend_fp8
    # exponents are required; lists as for msa_attend
    assert at(ctypes.byref(d), ok, None, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == 1
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, ok, None, ok, big, None) == 1
    assert at(ctypes.byref(d), odd, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == 4
    assert at(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, None, ok,
              ctypes.c_size_t(1), None) == 5
    empty = _dims(total_q=0, max_q_len=0)
    assert at(ctypes.byref(empty), None, None, None, None, None, None, None, None, None, None, None,
              None, None, None, 0, None) == 0


def test_prefill_index_kv_head_limit_rejected_on_host():
    """The prefill index kernels score all groups of a query in one workgroup
    (512 (query, group) rows for bf16 keys, 256 for 8-bit and 4-bit keys), so
    a larger KV head count on that path (max_q_len * num_kv_heads > 128,
    which every count above 128 is) is refused before any launch."""
    P = ctypes.c_void_p
    ok = P(0x10000)
    big = ctypes.c_size_t(1 << 40)
    sel, s8, s4 = lib.msa_index_select, lib.msa_index_select_fp8, lib.msa_index_select_q8k4

    def dims(G, q_len):
        return _dims(num_q_heads=G, num_kv_heads=G, total_q=q_len, max_q_len=q_len)

    for G, bf16_status, q8_status in ((1024, 3, 3), (512, None, 3)):
        d = dims(G, 256)
        if bf16_status is not None:
            assert sel(ctypes.byref(d), ok, ok, ok, ok, ok, None, ok, big, None) == bf16_status
            assert "512" in lib.msa_last_error().decode()
        assert s8(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == q8_status
        assert "256" in lib.msa_last_error().decode()
        assert s4(ctypes.byref(d), ok, ok, ok, ok, ok, ok, ok, None, ok, big, None) == q8_status
