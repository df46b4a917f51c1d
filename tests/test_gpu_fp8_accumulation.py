"""The 8-bit matrix cores' summation, observed through the public ABI.

msa_index_select_fp8 / _q8k4 report each selected block's score.  With
neutral exponents (2^0) and a key block in which one token carries the
products (the others are zero), that score is the matrix instruction's sum
of that token's dot product, in fp32.  The selection tests accept a GPU
selection that differs from the oracle's only within 2^-10 * sum |q_c k_c|
of the exact scores; this file pins the summation model behind that bound:
products are summed in groups of 8 consecutive elements, each group in
fixed point aligned to its largest product with 13 bits kept below that
product's leading bit (the rest dropped), and the groups are added in fp32;
products of subnormal E4M3 inputs are exact.  So each group loses less than
7 * 2^-13 of its largest product, below 2^-10 * sum |q_c k_c|.

Every case is a sequence of 256 tokens whose block-1 queries all carry the
case's query codes; block 0's token 0 carries the key codes.  The prefill
kernels score it (all 256 queries of a sequence: more than 128 rows), and so
does the decode kernel (one query at position 255).
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from oracle import fp4_index as F4
from oracle import fp8_index as F8

pytestmark = pytest.mark.gpu

from gpu_helpers import log  # noqa: E402

DI = 128
E4M3 = {448.0: 0x7E, 1.0: 0x38, 1.5 * 2 ** -5: 0x14, 2.0 ** -6: 0x08, 2.0 ** -9: 0x01}
E2M1 = {1.0: 0x2, 6.0: 0x7}

# (name, {element: query value}, {element: key value} (default 1.0), expected sum)
CASES = [
    ("last_bit_dropped", {0: 448.0, 1: 1.5 * 2 ** -5}, {}, 448.0 + 2 ** -5),
    ("below_13_bits_vanishes", {0: 448.0, 1: 2.0 ** -6}, {}, 448.0),
    ("next_group_exact", {0: 448.0, 8: 2.0 ** -6}, {}, 448.0 + 2 ** -6),
    ("subnormals_exact", {c: 2.0 ** -9 for c in range(8)}, {}, 8 * 2.0 ** -9),
]
CASES_FP8 = CASES + [
    ("large_product_swallows_group", {0: 448.0, **{c: 2.0 ** -9 for c in range(1, 8)}},
     {0: 448.0}, 448.0 * 448.0),
]
CASES_K4 = CASES + [
    ("large_product_swallows_group", {0: 448.0, **{c: 2.0 ** -9 for c in range(1, 8)}},
     {0: 6.0}, 448.0 * 6.0),
]


def _setup(cases, decode, k4, rng_cases=0, seed=0):
    """Codes for the cases (plus rng_cases random positive-code rows)."""
    n = len(cases) + rng_cases
    L = 256
    lq = 1 if decode else L
    dims = msa.make_dims(batch=n, num_q_heads=1, num_kv_heads=1, head_dim=64, index_dim=DI, top_k=2,
                         total_q=n * lq, total_k=n * L, max_q_len=lq, max_k_len=L)
    dev = torch.device("cuda:0")
    qc = np.zeros((n, DI), np.uint8)
    kv = np.zeros((n, DI))            # key values of token 0 of each sequence
    qv = np.zeros((n, DI))
    rng = np.random.default_rng(seed)
    for i in range(n):
        if i < len(cases):
            _, qd, kd, _ = cases[i]
            for c, x in qd.items():
                qc[i, c] = E4M3[x]
                qv[i, c] = x
            for c in range(DI):
                kv[i, c] = kd.get(c, 1.0)
        else:
            # positive codes of every magnitude (no NaN), random key values on the grid
            qc[i] = rng.integers(0x01, 0x7F, size=DI)
            qv[i] = F8.e4m3_table()[qc[i]]
            kv[i] = (rng.choice([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], size=DI) if k4 else
                     F8.e4m3_table()[rng.integers(0x01, 0x7F, size=DI)])
    cuq = torch.arange(0, n * lq + 1, lq, dtype=torch.int32, device=dev)
    cuk = torch.arange(0, n * L + 1, L, dtype=torch.int32, device=dev)
    q_rows = np.zeros((n * lq, 1, DI), np.uint8)
    for i in range(n):
        first = (L - lq) if decode else 128          # block-1 queries carry the codes
        q_rows[i * lq + (first - (L - lq)): (i + 1) * lq, 0] = qc[i]
    if k4:
        qk = msa.Q8K4Index(dims, dev)
        kcodes = np.zeros((n * L, DI), np.uint8)
        for i in range(n):
            kcodes[i * L] = F4.e2m1_encode(kv[i])
        qk.k_idx4.copy_(torch.from_numpy(F4.pack(kcodes)))
        qk.k_exp4.fill_(127)
        store = qk
    else:
        fp8 = msa.Fp8Index(dims, dev)
        kcodes = np.zeros((n * L, DI), np.uint8)
        for i in range(n):
            kcodes[i * L] = F8.e4m3_encode(kv[i])
        fp8.k_idx8.copy_(torch.from_numpy(kcodes))
        fp8.k_exp.fill_(127)
        store = fp8
    store.q_idx8.copy_(torch.from_numpy(q_rows))
    store.q_exp.fill_(127)
    sel = torch.empty((n * lq, 1, 2), dtype=torch.int32, device=dev)
    score = torch.empty((n * lq, 1, 2), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.workspace_size(dims, msa.OP_INDEX_SELECT), dtype=torch.uint8, device=dev)
    if k4:
        msa.index_select_q8k4(dims, store, cuq, cuk, sel, score, ws)
    else:
        msa.index_select_fp8(dims, store, cuq, cuk, sel, score, ws)
    torch.cuda.synchronize()
    last = np.arange(1, n + 1) * lq - 1              # a block-1 query of each sequence
    s = score.cpu().numpy()[last, 0, 0]
    assert (sel.cpu().numpy()[last, 0] == [0, 1]).all()
    return s, qv, kv


@pytest.mark.parametrize("decode", [False, True], ids=["prefill", "decode"])
@pytest.mark.parametrize("k4", [False, True], ids=["e4m3-keys", "e2m1-keys"])
def test_fp8_matrix_core_summation_model(k4, decode):
    cases = CASES_K4 if k4 else CASES_FP8
    got, qv, kv = _setup(cases, decode, k4, rng_cases=24, seed=5 + 2 * k4 + decode)
    for i, (name, _, _, want) in enumerate(cases):
        log(f"[acc {'k4' if k4 else 'fp8'} {'decode' if decode else 'prefill'}] {name}: "
            f"{got[i]!r} (model {want!r}, exact {float(qv[i] @ kv[i])!r})")
        assert got[i] == np.float32(want), (name, got[i], want)
    # random positive codes: within the documented bound of the exact dot product, and
    # never above it (the dropped bits only lower a positive sum)
    n0 = len(cases)
    exact = np.einsum("ij,ij->i", qv[n0:], kv[n0:])
    bound = 2.0 ** -10 * np.einsum("ij,ij->i", np.abs(qv[n0:]), np.abs(kv[n0:]))
    err = got[n0:] - exact
    log(f"[acc] random rows: max |err| / bound {float(np.max(np.abs(err) / bound)):.3f}")
    assert np.all(np.abs(err) <= bound)
    # positive products: the dropped bits only lower the sum; the fp32 additions of the
    # 16 group sums may round up, by less than 16 * 2^-24 of the total
    assert np.all(err <= bound * 2.0 ** -10)
