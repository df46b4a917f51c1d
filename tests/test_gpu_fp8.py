"""GPU parity of the quantised (FP8 E4M3) Index Branch against the oracle.

The oracle quantises the same bf16 inputs itself (oracle/fp8_index.py) and
runs the unquantised oracle on its dequantised values; nothing it uses comes
from the GPU.  Checked: the E4M3 codes and E8M0 exponents bit for bit; the
selection against the exact scores of the dequantised values, allowing only
the choices the fp8 matrix cores' error bound (below) leaves open, with the
reported block scores inside that bound; the output of the whole forward
against the oracle's Main Branch on the selection made.
Small cases check every row; the full-size workloads check sampled rows in
the configuration the benchmark times, quantising only what the oracle reads.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, sample_rows, workload
from oracle import fp8_index as F
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, log  # noqa: E402

# Error model of gfx950's fp8 matrix cores (measured with an in-bounds probe of
# the 32x32x64 and 32x32x16 fp8 MFMAs, which give identical results): the 64
# products of a contraction are summed in groups of 8, each group in fixed
# point aligned to its largest product, keeping 13 bits below that product's
# leading bit; subnormal E4M3 inputs are exact.  Up to 7 products per group
# lose less than 2^-13 of the group's largest |product| each, so a token score
# is within 7 * 2^-13 * sum|q_c k_c| (< 2^-10 of it, fp32 rounding included)
# of the exact dot product of the dequantised values.
FP8_DOT_REL = 2.0 ** -10


def fp8_block_bounds(P, r):
    """Per (group, block): the largest error bound of the block's token scores."""
    b, p, ko = int(P.seq[r]), int(P.pos[r]), int(P.koff[r])
    lk = int(P.cu_k[b + 1] - P.cu_k[b])
    qa = np.abs(np.asarray(P.q_idx[r], dtype=np.float64))
    ka = np.abs(np.asarray(P.k_idx[ko:ko + lk][: p + 1], dtype=np.float64))
    return FP8_DOT_REL * O.block_max_pool(qa @ ka.T, p, P.block)


def check_selection_fp8(P, rows, gsel, gscore, ref):
    """The GPU selection must hold the local block and top_k - 1 others such
    that every chosen block could still outrank every unchosen one after each
    score moves by its error bound; the reported scores must be within their
    bounds.  Returns (bad rows, rows whose selection differs from the oracle's)."""
    bad, differ = [], []
    for i, r in enumerate(rows):
        beta_p = int(P.pos[r]) // P.block
        B = fp8_block_bounds(P, r)
        for g in range(P.G):
            S = ref["S"][i][g]
            mine = [int(x) for x in gsel[i, g] if x >= 0]
            want = [int(x) for x in ref["sel"][i, g] if x >= 0]
            if sorted(mine) != list(gsel[i, g][:len(mine)]) or len(mine) != len(want) \
                    or beta_p not in mine or len(set(mine)) != len(mine) or max(mine) > beta_p:
                bad.append((r, g, "malformed", mine, want))
                continue
            if mine != want:
                differ.append((r, g))
                chosen = [x for x in mine if x != beta_p]
                others = [z for z in range(beta_p) if z not in chosen]
                lo = min(S[x] + B[g][x] for x in chosen)
                hi = max((S[z] - B[g][z] for z in others), default=-np.inf)
                if lo < hi:
                    bad.append((r, g, "not a top set within the bounds", mine, want))
            n = len(mine)
            sc = gscore[i, g]
            if not (np.isinf(sc[n - 1]) and sc[n - 1] > 0 and np.all(np.isnan(sc[n:]))):
                bad.append((r, g, "local/padding scores", list(sc)))
            for s_, x in zip(sc[:n - 1], mine[:n - 1]):
                if abs(float(s_) - S[x]) > B[g][x] + 1e-6 * abs(S[x]):
                    bad.append((r, g, "score outside bound", x, float(s_), S[x], B[g][x]))
    return bad, differ


def check_rows_fp8(P, rows, bufs_sel, bufs_score, ref, out, lse, tag):
    bad, differ = check_selection_fp8(P, rows, bufs_sel, bufs_score, ref)
    log(f"[{tag}] selection: invalid {len(bad)}; differing from the oracle within the error "
        f"bound {len(differ)} of {len(rows) * P.G}")
    assert not bad, bad[:3]
    # Main Branch: against the oracle on the selection the GPU made (identical
    # to the oracle's own selection on all other rows)
    ref_out, ref_lse = ref["out"].copy(), ref["lse"].copy()
    pos = {r: i for i, r in enumerate(rows)}
    for r in sorted({r for r, _ in differ}):
        i = pos[r]
        ref_out[i], ref_lse[i] = P.attend_with_selection(r, bufs_sel[i])
    check_out(out, ref_out, lse, ref_lse, tag)


def _nb(t):
    lk = np.diff(t["cu_seqlens_k"].cpu().numpy())
    return int((lk.max() + 127) // 128)


def _run_fp8(w, t, q_chunk=0):
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = msa.dims_for(w, q_chunk=q_chunk)
    bufs = msa.Buffers(dims, dev, want_scores=True)
    fp8 = msa.Fp8Index(dims, dev)
    msa.msa_forward(dims, g["q"], g["k"], g["v"], g["q_idx"], g["k_idx"], g["cu_seqlens_q"],
                    g["cu_seqlens_k"], bufs, fp8=fp8)
    torch.cuda.synchronize()
    return dims, bufs, fp8


def _check_codes(fp8, qc, qe, kc, ke, tag):
    gq, gqe = fp8.q_idx8.cpu().numpy(), fp8.q_exp.cpu().numpy()
    gk, gke = fp8.k_idx8.cpu().numpy(), fp8.k_exp.cpu().numpy()
    nq = int((gq != qc).sum())
    nk = int((gk != kc).sum())
    log(f"[{tag}] code mismatches q {nq}/{qc.size} k {nk}/{kc.size}")
    assert np.array_equal(gqe, qe)
    assert np.array_equal(gke, ke)
    assert nq == 0 and nk == 0


def _full_check(w, tag, q_chunk=0, plant=None):
    log(f"[{tag}] lens k={w.seq_k_lens} q={w.seq_q_lens} Hq={w.num_q_heads} G={w.num_kv_heads} "
        f"d={w.head_dim} di={w.index_dim} k={w.top_k} chunk={q_chunk}")
    t = generate(w, "cpu")
    if plant:
        plant(t)
    dims, bufs, fp8 = _run_fp8(w, t, q_chunk)
    cu_q, cu_k = t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy()
    qc, qe = F.quantize_q_idx(t["q_idx"].double().numpy())
    kc, ke = F.quantize_k_idx(t["k_idx"].double().numpy(), cu_k, _nb(t))
    _check_codes(fp8, qc, qe, kc, ke, tag)
    f = lambda x: x.double().numpy()
    P = O.Problem(f(t["q"]), f(t["k"]), f(t["v"]), F.dequantize_q_idx(qc, qe),
                  F.dequantize_k_idx(kc, ke, cu_k), cu_q, cu_k, w.top_k)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    check_rows_fp8(P, rows, bufs.sel.cpu().numpy(), bufs.sel_score.cpu().numpy(), ref,
                   bufs.out.float().cpu().numpy(), bufs.lse.cpu().numpy(), tag)
    return t, bufs, fp8


def test_fp8_tiny():
    _full_check(workload("tiny"), "fp8-tiny")


def test_fp8_ragged_prefill_di64():
    w = custom([1500, 900, 130, 128, 3000, 257], [1500, 300, 130, 1, 2000, 200], num_q_heads=8,
               num_kv_heads=2, head_dim=64, index_dim=64, top_k=5, seed=41, qkv_std=1.0)
    _full_check(w, "fp8-ragged")


def test_fp8_gqa8_di128():
    w = custom([2200, 700], [2200, 700], num_q_heads=64, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=16, seed=42, qkv_std=1.0)
    _full_check(w, "fp8-gqa8")


def test_fp8_three_groups_di32_k32():
    w = custom([5000], [5000], num_q_heads=12, num_kv_heads=3, head_dim=64, index_dim=32,
               top_k=32, seed=43, qkv_std=1.0)
    _full_check(w, "fp8-g3")


def test_fp8_decode_path():
    w = custom([5000, 20000, 128, 300, 129], [1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=44, qkv_std=1.0)
    _full_check(w, "fp8-decode")


def test_fp8_multi_token_decode_di32():
    w = custom([9000, 4100], [4, 3], num_q_heads=32, num_kv_heads=8, head_dim=64, index_dim=32,
               top_k=6, seed=45, qkv_std=1.0)
    _full_check(w, "fp8-mtd")


def test_fp8_degenerate_rows_and_blocks():
    """All-zero, tiny and huge index rows, an all-zero and a one-token key
    block, signed zeros."""
    w = custom([1300, 700], [1300, 700], num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=64,
               top_k=4, seed=46, qkv_std=1.0)

    def plant(t):
        qi, ki = t["q_idx"], t["k_idx"]
        qi[5, 0] = 0.0
        qi[6, 1] = -0.0
        qi[700, 0] *= 1e-20
        qi[701, 1] *= 1e20
        qi[702, 0, ::2] = 0.0
        ki[128 * 3:128 * 4] = 0.0                  # sequence 0, block 3: all zero
        ki[1300 + 128 * 2:1300 + 128 * 3] *= 1e-12  # sequence 1, block 2: tiny
        ki[1300 + 5] *= 1e15                        # one huge key in sequence 1, block 0
        t["q_idx"], t["k_idx"] = qi, ki

    _full_check(w, "fp8-degenerate", plant=plant)


def test_fp8_chunking_is_bitwise_invisible():
    w = custom([3000, 1000], [1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128, index_dim=64,
               top_k=4, seed=47, qkv_std=1.0)
    t = generate(w, "cpu")
    _, a, _ = _run_fp8(w, t, q_chunk=0)
    _, b, _ = _run_fp8(w, t, q_chunk=1)
    assert torch.equal(a.sel, b.sel) and torch.equal(a.out, b.out)


def test_fp8_decode_on_a_quantised_key_cache():
    """Keys quantised once (queries left out), then steps that quantise only
    their queries: the same selection and output as quantising both."""
    w = custom([7000, 3000, 12000], [1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=16, seed=49, qkv_std=1.0)
    t = generate(w, "cpu")
    dims, ref, ref8 = _run_fp8(w, t)
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    fp8 = msa.Fp8Index(dims, dev)
    fp8.q_idx8.fill_(0x7F)     # NaN codes: must be overwritten by the query-only calls
    msa.index_quantize_fp8(dims, None, g["k_idx"], g["cu_seqlens_k"], fp8)
    torch.cuda.synchronize()
    assert torch.equal(fp8.k_idx8, ref8.k_idx8) and torch.equal(fp8.k_exp, ref8.k_exp)
    assert int((fp8.q_idx8 == 0x7F).sum()) == fp8.q_idx8.numel()   # queries untouched
    bufs = msa.Buffers(dims, dev, want_scores=True)
    for _ in range(2):
        msa.msa_forward(dims, g["q"], g["k"], g["v"], g["q_idx"], None, g["cu_seqlens_q"],
                        g["cu_seqlens_k"], bufs, fp8=fp8)
        torch.cuda.synchronize()
        assert torch.equal(fp8.q_idx8, ref8.q_idx8) and torch.equal(fp8.q_exp, ref8.q_exp)
        assert torch.equal(bufs.sel, ref.sel) and torch.equal(bufs.out, ref.out)


def test_fp8_on_exact_values_equals_bf16_path():
    """Index inputs that are already E4M3 values with power-of-two block
    scales: the quantised path selects exactly what the bf16 path selects."""
    w = custom([2600, 900], [2600, 900], num_q_heads=16, num_kv_heads=4, head_dim=64,
               index_dim=128, top_k=8, seed=48, qkv_std=1.0)
    t = generate(w, "cpu")
    cu_k = t["cu_seqlens_k"].numpy()
    qc, qe = F.quantize_q_idx(t["q_idx"].double().numpy())
    kc, ke = F.quantize_k_idx(t["k_idx"].double().numpy(), cu_k, _nb(t))
    t["q_idx"] = torch.from_numpy(F.dequantize_q_idx(qc, qe)).to(torch.bfloat16)
    t["k_idx"] = torch.from_numpy(F.dequantize_k_idx(kc, ke, cu_k)).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = msa.dims_for(w)
    a = msa.Buffers(dims, dev, want_scores=True)
    msa.msa_forward(dims, g["q"], g["k"], g["v"], g["q_idx"], g["k_idx"], g["cu_seqlens_q"],
                    g["cu_seqlens_k"], a)
    _, b, _ = _run_fp8(w, t)
    torch.cuda.synchronize()
    assert torch.equal(a.sel, b.sel)


# ---------------------------------------------------------------------------
# full sizes: sampled rows; the oracle quantises only what it reads
# ---------------------------------------------------------------------------
class _DeqQ:
    """q_idx rows dequantised on demand (one scale per (row, group))."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, r):
        x = self.t[int(r)].double().cpu().numpy()[None]
        c, e = F.quantize_q_idx(x)
        return F.dequantize_q_idx(c, e)[0]


class _DeqK:
    """k_idx of one sequence, quantised and dequantised on demand: the oracle
    slices exactly a sequence's rows [cu_k[b], cu_k[b+1]), whose blocks start
    at the slice start."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)
        self.cache = {}

    def __getitem__(self, sl):
        assert isinstance(sl, slice)
        key = (sl.start, sl.stop)
        if key not in self.cache:
            x = self.t[sl].double().cpu().numpy()
            cu = np.array([0, len(x)])
            nb = (len(x) + 127) // 128
            c, e = F.quantize_k_idx(x, cu, nb)
            self.cache[key] = F.dequantize_k_idx(c, e, cu)
        return self.cache[key]


def _sampled_fp8(name, rows_fn):
    w = workload(name)
    log(f"[fp8-{name}] generating {w.note}")
    t = generate(w, "cuda:0")
    dims = msa.dims_for(w)
    bufs = msa.Buffers(dims, t["q"].device, want_scores=True)
    fp8 = msa.Fp8Index(dims, t["q"].device)
    msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                    t["cu_seqlens_k"], bufs, fp8=fp8)
    torch.cuda.synchronize()
    rows = rows_fn(w)
    log(f"[fp8-{name}] forward done; oracle on {len(rows)} rows")
    # codes of the sampled query rows and of the first sequence's first blocks
    ridx = torch.as_tensor(rows, device="cuda:0", dtype=torch.long)
    qc, qe = F.quantize_q_idx(t["q_idx"].index_select(0, ridx).double().cpu().numpy())
    assert np.array_equal(fp8.q_idx8.index_select(0, ridx).cpu().numpy(), qc)
    assert np.array_equal(fp8.q_exp.index_select(0, ridx).cpu().numpy(), qe)
    n0 = min(int(w.seq_k_lens[0]), 128 * 64)
    kc, ke = F.quantize_k_idx(t["k_idx"][:n0].double().cpu().numpy(), np.array([0, n0]),
                              (n0 + 127) // 128)
    assert np.array_equal(fp8.k_idx8[:n0].cpu().numpy(), kc)
    assert np.array_equal(fp8.k_exp[0, :(n0 + 127) // 128].cpu().numpy(), ke[0])
    from gpu_helpers import LazyRows
    P = O.Problem(LazyRows(t["q"]), LazyRows(t["k"]), LazyRows(t["v"]), _DeqQ(t["q_idx"]),
                  _DeqK(t["k_idx"]), t["cu_seqlens_q"].cpu().numpy(), t["cu_seqlens_k"].cpu().numpy(),
                  w.top_k)
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.index_select(0, ridx).cpu().numpy()
    score = bufs.sel_score.index_select(0, ridx).cpu().numpy()
    out = bufs.out.index_select(0, ridx).float().cpu().numpy()
    lse = bufs.lse.index_select(0, ridx).cpu().numpy()
    check_rows_fp8(P, rows, sel, score, ref, out, lse, f"fp8-{name}")


def test_fp8_p128k_sampled():
    _sampled_fp8("p128k", lambda w: sample_rows(w, 24))


def test_fp8_decode_sampled():
    # eight of the 32 sequences (each quantised whole by the oracle)
    _sampled_fp8("decode", lambda w: list(range(0, w.total_q, 4)))


def test_fp8_verification_shape():
    w = custom([7000, 4100, 300, 2049], [8, 8, 5, 8], num_q_heads=32, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=8, seed=50, qkv_std=1.0)
    _full_check(w, "fp8-verify8")
