"""GPU parity of the index projections (msa_index_project) against the oracle.

Element by element: every bf16 output must equal the oracle's rounding of the
exact product sum, except where the exact sum lies within the fp32
accumulation bound eps = D * 2^-24 * sum |x_c w_c| of a bf16 rounding
boundary; there the output must be within eps + one unit in the last place of
the exact sum (with cancellation eps can span many bf16 units of a small
result).  End to end (projections ->
index select -> lists -> attend), the selection is checked against the
oracle's own projections with the score bound those possible one-ulp
differences allow (computed from the oracle's values alone).
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, generate_projection, workload
from oracle import msa_oracle as O
from oracle import projections as PR

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, log  # noqa: E402


def _ulp(y):
    _, e = np.frexp(np.abs(y))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def _eps(s_abs, D):
    """fp32 accumulation bound of a D-term sum of products with sum |p| = s_abs."""
    return D * 2.0 ** -24 * s_abs + 1e-300


def _near_boundary(y, s_abs, D):
    """Values whose bf16 rounding the fp32-accumulated sum may flip."""
    r = PR.bf16_round(y)
    return (_ulp(y) / 2 - np.abs(y - r)) <= _eps(s_abs, D)


def _freedom(y, s_abs, D):
    """A-priori bound of |GPU output - oracle output| per element."""
    return np.where(_near_boundary(y, s_abs, D), _eps(s_abs, D) + 1.5 * _ulp(y), 0.0)


def _check_elementwise(gpu, y, s_abs, D, what):
    r = PR.bf16_round(y)
    diff = gpu != r
    n = int(diff.sum())
    log(f"[{what}] {n} of {gpu.size} outputs differ from the oracle's rounding")
    if n:
        near = _near_boundary(y, s_abs, D)
        ok = near & (np.abs(gpu - y) <= _eps(s_abs, D) + _ulp(y))
        assert np.all(ok[diff]), (what, np.argwhere(diff & ~ok)[:5])


def _run(w, D, t, p, prefill_k_fill=None):
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    gp = {k: v.to(dev) for k, v in p.items()}
    dims = msa.dims_for(w)
    q_idx = torch.empty((w.total_q, w.num_kv_heads, w.index_dim), dtype=torch.bfloat16, device=dev)
    k_idx = g["k_idx"].clone() if prefill_k_fill is None else \
        torch.full((w.total_k, w.index_dim), prefill_k_fill, dtype=torch.bfloat16, device=dev)
    msa.index_project(dims, gp["x"], gp["w_q"], gp["w_k"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                      q_idx, k_idx)
    torch.cuda.synchronize()
    return dims, g, gp, q_idx, k_idx


def _oracle(w, t, p, D):
    x = p["x"].double().numpy()
    wq, wk = p["w_q"].double().numpy(), p["w_k"].double().numpy()
    cu_q, cu_k = t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy()
    q, rows = PR.project(x, wq, wk, cu_q, cu_k, w.total_k, w.num_kv_heads)
    yq, sq = x @ wq.T, np.abs(x) @ np.abs(wq).T
    yk, sk = x @ wk.T, np.abs(x) @ np.abs(wk).T
    return q, rows, (yq, sq), (yk, sk)


def _key_rows(t, w):
    cu_q, cu_k = t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy()
    out = []
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        out += [cu_k[b] + lk - lq + i for i in range(lq)]
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("case", [
    dict(k=[300, 129, 1000], q=[300, 129, 1000], G=2, di=64, D=256),
    dict(k=[700], q=[700], G=1, di=32, D=64),            # partial feature tile, 2 K steps
    dict(k=[1100, 257], q=[1100, 257], G=8, di=128, D=1024),
    dict(k=[5000, 300, 129], q=[1, 2, 1], G=8, di=128, D=512),   # decode: new keys appended
    dict(k=[2000, 300, 129], q=[200, 300, 12], G=4, di=64, D=448),  # few-token kernel, 16 tiles
    dict(k=[512], q=[512], G=2, di=32, D=192),            # largest few-token case
    dict(k=[513], q=[513], G=2, di=32, D=192),            # smallest large-tile case
    dict(k=[4000] * 32, q=[1] * 32, G=8, di=128, D=8192),  # decode at full width: 15 K slices
    dict(k=[300, 200], q=[3, 2], G=2, di=32, D=64),       # one K chunk: three waves idle
    dict(k=[900, 400], q=[100, 160], G=4, di=64, D=320),  # 5 K chunks over 4 waves
    # mid-size steps: the large-tile kernel splits K when its tiles would leave CUs idle
    dict(k=[1200, 700, 100], q=[1200, 700, 100], G=8, di=128, D=4096),  # 7 slices, the last shorter
    dict(k=[640], q=[640], G=8, di=128, D=8192),          # 13 slices of 20 stages
    dict(k=[1100], q=[1100], G=2, di=64, D=1344),         # 2 slices of 22 and 20 stages
    dict(k=[5000, 3000], q=[400, 300], G=8, di=128, D=2048),  # 4 slices; new keys appended
])
def test_projection_elementwise(case):
    w = custom(case["k"], case["q"], num_q_heads=case["G"] * 4, num_kv_heads=case["G"],
               head_dim=64, index_dim=case["di"], top_k=4, seed=51, qkv_std=1.0)
    D = case["D"]
    t = generate(w, "cpu")
    p = generate_projection(w, D, "cpu")
    log(f"[proj] lens k={w.seq_k_lens} q={w.seq_q_lens} G={w.num_kv_heads} di={w.index_dim} D={D}")
    dims, g, gp, q_idx, k_idx = _run(w, D, t, p, prefill_k_fill=-7.0)
    q, rows, (yq, sq), (yk, sk) = _oracle(w, t, p, D)
    _check_elementwise(q_idx.double().cpu().numpy().reshape(w.total_q, -1), yq, sq, D, "q_idx")
    kr = _key_rows(t, w)
    kg = k_idx.double().cpu().numpy()
    _check_elementwise(kg[kr], yk, sk, D, "k_idx")
    untouched = np.ones(w.total_k, dtype=bool)
    untouched[kr] = False
    assert np.all(kg[untouched] == -7.0)


def test_split_path_is_deterministic_and_ignores_workspace_contents():
    # the few-token path sums K slices through the workspace in a fixed order
    w = custom([3000] * 16, [4] * 16, num_q_heads=32, num_kv_heads=8, head_dim=64, index_dim=128,
               top_k=4, seed=53, qkv_std=1.0)
    D = 4096
    t = generate(w, "cpu")
    p = generate_projection(w, D, "cpu")
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    gp = {k: v.to(dev) for k, v in p.items()}
    dims = msa.dims_for(w)
    need = msa.workspace_size(dims, msa.OP_INDEX_PROJECT)
    assert need > 0
    outs = []
    for fill in (float("nan"), 1e30, 0.0):
        ws = torch.full((need // 4,), fill, dtype=torch.float32, device=dev).view(torch.uint8)
        q_idx = torch.empty((w.total_q, w.num_kv_heads, w.index_dim), dtype=torch.bfloat16, device=dev)
        k_idx = torch.zeros((w.total_k, w.index_dim), dtype=torch.bfloat16, device=dev)
        msa.index_project(dims, gp["x"], gp["w_q"], gp["w_k"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                          q_idx, k_idx, workspace=ws)
        torch.cuda.synchronize()
        outs.append((q_idx, k_idx))
    for q_idx, k_idx in outs[1:]:
        assert torch.equal(q_idx, outs[0][0]) and torch.equal(k_idx, outs[0][1])
    q, rows, (yq, sq), (yk, sk) = _oracle(w, t, p, D)
    _check_elementwise(outs[0][0].double().cpu().numpy().reshape(w.total_q, -1), yq, sq, D, "q_idx")


def test_mid_size_split_matches_unsplit_within_rounding():
    """Up to a few thousand tokens the large-tile kernel sums slices of K through
    the workspace; with a workspace too small for them it runs unsplit.  Both
    are checked against the oracle element by element; the split run is
    deterministic and ignores what the workspace held before."""
    w = custom([1500, 600], [1500, 600], num_q_heads=32, num_kv_heads=8, head_dim=64,
               index_dim=128, top_k=4, seed=54, qkv_std=1.0)
    D = 4096
    t = generate(w, "cpu")
    p = generate_projection(w, D, "cpu")
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    gp = {k: v.to(dev) for k, v in p.items()}
    dims = msa.dims_for(w)
    F = 9 * 128
    # 2100 tokens: 5 x 9 tiles of 512 tokens x 128 features -> 256 // 45 = 5 slices of K
    need = msa.workspace_size(dims, msa.OP_INDEX_PROJECT)
    assert need == 5 * w.total_q * F * 4

    def run(ws):
        q_idx = torch.empty((w.total_q, w.num_kv_heads, w.index_dim), dtype=torch.bfloat16, device=dev)
        k_idx = torch.zeros((w.total_k, w.index_dim), dtype=torch.bfloat16, device=dev)
        msa.index_project(dims, gp["x"], gp["w_q"], gp["w_k"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                          q_idx, k_idx, workspace=ws)
        torch.cuda.synchronize()
        return q_idx, k_idx

    split = [run(torch.full((need // 4,), fill, dtype=torch.float32, device=dev).view(torch.uint8))
             for fill in (float("nan"), 1e30)]
    assert torch.equal(split[0][0], split[1][0]) and torch.equal(split[0][1], split[1][1])
    unsplit = run(torch.empty(need - 16, dtype=torch.uint8, device=dev))
    q, rows, (yq, sq), (yk, sk) = _oracle(w, t, p, D)
    kr = _key_rows(t, w)
    for what, (q_idx, k_idx) in (("split", split[0]), ("unsplit", unsplit)):
        _check_elementwise(q_idx.double().cpu().numpy().reshape(w.total_q, -1), yq, sq, D,
                           f"q_idx {what}")
        _check_elementwise(k_idx.double().cpu().numpy()[kr], yk, sk, D, f"k_idx {what}")
    # the two differ by fp32 summation order only, so most outputs agree exactly
    same = (split[0][0] == unsplit[0]).float().mean().item()
    log(f"[proj] split vs unsplit: {same:.4f} of q_idx outputs identical")
    assert same > 0.9


def test_projection_model_width_8192_sampled():
    w = custom([4096], [4096], num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128,
               top_k=16, seed=52, qkv_std=1.0)
    D = 8192
    t = generate(w, "cpu")
    p = generate_projection(w, D, "cpu")
    dims, g, gp, q_idx, k_idx = _run(w, D, t, p)
    rows = np.arange(0, w.total_q, 37)
    x = p["x"].double().numpy()[rows]
    wq, wk = p["w_q"].double().numpy(), p["w_k"].double().numpy()
    _check_elementwise(q_idx.double().cpu().numpy().reshape(w.total_q, -1)[rows], x @ wq.T,
                       np.abs(x) @ np.abs(wq).T, D, "q_idx D=8192")
    _check_elementwise(k_idx.double().cpu().numpy()[rows], x @ wk.T, np.abs(x) @ np.abs(wk).T, D,
                       "k_idx D=8192")


def test_projection_then_forward_end_to_end():
    """x -> projections -> selection -> attention, against the oracle run on its
    own projections; a differing selection is accepted only where the one-ulp
    freedom of the projections could reorder the blocks."""
    w = custom([1500, 900], [1500, 900], num_q_heads=16, num_kv_heads=4, head_dim=64,
               index_dim=64, top_k=5, seed=53, qkv_std=1.0)
    D = 512
    t = generate(w, "cpu")
    p = generate_projection(w, D, "cpu")
    dims, g, gp, q_idx, k_idx = _run(w, D, t, p, prefill_k_fill=0.0)
    bufs = msa.Buffers(dims, g["q"].device, want_scores=True)
    msa.msa_forward(dims, g["q"], g["k"], g["v"], q_idx, k_idx, g["cu_seqlens_q"],
                    g["cu_seqlens_k"], bufs)
    torch.cuda.synchronize()
    q, rows, (yq, sq), (yk, sk) = _oracle(w, t, p, D)
    kor = np.stack([rows[r] for r in range(w.total_k)])
    f = lambda x_: x_.double().numpy()
    P = O.Problem(f(t["q"]), f(t["k"]), f(t["v"]), q, kor, t["cu_seqlens_q"].numpy(),
                  t["cu_seqlens_k"].numpy(), w.top_k)
    # a-priori per-element freedom of the GPU projections
    dq = _freedom(yq, sq, D).reshape(q.shape)
    dk = _freedom(yk, sk, D)
    rows_all = list(range(w.total_q))
    ref = P.run(rows_all, want_scores=True)
    sel = bufs.sel.cpu().numpy()
    bad, differ = [], []
    for i, r in enumerate(rows_all):
        pp = int(P.pos[r])
        ko = int(P.koff[r])
        beta_p = pp // 128
        kq = np.abs(kor[ko:ko + pp + 1])
        for gg in range(P.G):
            mine = [int(x_) for x_ in sel[i, gg] if x_ >= 0]
            want = [int(x_) for x_ in ref["sel"][i, gg] if x_ >= 0]
            if mine == want:
                continue
            differ.append((r, gg))
            tok = dq[r, gg] @ kq.T + np.abs(q[r, gg]) @ dk[ko:ko + pp + 1].T \
                + dq[r, gg] @ dk[ko:ko + pp + 1].T
            B = O.block_max_pool(tok[None, :], pp)[0]
            S = ref["S"][i][gg]
            chosen = [x_ for x_ in mine if x_ != beta_p]
            others = [z for z in range(beta_p) if z not in chosen]
            if beta_p not in mine or len(mine) != len(want) or \
                    min(S[x_] + B[x_] for x_ in chosen) < max((S[z] - B[z] for z in others), default=-np.inf):
                bad.append((r, gg, mine, want))
    log(f"[proj e2e] selections differing within the projection bound: {len(differ)}; invalid {len(bad)}")
    assert not bad, bad[:3]
    ref_out, ref_lse = ref["out"].copy(), ref["lse"].copy()
    for r in sorted({r for r, _ in differ}):
        ref_out[r], ref_lse[r] = P.attend_with_selection(r, sel[r])
    check_out(bufs.out.float().cpu().numpy(), ref_out, bufs.lse.cpu().numpy(), ref_lse, "proj e2e")
