"""The hot path captured as a HIP graph: every replay, with eager work and
synchronisations between replays, must equal the eager result bitwise."""
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate

pytestmark = pytest.mark.gpu

from gpu_helpers import log  # noqa: E402


@pytest.mark.parametrize("case", ["decode", "prefill"])
def test_graph_replays_match_eager(case):
    if case == "decode":
        w = custom([9000, 20000, 300, 4100], [1, 1, 1, 1], num_q_heads=32, num_kv_heads=8,
                   head_dim=128, index_dim=128, top_k=16, seed=41, qkv_std=1.0)
    else:
        w = custom([3000, 1200], [3000, 1200], num_q_heads=16, num_kv_heads=2, head_dim=128,
                   index_dim=64, top_k=8, seed=42, qkv_std=1.0)
    log(f"[graph:{case}] lens {w.seq_k_lens}/{w.seq_q_lens}")
    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in generate(w, "cpu").items()}
    dims = msa.dims_for(w)
    bufs = msa.Buffers(dims, dev, want_scores=True)

    def step():
        msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                        t["cu_seqlens_k"], bufs)

    step()
    torch.cuda.synchronize()
    ref = {n: getattr(bufs, n).clone() for n in ("sel", "sel_score", "offsets", "out", "lse")}
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for n in ("sel", "sel_score", "out", "lse"):
            getattr(bufs, n).zero_()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, v in ref.items():
            assert torch.equal(getattr(bufs, n).nan_to_num(), v.nan_to_num()), (rep, n)
    log(f"[graph:{case}] 4 replays equal the eager result")
