"""Prefill index selection on short sequences: query tiles with every count of
earlier key blocks from 0 to 8.

The prefill index kernels stream a sequence's earlier key blocks in trips of
three steps that are never cut short: the loads of the blocks past the last
earlier one are clamped to it, and the steps past it score that copy again
and insert nothing into the top-k lists.  Sequences of 1 to 9 blocks (some
with ragged tails), with 8 groups (a query tile of 64 queries: half a block),
give tiles whose count of earlier blocks takes every value from 0 to 8, so
every position of the last trip is exercised.  Each index precision is
checked against the oracle on every row; the bf16 and E4M3 kernels also run
on a paged cache in scrambled page order, whose results must be bit-identical.
"""
import pytest

from msa_inputs import custom

pytestmark = pytest.mark.gpu

LENS = [128, 133, 256, 333, 384, 385, 512, 740, 768, 960, 1024, 1155]


def _w(seed):
    return custom(LENS, LENS, num_q_heads=16, num_kv_heads=8, head_dim=64, index_dim=128, top_k=4,
                  seed=seed, qkv_std=1.0)


def test_short_sequences_bf16():
    from test_gpu_parity import _full_check
    _full_check(_w(901), tag="short-bf16")


def test_short_sequences_fp8():
    from test_gpu_fp8 import _full_check
    _full_check(_w(902), "short-fp8")


def test_short_sequences_q8k4():
    from test_gpu_q8k4 import _full_check
    _full_check(_w(903), "short-q8k4")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_short_sequences_paged(fp8):
    from test_gpu_paged import _check_paged
    _check_paged(_w(904 + fp8), f"short-paged-{'fp8' if fp8 else 'bf16'}", fp8=fp8)
