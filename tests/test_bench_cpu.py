"""Host-side pieces of bench.py: the closed-form visible-pair counts that turn
kernel time into mask-adjusted TFLOP/s must equal the pairs the oracle's
visibility predicate admits.

For the one-rank workloads the oracle count is taken over the rank's own rows
(global positions from oracle/index_ref.py) against every key, at reduced S
with the workloads' ring layout, degree and mask."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import seeded_inputs as si  # noqa: E402
from oracle import index_ref as ix  # noqa: E402
from oracle.attention_ref import visibility, visible_pair_count  # noqa: E402


def _rank_pairs(w):
    pos_q = torch.tensor(ix.rank_positions(w.impl, w.S, w.ring_degree, w.rank, w.stripe_block))
    pos_k = torch.arange(w.S)
    return int(visibility(pos_q, pos_k, causal=w.causal, window=w.window, n_sink=w.n_sink,
                          cu_seqlens=w.cu_seqlens).sum())


@pytest.mark.parametrize("w", [
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=2048),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=2048, rank=3),
    si.WORKLOADS["stripe_mqa"].scaled(S=2048),
    si.WORKLOADS["stripe_mqa"].scaled(S=2048, rank=7),
    si.WORKLOADS["stripe_mqa"].scaled(S=2048, stripe_block=4),
    si.WORKLOADS["stripe_mqa"].scaled(S=4096, stripe_block=16, rank=5),
    si.WORKLOADS["stripe_mqa"].scaled(S=2048, stripe_block=2, ring_degree=4, rank=3),
], ids=lambda w: f"{w.name}-b{w.stripe_block}-r{w.rank}")
def test_one_rank_pair_count_matches_oracle(w):
    assert bench.visible_pairs_per_head(w) == _rank_pairs(w)


@pytest.mark.parametrize("name", ["zigzag_causal_small", "ring_swa", "varlen_streaming"])
def test_all_rank_pair_count_matches_oracle(name):
    w = si.WORKLOADS[name]  # full size: S <= 8192 counts in well under a second
    assert bench.visible_pairs_per_head(w) == visible_pair_count(
        w.S, causal=w.causal, window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens)


def test_full_size_counts_are_the_stated_ones():
    # the per-head pair totals that the mask-adjusted FLOP of the two one-rank
    # workloads are quoted on (zigzag: 2Nc^2 + c; stripe b=1: N L (L-1)/2 + (r+1) L)
    assert bench.visible_pairs_per_head(si.WORKLOADS["usp_zigzag_gqa"]) == 2_147_500_032
    assert bench.visible_pairs_per_head(si.WORKLOADS["stripe_mqa"]) == 68_719_083_520


def test_copy_byte_counts():
    # USP: one strided gather per tensor, ring rank 0's q rows and every k / v
    # piece, head group u only (q 2 x 32768 x 16 x 256 B, k and v 2 x 131072 x 4 x 256 B each)
    perm, relay = bench.step_bytes(si.WORKLOADS["usp_zigzag_gqa"])
    assert perm == 805_306_368 and relay == 0
    perm, relay = bench.step_bytes(si.WORKLOADS["stripe_mqa"])
    assert perm == 1_610_612_736 and relay == 0


def test_gpus_other_than_one_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
