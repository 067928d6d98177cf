"""Pins for oracle/index_ref: token orders of the ring layouts and the Ulysses relayout.

Checked against the example the Long Context Attention notes print (stripe,
16 tokens on 4 devices), the claims the same notes make about the zigzag fold
(every Q_i/K_j block is whole; work per card is nearly equal) and about the
striped rounds (only when host_id < round are the first query and last key
dropped), and bijection / inverse / slice invariants.
"""
import json
import os

import pytest
import torch

from oracle import index_ref as ix
from oracle.attention_ref import visibility

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_stripe_example_from_notes():
    g = _golden("stripe_16_tokens_4_devices.json")
    assert ix.rank_positions("stripe", g["S"], g["N"], g["rank"], 1) == g["stripe_positions"]
    assert ix.rank_positions("basic", g["S"], g["N"], g["rank"]) == g["contiguous_positions"]


@pytest.mark.parametrize("impl,b", [("basic", 1), ("zigzag", 1), ("stripe", 1), ("stripe", 2), ("stripe", 3)])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 8])
def test_bijection_and_inverse(impl, b, N):
    unit = {"basic": N, "zigzag": 2 * N, "stripe": N * b}[impl]
    S = unit * 5
    perm = ix.permutation(impl, S, N, b)
    assert sorted(perm) == list(range(S))
    L = S // N
    for idx, p in enumerate(perm):
        assert ix.owner(impl, S, N, p, b) == (idx // L, idx % L)


@pytest.mark.parametrize("impl", ["basic", "zigzag", "stripe"])
def test_permute_rows_roundtrip_and_extract(impl):
    N, S = 4, 32
    x = torch.arange(2 * S * 3).reshape(2, S, 3)
    y = ix.permute_rows(x, impl, N)
    assert torch.equal(ix.unpermute_rows(y, impl, N), x)
    L = S // N
    for r in range(N):
        assert torch.equal(ix.extract_rows(x, impl, N, 1, r), y[:, r * L:(r + 1) * L])
    # hybrid: global rank g = r*ud + u takes the u-th contiguous piece of ring shard r
    ud = 2
    for g in range(N * ud):
        r, u = divmod(g, ud)
        piece = y[:, r * L + u * (L // ud): r * L + (u + 1) * (L // ud)]
        assert torch.equal(ix.extract_rows(x, impl, N, ud, g), piece)


def test_basic_is_identity():
    assert ix.permutation("basic", 24, 4) == list(range(24))


def test_zigzag_fold_pairs_chunks():
    # The fold puts chunk a and chunk 2N-1-a on the same card, first half first.
    N, S = 4, 16
    c = S // (2 * N)
    for r in range(N):
        pos = ix.rank_positions("zigzag", S, N, r)
        chunks = sorted({p // c for p in pos})
        assert chunks == [r, 2 * N - 1 - r]
        assert pos == sorted(pos)


def _block_masks(impl, S, N, b=1):
    pos = [torch.tensor(ix.rank_positions(impl, S, N, r, b)) for r in range(N)]
    return {(i, j): visibility(pos[i], pos[j], causal=True, window=0, n_sink=0)
            for i in range(N) for j in range(N)}


@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_zigzag_blocks_are_whole_and_work_is_equal(N):
    c = 3
    S = 2 * N * c
    masks = _block_masks("zigzag", S, N)
    L = 2 * c
    tri = torch.tril(torch.ones(L, L, dtype=torch.bool))
    per_rank = []
    for i in range(N):
        work = 0
        for j in range(N):
            m = masks[(i, j)]
            work += int(m.sum())
            if i == j:
                assert torch.equal(m, tri)                   # one causal triangle
            elif j < i:                                      # all queries x first half of keys
                assert m[:, :c].all() and not m[:, c:].any()
            else:                                            # second half of queries x all keys
                assert m[c:, :].all() and not m[:c, :].any()
        per_rank.append(work)
    assert len(set(per_rank)) == 1
    assert per_rank[0] == 2 * N * c * c + c


@pytest.mark.parametrize("N", [2, 4, 8])
def test_stripe_rounds_drop_first_query_last_key_when_host_lt_round(N):
    L = 5
    S = N * L
    masks = _block_masks("stripe", S, N)
    causal = torch.tril(torch.ones(L, L, dtype=torch.bool))
    strict = torch.tril(torch.ones(L, L, dtype=torch.bool), diagonal=-1)
    for i in range(N):
        for s in range(N):
            j = (i - s) % N
            m = masks[(i, j)]
            if i < s:
                # strict triangle == the causal one without its first query row and last key column
                assert torch.equal(m, strict)
                assert torch.equal(m[1:, :-1], causal[:-1, :-1])
            else:
                assert torch.equal(m, causal)


def test_stripe_work_nearly_equal():
    N, L = 4, 16
    S = N * L
    masks = _block_masks("stripe", S, N)
    work = [sum(int(masks[(i, j)].sum()) for j in range(N)) for i in range(N)]
    for i in range(N):
        assert work[i] == N * L * (L - 1) // 2 + (i + 1) * L
    assert max(work) - min(work) == (N - 1) * L


def test_contiguous_layout_is_unbalanced():
    # The imbalance the striped / zigzag layouts remove (notes, section "Problem").
    N, L = 4, 4
    masks = _block_masks("basic", N * L, N)
    work = [sum(int(masks[(i, j)].sum()) for j in range(N)) for i in range(N)]
    assert work == sorted(work) and work[0] < work[-1]


@pytest.mark.parametrize("ud", [1, 2, 4])
def test_ulysses_relayout_roundtrip(ud):
    B, Ls, H, D = 2, 3, 8, 4
    shards = [torch.randn(B, Ls, H, D) for _ in range(ud)]
    for u in range(ud):
        y = ix.ulysses_seq_to_head(shards, u)
        assert y.shape == (B, ud * Ls, H // ud, D)
        for up in range(ud):
            for s in range(Ls):
                for hp in range(H // ud):
                    assert torch.equal(y[:, up * Ls + s, hp], shards[up][:, s, u * (H // ud) + hp])
        back = [torch.zeros(B, Ls, H, D) for _ in range(ud)]
        ix.ulysses_head_to_seq(y, u, back)
        for up in range(ud):
            sl = slice(u * (H // ud), (u + 1) * (H // ud))
            assert torch.equal(back[up][:, :, sl], shards[up][:, :, sl])
    # the ud head groups partition the heads: scattering every group rebuilds the shards
    back = [torch.zeros(B, Ls, H, D) for _ in range(ud)]
    for u in range(ud):
        ix.ulysses_head_to_seq(ix.ulysses_seq_to_head(shards, u), u, back)
    for up in range(ud):
        assert torch.equal(back[up], shards[up])
    if ud == 1:
        assert torch.equal(ix.ulysses_seq_to_head(shards, 0), shards[0])


def test_divisibility_errors():
    with pytest.raises(ValueError):
        ix.rank_positions("zigzag", 12, 4, 0)
    with pytest.raises(ValueError):
        ix.rank_positions("stripe", 12, 4, 0, 2)
    with pytest.raises(ValueError):
        ix.rank_positions("basic", 10, 4, 0)
