"""Pins of the decode oracle (oracle/decode_ref.py).

- the decode rows equal the corresponding rows of full attention over the
  sequence (attention_ref, itself pinned by brute force and SDPA), and torch
  SDPA in float64 with an explicit mask on the decode rows;
- brute force with scalar loops on tiny caches;
- the tree-merged split partials equal the unsplit result for any piece
  size and ragged cache lengths, and equal a left-to-right merge (notes,
  section "Tree Attention": max and logsumexp are associative);
- a piece beyond a row's cache is (0, -inf) and changes nothing;
- closed forms: a cache of one key returns that key's value; window 1 gives
  each query its own key's value;
- a planted mistake (queries one position too early) fails the pins.
"""
import math

import pytest
import torch

from oracle.attention_ref import attention_ref, visibility
from oracle.decode_ref import decode_ref, decode_split_ref, tree_merge_ref
from oracle.ring_ref import block_attention_ref, merge_ref


def _cache(B, S, Lq, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Lq, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("Lq", [1, 3])
@pytest.mark.parametrize("window,n_sink", [(0, 0), (7, 0), (5, 2)])
def test_decode_rows_equal_full_attention_rows(Lq, window, n_sink):
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 16
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=1)
    # the full sequence whose last Lq query rows are the decode queries
    g = torch.Generator().manual_seed(2)
    qf = torch.randn(B, S, Hq, D, generator=g).to(torch.bfloat16)
    qf[:, S - Lq:] = q
    O, L = decode_ref(q, k, v, softmax_scale=0.3, window=window, n_sink=n_sink)
    Of, Lf = attention_ref(qf, k, v, softmax_scale=0.3, causal=True, window=window, n_sink=n_sink,
                           rows=list(range(S - Lq, S)))
    assert torch.allclose(O, Of, atol=1e-12) and torch.allclose(L, Lf, atol=1e-12)


def test_decode_ragged_lengths_against_sdpa():
    B, S, Lq, Hq, Hkv, D = 3, 33, 2, 4, 1, 8
    lens = [33, 10, 2]
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=3)
    O, L = decode_ref(q, k, v, lens, softmax_scale=0.5, window=6, n_sink=1)
    for b, n in enumerate(lens):
        pq = torch.arange(n - Lq, n)
        mask = visibility(pq, torch.arange(n), causal=True, window=6, n_sink=1)
        qb = q[b].double().transpose(0, 1)                                   # [Hq,Lq,D]
        kb = k[b, :n].double().repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
        vb = v[b, :n].double().repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=0.5)
        assert torch.allclose(O[b].transpose(0, 1), ref, atol=1e-10)
        s = (qb @ kb.transpose(1, 2)) * 0.5
        s = s.masked_fill(~mask, -math.inf)
        assert torch.allclose(L[b], torch.logsumexp(s, dim=-1), atol=1e-10)


def test_decode_brute_force_tiny():
    B, S, Lq, Hq, Hkv, D = 1, 6, 2, 2, 1, 3
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=4)
    O, L = decode_ref(q, k, v, softmax_scale=0.7)
    for h in range(Hq):
        for t in range(Lq):
            pq = S - Lq + t
            s = [0.7 * math.fsum(float(q[0, t, h, d]) * float(k[0, u, 0, d]) for d in range(D))
                 for u in range(pq + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for d in range(D):
                o = math.fsum(w[u] * float(v[0, u, 0, d]) for u in range(pq + 1)) / z
                assert abs(o - float(O[0, t, h, d])) < 1e-12
            assert abs(m + math.log(z) - float(L[0, h, t])) < 1e-12


@pytest.mark.parametrize("split_keys", [1, 5, 8, 64])
def test_tree_merged_splits_equal_decode(split_keys):
    B, S, Lq, Hq, Hkv, D = 3, 50, 2, 4, 2, 8
    lens = [50, 17, 3]
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=5)
    O, L = decode_ref(q, k, v, lens, window=9, n_sink=2)
    Op, Lp = decode_split_ref(q, k, v, lens, split_keys=split_keys, window=9, n_sink=2)
    assert Op.shape[0] == (S + split_keys - 1) // split_keys
    Ot, Lt = tree_merge_ref(Op, Lp)
    assert torch.allclose(Ot, O, atol=1e-12) and torch.allclose(Lt, L, atol=1e-12)
    # a left-to-right merge gives the same result
    Os, Ls = Op[0], Lp[0]
    for i in range(1, Op.shape[0]):
        Os, Ls = merge_ref(Os, Ls, Op[i], Lp[i])
    assert torch.allclose(Os, O, atol=1e-12) and torch.allclose(Ls, L, atol=1e-12)


def test_pieces_beyond_the_cache_are_empty():
    B, S, Lq, Hq, Hkv, D = 2, 32, 1, 2, 1, 4
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=6)
    Op, Lp = decode_split_ref(q, k, v, [32, 9], split_keys=8)
    assert torch.isinf(Lp[2:, 1]).all() and (Lp[2:, 1] < 0).all()
    assert float(Op[2:, 1].abs().max()) == 0.0
    assert torch.isfinite(Lp[:, 0]).all()


def test_closed_forms():
    B, S, Lq, Hq, Hkv, D = 2, 12, 3, 2, 2, 4
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=7)
    O, L = decode_ref(q[:, :1], k, v, [1, 1])                 # one key in the cache
    assert torch.allclose(O[:, 0], v[:, 0].double(), atol=1e-12)
    O, L = decode_ref(q, k, v, window=1)                      # each query sees itself only
    for t in range(Lq):
        assert torch.allclose(O[:, t], v[:, S - Lq + t].double(), atol=1e-12)


def test_planted_mistake_is_caught():
    # placing the queries one position early drops the newest key from the last query
    B, S, Lq, Hq, Hkv, D = 1, 20, 1, 2, 1, 8
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=8)
    O, _ = decode_ref(q, k, v)
    wrong, _ = block_attention_ref(q, k, v, [S - 2], list(range(S)), scale=D ** -0.5, causal=True, window=0,
                                   n_sink=0)
    assert not torch.allclose(O, wrong, atol=1e-6)
