"""Pins for oracle/ring_ref: the ring decomposition and the partial merge.

* the ring-decomposed result equals unpartitioned attention (notes, section
  "Ring Attention": the pass completes once every host saw every KV piece;
  block order is free) for every layout, ring size and mask kind;
* the merge is order- and tree-shape independent (notes, section "Tree
  Attention": max and logsumexp are associative);
* a partial with no visible key is (0, -inf) and leaves the other unchanged;
* N = 1 is plain attention.
"""
import math
import random

import pytest
import torch

from oracle import index_ref as ix
from oracle.attention_ref import attention_ref
from oracle.ring_ref import block_attention_ref, merge_ref, ring_forward_ref


def _inputs(B, S, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    return q, k, v


def _close(a, b, tol=1e-12):
    assert torch.equal(torch.isinf(a), torch.isinf(b))
    fa, fb = a[torch.isfinite(a)], b[torch.isfinite(b)]
    assert torch.allclose(fa, fb, atol=tol, rtol=0)


@pytest.mark.parametrize("impl,b", [("basic", 1), ("zigzag", 1), ("stripe", 1), ("stripe", 2)])
@pytest.mark.parametrize("N", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_equals_full_attention(impl, b, N, causal):
    unit = {"basic": N, "zigzag": 2 * N, "stripe": N * b}[impl]
    S = unit * 4
    q, k, v = _inputs(2, S, 4, 2, 8, seed=N * 10 + (impl == "zigzag"))
    O, L = attention_ref(q, k, v, causal=causal)
    Or, Lr = ring_forward_ref(q, k, v, impl=impl, N=N, stripe_block=b, causal=causal)
    _close(O, Or)
    _close(L, Lr)


@pytest.mark.parametrize("impl", ["basic", "zigzag", "stripe"])
@pytest.mark.parametrize("window,n_sink", [(5, 0), (7, 2), (3, 4)])
def test_ring_window_sink_equals_full(impl, window, n_sink):
    N = 4
    S = 32
    q, k, v = _inputs(1, S, 2, 1, 8, seed=window + n_sink)
    O, L = attention_ref(q, k, v, window=window, n_sink=n_sink)
    Or, Lr = ring_forward_ref(q, k, v, impl=impl, N=N, window=window, n_sink=n_sink)
    _close(O, Or)
    _close(L, Lr)


def test_ring_varlen_equals_full():
    cu = [0, 5, 19, 20, 32]
    q, k, v = _inputs(1, 32, 4, 4, 8, seed=31)
    O, L = attention_ref(q[0], k[0], v[0], window=6, n_sink=2, cu_seqlens=cu)
    Or, Lr, parts = ring_forward_ref(q[0], k[0], v[0], impl="basic", N=4, window=6, n_sink=2,
                                     cu_seqlens=cu, return_partials=True)
    _close(O, Or)
    _close(L, Lr)
    # some steps have no visible key for some rows: their partial is (0, -inf)
    saw_empty = False
    for steps in parts:
        for (_j, Os, Ls) in steps:
            empty = torch.isinf(Ls)                    # [B,H,L]
            if empty.any():
                saw_empty = True
                assert (Ls[empty] < 0).all()
                assert (Os.transpose(1, 2)[empty] == 0).all()
    assert saw_empty


@pytest.mark.parametrize("impl,N,b", [("zigzag", 4, 1), ("zigzag", 2, 1), ("stripe", 4, 1), ("stripe", 2, 3)])
@pytest.mark.parametrize("kw", [dict(causal=True), dict(window=6, n_sink=2), dict()])
def test_ring_varlen_any_layout_equals_full(impl, N, b, kw):
    # the ring layout applied to the packed token axis, masks from global positions
    cu = [0, 5, 19, 20, 48]
    q, k, v = _inputs(1, 48, 4, 2, 8, seed=32)
    O, L = attention_ref(q[0], k[0], v[0], cu_seqlens=cu, **kw)
    Or, Lr = ring_forward_ref(q[0], k[0], v[0], impl=impl, N=N, stripe_block=b, cu_seqlens=cu, **kw)
    _close(O, Or)
    _close(L, Lr)


def test_ring_one_host_is_plain_attention():
    q, k, v = _inputs(1, 12, 2, 2, 8, seed=37)
    O, L = attention_ref(q, k, v, causal=True)
    Or, Lr = ring_forward_ref(q, k, v, impl="zigzag", N=1, causal=True)
    assert torch.equal(O, Or) and torch.equal(L, Lr)


def _random_partials(n, B=1, L=7, H=3, D=5, seed=0, empties=True):
    g = torch.Generator().manual_seed(seed)
    parts = []
    for i in range(n):
        o = torch.randn(B, L, H, D, generator=g, dtype=torch.float64)
        lse = torch.randn(B, H, L, generator=g, dtype=torch.float64) * 3
        if empties:
            dead = torch.rand(B, H, L, generator=g) < 0.25
            lse = lse.masked_fill(dead, -math.inf)
            o = o.masked_fill(dead.transpose(1, 2).unsqueeze(-1), 0.0)
        parts.append((o, lse))
    return parts


def _reduce_tree(parts, rng):
    parts = list(parts)
    while len(parts) > 1:
        i = rng.randrange(len(parts) - 1)
        a, b = parts[i], parts[i + 1]
        parts[i:i + 2] = [merge_ref(a[0], a[1], b[0], b[1])]
    return parts[0]


def test_merge_is_order_and_tree_independent():
    parts = _random_partials(6, seed=41)
    ref = parts[0]
    for p in parts[1:]:
        ref = merge_ref(ref[0], ref[1], p[0], p[1])
    # closed form of the merged result: LSE = log sum exp over partials, O = weighted mean
    lse_stack = torch.stack([p[1] for p in parts])
    lse_cf = torch.logsumexp(lse_stack, dim=0)
    _close(ref[1], lse_cf)
    rng = random.Random(5)
    for _ in range(20):
        order = list(parts)
        rng.shuffle(order)
        out = _reduce_tree(order, rng)
        _close(out[0], ref[0])
        _close(out[1], ref[1])


def test_merge_with_empty_partial_is_identity():
    (o, lse), = _random_partials(1, seed=43, empties=False)
    empty_o = torch.zeros_like(o)
    empty_l = torch.full_like(lse, -math.inf)
    mo, ml = merge_ref(o, lse, empty_o, empty_l)
    assert torch.allclose(mo, o, atol=1e-15, rtol=0) and torch.equal(ml, lse)
    mo, ml = merge_ref(empty_o, empty_l, o, lse)
    assert torch.allclose(mo, o, atol=1e-15, rtol=0) and torch.equal(ml, lse)
    mo, ml = merge_ref(empty_o, empty_l, empty_o, empty_l)
    assert (mo == 0).all() and torch.isinf(ml).all()


def test_merge_of_split_keys_is_attention():
    # splitting the keys of one softmax into two partials and merging gives the whole
    q, k, v = _inputs(1, 16, 2, 2, 8, seed=47)
    pos = list(range(16))
    full = block_attention_ref(q, k, v, pos, pos, scale=0.3, causal=True, window=0, n_sink=0)
    a = block_attention_ref(q, k[:, :9], v[:, :9], pos, pos[:9], scale=0.3, causal=True, window=0, n_sink=0)
    b = block_attention_ref(q, k[:, 9:], v[:, 9:], pos, pos[9:], scale=0.3, causal=True, window=0, n_sink=0)
    mo, ml = merge_ref(a[0], a[1], b[0], b[1])
    _close(mo, full[0])
    _close(ml, full[1])


def test_usp_one_rank_share_slices_full_attention():
    # one global rank's share: its ring rank's rows, its ulysses head group
    S, Hq, Hkv, D, rd, ud = 32, 4, 2, 8, 2, 2
    q, k, v = _inputs(1, S, Hq, Hkv, D, seed=53)
    O, L = attention_ref(q, k, v, causal=True)
    for r in range(rd):
        rows = ix.rank_positions("zigzag", S, rd, r)
        for u in range(ud):
            heads = list(range(u * Hq // ud, (u + 1) * Hq // ud))
            Os, Ls = attention_ref(q, k, v, causal=True, rows=rows, heads=heads)
            _close(Os, O[:, rows][:, :, heads])
            _close(Ls, L[:, heads][:, :, rows])
