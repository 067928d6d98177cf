"""Pins of the backward oracle (oracle/backward_ref.py).

- torch autograd through scaled_dot_product_attention in float64 on the CPU
  (a library routine differentiating the forward definition, independent of
  the hand-derived formulas), every mask kind;
- central finite differences of <O, dO> on tiny inputs (brute force);
- the ring decomposition (every layout, GQA, window, sinks, varlen) summing to
  the unpartitioned gradients;
- closed forms: dO = 0 gives zero gradients; a window of 1 gives dQ = dK = 0,
  dV = dO; GQA gradients of a shared KV head equal the sum over its query
  heads of the gradients with the KV head copied per query head.
"""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle.attention_ref import visibility  # noqa: E402
from oracle.backward_ref import attention_bwd_ref, block_attention_bwd_ref, ring_backward_ref  # noqa: E402


def _rand(*shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _autograd(q, k, v, dout, scale, causal, window, n_sink, cu_seqlens=None):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    pos = torch.arange(S)
    mask = visibility(pos, pos, causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu_seqlens)
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    ke = kg.repeat_interleave(Hq // Hkv, dim=2)
    ve = vg.repeat_interleave(Hq // Hkv, dim=2)
    o = torch.nn.functional.scaled_dot_product_attention(
        qg.transpose(1, 2), ke.transpose(1, 2), ve.transpose(1, 2), attn_mask=mask, scale=scale)
    o = o.transpose(1, 2)
    (o * dout).sum().backward()
    return qg.grad, kg.grad, vg.grad


MASKS = [dict(causal=False, window=0, n_sink=0), dict(causal=True, window=0, n_sink=0),
         dict(causal=False, window=5, n_sink=0), dict(causal=False, window=4, n_sink=2)]


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: f"c{int(m['causal'])}w{m['window']}s{m['n_sink']}")
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_matches_autograd(mask, hq, hkv):
    B, S, D = 2, 23, 8
    q, k, v, do = _rand(B, S, hq, D, seed=1), _rand(B, S, hkv, D, seed=2), _rand(B, S, hkv, D, seed=3), \
        _rand(B, S, hq, D, seed=4)
    scale = 0.37
    dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, do, softmax_scale=scale, **mask)
    aq, ak, av = _autograd(q, k, v, do, scale, **mask)
    for a, b in ((dq, aq), (dk, ak), (dv, av)):
        assert torch.allclose(a, b, atol=1e-10, rtol=1e-10), float((a - b).abs().max())


def test_matches_autograd_varlen():
    S, H, D = 30, 2, 4
    cu = [0, 7, 19, 30]
    q, k, v, do = (_rand(1, S, H, D, seed=s) for s in (5, 6, 7, 8))
    dq, dk, dv, _, _ = attention_bwd_ref(q[0], k[0], v[0], do[0], softmax_scale=0.5, window=6, n_sink=2,
                                         cu_seqlens=cu)
    aq, ak, av = _autograd(q, k, v, do, 0.5, False, 6, 2, cu_seqlens=cu)
    for a, b in ((dq, aq[0]), (dk, ak[0]), (dv, av[0])):
        assert torch.allclose(a, b, atol=1e-10, rtol=1e-10)


def test_finite_differences():
    B, S, H, D = 1, 6, 1, 3
    q, k, v, do = (_rand(B, S, H, D, seed=s) for s in (11, 12, 13, 14))
    scale, kw = 0.8, dict(causal=True, window=0, n_sink=0)
    dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, do, softmax_scale=scale, **kw)

    def loss(q_, k_, v_):
        from oracle.attention_ref import attention_ref
        o, _ = attention_ref(q_, k_, v_, softmax_scale=scale, **kw)
        return float((o * do).sum())

    h = 1e-6
    for name, t, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0, 0), (0, 3, 0, 1), (0, 5, 0, 2)]:
            tp, tm = t.clone(), t.clone()
            tp[idx] += h
            tm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = tp, tm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - float(g[idx])) < 1e-6, (name, idx, fd, float(g[idx]))


@pytest.mark.parametrize("impl,N,b,kw", [
    ("zigzag", 4, 1, dict(causal=True)),
    ("stripe", 3, 1, dict(causal=True)),
    ("stripe", 2, 3, dict(causal=True)),
    ("basic", 4, 1, dict(causal=False, window=9)),
    ("basic", 2, 1, dict(causal=False, window=7, n_sink=3)),
])
def test_ring_decomposition_sums_to_full(impl, N, b, kw):
    B, S, Hq, Hkv, D = 1, 48, 4, 2, 4
    q, do = _rand(B, S, Hq, D, seed=21), _rand(B, S, Hq, D, seed=24)
    k, v = _rand(B, S, Hkv, D, seed=22), _rand(B, S, Hkv, D, seed=23)
    full = attention_bwd_ref(q, k, v, do, softmax_scale=0.4, **kw)[:3]
    ring = ring_backward_ref(q, k, v, do, impl=impl, N=N, stripe_block=b, softmax_scale=0.4, **kw)
    for a, r in zip(full, ring):
        assert torch.allclose(a, r, atol=1e-12, rtol=1e-12)


def test_ring_decomposition_varlen():
    S, H, D = 40, 2, 4
    cu = [0, 9, 25, 40]
    q, k, v, do = (_rand(S, H, D, seed=s) for s in (31, 32, 33, 34))
    full = attention_bwd_ref(q, k, v, do, window=6, n_sink=2, cu_seqlens=cu)[:3]
    ring = ring_backward_ref(q, k, v, do, impl="basic", N=4, window=6, n_sink=2, cu_seqlens=cu)
    for a, r in zip(full, ring):
        assert torch.allclose(a, r, atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("impl,N,b", [("zigzag", 4, 1), ("stripe", 2, 3)])
def test_ring_decomposition_varlen_any_layout(impl, N, b):
    S, H, D = 48, 2, 4
    cu = [0, 9, 25, 48]
    q, k, v, do = (_rand(S, H, D, seed=s) for s in (35, 36, 37, 38))
    full = attention_bwd_ref(q, k, v, do, causal=True, cu_seqlens=cu)[:3]
    ring = ring_backward_ref(q, k, v, do, impl=impl, N=N, stripe_block=b, causal=True, cu_seqlens=cu)
    for a, r in zip(full, ring):
        assert torch.allclose(a, r, atol=1e-12, rtol=1e-12)


def test_zero_upstream_gradient():
    q, k, v = (_rand(1, 10, 2, 4, seed=s) for s in (41, 42, 43))
    grads = attention_bwd_ref(q, k, v, torch.zeros(1, 10, 2, 4, dtype=torch.float64), causal=True)[:3]
    assert all(float(g.abs().max()) == 0.0 for g in grads)


def test_window_one_closed_form():
    # each query sees only itself: P = 1, so dV = dO, and dS = P (dP - delta) = 0
    q, k, v, do = (_rand(2, 9, 3, 4, seed=s) for s in (51, 52, 53, 54))
    dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, do, window=1)
    assert float(dq.abs().max()) < 1e-12 and float(dk.abs().max()) < 1e-12
    assert torch.allclose(dv, do, atol=1e-12)


def test_gqa_sums_over_group():
    B, S, Hq, Hkv, D = 1, 12, 4, 2, 4
    q, do = _rand(B, S, Hq, D, seed=61), _rand(B, S, Hq, D, seed=64)
    k, v = _rand(B, S, Hkv, D, seed=62), _rand(B, S, Hkv, D, seed=63)
    dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, do, causal=True)
    ke, ve = k.repeat_interleave(2, dim=2), v.repeat_interleave(2, dim=2)
    eq, ek, ev, _, _ = attention_bwd_ref(q, ke, ve, do, causal=True)
    assert torch.allclose(dq, eq, atol=1e-12)
    assert torch.allclose(dk, ek.view(B, S, Hkv, 2, D).sum(3), atol=1e-12)
    assert torch.allclose(dv, ev.view(B, S, Hkv, 2, D).sum(3), atol=1e-12)


def test_planted_mistake_is_caught():
    # dropping delta (dS = P * dP) must break the autograd pin
    B, S, H, D = 1, 11, 2, 4
    q, k, v, do = (_rand(B, S, H, D, seed=s) for s in (71, 72, 73, 74))
    _, _, _, _, lse = attention_bwd_ref(q, k, v, do, causal=True)
    pos = list(range(S))
    wrong = block_attention_bwd_ref(q, k, v, do, lse, torch.zeros(B, H, S, dtype=torch.float64), pos, pos,
                                    scale=D ** -0.5, causal=True, window=0, n_sink=0)
    aq, _, _ = _autograd(q, k, v, do, D ** -0.5, True, 0, 0)
    assert not torch.allclose(wrong[0], aq, atol=1e-6)
