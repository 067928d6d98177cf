"""Pins of the score modifiers in the oracle (softcap, ALiBi; YunChang
README "2. Usage" passes ``softcap`` and ``alibi_slopes`` to the attention
call, read with flash-attention's meaning: softcap * tanh(s / softcap), then
minus slope_h * |p_q - p_k|).

- ALiBi against torch SDPA in float64 with the bias as an additive mask;
- softcap and ALiBi by scalar brute force on tiny inputs;
- limits: softcap -> infinity and slope 0 give plain attention; a steep
  causal ALiBi slope leaves each query its own value;
- the backward against autograd of an explicit float64 forward with tanh and
  the bias, for every mask kind;
- the ring decompositions (forward and backward) and decode with both
  modifiers equal the unpartitioned results;
- a planted mistake (bias sign flipped) fails.
"""
import math

import pytest
import torch

from oracle.attention_ref import attention_ref, visibility
from oracle.backward_ref import attention_bwd_ref, ring_backward_ref
from oracle.decode_ref import decode_ref, decode_split_ref, tree_merge_ref
from oracle.ring_ref import ring_forward_ref


def _rand(*shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


SLOPES = torch.tensor([0.5, 0.25, 0.125, 0.0625], dtype=torch.float64)


@pytest.mark.parametrize("kw", [dict(causal=True), dict(causal=False), dict(window=5, n_sink=2)])
def test_alibi_against_sdpa_additive_mask(kw):
    B, S, H, D = 2, 19, 4, 8
    q, k, v = (_rand(B, S, H, D, seed=s) for s in (1, 2, 3))
    O, L = attention_ref(q, k, v, softmax_scale=0.4, alibi_slopes=SLOPES, **kw)
    pos = torch.arange(S)
    vis = visibility(pos, pos, causal=kw.get("causal", False), window=kw.get("window", 0),
                     n_sink=kw.get("n_sink", 0))
    bias = -SLOPES.view(H, 1, 1) * (pos[:, None] - pos[None, :]).abs().double()       # [H,S,S]
    mask = bias.masked_fill(~vis, -math.inf)
    ref = torch.nn.functional.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2),
                                                           v.transpose(1, 2), attn_mask=mask, scale=0.4)
    assert torch.allclose(O, ref.transpose(1, 2), atol=1e-10)
    s = (q.transpose(1, 2) @ k.transpose(1, 2).transpose(2, 3)) * 0.4 + mask
    assert torch.allclose(L, torch.logsumexp(s, dim=-1), atol=1e-10)


def test_softcap_and_alibi_brute_force():
    S, H, D, cap = 6, 2, 3, 0.7
    q, k, v = (_rand(1, S, H, D, seed=s) for s in (4, 5, 6))
    slopes = torch.tensor([0.3, 0.9], dtype=torch.float64)
    O, L = attention_ref(q, k, v, softmax_scale=1.1, causal=True, softcap=cap, alibi_slopes=slopes)
    for h in range(H):
        for t in range(S):
            s = []
            for u in range(t + 1):
                x = 1.1 * math.fsum(float(q[0, t, h, d]) * float(k[0, u, h, d]) for d in range(D))
                s.append(cap * math.tanh(x / cap) - float(slopes[h]) * (t - u))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for d in range(D):
                o = math.fsum(w[u] * float(v[0, u, h, d]) for u in range(t + 1)) / z
                assert abs(o - float(O[0, t, h, d])) < 1e-12
            assert abs(m + math.log(z) - float(L[0, h, t])) < 1e-12


def test_limits():
    B, S, H, D = 1, 16, 4, 8
    q, k, v = (_rand(B, S, H, D, seed=s) for s in (7, 8, 9))
    O0, L0 = attention_ref(q, k, v, causal=True)
    O1, L1 = attention_ref(q, k, v, causal=True, softcap=1e5)
    assert torch.allclose(O0, O1, atol=1e-8) and torch.allclose(L0, L1, atol=1e-8)
    O2, L2 = attention_ref(q, k, v, causal=True, alibi_slopes=torch.zeros(H, dtype=torch.float64))
    assert torch.equal(O0, O2) and torch.equal(L0, L2)
    O3, _ = attention_ref(q, k, v, causal=True, alibi_slopes=torch.full((H,), 200.0, dtype=torch.float64))
    assert torch.allclose(O3, v.double(), atol=1e-12)       # each query keeps its own value


@pytest.mark.parametrize("kw", [dict(causal=True), dict(causal=False), dict(window=4, n_sink=1)])
def test_backward_against_autograd(kw):
    B, S, H, D, cap, scale = 1, 13, 4, 8, 1.5, 0.45
    q, k, v, do = (_rand(B, S, H, D, seed=s) for s in (11, 12, 13, 14))
    dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, do, softmax_scale=scale, softcap=cap, alibi_slopes=SLOPES, **kw)
    pos = torch.arange(S)
    vis = visibility(pos, pos, causal=kw.get("causal", False), window=kw.get("window", 0),
                     n_sink=kw.get("n_sink", 0))
    bias = -SLOPES.view(H, 1, 1) * (pos[:, None] - pos[None, :]).abs().double()
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    s = (qg.transpose(1, 2) @ kg.transpose(1, 2).transpose(2, 3)) * scale           # [B,H,S,S]
    s = cap * torch.tanh(s / cap) + bias
    s = s.masked_fill(~vis, -math.inf)
    o = torch.softmax(s, dim=-1) @ vg.transpose(1, 2)
    (o.transpose(1, 2) * do).sum().backward()
    for a, b in ((dq, qg.grad), (dk, kg.grad), (dv, vg.grad)):
        assert torch.allclose(a, b, atol=1e-10), float((a - b).abs().max())


@pytest.mark.parametrize("impl,N,b", [("zigzag", 4, 1), ("stripe", 2, 3), ("basic", 3, 1)])
def test_ring_with_mods_equals_full(impl, N, b):
    B, S, Hq, Hkv, D = 1, 48, 4, 2, 8
    q = _rand(B, S, Hq, D, seed=21)
    k, v = _rand(B, S, Hkv, D, seed=22), _rand(B, S, Hkv, D, seed=23)
    do = _rand(B, S, Hq, D, seed=24)
    kw = dict(causal=True, softcap=2.0, alibi_slopes=SLOPES)
    O, L = attention_ref(q, k, v, **kw)
    Or, Lr = ring_forward_ref(q, k, v, impl=impl, N=N, stripe_block=b, **kw)
    assert torch.allclose(O, Or, atol=1e-12) and torch.allclose(L, Lr, atol=1e-12)
    full = attention_bwd_ref(q, k, v, do, **kw)[:3]
    ring = ring_backward_ref(q, k, v, do, impl=impl, N=N, stripe_block=b, **kw)
    for a, r in zip(full, ring):
        assert torch.allclose(a, r, atol=1e-12)


def test_decode_with_mods_equals_full_rows():
    B, S, Lq, Hq, Hkv, D = 2, 40, 2, 4, 2, 8
    q = _rand(B, Lq, Hq, D, seed=31)
    k, v = _rand(B, S, Hkv, D, seed=32), _rand(B, S, Hkv, D, seed=33)
    qf = _rand(B, S, Hq, D, seed=34)
    qf[:, S - Lq:] = q
    kw = dict(softcap=3.0, alibi_slopes=SLOPES)
    O, L = decode_ref(q, k, v, **kw)
    Of, Lf = attention_ref(qf, k, v, causal=True, rows=list(range(S - Lq, S)), **kw)
    assert torch.allclose(O, Of, atol=1e-12) and torch.allclose(L, Lf, atol=1e-12)
    Ot, Lt = tree_merge_ref(*decode_split_ref(q, k, v, split_keys=7, **kw))
    assert torch.allclose(Ot, O, atol=1e-12) and torch.allclose(Lt, L, atol=1e-12)


def test_planted_mistake_is_caught():
    B, S, H, D = 1, 12, 4, 8
    q, k, v = (_rand(B, S, H, D, seed=s) for s in (41, 42, 43))
    O, _ = attention_ref(q, k, v, causal=True, alibi_slopes=SLOPES)
    wrong, _ = attention_ref(q, k, v, causal=True, alibi_slopes=-SLOPES)
    assert not torch.allclose(O, wrong, atol=1e-3)
