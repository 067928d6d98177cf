"""Float64 CPU reference for the backward pass of masked softmax attention and
its ring decomposition.

Test infrastructure only (see ``oracle/__init__``).

Long Context Attention notes, section "Ring Attention": the forward keeps Q,
K, V, the output and the log-sum-exp for the backward, and the backward runs
the same ring, the KV pieces (and their gradients) travelling between hosts.

The backward of O = softmax(S) V with S = scale * Q K^T (non-visible scores
-inf) is the chain rule written out, per (batch row, head):

    P     = exp(S - LSE)                 (LSE per query row)
    dV    = P^T dO
    dP    = dO V^T
    delta = rowsum(P * dP) = rowsum(dO * O)
    dS    = P * (dP - delta)
    dQ    = scale * dS K,     dK = scale * dS^T Q

With GQA / MQA, dK and dV of a KV head sum over the query heads that share it.
Because P uses the final LSE and delta, the terms of a ring step (one query
piece against one KV piece) add up over the steps: dQ of a host is the sum of
its steps' dQ, and dK / dV of a KV piece the sum over the hosts that saw it.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

from .attention_ref import apply_score_mods, visibility
from .index_ref import rank_positions
from .ring_ref import ring_forward_ref


def block_attention_bwd_ref(q_loc: torch.Tensor, k_loc: torch.Tensor, v_loc: torch.Tensor,
                            dout_loc: torch.Tensor, lse_loc: torch.Tensor, delta_loc: torch.Tensor,
                            pos_q: Sequence[int], pos_k: Sequence[int], *, scale: float, causal: bool,
                            window: int, n_sink: int, cu_seqlens: Optional[Sequence[int]] = None,
                            softcap: float = 0.0, alibi_slopes: Optional[torch.Tensor] = None):
    """One ring step's gradient terms.  q_loc / dout_loc [B,Lq,Hq,D], k_loc /
    v_loc [B,Lk,Hkv,D], lse_loc / delta_loc [B,Hq,Lq] (the final LSE and delta
    of those query rows).  Returns (dq [B,Lq,Hq,D], dk [B,Lk,Hkv,D], dv) in
    float64.  With softcap the score is c * tanh(s / c), whose derivative
    1 - tanh^2 multiplies dS; the ALiBi bias is constant in q and k."""
    B, Lq, Hq, D = q_loc.shape
    Lk, Hkv = k_loc.shape[1], k_loc.shape[2]
    group = Hq // Hkv
    mask = visibility(torch.tensor(list(pos_q)), torch.tensor(list(pos_k)), causal=causal, window=window,
                      n_sink=n_sink, cu_seqlens=cu_seqlens)
    dq = torch.zeros((B, Lq, Hq, D), dtype=torch.float64)
    dk = torch.zeros((B, Lk, Hkv, D), dtype=torch.float64)
    dv = torch.zeros((B, Lk, Hkv, D), dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qh, kh, vh = q_loc[b, :, h].double(), k_loc[b, :, g].double(), v_loc[b, :, g].double()
            doh = dout_loc[b, :, h].double()
            lse = lse_loc[b, h].double().unsqueeze(1)
            delta = delta_loc[b, h].double().unsqueeze(1)
            s = (qh @ kh.T) * scale
            t = torch.tanh(s / softcap) if softcap > 0 else None
            if softcap > 0 or alibi_slopes is not None:
                s = apply_score_mods(s.unsqueeze(0), torch.tensor(list(pos_q)), torch.tensor(list(pos_k)),
                                     softcap=softcap,
                                     alibi_slopes=None if alibi_slopes is None else alibi_slopes[h:h + 1])[0]
            # rows with no visible key anywhere have LSE = -inf: P = 0 there
            lse_safe = torch.where(torch.isfinite(lse), lse, torch.zeros_like(lse))
            p = torch.where(mask & torch.isfinite(lse), torch.exp(s - lse_safe), torch.zeros_like(s))
            dv[b, :, g] += p.T @ doh
            dp = doh @ vh.T
            ds = p * (dp - delta)
            if t is not None:
                ds = ds * (1.0 - t * t)
            dq[b, :, h] = scale * (ds @ kh)
            dk[b, :, g] += scale * (ds.T @ qh)
    return dq, dk, dv


def attention_bwd_ref(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, *,
                      softmax_scale: Optional[float] = None, causal: bool = False, window: int = 0,
                      n_sink: int = 0, cu_seqlens: Optional[Sequence[int]] = None, softcap: float = 0.0,
                      alibi_slopes: Optional[torch.Tensor] = None):
    """Unpartitioned gradients of natural-order attention ([B,S,H,D], or varlen
    [T,H,D] with cu_seqlens).  Returns (dq, dk, dv, O, LSE) in float64."""
    varlen = cu_seqlens is not None
    qb, kb, vb, db = (t.unsqueeze(0) if varlen else t for t in (q, k, v, dout))
    B, S, Hq, D = qb.shape
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    O, LSE = ring_forward_ref(qb[0] if varlen else qb, kb[0] if varlen else kb, vb[0] if varlen else vb,
                              impl="basic", N=1, softmax_scale=scale, causal=causal, window=window,
                              n_sink=n_sink, cu_seqlens=cu_seqlens, softcap=softcap, alibi_slopes=alibi_slopes)
    Ob = O.unsqueeze(0) if varlen else O
    Lb = LSE.unsqueeze(0) if varlen else LSE
    delta = (db.double() * Ob).sum(-1).transpose(1, 2)               # [B,Hq,S]
    pos = list(range(S))
    dq, dk, dv = block_attention_bwd_ref(qb, kb, vb, db, Lb, delta, pos, pos, scale=scale, causal=causal,
                                         window=window, n_sink=n_sink, cu_seqlens=cu_seqlens, softcap=softcap,
                                         alibi_slopes=alibi_slopes)
    if varlen:
        dq, dk, dv = dq[0], dk[0], dv[0]
    return dq, dk, dv, O, LSE


def ring_backward_ref(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, *, impl: str,
                      N: int, stripe_block: int = 1, softmax_scale: Optional[float] = None,
                      causal: bool = False, window: int = 0, n_sink: int = 0,
                      cu_seqlens: Optional[Sequence[int]] = None, softcap: float = 0.0,
                      alibi_slopes: Optional[torch.Tensor] = None):
    """The backward run as the ring runs the forward: host i, round s, KV piece
    j = (i - s) mod N; each step's dQ stays on host i, its dK / dV belong to
    piece j.  Natural-order (dq, dk, dv) in float64."""
    varlen = cu_seqlens is not None
    qb, kb, vb, db = (t.unsqueeze(0) if varlen else t for t in (q, k, v, dout))
    B, S, Hq, D = qb.shape
    Hkv = kb.shape[2]
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    O, LSE = ring_forward_ref(q, k, v, impl=impl, N=N, stripe_block=stripe_block, softmax_scale=scale,
                              causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu_seqlens, softcap=softcap,
                              alibi_slopes=alibi_slopes)
    Ob = O.unsqueeze(0) if varlen else O
    Lb = LSE.unsqueeze(0) if varlen else LSE
    delta = (db.double() * Ob).sum(-1).transpose(1, 2)
    pos = [rank_positions(impl, S, N, r, stripe_block) for r in range(N)]
    dq = torch.zeros((B, S, Hq, D), dtype=torch.float64)
    dk = torch.zeros((B, S, Hkv, D), dtype=torch.float64)
    dv = torch.zeros((B, S, Hkv, D), dtype=torch.float64)
    for i in range(N):
        for s in range(N):
            j = (i - s) % N
            gq, gk, gv = block_attention_bwd_ref(qb[:, pos[i]], kb[:, pos[j]], vb[:, pos[j]], db[:, pos[i]],
                                                 Lb[:, :, pos[i]], delta[:, :, pos[i]], pos[i], pos[j],
                                                 scale=scale, causal=causal, window=window, n_sink=n_sink,
                                                 cu_seqlens=cu_seqlens, softcap=softcap, alibi_slopes=alibi_slopes)
            dq[:, pos[i]] += gq
            dk[:, pos[j]] += gk
            dv[:, pos[j]] += gv
    if varlen:
        dq, dk, dv = dq[0], dk[0], dv[0]
    return dq, dk, dv
