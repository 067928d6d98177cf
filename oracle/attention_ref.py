"""The definition: naive masked softmax attention in float64 on global positions.

Test infrastructure only (see ``oracle/__init__``).

What is computed, for batch row b, query head h and query position p_q:

    s_k   = scale * sum_d q[b,p_q,h,d] * k[b,p_k,g(h),d]     (float64)
    s_k   = -inf where key p_k is not visible from p_q
    m     = max_k s_k,   l = sum_k exp(s_k - m)
    O     = sum_k exp(s_k - m) * v[b,p_k,g(h),:] / l
    LSE   = m + ln l                    (natural log; -inf and O = 0 if no key)

with g(h) = h // (Hq // Hkv) (contiguous GQA/MQA groups) and scale defaulting
to 1/sqrt(D) (ring sliding-window README, argument ``softmax_scale``).  The
log-sum-exp is the per-row statistic the Long Context Attention notes list
among what must be kept ("Motivation": QKV, output, LSE and dout).

Visibility of key p_k from query p_q (``visibility``):
  * same sequence: with ``cu_seqlens`` (global over the whole packed batch,
    ring sliding-window README, varlen section) both positions lie in the
    same [cu[i], cu[i+1]); otherwise the batch row is the sequence;
  * causal (YunChang README, "2. Usage": zigzag/stripe balance causal=True):
    p_k <= p_q;
  * sliding window of W keys (ring sliding-window README, ``window_size``:
    the number of tokens each query attends to): p_q - W < p_k <= p_q, i.e.
    the query itself and the W-1 before it, so each query sees min(W, p+1)
    keys of its sequence;
  * attention sink (ring sliding-window README, streaming-LLM section: every
    query also attends to the first token): with ``n_sink`` sinks, keys whose
    offset from their sequence start is < n_sink are visible as well (still
    p_k <= p_q).  A window implies the causal band.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import torch


def seq_index(pos: torch.Tensor, cu_seqlens: Optional[Sequence[int]]) -> torch.Tensor:
    """Index of the packed sequence each position belongs to (0 if not varlen)."""
    if cu_seqlens is None:
        return torch.zeros_like(pos)
    cu = torch.tensor(list(cu_seqlens), dtype=torch.long)
    return torch.searchsorted(cu, pos, right=True) - 1


def visibility(pos_q: torch.Tensor, pos_k: torch.Tensor, *, causal: bool, window: int,
               n_sink: int, cu_seqlens: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Boolean [len(pos_q), len(pos_k)]: True where key pos_k[j] is visible from query pos_q[i]."""
    pq = pos_q.long()[:, None]
    pk = pos_k.long()[None, :]
    sq = seq_index(pos_q.long(), cu_seqlens)
    sk = seq_index(pos_k.long(), cu_seqlens)
    vis = sq[:, None] == sk[None, :]
    if causal or window > 0:
        vis &= pk <= pq
    if window > 0:
        if cu_seqlens is None:
            start_q = torch.zeros_like(pq)
        else:
            cu = torch.tensor(list(cu_seqlens), dtype=torch.long)
            start_q = cu[sq][:, None]
        in_window = (pq - pk) < window
        is_sink = (pk - start_q) < n_sink
        vis &= in_window | is_sink
    return vis


def apply_score_mods(s: torch.Tensor, pos_q: torch.Tensor, pos_k: torch.Tensor, *, softcap: float = 0.0,
                     alibi_slopes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The score modifiers of the attention call (YunChang README, "2. Usage": ``softcap`` and
    ``alibi_slopes`` arguments, read with flash-attention's meaning): scaled scores s [H,r,K] of the
    heads whose slopes are given ([H]) become softcap * tanh(s / softcap) when softcap > 0, then
    minus slope_h * |p_q - p_k| on global positions."""
    if softcap > 0:
        s = softcap * torch.tanh(s / softcap)
    if alibi_slopes is not None:
        dist = (pos_q.long()[:, None] - pos_k.long()[None, :]).abs().to(torch.float64)      # [r,K]
        s = s - alibi_slopes.to(torch.float64).view(-1, 1, 1) * dist.unsqueeze(0)
    return s


def _as_batched(x: torch.Tensor, varlen: bool) -> torch.Tensor:
    return x.unsqueeze(0) if varlen else x


def attention_ref(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                  softmax_scale: Optional[float] = None, causal: bool = False,
                  window: int = 0, n_sink: int = 0,
                  cu_seqlens: Optional[Sequence[int]] = None,
                  rows: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None,
                  softcap: float = 0.0, alibi_slopes: Optional[torch.Tensor] = None,
                  block_bytes: int = 1 << 28):
    """Masked softmax attention in float64 over natural-order tensors.

    q [B,S,Hq,D], k/v [B,S,Hkv,D]; with ``cu_seqlens`` q is [T,Hq,D] and k/v
    [T,Hkv,D].  ``rows`` restricts the computation to those query positions,
    ``heads`` to those query heads (outputs keep that order).  ``softcap`` and
    ``alibi_slopes`` ([Hq]) modify the scaled scores (apply_score_mods).

    Returns (O, LSE) in float64: O [B,R,H',D] and LSE [B,H',R]; varlen drops B.
    """
    varlen = cu_seqlens is not None
    qb = _as_batched(q, varlen)
    kb = _as_batched(k, varlen)
    vb = _as_batched(v, varlen)
    B, S, Hq, D = qb.shape
    Hkv = kb.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if varlen and (cu_seqlens[0] != 0 or cu_seqlens[-1] != S):
        raise ValueError("cu_seqlens must start at 0 and end at the total length")
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    rows_t = torch.arange(S) if rows is None else torch.tensor(list(rows), dtype=torch.long)
    heads_t = torch.arange(Hq) if heads is None else torch.tensor(list(heads), dtype=torch.long)
    group = Hq // Hkv
    kv_head = heads_t // group
    R = rows_t.numel()
    H = heads_t.numel()
    O = torch.zeros((B, R, H, D), dtype=torch.float64)
    LSE = torch.full((B, H, R), -math.inf, dtype=torch.float64)
    pos_k_all = torch.arange(S)
    rb = max(1, min(R, block_bytes // max(1, H * S * 8)))
    for b in range(B):
        kh = kb[b].index_select(1, kv_head).to(torch.float64).permute(1, 0, 2)   # [H,S,D]
        vh = vb[b].index_select(1, kv_head).to(torch.float64).permute(1, 0, 2)   # [H,S,D]
        for r0 in range(0, R, rb):
            pr = rows_t[r0:r0 + rb]
            mask = visibility(pr, pos_k_all, causal=causal, window=window,
                              n_sink=n_sink, cu_seqlens=cu_seqlens)          # [r,S]
            cols = torch.nonzero(mask.any(0)).flatten()
            if cols.numel() == 0:
                continue
            k_lo, k_hi = int(cols[0]), int(cols[-1]) + 1    # invisible columns add exp(-inf)=0
            qh = qb[b, pr][:, heads_t].to(torch.float64).permute(1, 0, 2)      # [H,r,D]
            s = torch.matmul(qh, kh[:, k_lo:k_hi].transpose(1, 2)) * scale     # [H,r,K]
            if softcap > 0 or alibi_slopes is not None:
                s = apply_score_mods(s, pr, pos_k_all[k_lo:k_hi], softcap=softcap,
                                     alibi_slopes=None if alibi_slopes is None else alibi_slopes[heads_t])
            s = s.masked_fill(~mask[:, k_lo:k_hi].unsqueeze(0), -math.inf)
            m = s.amax(dim=2, keepdim=True)
            has = torch.isfinite(m)
            m_safe = torch.where(has, m, torch.zeros_like(m))
            e = torch.exp(s - m_safe)
            l = e.sum(dim=2, keepdim=True)
            o = torch.matmul(e, vh[:, k_lo:k_hi]) / torch.where(has, l, torch.ones_like(l))
            lse = torch.where(has, m_safe + torch.log(l), torch.full_like(l, -math.inf))
            O[b, r0:r0 + pr.numel()] = torch.where(has, o, torch.zeros_like(o)).permute(1, 0, 2)
            LSE[b, :, r0:r0 + pr.numel()] = lse.squeeze(2)
    if varlen:
        return O[0], LSE[0]
    return O, LSE


def visible_pair_count(S: int, *, causal: bool, window: int, n_sink: int,
                       cu_seqlens: Optional[Sequence[int]] = None, block: int = 1024) -> int:
    """Number of visible (query, key) pairs for one (batch row, head)."""
    pos = torch.arange(S)
    total = 0
    for r0 in range(0, S, block):
        total += int(visibility(pos[r0:r0 + block], pos, causal=causal, window=window,
                                n_sink=n_sink, cu_seqlens=cu_seqlens).sum())
    return total
