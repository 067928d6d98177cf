"""Ring-decomposed float64 reference: per-step partials and their merge.

Test infrastructure only (see ``oracle/__init__``).

Long Context Attention notes, section "Ring Attention": the sequence is cut
into N pieces on N hosts that form a ring and pass KV pieces around it; the
order in which the blocks are computed is free, and the pass is complete once
every host has seen every KV piece.  Section "Tree Attention": the softmax's
max and logsumexp are associative, so partial results combine in any order.

Here host i holds query piece i; at round s it holds the KV piece of host
j = (i - s) mod N (the KV moves one host along the ring per round), computes
the block's partial (O_s, LSE_s) with the mask that the global positions of
its rows and keys imply, and folds it into its running result with

    M = max(L_a, L_b),   L = M + ln(exp(L_a - M) + exp(L_b - M)),
    O = exp(L_a - L) * O_a + exp(L_b - L) * O_b,

a partial with L = -inf (no visible key) leaving the other unchanged.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import torch

from .attention_ref import apply_score_mods, visibility
from .index_ref import rank_positions


def block_attention_ref(q_loc: torch.Tensor, k_loc: torch.Tensor, v_loc: torch.Tensor,
                        pos_q: Sequence[int], pos_k: Sequence[int], *, scale: float,
                        causal: bool, window: int, n_sink: int,
                        cu_seqlens: Optional[Sequence[int]] = None, softcap: float = 0.0,
                        alibi_slopes: Optional[torch.Tensor] = None):
    """One ring step: q_loc [B,Lq,Hq,D] against k_loc/v_loc [B,Lk,Hkv,D] whose
    rows sit at global positions pos_q / pos_k.  Returns the partial
    (O [B,Lq,Hq,D], LSE [B,Hq,Lq]) in float64.  softcap / alibi_slopes ([Hq])
    as in attention_ref."""
    B, Lq, Hq, D = q_loc.shape
    Hkv = k_loc.shape[2]
    group = Hq // Hkv
    mask = visibility(torch.tensor(list(pos_q)), torch.tensor(list(pos_k)),
                      causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu_seqlens)
    O = torch.zeros((B, Lq, Hq, D), dtype=torch.float64)
    LSE = torch.full((B, Hq, Lq), -math.inf, dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            qh = q_loc[b, :, h].double()              # [Lq,D]
            kh = k_loc[b, :, h // group].double()     # [Lk,D]
            vh = v_loc[b, :, h // group].double()
            s = (qh @ kh.T) * scale
            if softcap > 0 or alibi_slopes is not None:
                s = apply_score_mods(s.unsqueeze(0), torch.tensor(list(pos_q)), torch.tensor(list(pos_k)),
                                     softcap=softcap,
                                     alibi_slopes=None if alibi_slopes is None else alibi_slopes[h:h + 1])[0]
            s[~mask] = -math.inf
            live = mask.any(1)                        # rows with at least one visible key
            if not bool(live.any()):
                continue
            sl = s[live]
            m = sl.max(dim=1, keepdim=True).values
            p = torch.exp(sl - m)
            l = p.sum(dim=1, keepdim=True)
            O[b, live, h] = (p @ vh) / l
            LSE[b, h, live] = (m + torch.log(l)).squeeze(1)
    return O, LSE


def merge_ref(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor):
    """Associative combine of two partials.  o_* [B,L,H,D], lse_* [B,H,L]."""
    M = torch.maximum(lse_a, lse_b)
    M_safe = torch.where(torch.isfinite(M), M, torch.zeros_like(M))
    L = M_safe + torch.log(torch.exp(lse_a - M_safe) + torch.exp(lse_b - M_safe))
    L = torch.where(torch.isfinite(M), L, torch.full_like(L, -math.inf))
    L_safe = torch.where(torch.isfinite(L), L, torch.zeros_like(L))
    wa = torch.exp(lse_a - L_safe).transpose(1, 2).unsqueeze(-1)   # [B,L,H,1]
    wb = torch.exp(lse_b - L_safe).transpose(1, 2).unsqueeze(-1)
    O = wa * o_a + wb * o_b
    empty = ~torch.isfinite(L).transpose(1, 2).unsqueeze(-1)
    O = torch.where(empty, torch.zeros_like(O), O)
    return O, L


def ring_forward_ref(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, impl: str, N: int,
                     stripe_block: int = 1, softmax_scale: Optional[float] = None,
                     causal: bool = False, window: int = 0, n_sink: int = 0,
                     cu_seqlens: Optional[Sequence[int]] = None,
                     return_partials: bool = False, softcap: float = 0.0,
                     alibi_slopes: Optional[torch.Tensor] = None):
    """Virtual ring over N hosts on natural-order q/k/v ([B,S,H,D] or varlen
    [T,H,D]).  Returns the natural-order (O, LSE) in float64 and, if asked,
    partials[i][s] = (j, O_s, LSE_s) in host i's local order."""
    varlen = cu_seqlens is not None
    qb = q.unsqueeze(0) if varlen else q
    kb = k.unsqueeze(0) if varlen else k
    vb = v.unsqueeze(0) if varlen else v
    B, S, Hq, D = qb.shape
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    pos = [rank_positions(impl, S, N, r, stripe_block) for r in range(N)]
    O = torch.zeros((B, S, Hq, D), dtype=torch.float64)
    LSE = torch.full((B, Hq, S), -math.inf, dtype=torch.float64)
    partials: List[List[Tuple[int, torch.Tensor, torch.Tensor]]] = []
    for i in range(N):
        qi = qb[:, pos[i]]
        acc: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
        steps = []
        for s in range(N):
            j = (i - s) % N
            part = block_attention_ref(qi, kb[:, pos[j]], vb[:, pos[j]], pos[i], pos[j],
                                       scale=scale, causal=causal, window=window,
                                       n_sink=n_sink, cu_seqlens=cu_seqlens, softcap=softcap,
                                       alibi_slopes=alibi_slopes)
            steps.append((j, part[0], part[1]))
            acc = part if acc is None else merge_ref(acc[0], acc[1], part[0], part[1])
        partials.append(steps)
        O[:, pos[i]] = acc[0]
        LSE[:, :, pos[i]] = acc[1]
    if varlen:
        O, LSE = O[0], LSE[0]
    return (O, LSE, partials) if return_partials else (O, LSE)
