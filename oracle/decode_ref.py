"""Float64 CPU reference for decode-time attention over a KV cache, split
into pieces whose partial results are combined by a tree reduction.

Test infrastructure only (see ``oracle/__init__``).

Long Context Attention notes, section "Ring Attention": flash decoding is
ring attention's optimisation for inference (the KV is cut into pieces that
are processed independently and their partials combined).  Section "Tree
Attention": because the softmax's max and logsumexp are associative, the
partials of the pieces can be combined pairwise along a tree, in log2 of
the piece count rounds.

Decode here: batch row b holds a cache of kv_len[b] keys at positions
0 .. kv_len[b]-1, and Lq new queries that sit at its last Lq positions
(query t at kv_len[b] - Lq + t), each attending causally (and with the
optional window / sinks of the visibility rule) to the cache.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import torch

from .ring_ref import block_attention_ref, merge_ref


def _lens(kv_lens: Optional[Sequence[int]], B: int, S: int) -> List[int]:
    return [S] * B if kv_lens is None else [int(x) for x in kv_lens]


def decode_ref(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_lens: Optional[Sequence[int]] = None, *,
               softmax_scale: Optional[float] = None, window: int = 0, n_sink: int = 0, softcap: float = 0.0,
               alibi_slopes: Optional[torch.Tensor] = None):
    """q [B,Lq,Hq,D], cache k / v [B,S,Hkv,D] (row b valid up to kv_lens[b],
    default S).  Returns (O [B,Lq,Hq,D], LSE [B,Hq,Lq]) in float64: the
    definition, one block over each row's whole cache."""
    B, Lq, Hq, D = q.shape
    S = k.shape[1]
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    lens = _lens(kv_lens, B, S)
    O = torch.zeros((B, Lq, Hq, D), dtype=torch.float64)
    LSE = torch.full((B, Hq, Lq), -math.inf, dtype=torch.float64)
    for b in range(B):
        n = lens[b]
        pos_q = [n - Lq + t for t in range(Lq)]
        o, l = block_attention_ref(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], pos_q, list(range(n)),
                                   scale=scale, causal=True, window=window, n_sink=n_sink, softcap=softcap,
                                   alibi_slopes=alibi_slopes)
        O[b], LSE[b] = o[0], l[0]
    return O, LSE


def decode_split_ref(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_lens: Optional[Sequence[int]] = None, *,
                     split_keys: int, softmax_scale: Optional[float] = None, window: int = 0, n_sink: int = 0,
                     softcap: float = 0.0, alibi_slopes: Optional[torch.Tensor] = None):
    """Partials of the cache pieces [i*split_keys, (i+1)*split_keys) (cut at
    each row's kv_len): (O [n,B,Lq,Hq,D], LSE [n,B,Hq,Lq]) in float64; a piece
    with no visible key has LSE = -inf and O = 0."""
    B, Lq, Hq, D = q.shape
    S = k.shape[1]
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    lens = _lens(kv_lens, B, S)
    n = (S + split_keys - 1) // split_keys
    O = torch.zeros((n, B, Lq, Hq, D), dtype=torch.float64)
    LSE = torch.full((n, B, Hq, Lq), -math.inf, dtype=torch.float64)
    for i in range(n):
        for b in range(B):
            lo, hi = i * split_keys, min((i + 1) * split_keys, lens[b])
            if lo >= hi:
                continue
            pos_q = [lens[b] - Lq + t for t in range(Lq)]
            o, l = block_attention_ref(q[b:b + 1], k[b:b + 1, lo:hi], v[b:b + 1, lo:hi], pos_q,
                                       list(range(lo, hi)), scale=scale, causal=True, window=window,
                                       n_sink=n_sink, softcap=softcap, alibi_slopes=alibi_slopes)
            O[i, b], LSE[i, b] = o[0], l[0]
    return O, LSE


def tree_merge_ref(O_parts: torch.Tensor, LSE_parts: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Pairwise tree over the piece axis: round r merges piece i with piece
    i + 2^r for every i divisible by 2^(r+1), until one remains."""
    parts = [(O_parts[i].double(), LSE_parts[i].double()) for i in range(O_parts.shape[0])]
    stride = 1
    while stride < len(parts):
        for i in range(0, len(parts), 2 * stride):
            if i + stride < len(parts):
                parts[i] = merge_ref(parts[i][0], parts[i][1], parts[i + stride][0], parts[i + stride][1])
        stride *= 2
    return parts[0]
