"""Token-order formulas of the three ring layouts and the Ulysses relayout.

Test infrastructure only (see ``oracle/__init__``).  Plain Python integers; the
tensor helpers only index with the lists these functions build.

Layouts (S tokens, N virtual ring ranks, L = S // N tokens per rank):

* ``basic`` -- contiguous chunks: rank r holds positions [r*L, (r+1)*L).
  Long Context Attention notes, section "Ring Attention" (the sequence is cut
  into N pieces, one per host on a ring); ring sliding-window README (chunk i
  is placed on rank i).
* ``stripe`` -- striped permutation with block size b: the sequence is cut
  into blocks of b tokens and block beta goes to rank beta mod N, so with b=1
  rank r holds r, r+N, r+2N, ...  Long Context Attention notes, section
  "Solution" (16 tokens over 4 devices: device 0 holds 0, 4, 8, 12); section
  "Zig-Zag Attention" (block size 1 keeps the per-step mask a plain causal
  one).
* ``zigzag`` -- "fold the mask": 2N chunks of c = S/(2N) tokens; rank r holds
  chunk r followed by chunk 2N-1-r.  Long Context Attention notes, section
  "Zig-Zag Attention" (folding gives every (Q_i, K_j) pair a whole block and
  nearly equal work per card).  The figure on that page is missing; the
  reading (chunk r and its mirror 2N-1-r, in that order) is the one under
  which the page's claims hold, which ``tests/test_oracle_index.py`` checks.

Hybrid USP sharding (YunChang README, section "2. Usage": the extract
function takes (rank, world_size, rd, ud)): global rank g = r*ud + u holds the
u-th contiguous piece (of L/ud tokens) of ring rank r's shard.

Ulysses relayout (DeepSpeed-Ulysses all-to-all named in the YunChang README,
"Why not apply Ulysses and Ring Attention Individually?"): before attention
Ulysses rank u gathers the sequence pieces of all ud peers for its head group
[u*H/ud, (u+1)*H/ud); after attention the inverse scatters them back.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import torch

IMPLS = ("basic", "zigzag", "stripe")


def check_divisible(impl: str, S: int, N: int, b: int = 1) -> None:
    if N < 1 or S < 0:
        raise ValueError("bad S/N")
    if impl == "basic" and S % N:
        raise ValueError("basic layout needs S % N == 0")
    if impl == "zigzag" and S % (2 * N):
        raise ValueError("zigzag layout needs S % (2N) == 0")
    if impl == "stripe" and (b < 1 or S % (N * b)):
        raise ValueError("stripe layout needs S % (N*b) == 0")
    if impl not in IMPLS:
        raise ValueError(impl)


def global_position(impl: str, S: int, N: int, rank: int, t: int, b: int = 1) -> int:
    """Global sequence position of local row t on ring rank ``rank``."""
    L = S // N
    if not 0 <= t < L:
        raise IndexError(t)
    if impl == "basic":
        return rank * L + t
    if impl == "zigzag":
        c = S // (2 * N)
        if t < c:
            return rank * c + t
        return (2 * N - 1 - rank) * c + (t - c)
    if impl == "stripe":
        blk, off = divmod(t, b)
        return (blk * N + rank) * b + off
    raise ValueError(impl)


def owner(impl: str, S: int, N: int, p: int, b: int = 1) -> Tuple[int, int]:
    """(rank, local row) holding global position p -- the inverse map, written
    from the layout description rather than by inverting ``global_position``."""
    if not 0 <= p < S:
        raise IndexError(p)
    if impl == "basic":
        L = S // N
        return p // L, p % L
    if impl == "zigzag":
        c = S // (2 * N)
        chunk, off = divmod(p, c)
        if chunk < N:
            return chunk, off
        return 2 * N - 1 - chunk, c + off
    if impl == "stripe":
        blk, off = divmod(p, b)
        return blk % N, (blk // N) * b + off
    raise ValueError(impl)


def rank_positions(impl: str, S: int, N: int, rank: int, b: int = 1) -> List[int]:
    """Global positions of ring rank ``rank``'s rows, in local order."""
    check_divisible(impl, S, N, b)
    return [global_position(impl, S, N, rank, t, b) for t in range(S // N)]


def permutation(impl: str, S: int, N: int, b: int = 1) -> List[int]:
    """perm[i] = global position stored at rank-major index i = r*L + t."""
    out: List[int] = []
    for r in range(N):
        out.extend(rank_positions(impl, S, N, r, b))
    return out


def usp_positions(impl: str, S: int, rd: int, ud: int, g: int, b: int = 1) -> List[int]:
    """Positions held by global USP rank g = r*ud + u (ring rank r, piece u)."""
    r, u = divmod(g, ud)
    pos = rank_positions(impl, S, rd, r, b)
    Ls = len(pos) // ud
    if Ls * ud != len(pos):
        raise ValueError("ring shard not divisible by ulysses degree")
    return pos[u * Ls:(u + 1) * Ls]


# ---------------------------------------------------------------- tensors
def permute_rows(x: torch.Tensor, impl: str, N: int, b: int = 1, dim: int = 1) -> torch.Tensor:
    """Natural order -> rank-major order along ``dim`` (a gather)."""
    perm = permutation(impl, x.shape[dim], N, b)
    return x.index_select(dim, torch.tensor(perm, dtype=torch.long))


def unpermute_rows(y: torch.Tensor, impl: str, N: int, b: int = 1, dim: int = 1) -> torch.Tensor:
    """Rank-major order -> natural order along ``dim`` (a scatter)."""
    perm = permutation(impl, y.shape[dim], N, b)
    out = torch.empty_like(y)
    idx = torch.tensor(perm, dtype=torch.long)
    out.index_copy_(dim, idx, y)
    return out


def extract_rows(x: torch.Tensor, impl: str, rd: int, ud: int, g: int, b: int = 1, dim: int = 1) -> torch.Tensor:
    """Global USP rank g's shard of a natural-order tensor (the extract call)."""
    pos = usp_positions(impl, x.shape[dim], rd, ud, g, b)
    return x.index_select(dim, torch.tensor(pos, dtype=torch.long))


def ulysses_seq_to_head(shards: Sequence[torch.Tensor], u: int) -> torch.Tensor:
    """Gather for Ulysses rank u.  shards[u'] is [B, Ls, H, D] (peer u's
    sequence piece, all heads); returns [B, ud*Ls, H/ud, D] with
    Y[b, u'*Ls + s, h', d] = shards[u'][b, s, u*H/ud + h', d]."""
    ud = len(shards)
    B, Ls, H, D = shards[0].shape
    Hg = H // ud
    if Hg * ud != H:
        raise ValueError("ulysses degree must divide the head count")
    out = torch.empty((B, ud * Ls, Hg, D), dtype=shards[0].dtype)
    for up in range(ud):
        out[:, up * Ls:(up + 1) * Ls] = shards[up][:, :, u * Hg:(u + 1) * Hg]
    return out


def ulysses_head_to_seq(y: torch.Tensor, u: int, shards_out: Sequence[torch.Tensor]) -> None:
    """Scatter for Ulysses rank u: the inverse of ``ulysses_seq_to_head``.
    Writes only head group u of each shard: shards_out[u'][b, s, u*Hg + h', d]
    = y[b, u'*Ls + s, h', d]."""
    ud = len(shards_out)
    B, Ls, H, D = shards_out[0].shape
    Hg = H // ud
    for up in range(ud):
        shards_out[up][:, :, u * Hg:(u + 1) * Hg] = y[:, up * Ls:(up + 1) * Ls]
