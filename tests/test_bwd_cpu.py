"""CPU tests of the backward entry points: host-side validation of
usp_attn_bwd_preprocess / usp_block_attn_bwd, and the transposed tile plan
of the dK / dV kernel (usp_plan_block_kv, host code) checked bit-exactly
against the oracle's visibility predicate.

No test here launches device work: every call either fails validation on the
host, returns before enqueueing anything (an EMPTY mask), or is the
host-only planner.
"""
import ctypes
import os

import pytest
import torch

import ulysses_sequence_attention_zigzag_amd as usp
from oracle import index_ref as ix
from oracle.attention_ref import visibility

pytestmark = pytest.mark.skipif(not os.path.exists(usp.LIB_PATH), reason="libusp.so not built")

FAKE = ctypes.c_void_p(0x10000)


def _status(fn, *args):
    st = fn(*args)
    return st, usp.lib().usp_last_error().decode()


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, do=FAKE, lse=FAKE, delta=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Lq=128,
             Lk=128, Hq=4, Hkv=2, D=128, scale=0.0, mask=usp.MASK["causal"], qmap=None, kmap=None, causal=0,
             window=0, n_sink=0, cud=None, cuh=None, nseq=0, softcap=0.0, alibi=None)
    a.update(kw)
    return _status(usp.lib().usp_block_attn_bwd, a["q"], a["k"], a["v"], a["do"], a["lse"], a["delta"], a["dq"],
                   a["dk"], a["dv"], a["B"], a["Lq"], a["Lk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["mask"],
                   a["qmap"], a["kmap"], a["causal"], a["window"], a["n_sink"], a["cud"], a["cuh"], a["nseq"],
                   a["softcap"], a["alibi"], a.get("ws"), a.get("ws_bytes", 0), None)


def test_block_attn_bwd_validation():
    for name in ("q", "k", "v", "do", "lse", "delta", "dq", "dk", "dv"):
        st, msg = _bwd(**{name: None})
        assert st == 1 and "null" in msg, name
    st, msg = _bwd(D=96)
    assert st == 2 and "head_dim" in msg
    st, msg = _bwd(Hq=3, Hkv=2)
    assert st == 1 and "multiple" in msg
    st, msg = _bwd(causal=1)
    assert st == 1 and "explicit" in msg
    st, msg = _bwd(scale=float("nan"))
    assert st == 1 and "finite" in msg
    st, msg = _bwd(mask=usp.MASK["positional"])
    assert st == 1 and "qmap" in msg
    qm = usp.posmap("zigzag", 4, 0, 512)
    km = usp.posmap("zigzag", 4, 1, 512)
    st, msg = _bwd(mask=usp.MASK["positional"], qmap=ctypes.byref(qm), kmap=ctypes.byref(km), Lq=64)
    assert st == 1 and "Lq == Lk" in msg
    cu = torch.tensor([0, 100, 512], dtype=torch.int32)
    st, msg = _bwd(mask=usp.MASK["positional"], qmap=ctypes.byref(qm), kmap=ctypes.byref(km),
                   cud=None, cuh=ctypes.c_void_p(cu.data_ptr()), nseq=2)
    assert st == 1 and "both" in msg
    # score modifiers are checked before anything is enqueued
    st, msg = _bwd(softcap=-0.5)
    assert st == 1 and "softcap" in msg
    st, msg = _bwd(alibi=FAKE)
    assert st == 1 and "POSITIONAL" in msg
    # an EMPTY mask adds nothing and enqueues nothing
    st, msg = _bwd(mask=usp.MASK["empty"])
    assert st == 0


def test_preprocess_validation():
    L = usp.lib()
    st, msg = _status(L.usp_attn_bwd_preprocess, None, 0, FAKE, FAKE, 1, 16, 2, 64, None)
    assert st == 1 and "null" in msg
    st, msg = _status(L.usp_attn_bwd_preprocess, FAKE, 0, FAKE, FAKE, 1, 16, 2, 60, None)
    assert st == 2 and "head_dim" in msg
    st, msg = _status(L.usp_attn_bwd_preprocess, FAKE, 0, FAKE, FAKE, 1, 16, 2, 96, None)
    assert st == 2 and "head_dim" in msg   # D/8 threads of a row must fit one wave in powers of two
    st, msg = _status(L.usp_attn_bwd_preprocess, FAKE, 7, FAKE, FAKE, 1, 16, 2, 64, None)
    assert st == 1 and "dtype" in msg
    st, msg = _status(L.usp_attn_bwd_preprocess, FAKE, 0, FAKE, FAKE, 1, 16, 0, 64, None)
    assert st == 1 and "sizes" in msg


# ------------------------------------------------------- transposed planner
def _check_kv_plan(Lq, Lk, vis, items, runs, tk, tq):
    """vis: bool [Lq, Lk] oracle visibility on local indices; items are key tiles."""
    covered = torch.zeros(Lk, dtype=torch.int32)
    costs = []
    for it in items.tolist():
        k_row0, u0, keys, krank, q_row0, qrank, rb, re_ = it
        assert k_row0 == u0 and q_row0 == 0 and 0 < keys <= tk
        covered[u0:u0 + keys] += 1
        rows = torch.zeros(Lq, dtype=torch.int32)
        cost = 0
        for r in runs[rb:re_].tolist():
            tb, te, full, _ = r
            assert 0 <= tb < te <= Lq
            rows[tb:te] += 1
            cost += te - tb
            if full:
                assert (te - tb) % tq == 0
                assert vis[tb:te, u0:u0 + keys].all(), (it, r)
        assert (rows <= 1).all(), "a query row appears in two runs"
        outside = vis[:, u0:u0 + keys][rows == 0]
        assert not outside.any(), it
        assert rb < re_
        costs.append((1 + cost) * keys)
    assert costs == sorted(costs, reverse=True)
    assert (covered <= 1).all()
    # keys without an item are seen by no query
    assert not vis[:, covered == 0].any()


CASES = [
    # impl, S, N, b, causal, window, n_sink, cu
    ("zigzag", 1024, 4, 1, True, 0, 0, None),
    ("zigzag", 2 * 4 * 200, 4, 1, True, 0, 0, None),
    ("stripe", 2048, 8, 1, True, 0, 0, None),
    ("stripe", 1536, 4, 3, True, 0, 0, None),
    ("basic", 8192, 8, 1, False, 1000, 0, None),
    ("basic", 8192, 4, 1, False, 1000, 4, [0, 512, 4000, 8192]),
    ("basic", 4096, 4, 1, True, 0, 0, [0, 1, 700, 701, 2900, 4096]),
    ("basic", 4096, 4, 1, False, 0, 0, [0, 1500, 4096]),
    ("basic", 3000, 3, 1, False, 130, 7, [0, 100, 1234, 3000]),
    ("zigzag", 1200, 3, 1, False, 0, 0, None),
    ("zigzag", 3072, 4, 1, False, 300, 2, None),
    ("zigzag", 4096, 4, 1, True, 0, 0, [0, 1, 700, 701, 2900, 4096]),      # varlen, packed-axis layout
    ("stripe", 3072, 4, 3, False, 200, 3, [0, 1000, 1100, 3072]),
    ("stripe", 2048, 8, 1, True, 0, 0, [0, 333, 2048]),
    ("basic", 2048, 2, 1, False, 64, 200, [0, 150, 1100, 2048]),   # sink runs wider than a tile
]


@pytest.mark.parametrize("case", CASES)
def test_kv_planner_against_oracle_visibility(case):
    impl, S, N, b, causal, window, n_sink, cu = case
    L = S // N
    for i in range(N):
        for j in {0, i, (i + 1) % N, N - 1}:
            qpos = torch.tensor(ix.rank_positions(impl, S, N, i, b))
            kpos = torch.tensor(ix.rank_positions(impl, S, N, j, b))
            vis = visibility(qpos, kpos, causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu)
            items, runs, tk, tq = usp.plan_block_kv(
                L, L, 128, mask="positional", qmap=usp.posmap(impl, N, i, S, b), kmap=usp.posmap(impl, N, j, S, b),
                causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu)
            assert tk == 128 and tq == 64
            _check_kv_plan(L, L, vis, items, runs, tk, tq)


@pytest.mark.parametrize("mask", ["full", "causal", "causal_strict", "empty"])
@pytest.mark.parametrize("Lq,Lk", [(256, 256), (300, 300), (200, 77), (64, 1000)])
def test_kv_planner_explicit_classes(mask, Lq, Lk):
    t = torch.arange(Lq)[:, None]
    u = torch.arange(Lk)[None, :]
    vis = {"full": torch.ones(Lq, Lk, dtype=torch.bool), "causal": u <= t, "causal_strict": u < t,
           "empty": torch.zeros(Lq, Lk, dtype=torch.bool)}[mask]
    items, runs, tk, tq = usp.plan_block_kv(Lq, Lk, 64, mask=mask)
    _check_kv_plan(Lq, Lk, vis, items, runs, tk, tq)


def test_kv_planner_full_runs_dominate_large_causal():
    # key tile i of a causal diagonal block: queries after the tile are fully visible
    S, N = 16384, 4
    L = S // N
    items, runs, tk, tq = usp.plan_block_kv(L, L, 128, qmap=usp.posmap("basic", N, 1, S),
                                            kmap=usp.posmap("basic", N, 1, S), causal=True)
    r = runs.tolist()
    full = sum(x[1] - x[0] for x in r if x[2])
    part = sum(x[1] - x[0] for x in r if not x[2])
    n = L // tk
    # each key tile sees its own tk rows partially and the rest after it fully
    assert part == n * tk and full == sum(L - (i + 1) * tk for i in range(n))


# ------------------------------------------------------- ring backward
def test_ring_bwd_validation_and_workspace():
    from test_abi_cpu import _ring_args
    L = usp.lib()

    def bargs(**kw):
        grads = {n: kw.pop(n, 0x20000) for n in ("dout", "dq", "dk", "dv")}
        b = usp.RingBwdArgs()
        b.fwd = _ring_args(**kw)
        b.dout, b.dq, b.dk, b.dv = grads["dout"], grads["dq"], grads["dk"], grads["dv"]
        return b

    for kw, code, word in [(dict(S=1020), 1, "zigzag"), (dict(D=80), 2, "head_dim"), (dict(q=None), 1, "null"),
                           (dict(dq=None), 1, "gradient"), (dict(dout=None), 1, "gradient")]:
        b = bargs(**kw)
        if "dq" not in kw and "dout" not in kw:
            assert L.usp_ring_bwd_workspace_size(ctypes.byref(b)) == 0
        st, msg = _status(L.usp_ring_bwd, ctypes.byref(b), None, 0, None)
        assert st == code and word in msg, (kw, st, msg)
    # natural-order zigzag, all ranks: permuted q, k, v (bf16), delta (natural and
    # rank-major), permuted dout and LSE, and three f32 accumulators
    b = bargs()
    need = L.usp_ring_bwd_workspace_size(ctypes.byref(b))
    S, Hq, Hkv, D = 1024, 8, 2, 128
    expect = S * (Hq + 2 * Hkv) * D * 2 + 2 * Hq * S * 4 + S * Hq * D * 2 + Hq * S * 4 + S * (Hq + 2 * Hkv) * D * 4

    def plan_bytes(cands, slots):   # items, run slots, candidate items, costs; each 256-byte aligned
        a = lambda x: (x + 255) // 256 * 256
        return a(cands * 32) + a(cands * slots * 16) + a(cands * 32) + a(cands * 8)

    # dQ and dK / dV plans: 4 steps x 4 ranks x 2 tiles of 128 (one per zigzag chunk), 2 chunks x 3 run slots
    plans = 2 * plan_bytes(32, 6)
    assert expect + plans <= need <= expect + plans + 16 * 256
    st, msg = _status(L.usp_ring_bwd, ctypes.byref(b), None, 0, None)
    assert st == 3 and "workspace" in msg
    st, msg = _status(L.usp_ring_bwd, ctypes.byref(b), ctypes.c_void_p(0x10010), need, None)
    assert st == 3 and "aligned" in msg
    # basic layout, rank-major input: only delta and the plans (one piece per rank: 3 run slots)
    b = bargs(impl=0, input_order=1)
    assert L.usp_ring_bwd_workspace_size(ctypes.byref(b)) == ((Hq * S * 4 + 255) // 256) * 256 + 2 * plan_bytes(32, 3)
