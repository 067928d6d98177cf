"""CPU tests of the C ABI: exported symbols, host-side validation and the
tile planner (usp_plan_block: the per-item planner the device planner kernels
run, built on the host), checked here bit-exactly against the oracle's
visibility predicate.

No test here launches device work: every call either fails validation on the
host before anything is enqueued, or is the host-only planner.  This
container has no GPU, so a call that got as far as enqueueing would return
USP_ERR_HIP (test_reaching_the_device_reports_hip shows it): a validation
status therefore also shows that nothing was enqueued.
"""
import ctypes
import os
import re

import pytest
import torch

import ulysses_sequence_attention_zigzag_amd as usp
from oracle import index_ref as ix
from oracle.attention_ref import visibility

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "usp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(usp.LIB_PATH), reason="libusp.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(usp_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_header_function():
    names = header_functions()
    assert "usp_ring_fwd" in names and "usp_block_attn_fwd" in names
    lib = ctypes.CDLL(usp.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(usp.EXPORTS) == names


def test_version_and_empty_error():
    assert usp.lib().usp_version().decode().startswith("usp-")


FAKE = ctypes.c_void_p(0x10000)
FAKE2 = ctypes.c_void_p(0x7f0000000000)


def _status(fn, *args):
    st = fn(*args)
    return st, usp.lib().usp_last_error().decode()


def test_permute_validation():
    L = usp.lib()
    st, msg = _status(L.usp_permute, None, FAKE, 1, 16, 8, 0, 1, 4, 1, 1, -1, 0, None)
    assert st == 1 and "null" in msg
    st, msg = _status(L.usp_permute, FAKE, FAKE2, 1, 12, 8, 0, 1, 4, 1, 1, -1, 0, None)
    assert st == 1 and "zigzag" in msg
    st, msg = _status(L.usp_permute, FAKE, FAKE2, 1, 12, 8, 0, 2, 4, 1, 2, -1, 0, None)
    assert st == 1 and "stripe" in msg
    st, msg = _status(L.usp_permute, FAKE, FAKE2, 1, 16, 8, 0, 7, 4, 1, 1, -1, 0, None)
    assert st == 1 and "impl" in msg
    st, msg = _status(L.usp_permute, FAKE, FAKE2, 1, 16, 8, 0, 0, 4, 3, 1, -1, 0, None)
    assert st == 1 and "ulysses" in msg
    st, msg = _status(L.usp_permute, FAKE, FAKE2, 1, 16, 8, 0, 0, 4, 1, 1, 4, 0, None)
    assert st == 1 and "rank" in msg
    st, msg = _status(L.usp_permute, FAKE, ctypes.c_void_p(0x10000 + 64), 1, 16, 8, 0, 0, 4, 1, 1, -1, 0, None)
    assert st == 1 and "overlap" in msg


def test_relayout_validation():
    L = usp.lib()
    arr9 = (ctypes.c_void_p * 9)(*[0x10000 * (i + 1) for i in range(9)])
    st, msg = _status(L.usp_ulysses_relayout, ctypes.cast(arr9, ctypes.c_void_p), FAKE2, 1, 4, 9, 8, 0, 9, 0, 0, None)
    assert st == 2 and "ulysses_degree" in msg
    arr = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    st, msg = _status(L.usp_ulysses_relayout, ctypes.cast(arr, ctypes.c_void_p), FAKE2, 1, 4, 5, 8, 0, 2, 0, 0, None)
    assert st == 1 and "divide" in msg
    st, msg = _status(L.usp_ulysses_relayout, ctypes.cast(arr, ctypes.c_void_p), FAKE2, 1, 4, 4, 8, 0, 2, 2, 0, None)
    assert st == 1 and "ulysses_rank" in msg
    st, msg = _status(L.usp_ulysses_relayout, ctypes.cast(arr, ctypes.c_void_p), FAKE2, 1, 4, 4, 8, 0, 2, 0, 3, None)
    assert st == 1 and "direction" in msg


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE2, lse=FAKE2, B=1, Lq=64, Lk=64, Hq=4, Hkv=2, D=128, scale=0.0,
             mask=usp.MASK["causal"], qmap=None, kmap=None, causal=0, window=0, n_sink=0, cud=None, cuh=None,
             nseq=0, dt=1, acc=0, softcap=0.0, alibi=None)
    a.update(kw)
    L = usp.lib()
    return _status(L.usp_block_attn_fwd, a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Lq"], a["Lk"],
                   a["Hq"], a["Hkv"], a["D"], a["scale"], a["mask"], a["qmap"], a["kmap"], a["causal"],
                   a["window"], a["n_sink"], a["cud"], a["cuh"], a["nseq"], a["dt"], a["acc"], a["softcap"],
                   a["alibi"], a.get("ws"), a.get("ws_bytes", 0), None)


def test_block_attn_validation():
    assert _attn(q=None)[0] == 1
    st, msg = _attn(D=96)
    assert st == 2 and "head_dim" in msg
    st, msg = _attn(Hq=3, Hkv=2)
    assert st == 1 and "multiple" in msg
    st, msg = _attn(dt=0, acc=1)
    assert st == 1 and "accumulate" in msg
    st, msg = _attn(causal=1)
    assert st == 1 and "explicit" in msg
    st, msg = _attn(mask=usp.MASK["positional"])
    assert st == 1 and "qmap" in msg
    qm = usp.posmap("zigzag", 4, 0, 512)
    km = usp.posmap("stripe", 4, 1, 512)
    st, msg = _attn(mask=usp.MASK["positional"], qmap=ctypes.byref(qm), kmap=ctypes.byref(km), Lq=128, Lk=128)
    assert st == 1 and "same layout" in msg
    km = usp.posmap("zigzag", 4, 1, 512)
    st, msg = _attn(mask=usp.MASK["positional"], qmap=ctypes.byref(qm), kmap=ctypes.byref(km), Lq=64, Lk=128)
    assert st == 1 and "Lq == Lk" in msg
    cu = torch.tensor([0, 100, 512], dtype=torch.int32)
    st, msg = _attn(mask=usp.MASK["positional"], qmap=ctypes.byref(qm), kmap=ctypes.byref(km), Lq=128, Lk=128,
                    cud=FAKE, cuh=ctypes.c_void_p(cu.data_ptr()), nseq=2, causal=1, B=2)
    assert st == 1 and "B == 1" in msg
    qb = usp.posmap("basic", 4, 0, 512)
    kb = usp.posmap("basic", 4, 1, 512)
    bad = torch.tensor([0, 300, 200], dtype=torch.int32)
    st, msg = _attn(mask=usp.MASK["positional"], qmap=ctypes.byref(qb), kmap=ctypes.byref(kb), Lq=128, Lk=128,
                    cud=FAKE, cuh=ctypes.c_void_p(bad.data_ptr()), nseq=2)
    assert st == 1 and "cu_seqlens" in msg
    st, msg = _attn(window=-1, mask=usp.MASK["positional"], qmap=ctypes.byref(qb), kmap=ctypes.byref(kb), Lq=128, Lk=128)
    assert st == 1 and "window" in msg
    # score modifiers: softcap finite and >= 0; ALiBi needs global positions, at most 2^22 of them
    for cap in (-1.0, float("nan"), float("inf")):
        st, msg = _attn(softcap=cap)
        assert st == 1 and "softcap" in msg, cap
    st, msg = _attn(alibi=FAKE)
    assert st == 1 and "POSITIONAL" in msg
    S = 1 << 23
    qb = usp.posmap("basic", 8, 0, S)
    kb = usp.posmap("basic", 8, 1, S)
    st, msg = _attn(mask=usp.MASK["positional"], qmap=ctypes.byref(qb), kmap=ctypes.byref(kb), Lq=S // 8,
                    Lk=S // 8, alibi=FAKE)
    assert st == 2 and "ALiBi" in msg


def test_block_workspace_sizes_and_checks():
    """Block calls take their tile plan's workspace from the caller: the size
    calls report it, and a missing or short workspace is USP_ERR_WORKSPACE
    before anything is enqueued."""
    L = usp.lib()
    need = L.usp_block_attn_fwd_workspace_size(300, 300, usp.MASK["causal"], None, None, 0, 0, 0, None, 0)
    # 2 query tiles of 256 rows: items, run slots (3 per tile), candidate items and costs, 256-byte aligned
    assert need == 4 * 256
    st, msg = _attn(Lq=300, Lk=300)
    assert st == 3 and "workspace" in msg
    st, msg = _attn(Lq=300, Lk=300, ws=FAKE, ws_bytes=need - 1)
    assert st == 3 and "workspace" in msg
    st, msg = _attn(Lq=300, Lk=300, ws=ctypes.c_void_p(0x10010), ws_bytes=need)
    assert st == 3 and "aligned" in msg
    # invalid arguments: size 0, and the call reports the reason
    assert L.usp_block_attn_fwd_workspace_size(300, 300, usp.MASK["causal"], None, None, 1, 0, 0, None, 0) == 0
    qm, km = usp.posmap("zigzag", 4, 1, 4096), usp.posmap("zigzag", 4, 2, 4096)
    nb = L.usp_block_attn_bwd_workspace_size(1024, 1024, usp.MASK["positional"], ctypes.byref(qm), ctypes.byref(km),
                                             1, 0, 0, None, 0)
    assert nb > 0
    args = [FAKE] * 9 + [1, 1024, 1024, 4, 4, 128, 0.0, usp.MASK["positional"], ctypes.byref(qm),
                         ctypes.byref(km), 1, 0, 0, None, None, 0, 0.0, None]
    st, msg = _status(L.usp_block_attn_bwd, *args, None, 0, None)
    assert st == 3 and "workspace" in msg
    # EMPTY has no work: no workspace needed
    assert L.usp_block_attn_bwd_workspace_size(64, 64, usp.MASK["empty"], None, None, 0, 0, 0, None, 0) == 0


def test_reaching_the_device_reports_hip():
    """Positive control for the 'nothing enqueued' tests: a valid call whose
    workspace is large enough goes on to enqueue, which this GPU-less
    container refuses, so the status is USP_ERR_HIP."""
    L = usp.lib()
    need = L.usp_block_attn_fwd_workspace_size(300, 300, usp.MASK["causal"], None, None, 0, 0, 0, None, 0)
    st, msg = _attn(Lq=300, Lk=300, ws=ctypes.c_void_p(0x100000), ws_bytes=need)
    assert st == 4, (st, msg)


def test_host_planning_allocates_nothing_on_device():
    # usp_plan_block is host-only: it works without a device
    n = ctypes.c_int64()
    st = usp.lib().usp_plan_block(256, 256, 128, usp.MASK["causal"], None, None, 0, 0, 0, None, 0, 0,
                                  None, 0, None, 0, ctypes.byref(n), ctypes.byref(ctypes.c_int64()),
                                  ctypes.byref(ctypes.c_int32()), ctypes.byref(ctypes.c_int32()))
    assert st == 0 and n.value > 0
    nc, slots, need = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_size_t()
    # the device planner's sizes without a workspace (no device work)
    st = usp.lib().usp_plan_block_device(256, 256, usp.MASK["causal"], None, None, 0, 0, 0, None, None, 0, 0, 0,
                                         None, 0, ctypes.byref(nc), ctypes.byref(slots), ctypes.byref(need), None)
    assert st == 0 and nc.value == 1 and slots.value == 3 and need.value > 0


def test_size_limits_are_rejected_before_device_work():
    """Shapes past the 32-bit offset limits fail validation (USP_ERR_UNSUPPORTED)
    instead of launching; the pointers are never touched."""
    L = usp.lib()
    # block attention: one batch row of k/v over 2 GiB (2^24 keys x 1 head x 128 x 2 B)
    st, msg = _attn(Lk=1 << 24, Hkv=1, Hq=1, mask=usp.MASK["full"])
    assert st == 2 and "2 GiB" in msg
    st, msg = _attn(B=1 << 16, Lq=1 << 16)
    assert st == 2 and "too large" in msg
    # permute: outer * S beyond the index range
    st, msg = _status(L.usp_permute, FAKE, FAKE2, 1 << 20, 1 << 14, 8, 0, 0, 4, 1, 1, -1, 0, None)
    assert st == 2 and "too large" in msg
    # merge: more (batch, row, head) groups than 32-bit indices
    st, msg = _status(L.usp_lse_merge, FAKE, FAKE, FAKE2, FAKE2, 1 << 12, 1 << 12, 1 << 8, 64, 0, 1 << 12, None)
    assert st == 2 and "too large" in msg
    # ring: one ring rank's k/v rows over 2 GiB
    a = _ring_args(S=1 << 26, Hq=8, Hkv=8, impl=0, ring_degree=2, causal=1)
    assert L.usp_ring_fwd_workspace_size(ctypes.byref(a)) == 0
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 2 and "2 GiB" in msg, msg
    # decode: one batch row of the cache over 2 GiB; more than 65535 batch rows
    dec = lambda B, S: _status(L.usp_decode_split_fwd, FAKE, FAKE, FAKE, None, None, FAKE2, FAKE2,
                               B, 1, S, 8, 1, 128, 1024, 0.0, 0, 0, 0.0, None, None)
    st, msg = dec(1, 1 << 24)
    assert st == 2 and "2 GiB" in msg, msg
    st, msg = dec(1 << 16, 1024)
    assert st == 2 and "rows or heads" in msg, msg


def test_merge_validation():
    L = usp.lib()
    st, msg = _status(L.usp_lse_merge, FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 128, 5, 11, None)
    assert st == 1 and "row range" in msg
    st, msg = _status(L.usp_lse_merge, FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 6, 0, 10, None)
    assert st == 2
    # a (row, head) of D/4 threads must fit in one wave of 64
    st, msg = _status(L.usp_lse_merge, FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 512, 0, 10, None)
    assert st == 2 and "dividing 64" in msg


def _ring_args(**kw):
    a = usp.RingArgs()
    a.q = a.k = a.v = 0x10000
    a.out = a.lse = 0x7f0000000000
    a.B, a.S, a.Hq, a.Hkv, a.D = 1, 1024, 8, 2, 128
    a.impl, a.ring_degree, a.ulysses_degree, a.stripe_block = 1, 4, 1, 1
    a.rank, a.ulysses_rank = -1, 0
    a.causal = 1
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_ring_validation_and_workspace():
    L = usp.lib()
    cases = [
        (dict(S=1020), 1, "zigzag"),
        (dict(D=80), 2, "head_dim"),
        (dict(ulysses_degree=2), 1, "all-ranks"),
        (dict(ulysses_degree=4, rank=0), 1, "divide"),
        (dict(rank=4), 1, "rank"),
        (dict(merge_mode=3), 1, "merge_mode"),
        (dict(q=None), 1, "null"),
    ]
    cases += [
        (dict(softcap=-2.0), 1, "softcap"),
        (dict(S=1 << 23, alibi_slopes=0x10000), 2, "ALiBi"),
    ]
    for kw, code, word in cases:
        a = _ring_args(**kw)
        assert L.usp_ring_fwd_workspace_size(ctypes.byref(a)) == 0
        st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
        assert st == code and word in msg, (kw, st, msg)
    # workspace: natural-order zigzag input needs permuted copies of q, k, v plus
    # an f32 accumulator in permuted order
    a = _ring_args()
    need = L.usp_ring_fwd_workspace_size(ctypes.byref(a))
    qkv = 1024 * (8 + 2 + 2) * 128 * 2
    acc = 1024 * 8 * 128 * 4 + 8 * 1024 * 4
    assert need >= qkv + acc
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 3 and "workspace" in msg
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), ctypes.c_void_p(0x10010), need, None)
    assert st == 3 and "aligned" in msg
    # pre-permuted f32 output of basic layout accumulates in place: the
    # workspace holds only the tile plans (4 steps x 4 ranks x 1 tile)
    a = _ring_args(impl=0, input_order=1, out_dtype=1)
    need = L.usp_ring_fwd_workspace_size(ctypes.byref(a))
    assert 0 < need <= 4 * 1024
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 3 and "workspace" in msg
    # out_layout: 0 or 1, and the sequence-shard layout is one rank's share
    for kw, word in ((dict(out_layout=2), "out_layout"), (dict(out_layout=1), "rank >= 0")):
        a = _ring_args(**kw)
        assert L.usp_ring_fwd_workspace_size(ctypes.byref(a)) == 0
        st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
        assert st == 1 and word in msg, (kw, msg)
    # staging entry point: the ring's argument checks, then its buffers
    st, msg = _status(L.usp_ring_stage, ctypes.byref(_ring_args(S=1020)), FAKE, FAKE, FAKE, None)
    assert st == 1 and "zigzag" in msg
    st, msg = _status(L.usp_ring_stage, ctypes.byref(_ring_args()), None, FAKE, FAKE, None)
    assert st == 1 and "staging" in msg
    # backward: same checks, its own workspace
    b = usp.RingBwdArgs()
    b.fwd = _ring_args()
    b.dout, b.dq, b.dk, b.dv = 0x10000, 0x20000, 0x30000, 0x40000
    need = L.usp_ring_bwd_workspace_size(ctypes.byref(b))
    assert need > 0
    st, msg = _status(L.usp_ring_bwd, ctypes.byref(b), ctypes.c_void_p(0x100000), need - 256, None)
    assert st == 3 and "workspace" in msg
    # packed qkv: multi-head only; the copies of q, k, v always take workspace
    a = _ring_args(qkv_packed=1)
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 1 and "Hq == Hkv" in msg
    a = _ring_args(qkv_packed=2)
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 1 and "qkv_packed" in msg
    a = _ring_args(qkv_packed=1, Hkv=8, k=None, v=None, impl=0, input_order=1, out_dtype=1)
    need = L.usp_ring_fwd_workspace_size(ctypes.byref(a))
    assert need >= 3 * 1024 * 8 * 128 * 2
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 3 and "workspace" in msg
    # varlen: cu_seqlens must end at S (and B must be 1)
    cu = torch.tensor([0, 500, 1000], dtype=torch.int32)
    a = _ring_args(cu_seqlens_dev=0x10000, cu_seqlens_host=cu.data_ptr(), nseq=2)
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 1 and "cu_seqlens" in msg
    cu = torch.tensor([0, 500, 1024], dtype=torch.int32)
    a = _ring_args(cu_seqlens_dev=0x10000, cu_seqlens_host=cu.data_ptr(), nseq=2, B=2)
    st, msg = _status(L.usp_ring_fwd, ctypes.byref(a), None, 0, None)
    assert st == 1 and "B == 1" in msg


# ---------------------------------------------------------------- planner
def _check_plan(Lq, Lk, qpos, kpos, vis, accumulate, items, runs, tn, tm=128):
    """vis: bool [Lq, Lk] oracle visibility on local indices."""
    covered = torch.zeros(Lq, dtype=torch.int32)
    costs = []
    for it in items.tolist():
        q_row0, t0, rows, qrank, k_row0, krank, rb, re_ = it
        assert q_row0 == t0 and 0 < rows <= tm
        covered[t0:t0 + rows] += 1
        keys = torch.zeros(Lk, dtype=torch.int32)
        cost = 0
        for r in runs[rb:re_].tolist():
            kb, ke, full, _ = r
            assert 0 <= kb < ke <= Lk
            keys[kb:ke] += 1
            cost += ke - kb
            if full:
                assert (ke - kb) % tn == 0
                assert vis[t0:t0 + rows, kb:ke].all(), (it, r)
        assert (keys <= 1).all(), "a key appears in two runs"
        # every visible key of every row lies inside a run
        outside = vis[t0:t0 + rows][:, keys == 0]
        assert not outside.any(), it
        costs.append((1 + cost) * rows)
    assert costs == sorted(costs, reverse=True)
    if accumulate:
        assert (covered <= 1).all()
        # rows without any item see no key
        assert not vis[covered == 0].any()
    else:
        assert (covered == 1).all()


CASES = [
    # impl, S, N, b, causal, window, n_sink, cu
    ("zigzag", 1024, 4, 1, True, 0, 0, None),
    ("zigzag", 2 * 4 * 200, 4, 1, True, 0, 0, None),      # chunk 200: ragged tiles
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
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_planner_against_oracle_visibility(case, accumulate):
    impl, S, N, b, causal, window, n_sink, cu = case
    L = S // N
    for i in range(N):
        for j in {0, i, (i + 1) % N, N - 1}:
            qpos = torch.tensor(ix.rank_positions(impl, S, N, i, b))
            kpos = torch.tensor(ix.rank_positions(impl, S, N, j, b))
            vis = visibility(qpos, kpos, causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu)
            items, runs, tm, tn = usp.plan_block(
                L, L, 128, mask="positional", qmap=usp.posmap(impl, N, i, S, b), kmap=usp.posmap(impl, N, j, S, b),
                causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu, accumulate=accumulate)
            assert tm in (128, 256) and tn == 128
            _check_plan(L, L, qpos, kpos, vis, accumulate, items, runs, tn, tm)


@pytest.mark.parametrize("mask", ["full", "causal", "causal_strict", "empty"])
@pytest.mark.parametrize("Lq,Lk", [(256, 256), (300, 300), (200, 77), (64, 1000)])
def test_planner_explicit_classes(mask, Lq, Lk):
    t = torch.arange(Lq)[:, None]
    u = torch.arange(Lk)[None, :]
    vis = {"full": torch.ones(Lq, Lk, dtype=torch.bool), "causal": u <= t, "causal_strict": u < t,
           "empty": torch.zeros(Lq, Lk, dtype=torch.bool)}[mask]
    for acc in (False, True):
        items, runs, tm, tn = usp.plan_block(Lq, Lk, 64, mask=mask, accumulate=acc)
        _check_plan(Lq, Lk, None, None, vis, acc, items, runs, tn, tm)


def test_planner_full_tiles_dominate_large_causal():
    # the bulk of a long causal zigzag block is planned as full tiles (no per-element mask)
    S, N = 16384, 4
    items, runs, tm, tn = usp.plan_block(S // N, S // N, 128, qmap=usp.posmap("zigzag", N, 1, S),
                                         kmap=usp.posmap("zigzag", N, 1, S), causal=True)
    r = runs.tolist()
    full = sum(x[1] - x[0] for x in r if x[2])
    part = sum(x[1] - x[0] for x in r if not x[2])
    # n q-tiles of tm rows: tile i sees tm*i keys fully and its tm-key diagonal partially
    n = (S // N) // tm
    assert part == n * tm and full == tm * n * (n - 1) // 2
