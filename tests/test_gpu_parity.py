"""GPU parity: every libusp entry point against the float64 oracle.

Bars: token permutations and relayouts bit-exact; attention output max abs
error <= 1e-2 and LSE max abs error <= 5e-3 against float64, with a -inf LSE
(row without visible key) matched exactly.  Inputs are bf16 N(0,1) from the
seeded generator; the kernels accumulate in fp32.
"""
import math
import sys

import pytest
import torch

import seeded_inputs as si
import ulysses_sequence_attention_zigzag_amd as usp
from oracle import index_ref as ix
from oracle.attention_ref import attention_ref
from oracle.ring_ref import block_attention_ref, merge_ref

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a device"
    usp.lib()  # raises if libusp.so is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_parity(out, lse, O_ref, L_ref, what=""):
    o = out.detach().float().cpu().double()
    l = lse.detach().cpu().double()
    assert not torch.isnan(o).any(), f"{what}: NaN in output"
    assert not torch.isnan(l).any(), f"{what}: NaN in LSE"
    ref_empty = torch.isinf(L_ref) & (L_ref < 0)
    got_empty = torch.isinf(l) & (l < 0)
    assert torch.equal(ref_empty, got_empty), f"{what}: -inf LSE rows differ"
    err_o = float((o - O_ref).abs().max()) if o.numel() else 0.0
    fin = ~ref_empty
    err_l = float((l[fin] - L_ref[fin]).abs().max()) if fin.any() else 0.0
    say(f"  {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= OUT_TOL, f"{what}: output error {err_o}"
    assert err_l <= LSE_TOL, f"{what}: LSE error {err_l}"


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


# ---------------------------------------------------------------- permute
@pytest.mark.parametrize("impl,N,b", [("zigzag", 4, 1), ("stripe", 8, 1), ("stripe", 4, 3), ("basic", 4, 1),
                                      ("zigzag", 3, 1)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute_bit_exact(impl, N, b, dtype):
    unit = {"basic": N, "zigzag": 2 * N, "stripe": N * b}[impl]
    S = unit * 40
    x = si.randn_bf16((2, S, 3, 64), seed=5, stream=0).to(dtype)
    xd = x.cuda()
    y = usp.permute(xd, impl, N, stripe_block=b)
    assert torch.equal(bits(y.cpu()), bits(ix.permute_rows(x, impl, N, b)))
    back = usp.permute(y, impl, N, stripe_block=b, inverse=True)
    assert torch.equal(bits(back.cpu()), bits(x))
    for ud in (1, 2):
        for g in range(N * ud):
            e = usp.permute(xd, impl, N, stripe_block=b, ulysses_degree=ud, rank=g)
            assert torch.equal(bits(e.cpu()), bits(ix.extract_rows(x, impl, N, ud, g, b)))
            full = torch.full_like(xd, float("nan"))
            usp.permute(e, impl, N, stripe_block=b, ulysses_degree=ud, rank=g, inverse=True, S_global=S, out=full)
            pos = ix.usp_positions(impl, S, N, ud, g, b)
            assert torch.equal(bits(full.cpu()[:, pos]), bits(x[:, pos]))


def test_permute_lse_layout_rows_of_one_float():
    # the LSE [B,H,S] is permuted along its last axis (rows of 4 bytes)
    S, N = 64, 4
    x = torch.randn(2, 5, S)
    y = usp.permute(x.cuda(), "zigzag", N, dim=2)
    assert torch.equal(y.cpu(), ix.permute_rows(x, "zigzag", N, 1, dim=2))


@pytest.mark.parametrize("ud,H", [(1, 4), (2, 8), (4, 8), (2, 6)])
def test_ulysses_relayout_bit_exact(ud, H):
    B, Ls, D = 2, 48, 64
    shards = [si.randn_bf16((B, Ls, H, D), seed=7, stream=i) for i in range(ud)]
    sd = [s.cuda() for s in shards]
    for u in range(ud):
        local = torch.empty((B, ud * Ls, H // ud, D), dtype=torch.bfloat16, device="cuda")
        usp.ulysses_relayout(sd, local, u, 0)
        assert torch.equal(bits(local.cpu()), bits(ix.ulysses_seq_to_head(shards, u)))
        back = [torch.zeros_like(s) for s in sd]
        usp.ulysses_relayout(back, local, u, 1)
        ref = [torch.zeros_like(s) for s in shards]
        ix.ulysses_head_to_seq(ix.ulysses_seq_to_head(shards, u), u, ref)
        for a, r in zip(back, ref):
            assert torch.equal(bits(a.cpu()), bits(r))


# ---------------------------------------------------------------- block attention
def _qkv(B, Lq, Lk, Hq, Hkv, D, seed):
    q = si.randn_bf16((B, Lq, Hq, D), seed, 0)
    k = si.randn_bf16((B, Lk, Hkv, D), seed, 1)
    v = si.randn_bf16((B, Lk, Hkv, D), seed, 2)
    return q, k, v


EXPLICIT = [
    # mask, B, Lq, Lk, Hq, Hkv, D
    ("full", 1, 32, 32, 1, 1, 64),
    ("full", 2, 300, 200, 4, 2, 128),
    ("causal", 1, 256, 256, 2, 2, 64),
    ("causal", 2, 333, 333, 4, 1, 128),
    ("causal_strict", 1, 300, 300, 3, 1, 128),
    ("causal_strict", 1, 257, 257, 2, 2, 64),
    ("empty", 1, 130, 130, 2, 1, 64),
]


def _explicit_ref(mask, q, k, v, scale):
    Lq, Lk = q.shape[1], k.shape[1]
    if mask == "full":
        pos_q, pos_k, causal = list(range(Lq)), list(range(Lk)), False
    elif mask == "causal":
        pos_q, pos_k, causal = list(range(Lq)), list(range(Lk)), True
    elif mask == "causal_strict":
        pos_q, pos_k, causal = list(range(Lq)), list(range(1, Lk + 1)), True
    else:
        pos_q, pos_k, causal = list(range(Lq)), list(range(10**6, 10**6 + Lk)), True
    return block_attention_ref(q, k, v, pos_q, pos_k, scale=scale, causal=causal, window=0, n_sink=0)


@pytest.mark.parametrize("case", EXPLICIT)
def test_block_attn_explicit_classes(case):
    mask, B, Lq, Lk, Hq, Hkv, D = case
    say(f"block_attn explicit {case}")
    q, k, v = _qkv(B, Lq, Lk, Hq, Hkv, D, seed=11)
    scale = D ** -0.5
    O_ref, L_ref = _explicit_ref(mask, q, k, v, scale)
    out, lse = usp.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask=mask)
    assert_parity(out, lse, O_ref, L_ref, f"{mask}")
    # bf16 output: same partial rounded to bf16 (|o| < 4 here, so within the bar)
    outb, lseb = usp.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask=mask, out_dtype=torch.bfloat16)
    assert_parity(outb, lseb, O_ref, L_ref, f"{mask} bf16 out")


POSITIONAL = [
    # impl, S, N, b, causal, window, n_sink, cu, Hq, Hkv, D
    ("zigzag", 1024, 4, 1, True, 0, 0, None, 4, 4, 64),
    ("zigzag", 2 * 4 * 200, 4, 1, True, 0, 0, None, 4, 2, 128),
    ("stripe", 2048, 8, 1, True, 0, 0, None, 4, 1, 128),
    ("stripe", 1536, 4, 3, True, 0, 0, None, 2, 1, 64),
    ("basic", 4096, 4, 1, False, 300, 0, None, 2, 2, 128),
    ("basic", 4096, 4, 1, False, 300, 4, [0, 512, 2000, 4096], 2, 2, 128),
    ("basic", 3000, 3, 1, True, 0, 0, [0, 1, 700, 701, 2900, 3000], 2, 1, 64),
    ("zigzag", 3072, 4, 1, False, 300, 2, None, 2, 2, 128),
    # striped blocks (stepped positions) under window, sink and varlen masks:
    # partial tiles whose visible keys are intervals of the inverse position map
    ("stripe", 4096, 4, 8, False, 300, 3, None, 2, 1, 128),
    ("stripe", 3072, 4, 3, False, 250, 2, [0, 700, 2000, 3072], 2, 2, 128),
    ("stripe", 2048, 8, 16, True, 0, 0, None, 4, 1, 128),
    # window masks at D = 64 (the kernel's windowed instantiation)
    ("basic", 4096, 4, 1, False, 200, 2, [0, 300, 2500, 4096], 4, 2, 64),
    ("zigzag", 2048, 2, 1, False, 700, 0, None, 2, 1, 64),
]


@pytest.mark.parametrize("case", POSITIONAL)
def test_block_attn_positional_steps(case):
    impl, S, N, b, causal, window, n_sink, cu, Hq, Hkv, D = case
    say(f"block_attn positional {case}")
    L = S // N
    B = 1
    q, k, v = _qkv(B, L, L, Hq, Hkv, D, seed=13)
    scale = 0.1
    i = N - 1
    for j in sorted({0, i, (i + 1) % N, N // 2}):
        pos_q = ix.rank_positions(impl, S, N, i, b)
        pos_k = ix.rank_positions(impl, S, N, j, b)
        O_ref, L_ref = block_attention_ref(q, k, v, pos_q, pos_k, scale=scale, causal=causal, window=window,
                                           n_sink=n_sink, cu_seqlens=cu)
        out, lse = usp.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask="positional",
                                      qmap=usp.posmap(impl, N, i, S, b), kmap=usp.posmap(impl, N, j, S, b),
                                      causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu,
                                      softmax_scale=scale)
        assert_parity(out, lse, O_ref, L_ref, f"i={i} j={j}")


def test_block_attn_accumulate_matches_merge():
    say("block_attn accumulate")
    S, N, Hq, Hkv, D = 2048, 4, 4, 2, 128
    L = S // N
    q, k, v = _qkv(1, L, L, Hq, Hkv, D, seed=17)
    k2 = si.randn_bf16(k.shape, 17, 5)
    v2 = si.randn_bf16(v.shape, 17, 6)
    qm = usp.posmap("zigzag", N, 1, S)
    parts = []
    for kk, vv, j in ((k, v, 1), (k2, v2, 2)):
        parts.append(block_attention_ref(q, kk, vv, ix.rank_positions("zigzag", S, N, 1),
                                         ix.rank_positions("zigzag", S, N, j), scale=D ** -0.5, causal=True,
                                         window=0, n_sink=0))
    O_ref, L_ref = merge_ref(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    out, lse = usp.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), qmap=qm, kmap=usp.posmap("zigzag", N, 1, S),
                                  causal=True)
    usp.block_attn_fwd(q.cuda(), k2.cuda(), v2.cuda(), qmap=qm, kmap=usp.posmap("zigzag", N, 2, S), causal=True,
                       accumulate=True, out=out, lse=lse)
    assert_parity(out, lse, O_ref, L_ref, "accumulate")


@pytest.mark.parametrize("D", [8, 64, 128, 256])
def test_lse_merge_kernel(D):
    say(f"lse_merge D={D}")
    g = torch.Generator().manual_seed(3)
    B, L, H = 2, 300, 3
    oa = torch.randn(B, L, H, D, generator=g, dtype=torch.float64)
    ob = torch.randn(B, L, H, D, generator=g, dtype=torch.float64)
    la = torch.randn(B, H, L, generator=g, dtype=torch.float64) * 4
    lb = torch.randn(B, H, L, generator=g, dtype=torch.float64) * 4
    dead_a = torch.rand(B, H, L, generator=g) < 0.2
    dead_b = torch.rand(B, H, L, generator=g) < 0.2
    la[dead_a] = -math.inf
    lb[dead_b] = -math.inf
    oa[dead_a.transpose(1, 2)] = 0
    ob[dead_b.transpose(1, 2)] = 0
    # round inputs to fp32 first so both sides start from the same values
    oa, ob, la, lb = (t.float().double() for t in (oa, ob, la, lb))
    O_ref, L_ref = merge_ref(oa, la, ob, lb)
    rb, re_ = 37, 251
    O_exp, L_exp = oa.clone(), la.clone()
    O_exp[:, rb:re_] = O_ref[:, rb:re_]
    L_exp[:, :, rb:re_] = L_ref[:, :, rb:re_]
    oad, lad = oa.float().cuda(), la.float().cuda()
    usp.lse_merge(oad, lad, ob.float().cuda(), lb.float().cuda(), rb, re_)
    o = oad.cpu().double()
    l = lad.cpu().double()
    assert torch.equal(torch.isinf(l), torch.isinf(L_exp))
    fin = torch.isfinite(L_exp)
    assert float((l[fin] - L_exp[fin]).abs().max()) < 1e-5
    assert float((o - O_exp).abs().max()) < 1e-5


# ---------------------------------------------------------------- HIP graph
@pytest.mark.parametrize("w", [si.WORKLOADS["zigzag_causal_small"],
                               si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4),
                               # window masks: the 4-wave kernel form
                               si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=2, window=300,
                                                                       cu_seqlens=[0, 300, 1200, 2048])],
                         ids=lambda w: w.name)
def test_ring_graph_replay(w):
    """usp_ring_fwd recorded into a HIP graph: every replay, with eager calls
    and synchronisations between them, gives the eager result bit for bit."""
    say(f"graph replay {w.name}")
    q, k, v = w.make_inputs()
    call = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                        ulysses_degree=w.ulysses_degree, causal=w.causal, window=w.window, n_sink=w.n_sink,
                        cu_seqlens=w.cu_seqlens, softmax_scale=w.softmax_scale or 0.0,
                        rank=w.rank, ulysses_rank=w.ulysses_rank)
    out, lse = call.run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.cpu().clone(), lse.cpu().clone()
    O_ref, L_ref = _oracle_share(w, q, k, v)
    assert_parity(ref_o, ref_l, O_ref, L_ref, "eager")
    graph = call.capture()
    for i in range(3):
        call.out.zero_()
        call.lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out.cpu(), ref_o) and torch.equal(call.lse.cpu(), ref_l), f"replay {i}"
        call.run()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(call.out.cpu(), ref_o) and torch.equal(call.lse.cpu(), ref_l), f"eager {i}"


# ---------------------------------------------------------------- zero-length inputs
@pytest.mark.parametrize("D", [64, 128])
def test_block_attn_zero_length(D):
    """A step with no keys: every row has no visible key, so its partial is
    (O = 0, LSE = -inf), the empty-row convention of the definition, and
    merging it changes nothing; a step with no queries enqueues nothing."""
    say(f"zero-length block D={D}")
    g = torch.Generator().manual_seed(5)
    q = torch.randn(2, 70, 4, D, generator=g).to(torch.bfloat16).cuda()
    k0 = torch.empty(2, 0, 2, D, dtype=torch.bfloat16, device="cuda")
    for mask in ("full", "causal", "empty"):
        out = torch.full((2, 70, 4, D), 7.0, device="cuda")
        lse = torch.full((2, 4, 70), 7.0, device="cuda")
        usp.block_attn_fwd(q, k0, k0, mask=mask, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), torch.zeros(2, 70, 4, D)), mask
        assert bool(torch.all(torch.isneginf(lse.cpu()))), mask
    # accumulate: the empty partial leaves the running result as it was
    out = torch.randn(2, 70, 4, D, generator=g).cuda()
    lse = torch.randn(2, 4, 70, generator=g).cuda()
    o0, l0 = out.clone(), lse.clone()
    usp.block_attn_fwd(q, k0, k0, mask="full", accumulate=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o0) and torch.equal(lse, l0)
    # no queries
    qe = torch.empty(2, 0, 4, D, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(2, 33, 2, D, generator=g).to(torch.bfloat16).cuda()
    oe, le = usp.block_attn_fwd(qe, k, k, mask="full")
    torch.cuda.synchronize()
    assert oe.shape == (2, 0, 4, D) and le.shape == (2, 4, 0)


def test_copy_and_merge_zero_length():
    """Permute of zero batch rows and a merge over an empty row range change nothing."""
    say("zero-length permute / merge")
    x = torch.empty(0, 64, 3, 8, dtype=torch.bfloat16, device="cuda")
    y = usp.permute(x, "zigzag", 4)
    torch.cuda.synchronize()
    assert y.shape == x.shape
    g = torch.Generator().manual_seed(6)
    oa = torch.randn(1, 40, 2, 64, generator=g).cuda()
    la = torch.randn(1, 2, 40, generator=g).cuda()
    o0, l0 = oa.clone(), la.clone()
    usp.lse_merge(oa, la, torch.randn_like(oa), torch.randn_like(la), 17, 17)
    torch.cuda.synchronize()
    assert torch.equal(oa, o0) and torch.equal(la, l0)


# ---------------------------------------------------------------- virtual ring, end to end
def _run_ring(w: si.Workload, q, k, v, **kw):
    call = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                        ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                        window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens,
                        softmax_scale=w.softmax_scale or 0.0, rank=w.rank, ulysses_rank=w.ulysses_rank, **kw)
    out, lse = call.run()
    torch.cuda.synchronize()
    return out, lse


def _oracle_share(w: si.Workload, q, k, v, rows=None):
    """Oracle rows of the workload's output, in the library's output order."""
    if w.rank < 0:
        return attention_ref(q, k, v, softmax_scale=w.scale, causal=w.causal, window=w.window,
                             n_sink=w.n_sink, cu_seqlens=w.cu_seqlens)
    pos = ix.rank_positions(w.impl, w.S, w.ring_degree, w.rank, w.stripe_block)
    Hl = w.Hq // w.ulysses_degree
    heads = list(range(w.ulysses_rank * Hl, (w.ulysses_rank + 1) * Hl))
    sel = pos if rows is None else [pos[t] for t in rows]
    return attention_ref(q, k, v, softmax_scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink,
                         cu_seqlens=w.cu_seqlens, rows=sel, heads=heads)


SMALL_RING = [
    si.WORKLOADS["zigzag_causal_small"],
    si.WORKLOADS["ring_swa"].scaled(B=1, S=2048, Hq=4, Hkv=4, window=300),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=4, window=250, cu_seqlens=[0, 128, 1000, 2048]),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4, rank=3, ulysses_rank=1),
    si.WORKLOADS["stripe_mqa"].scaled(S=8192, Hq=4, Hkv=1),
    si.WORKLOADS["stripe_mqa"].scaled(S=8192, Hq=4, Hkv=1, rank=7),
    si.WORKLOADS["stripe_mqa"].scaled(S=4096, Hq=2, Hkv=1, stripe_block=4, ring_degree=4, rank=-1),
    si.WORKLOADS["zigzag_causal_small"].scaled(rank=-1, ring_degree=3, S=1200, Hq=2, Hkv=1, D=128),
    # varlen with the zigzag / stripe layouts over the packed token axis
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=2, window=250, cu_seqlens=[0, 128, 1000, 2048],
                                            impl="zigzag"),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=1, window=0, n_sink=0, causal=True,
                                            cu_seqlens=[0, 700, 701, 2048], impl="stripe", stripe_block=4),
    # Ulysses head groups with every layout: the staging gathers ring-ordered
    # rows of head group u in one strided pass
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4, ulysses_degree=4, rank=1, ulysses_rank=2),
    si.WORKLOADS["stripe_mqa"].scaled(S=4096, Hq=4, Hkv=2, ring_degree=4, ulysses_degree=2, rank=2,
                                      ulysses_rank=1),
    si.WORKLOADS["ring_swa"].scaled(S=2048, Hq=4, Hkv=4, window=300, ulysses_degree=2, rank=5, ulysses_rank=1),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=2, window=250, cu_seqlens=[0, 128, 1000, 2048],
                                            impl="zigzag", ulysses_degree=2, rank=1, ulysses_rank=0),
]


@pytest.mark.parametrize("w", SMALL_RING, ids=lambda w: f"{w.name}-S{w.S}-r{w.rank}-u{w.ulysses_degree}.{w.ulysses_rank}")
@pytest.mark.parametrize("merge_mode", [0, 1])
def test_ring_small_full_oracle(w, merge_mode):
    say(f"ring {w.name} S={w.S} rank={w.rank} merge_mode={merge_mode}")
    q, k, v = w.make_inputs()
    O_ref, L_ref = _oracle_share(w, q, k, v)
    out, lse = _run_ring(w, q, k, v, merge_mode=merge_mode)
    assert_parity(out, lse, O_ref, L_ref, w.name)


DEGENERATE = [
    # one rank: the ring is plain attention (ragged length, D 64)
    si.WORKLOADS["zigzag_causal_small"].scaled(impl="basic", ring_degree=1, S=777, Hq=2, Hkv=1, rank=-1),
    # zigzag chunks of one token and stripes of one token per rank
    si.WORKLOADS["zigzag_causal_small"].scaled(S=8, ring_degree=4, Hq=2, Hkv=2, D=128, rank=-1),
    si.WORKLOADS["stripe_mqa"].scaled(S=8, ring_degree=8, Hq=2, Hkv=1, rank=-1),
    # a window of one key: every query sees only itself
    si.WORKLOADS["ring_swa"].scaled(B=1, S=512, Hq=2, Hkv=2, ring_degree=2, window=1),
]


@pytest.mark.parametrize("w", DEGENERATE, ids=lambda w: f"{w.name}-{w.impl}-N{w.ring_degree}-S{w.S}-W{w.window}")
def test_ring_degenerate_cases(w):
    say(f"degenerate ring {w.impl} N={w.ring_degree} S={w.S} W={w.window}")
    q, k, v = w.make_inputs()
    O_ref, L_ref = _oracle_share(w, q, k, v)
    out, lse = _run_ring(w, q, k, v)
    assert_parity(out, lse, O_ref, L_ref, "degenerate")
    if w.window == 1:
        # closed form: O = v of the query's own position, LSE = scale * q . k_self
        rep = w.Hq // w.Hkv
        vs = v.float().repeat_interleave(rep, dim=2)
        ks = k.float().repeat_interleave(rep, dim=2)
        assert float((out.cpu() - vs).abs().max()) <= 1e-6
        l_self = (q.float() * ks).sum(-1).transpose(1, 2) * w.scale
        assert float((lse.cpu() - l_self).abs().max()) <= 1e-4


@pytest.mark.parametrize("w", [si.WORKLOADS["zigzag_causal_small"], SMALL_RING[3]], ids=lambda w: w.name)
def test_ring_permuted_input_and_bf16_output(w):
    q, k, v = w.make_inputs()
    O_ref, L_ref = _oracle_share(w, q, k, v)
    qp, kp, vp = (ix.permute_rows(t, w.impl, w.ring_degree, w.stripe_block) for t in (q, k, v))
    out, lse = _run_ring(w, qp, kp, vp, input_order="permuted")
    if w.rank < 0:
        out = ix.unpermute_rows(out.cpu(), w.impl, w.ring_degree, w.stripe_block)
        lse = ix.unpermute_rows(lse.cpu(), w.impl, w.ring_degree, w.stripe_block, dim=2)
    assert_parity(out, lse, O_ref, L_ref, "permuted input")
    out, lse = _run_ring(w, q, k, v, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    assert_parity(out, lse, O_ref, L_ref, "bf16 output")


# both attention kernels: positions linear in every run (zigzag, USP) and
# striped blocks of 4 tokens (per-element positions), all ranks in one launch
@pytest.mark.parametrize("w", [SMALL_RING[3], SMALL_RING[7]], ids=lambda w: f"{w.name}-b{w.stripe_block}")
def test_ring_deterministic_and_writes_every_row(w):
    q, k, v = w.make_inputs()
    call = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                        ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=True,
                        rank=w.rank)
    call.out.fill_(float("nan"))
    call.lse.fill_(float("nan"))
    o1, l1 = (t.clone() for t in call.run())
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    for _ in range(4):
        o2, l2 = call.run()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["zigzag_causal_small", "ring_swa", "varlen_streaming"])
def test_workload_full_size_full_oracle(name):
    w = si.WORKLOADS[name]
    say(f"full-size {name}")
    q, k, v = w.make_inputs()
    out, lse = _run_ring(w, q, k, v)
    O_ref, L_ref = _oracle_share(w, q, k, v)
    assert_parity(out, lse, O_ref, L_ref, name)


@pytest.mark.parametrize("name,scaled", [("usp_zigzag_gqa", dict(S=16384)), ("stripe_mqa", dict(S=32768))])
def test_large_workloads_scaled_full_oracle(name, scaled):
    w = si.WORKLOADS[name].scaled(**scaled)
    say(f"scaled {name} {scaled}")
    q, k, v = w.make_inputs()
    out, lse = _run_ring(w, q, k, v)
    O_ref, L_ref = _oracle_share(w, q, k, v)
    assert_parity(out, lse, O_ref, L_ref, f"{name} scaled")


def full_size_rows(w: si.Workload, total: int, seed: int):
    """Local rows of the rank for the full-size checks: the first eight rows,
    the rows around the zigzag chunk boundary and the last rows, two whole
    256-row work items of the attention kernel (zigzag: one in each chunk,
    i.e. a tile that meets only the diagonal step and one that meets every
    step; striped: the first tile and one in the middle), and seeded random
    rows up to `total`."""
    L = w.S // w.ring_degree
    rows = set(range(8)) | {L - 2, L - 1}
    if w.impl == "zigzag":
        c = L // 2
        rows |= {c - 2, c - 1, c, c + 1}
        items = [(c // 2) // 256 * 256, c + (c // 4) // 256 * 256]
    else:
        items = [0, (L // 2) // 256 * 256]
    for t0 in items:
        rows |= set(range(t0, t0 + 256))
    g = torch.Generator().manual_seed(seed)
    while len(rows) < total:
        rows |= set(torch.randint(0, L, (total - len(rows),), generator=g).tolist())
    return sorted(rows), items


def oracle_rows_sorted(w: si.Workload, q, k, v, heads, rows):
    """Oracle (O, LSE) of the rank's local rows, computed over the rows' global
    positions in increasing order (so each block of rows spans few keys), and
    returned in the order of `rows`."""
    pos = ix.rank_positions(w.impl, w.S, w.ring_degree, w.rank, w.stripe_block)
    order = sorted(range(len(rows)), key=lambda i: pos[rows[i]])
    sel = [pos[rows[i]] for i in order]
    O, LSE = attention_ref(q, k, v, softmax_scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink,
                           cu_seqlens=w.cu_seqlens, rows=sel, heads=heads, block_bytes=1 << 32)
    back = torch.empty(len(rows), dtype=torch.long)
    back[torch.tensor(order)] = torch.arange(len(rows))
    return O[:, back], LSE[:, :, back]


@pytest.mark.parametrize("name,n_rows", [("usp_zigzag_gqa", 2048), ("stripe_mqa", 1024)])
def test_large_workloads_full_size_sampled_rows(name, n_rows):
    """The two large one-rank workloads at full size, in the configuration
    bench.py times (the USP share with the Ulysses head -> seq output layout):
    every head of n_rows local rows against the float64 oracle."""
    w = si.WORKLOADS[name]
    say(f"full-size {name}: generating inputs")
    q, k, v = w.make_inputs()
    seq = w.ulysses_degree > 1
    out, lse = _run_ring(w, q, k, v, out_layout="seq" if seq else "heads")
    Hl = w.Hq // w.ulysses_degree
    heads = list(range(w.ulysses_rank * Hl, (w.ulysses_rank + 1) * Hl))
    if seq:
        out = out[:, :, heads[0]:heads[-1] + 1]
        lse = lse[:, heads[0]:heads[-1] + 1]
    out, lse = out.cpu(), lse.cpu()
    rows, items = full_size_rows(w, n_rows, seed=99)
    say(f"full-size {name}: oracle on {len(rows)} rows (whole items at {items})")
    O_ref, L_ref = oracle_rows_sorted(w, q, k, v, heads, rows)
    idx = torch.tensor(rows)
    assert_parity(out[:, idx], lse[:, :, idx], O_ref, L_ref, f"{name} {len(rows)} rows")


# ---------------------------------------------------------------- packed qkv input
PACKED = [
    si.WORKLOADS["zigzag_causal_small"],
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=8),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=4, Hkv=4, rank=2, ulysses_rank=1),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=4, window=250, cu_seqlens=[0, 128, 1000, 2048]),
]


@pytest.mark.parametrize("w", PACKED, ids=lambda w: f"{w.name}-S{w.S}-r{w.rank}")
def test_ring_packed_qkv(w):
    say(f"packed qkv {w.name} S={w.S} rank={w.rank}")
    q, k, v = w.make_inputs()
    O_ref, L_ref = _oracle_share(w, q, k, v)
    qkv = torch.stack([q, k, v], dim=-3).contiguous()          # [B,S,3,H,D] or [T,3,H,D]
    call = usp.RingCall(qkv.cuda(), None, None, impl=w.impl, ring_degree=w.ring_degree,
                        ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                        window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens,
                        softmax_scale=w.softmax_scale or 0.0, rank=w.rank, ulysses_rank=w.ulysses_rank,
                        qkv_packed=True)
    out, lse = call.run()
    torch.cuda.synchronize()
    assert_parity(out, lse, O_ref, L_ref, "packed")
