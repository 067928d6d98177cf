"""GPU parity of the backward entry points against the float64 oracle
(oracle/backward_ref.py).

Bar (derived from the arithmetic): the kernels take bf16 q, k, v, dO, round
P and dS to bf16 before the gradient products (relative error at most 2^-9
each) and accumulate in fp32, so an entry's error is at most about
2^-9 * sum |terms| and in practice far less; the bar is
    max |grad - ref| <= 1e-2 * max |ref|      per gradient tensor,
which a dropped term, a wrong sign, a wrong mask or a transposed operand
exceeds by an order of magnitude.  delta (fp32 sum of bf16 x bf16/f32
products) must be within 1e-5 * sum |dO * O| per row.  LSE and delta given to
the kernels come from the oracle's forward in float64, rounded to f32.
"""
import sys

import pytest
import torch

import seeded_inputs as si
import ulysses_sequence_attention_zigzag_amd as usp
from oracle import index_ref as ix
from oracle.attention_ref import attention_ref
from oracle.backward_ref import attention_bwd_ref, block_attention_bwd_ref, ring_backward_ref
from oracle.ring_ref import block_attention_ref

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a device"
    usp.lib()  # raises if libusp.so is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_grad(got, ref, what):
    g = got.detach().cpu().double()
    assert not torch.isnan(g).any(), f"{what}: NaN"
    scale = float(ref.abs().max()) if ref.numel() else 0.0
    err = float((g - ref).abs().max()) if ref.numel() else 0.0
    say(f"  {what}: max|ref|={scale:.3e} max|err|={err:.3e} ({err / max(scale, 1e-30):.2e} rel)")
    if scale == 0.0:
        assert err == 0.0, f"{what}: expected zeros"
    else:
        assert err <= GRAD_TOL * scale, f"{what}: error {err} > {GRAD_TOL} * {scale}"


def _inputs(B, Lq, Lk, Hq, Hkv, D, seed):
    q = si.randn_bf16((B, Lq, Hq, D), seed, 0)
    k = si.randn_bf16((B, Lk, Hkv, D), seed, 1)
    v = si.randn_bf16((B, Lk, Hkv, D), seed, 2)
    do = si.randn_bf16((B, Lq, Hq, D), seed, 3)
    return q, k, v, do


def _delta(do, O):
    return (do.double() * O.double()).sum(-1).transpose(1, 2).contiguous()   # [B,H,L]


# ---------------------------------------------------------------- delta
@pytest.mark.parametrize("B,L,H,D", [(1, 1, 1, 64), (2, 333, 3, 128), (1, 1000, 4, 64), (1, 77, 5, 8),
                                     (2, 65, 3, 256)])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
def test_preprocess_delta(B, L, H, D, odt):
    say(f"delta B={B} L={L} H={H} D={D} {odt}")
    o = si.randn_bf16((B, L, H, D), 3, 0).to(odt)
    do = si.randn_bf16((B, L, H, D), 3, 1)
    delta = usp.attn_bwd_preprocess(o.cuda(), do.cuda())
    ref = _delta(do, o)
    bound = 1e-5 * (do.double() * o.double()).abs().sum(-1).transpose(1, 2)
    err = (delta.cpu().double() - ref).abs()
    say(f"  max err {float(err.max()):.3e}")
    assert (err <= bound + 1e-30).all()


# ---------------------------------------------------------------- block backward
EXPLICIT = [
    # mask, B, Lq, Lk, Hq, Hkv, D
    ("full", 1, 32, 32, 1, 1, 64),
    ("full", 2, 300, 200, 4, 2, 128),
    ("causal", 1, 256, 256, 2, 2, 64),
    ("causal", 2, 333, 333, 4, 1, 128),
    ("causal_strict", 1, 300, 300, 3, 1, 128),
    ("causal_strict", 1, 257, 257, 2, 2, 64),
    ("full", 1, 64, 1000, 2, 1, 128),
]


def _explicit_pos(mask, Lq, Lk):
    if mask == "full":
        return list(range(Lq)), list(range(Lk)), False
    if mask == "causal":
        return list(range(Lq)), list(range(Lk)), True
    return list(range(Lq)), list(range(1, Lk + 1)), True


@pytest.mark.parametrize("case", EXPLICIT)
def test_block_bwd_explicit_classes(case):
    mask, B, Lq, Lk, Hq, Hkv, D = case
    say(f"block_bwd explicit {case}")
    q, k, v, do = _inputs(B, Lq, Lk, Hq, Hkv, D, seed=21)
    scale = D ** -0.5
    pq, pk, causal = _explicit_pos(mask, Lq, Lk)
    O, LSE = block_attention_ref(q, k, v, pq, pk, scale=scale, causal=causal, window=0, n_sink=0)
    delta = _delta(do, O)
    rq, rk, rv = block_attention_bwd_ref(q, k, v, do, LSE, delta, pq, pk, scale=scale, causal=causal, window=0,
                                         n_sink=0)
    dq, dk, dv = usp.block_attn_bwd(q.cuda(), k.cuda(), v.cuda(), do.cuda(), LSE.float().cuda(),
                                    delta.float().cuda(), mask=mask)
    torch.cuda.synchronize()
    assert_grad(dq, rq, "dq")
    assert_grad(dk, rk, "dk")
    assert_grad(dv, rv, "dv")


def test_block_bwd_accumulates_and_empty_is_noop():
    say("block_bwd accumulate / empty")
    B, L, Hq, Hkv, D = 1, 200, 2, 1, 64
    q, k, v, do = _inputs(B, L, L, Hq, Hkv, D, seed=23)
    pos = list(range(L))
    O, LSE = block_attention_ref(q, k, v, pos, pos, scale=D ** -0.5, causal=True, window=0, n_sink=0)
    delta = _delta(do, O)
    rq, rk, rv = block_attention_bwd_ref(q, k, v, do, LSE, delta, pos, pos, scale=D ** -0.5, causal=True,
                                         window=0, n_sink=0)
    g = torch.Generator().manual_seed(5)
    init = [torch.randn(t.shape, generator=g, dtype=torch.float32) for t in (rq, rk, rv)]
    dq, dk, dv = (t.clone().cuda() for t in init)
    args = (q.cuda(), k.cuda(), v.cuda(), do.cuda(), LSE.float().cuda(), delta.float().cuda())
    usp.block_attn_bwd(*args, dq=dq, dk=dk, dv=dv, mask="causal")
    before = [t.clone() for t in (dq, dk, dv)]
    usp.block_attn_bwd(*args, dq=dq, dk=dk, dv=dv, mask="empty")
    torch.cuda.synchronize()
    for a, b in zip(before, (dq, dk, dv)):
        assert torch.equal(a, b)
    for got, i0, ref, name in zip((dq, dk, dv), init, (rq, rk, rv), ("dq", "dk", "dv")):
        assert_grad(got.cpu() - i0, ref, name + " accumulated")


def _forward_ref(q, k, v, scale, causal, window, n_sink, cu):
    """Float64 (O [B,S,H,D], LSE [B,H,S]) of natural-order q, k, v (varlen: B = 1)."""
    if cu is None:
        return attention_ref(q, k, v, softmax_scale=scale, causal=causal, window=window, n_sink=n_sink)
    O, LSE = attention_ref(q[0], k[0], v[0], softmax_scale=scale, causal=causal, window=window, n_sink=n_sink,
                           cu_seqlens=cu)
    return O.unsqueeze(0), LSE.unsqueeze(0)


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
]


@pytest.mark.parametrize("case", POSITIONAL)
def test_block_bwd_positional_steps(case):
    impl, S, N, b, causal, window, n_sink, cu, Hq, Hkv, D = case
    say(f"block_bwd positional {case}")
    B, scale = 1, 0.1
    q, k, v, do = _inputs(B, S, S, Hq, Hkv, D, seed=25)
    O, LSE = _forward_ref(q, k, v, scale, causal, window, n_sink, cu)
    delta = _delta(do, O)
    i = N - 1
    pos_q = ix.rank_positions(impl, S, N, i, b)
    qi, doi = q[:, pos_q].contiguous(), do[:, pos_q].contiguous()
    lse_i, del_i = LSE[:, :, pos_q].contiguous(), delta[:, :, pos_q].contiguous()
    for j in sorted({0, i, (i + 1) % N, N // 2}):
        pos_k = ix.rank_positions(impl, S, N, j, b)
        kj, vj = k[:, pos_k].contiguous(), v[:, pos_k].contiguous()
        rq, rk, rv = block_attention_bwd_ref(qi, kj, vj, doi, lse_i, del_i, pos_q, pos_k, scale=scale,
                                             causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu)
        dq, dk, dv = usp.block_attn_bwd(qi.cuda(), kj.cuda(), vj.cuda(), doi.cuda(), lse_i.float().cuda(),
                                        del_i.float().cuda(), qmap=usp.posmap(impl, N, i, S, b),
                                        kmap=usp.posmap(impl, N, j, S, b), causal=causal, window=window,
                                        n_sink=n_sink, cu_seqlens=cu, softmax_scale=scale)
        torch.cuda.synchronize()
        assert_grad(dq, rq, f"i={i} j={j} dq")
        assert_grad(dk, rk, f"i={i} j={j} dk")
        assert_grad(dv, rv, f"i={i} j={j} dv")


# ---------------------------------------------------------------- ring of block calls
RING = [
    # impl, S, N, b, causal, window, n_sink, cu, Hq, Hkv, D
    ("zigzag", 1200, 3, 1, True, 0, 0, None, 2, 1, 128),
    ("zigzag", 1024, 4, 1, True, 0, 0, None, 4, 2, 64),
    ("stripe", 2048, 4, 1, True, 0, 0, None, 4, 1, 128),
    ("stripe", 1536, 4, 3, True, 0, 0, None, 2, 2, 64),
    ("basic", 2048, 4, 1, False, 250, 4, [0, 128, 1000, 2048], 2, 2, 128),
    ("zigzag", 2048, 4, 1, True, 0, 0, [0, 128, 1000, 2048], 2, 1, 128),
    ("stripe", 1536, 4, 3, False, 200, 3, [0, 700, 1536], 2, 2, 64),
]


def _ring_gpu(impl, S, N, b, causal, window, n_sink, cu, q, k, v, do, LSE, delta, scale):
    """The backward ring on one device: host i at round s meets KV piece
    (i - s) mod N; dQ stays with host i, dK / dV with the piece."""
    pos = [ix.rank_positions(impl, S, N, r, b) for r in range(N)]
    dev = lambda t: t.contiguous().cuda()  # noqa: E731
    qs = [dev(q[:, p]) for p in pos]
    dos = [dev(do[:, p]) for p in pos]
    ks = [dev(k[:, p]) for p in pos]
    vs = [dev(v[:, p]) for p in pos]
    lses = [dev(LSE[:, :, p].float()) for p in pos]
    dels = [dev(delta[:, :, p].float()) for p in pos]
    dq = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in qs]
    dk = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in ks]
    dv = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in ks]
    for s in range(N):
        for i in range(N):
            j = (i - s) % N
            usp.block_attn_bwd(qs[i], ks[j], vs[j], dos[i], lses[i], dels[i], dq=dq[i], dk=dk[j], dv=dv[j],
                               qmap=usp.posmap(impl, N, i, S, b), kmap=usp.posmap(impl, N, j, S, b),
                               causal=causal, window=window, n_sink=n_sink, cu_seqlens=cu, softmax_scale=scale)
    torch.cuda.synchronize()
    out = []
    for parts, like in ((dq, q), (dk, k), (dv, v)):
        full = torch.zeros(like.shape, dtype=torch.float64)
        for r in range(N):
            full[:, pos[r]] = parts[r].cpu().double()
        out.append(full)
    return out


@pytest.mark.parametrize("case", RING)
def test_ring_bwd_of_block_calls(case):
    impl, S, N, b, causal, window, n_sink, cu, Hq, Hkv, D = case
    say(f"ring_bwd {case}")
    scale = D ** -0.5
    q, k, v, do = _inputs(1, S, S, Hq, Hkv, D, seed=27)
    O, LSE = _forward_ref(q, k, v, scale, causal, window, n_sink, cu)
    if cu is None:
        ref = ring_backward_ref(q, k, v, do, impl=impl, N=N, stripe_block=b, softmax_scale=scale, causal=causal,
                                window=window, n_sink=n_sink)
    else:
        ref = [t.unsqueeze(0) for t in ring_backward_ref(q[0], k[0], v[0], do[0], impl=impl, N=N,
                                                         stripe_block=b, softmax_scale=scale, causal=causal,
                                                         window=window, n_sink=n_sink, cu_seqlens=cu)]
    delta = _delta(do, O)
    got = _ring_gpu(impl, S, N, b, causal, window, n_sink, cu, q, k, v, do, LSE, delta, scale)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        assert_grad(g, r, name)


def test_block_bwd_deterministic():
    say("block_bwd deterministic")
    impl, S, N = "zigzag", 4096, 2
    L = S // N
    q, k, v, do = _inputs(1, L, L, 4, 1, 128, seed=29)
    lse = torch.full((1, 4, L), 9.0)
    delta = torch.randn((1, 4, L), generator=torch.Generator().manual_seed(3))
    args = [t.cuda() for t in (q, k, v, do, lse, delta)]
    kw = dict(qmap=usp.posmap(impl, N, 1, S), kmap=usp.posmap(impl, N, 0, S), causal=True)
    first = usp.block_attn_bwd(*args, **kw)
    for _ in range(3):
        again = usp.block_attn_bwd(*args, **kw)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


# ---------------------------------------------------------------- virtual ring backward
RING_BWD = [
    si.WORKLOADS["zigzag_causal_small"],
    si.WORKLOADS["ring_swa"].scaled(B=1, S=2048, Hq=4, Hkv=4, window=300),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=4, window=250, cu_seqlens=[0, 128, 1000, 2048]),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4, rank=3, ulysses_rank=1),
    si.WORKLOADS["stripe_mqa"].scaled(S=8192, Hq=4, Hkv=1, rank=7),
    si.WORKLOADS["stripe_mqa"].scaled(S=4096, Hq=2, Hkv=1, stripe_block=4, ring_degree=4, rank=-1),
    si.WORKLOADS["zigzag_causal_small"].scaled(rank=-1, ring_degree=3, S=1200, Hq=2, Hkv=1, D=128),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=2, window=250, cu_seqlens=[0, 128, 1000, 2048],
                                            impl="zigzag"),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=1, window=0, n_sink=0, causal=True,
                                            cu_seqlens=[0, 700, 701, 2048], impl="stripe", stripe_block=4),
    si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4, ulysses_degree=4, rank=1, ulysses_rank=2),
    si.WORKLOADS["stripe_mqa"].scaled(S=4096, Hq=4, Hkv=2, ring_degree=4, ulysses_degree=2, rank=2,
                                      ulysses_rank=1),
    # degenerate: one rank, the ring is plain attention
    si.WORKLOADS["zigzag_causal_small"].scaled(impl="basic", ring_degree=1, S=777, Hq=2, Hkv=1, rank=-1),
    # one rank with ring steps that see nothing: the dk / dv pieces of those
    # steps are zeros (window; causal pieces after the rank's own; varlen)
    si.WORKLOADS["ring_swa"].scaled(B=1, S=2048, Hq=2, Hkv=2, window=300, rank=5),
    si.WORKLOADS["zigzag_causal_small"].scaled(impl="basic", rank=1),
    si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=2, Hkv=1, window=250, cu_seqlens=[0, 128, 1000, 2048],
                                            rank=2),
    si.WORKLOADS["ring_swa"].scaled(B=1, S=2048, Hq=4, Hkv=2, window=300, rank=6, ulysses_degree=2,
                                    ulysses_rank=1),
]


def _ring_bwd_expected(w: si.Workload, q, k, v):
    """Oracle (O, LSE) in the forward's output format, dout of that shape,
    and the expected (dq, dk, dv) in usp_ring_bwd's output format."""
    kw = dict(softmax_scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens)
    if w.rank < 0:
        O, LSE = attention_ref(q, k, v, **kw)
        dout = si.randn_bf16(tuple(O.shape), w.seed, 3)
        dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, dout, **kw)
        return O, LSE, dout, (dq, dk, dv)
    N, ud, u = w.ring_degree, w.ulysses_degree, w.ulysses_rank
    Hl, Hkl = w.Hq // ud, w.Hkv // ud
    heads, kvh = list(range(u * Hl, (u + 1) * Hl)), list(range(u * Hkl, (u + 1) * Hkl))
    pos = [ix.rank_positions(w.impl, w.S, N, r, w.stripe_block) for r in range(N)]
    O, LSE = attention_ref(q, k, v, rows=pos[w.rank], heads=heads, **kw)
    dout = si.randn_bf16(tuple(O.shape), w.seed, 3)
    # the block oracle takes a batch dimension, which varlen tensors lack
    bat = (lambda t: t.unsqueeze(0)) if w.cu_seqlens is not None else (lambda t: t)
    qb, kb, vb, Ob, LSEb, dob = (bat(t) for t in (q, k, v, O, LSE, dout))
    qi = qb[:, pos[w.rank]][:, :, heads].contiguous()
    ks, vs = kb[:, :, kvh].contiguous(), vb[:, :, kvh].contiguous()
    dq, dk, dv = block_attention_bwd_ref(qi, ks, vs, dob, LSEb, _delta(dob, Ob), pos[w.rank], list(range(w.S)),
                                         scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink,
                                         cu_seqlens=w.cu_seqlens)
    perm = [p for r in range(N) for p in pos[r]]          # rank-major row order
    grads = (dq, dk[:, perm], dv[:, perm])
    if w.cu_seqlens is not None:
        grads = tuple(g[0] for g in grads)
    return O, LSE, dout, grads


@pytest.mark.parametrize("w", RING_BWD, ids=lambda w: f"{w.name}-S{w.S}-r{w.rank}-u{w.ulysses_rank}")
def test_ring_bwd_oracle_forward(w):
    """usp_ring_bwd given the oracle's forward output and LSE."""
    say(f"ring_bwd {w.name} S={w.S} rank={w.rank} u={w.ulysses_rank}")
    q, k, v = w.make_inputs()
    O, LSE, dout, ref = _ring_bwd_expected(w, q, k, v)
    fwd = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                       ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                       window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens,
                       softmax_scale=w.softmax_scale or 0.0, rank=w.rank, ulysses_rank=w.ulysses_rank)
    fwd.out.copy_(O.float())
    fwd.lse.copy_(LSE.float())
    bwd = usp.RingBwdCall(fwd, dout.cuda())
    # outputs and workspace start as NaN: a gradient row the call leaves
    # unwritten, or a workspace byte it reads before writing, shows
    for t in (bwd.dq, bwd.dk, bwd.dv):
        t.fill_(float("nan"))
    bwd.workspace.fill_(0xFF)
    got = bwd.run()
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        assert tuple(g.shape) == tuple(r.shape), (name, g.shape, r.shape)
        assert_grad(g, r, name)
    # a second run overwrites (does not accumulate into) the outputs
    again = bwd.run()
    torch.cuda.synchronize()
    for a_, b_ in zip(got, again):
        assert torch.equal(a_, b_)


def test_ring_bwd_window_one():
    """A window of one key: each query sees only itself, so P = 1, delta = dO . v
    = dP and the exact dQ and dK are 0 (dV = dO).  dP and delta are two f32
    sums of the same products in different orders, so the kernel's dS is their
    rounding difference: |dq_t| <= scale |dP_t - delta_t| max|k_t| with
    |dP - delta| <= 2 D 2^-24 sum_d |dO_d v_d| (f32 summation), and dk the same
    with q.  dV is compared with the usual relative bar."""
    w = si.WORKLOADS["ring_swa"].scaled(B=1, S=512, Hq=2, Hkv=2, ring_degree=2, window=1)
    say("ring_bwd window 1")
    q, k, v = w.make_inputs()
    O, LSE, dout, ref = _ring_bwd_expected(w, q, k, v)
    fwd = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree, window=w.window,
                       softmax_scale=w.softmax_scale or 0.0)
    fwd.out.copy_(O.float())
    fwd.lse.copy_(LSE.float())
    dq, dk, dv = usp.RingBwdCall(fwd, dout.cuda()).run()
    torch.cuda.synchronize()
    assert_grad(dv, ref[2], "dv")
    dsum = (dout.double() * v.double()).abs().sum(-1, keepdim=True)          # [B,S,H,1]
    ds_bound = 2 * w.D * 2.0 ** -24 * dsum
    for g, other, name in ((dq, k, "dq"), (dk, q, "dk")):
        bound = w.scale * ds_bound * other.double().abs().amax(-1, keepdim=True)
        err = (g.cpu().double() - 0.0).abs()
        say(f"  {name}: max|g|={float(err.max()):.3e}, max bound={float(bound.max()):.3e}")
        assert bool((err <= bound).all()), name


@pytest.mark.parametrize("w", [RING_BWD[0], RING_BWD[3], RING_BWD[6]],
                         ids=lambda w: f"{w.name}-S{w.S}-r{w.rank}")
def test_ring_fwd_then_bwd_end_to_end(w):
    """usp_ring_fwd then usp_ring_bwd on the device (bf16 forward output)."""
    say(f"ring fwd+bwd {w.name} S={w.S} rank={w.rank}")
    q, k, v = w.make_inputs()
    _, _, dout, ref = _ring_bwd_expected(w, q, k, v)
    fwd = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                       ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                       window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens,
                       softmax_scale=w.softmax_scale or 0.0, rank=w.rank, ulysses_rank=w.ulysses_rank,
                       out_dtype=torch.bfloat16)
    fwd.run()
    bwd = usp.RingBwdCall(fwd, dout.cuda())
    got = bwd.run()
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        assert_grad(g, r, name)
    # the same backward replayed from a HIP graph, with eager calls between
    # replays: the eager bits every time
    eager = [g.cpu().clone() for g in got]
    graph = bwd.capture()
    for i in range(2):
        for g in (bwd.dq, bwd.dk, bwd.dv):
            g.fill_(3.0)
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(g.cpu(), e) for g, e in zip((bwd.dq, bwd.dk, bwd.dv), eager)), f"replay {i}"
        bwd.run()
        torch.cuda.synchronize()
        assert all(torch.equal(g.cpu(), e) for g, e in zip((bwd.dq, bwd.dk, bwd.dv), eager)), f"eager {i}"


@pytest.mark.parametrize("w", [RING_BWD[0], RING_BWD[2], si.WORKLOADS["usp_zigzag_gqa"].scaled(S=4096, Hq=4, Hkv=4,
                                                                                           rank=1, ulysses_rank=1)],
                         ids=lambda w: f"{w.name}-S{w.S}-r{w.rank}")
def test_ring_bwd_packed_qkv(w):
    """usp_ring_bwd of a packed-qkv forward (oracle forward output and LSE given)."""
    say(f"ring_bwd packed {w.name} S={w.S} rank={w.rank}")
    q, k, v = w.make_inputs()
    O, LSE, dout, ref = _ring_bwd_expected(w, q, k, v)
    qkv = torch.stack([q, k, v], dim=-3).contiguous()
    fwd = usp.RingCall(qkv.cuda(), None, None, impl=w.impl, ring_degree=w.ring_degree,
                       ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                       window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens,
                       softmax_scale=w.softmax_scale or 0.0, rank=w.rank, ulysses_rank=w.ulysses_rank,
                       qkv_packed=True)
    fwd.out.copy_(O.float())
    fwd.lse.copy_(LSE.float())
    got = usp.RingBwdCall(fwd, dout.cuda()).run()
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        assert_grad(g, r, name)


# ---------------------------------------------------------------- full size, sampled
def _local_rows(w: si.Workload, seed: int, n: int):
    L = w.S // w.ring_degree
    rows = {0, 1, L // 2 - 1, L // 2, L - 1}
    g = torch.Generator().manual_seed(seed)
    rows |= set(torch.randint(0, L, (n,), generator=g).tolist())
    return sorted(rows)


# keys checked at full size: positions near the sequence end, so that the
# oracle can take every query that sees them, yet each is seen by hundreds
# (striped MQA: 8 heads over up to 2^20 keys per query) or about two
# thousand (USP share) of the rank's queries; with GQA the check covers two
# KV heads of the Ulysses rank (all query heads of those groups)
FULL_BWD = {
    "usp_zigzag_gqa": dict(keys=lambda S: [S - 1972, S - 1500, S - 1001, S - 640, S - 129, S - 2], kv_groups=[0, 3]),
    "stripe_mqa": dict(keys=lambda S: [S - 2048, S - 1601, S - 1024, S - 777, S - 256, S - 9], kv_groups=[0]),
}


@pytest.mark.parametrize("name", ["usp_zigzag_gqa", "stripe_mqa"])
def test_large_workloads_full_size_backward_sampled(name):
    """usp_ring_bwd at the workload's full size, after usp_ring_fwd on the
    device in the configuration bench.py times (the USP share with the Ulysses
    head -> seq output layout): dq on sampled query rows of the rank, and dk /
    dv of keys that hundreds to thousands of the rank's queries see, each
    accumulated over all of them (keys no query of the rank sees come back
    exactly zero)."""
    w = si.WORKLOADS[name]
    cfg = FULL_BWD[name]
    say(f"full-size backward {name}: generating inputs")
    q, k, v = w.make_inputs()
    seq = w.ulysses_degree > 1
    fwd = usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                       ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                       window=w.window, n_sink=w.n_sink, softmax_scale=w.softmax_scale or 0.0, rank=w.rank,
                       ulysses_rank=w.ulysses_rank, out_layout="seq" if seq else "heads")
    fwd.run()
    dout = si.randn_bf16(tuple(fwd.out.shape), w.seed, 3)
    dq, dk, dv = usp.RingBwdCall(fwd, dout.cuda()).run()
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    N, ud, u = w.ring_degree, w.ulysses_degree, w.ulysses_rank
    Hl, Hkl = w.Hq // ud, w.Hkv // ud
    group = w.Hq // w.Hkv
    heads, kvh = list(range(u * Hl, (u + 1) * Hl)), list(range(u * Hkl, (u + 1) * Hkl))
    if seq:
        dout = dout[:, :, heads[0]:heads[-1] + 1]          # this Ulysses rank's head group
    pos = ix.rank_positions(w.impl, w.S, N, w.rank, w.stripe_block)
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink)
    ks, vs = k[:, :, kvh].contiguous(), v[:, :, kvh].contiguous()

    def oracle_fwd(local_rows, hs):
        """float64 (O, LSE) and delta of the rank's local rows for query heads hs (positions in
        increasing order, every key)."""
        order = sorted(local_rows, key=lambda r: pos[r])
        O, LSE = attention_ref(q, k, v, softmax_scale=w.scale, causal=w.causal, window=w.window,
                               n_sink=w.n_sink, rows=[pos[r] for r in order], heads=hs, block_bytes=1 << 32)
        hl = [h - heads[0] for h in hs]
        do = dout[:, order][:, :, hl]
        delta = (do.double() * O).sum(-1).transpose(1, 2)
        return order, [pos[r] for r in order], LSE, do, delta

    # dq of sampled query rows: every key, every head of the Ulysses rank
    rows = _local_rows(w, seed=17, n=3)
    say(f"full-size backward {name}: oracle dq on {len(rows)} rows")
    order, p_rows, LSE, do, delta = oracle_fwd(rows, heads)
    qi = q[:, p_rows][:, :, heads].contiguous()
    dq_ref, _, _ = block_attention_bwd_ref(qi, ks, vs, do, LSE, delta, p_rows, list(range(w.S)), **kw)
    assert_grad(dq[:, order], dq_ref, "dq sampled")

    # dk / dv of the chosen keys, per checked KV head (its group of query heads)
    keys = sorted(cfg["keys"](w.S))
    allpos = [ix.rank_positions(w.impl, w.S, N, r, w.stripe_block) for r in range(N)]
    out_row = {p: i for i, p in enumerate(p for r in range(N) for p in allpos[r])}   # rank-major rows
    krow = torch.tensor([out_row[p] for p in keys])
    seers = [t for t in range(len(pos)) if pos[t] >= keys[0]]
    say(f"full-size backward {name}: oracle dk/dv on {len(keys)} keys seen by up to {len(seers)} query rows")
    for g in cfg["kv_groups"]:
        hs = [heads[g * group + i] for i in range(group)]
        order, p_s, LSE_s, do_s, delta_s = oracle_fwd(seers, hs)
        qs = q[:, p_s][:, :, hs].contiguous()
        kg, vg = ks[:, keys][:, :, g:g + 1].contiguous(), vs[:, keys][:, :, g:g + 1].contiguous()
        _, dk_ref, dv_ref = block_attention_bwd_ref(qs, kg, vg, do_s, LSE_s, delta_s, p_s, keys, **kw)
        n_seen = [sum(1 for pp in p_s if pp >= p) for p in keys]
        say(f"  kv head {g}: queries per key {n_seen}")
        assert_grad(dk[:, krow][:, :, g:g + 1], dk_ref, f"dk kv head {g}")
        assert_grad(dv[:, krow][:, :, g:g + 1], dv_ref, f"dv kv head {g}")
    # keys after the rank's last query: no query of the rank sees them
    last = max(pos)
    unseen = [p for p in range(last + 1, w.S)]
    if unseen:
        urow = torch.tensor([out_row[p] for p in unseen])
        assert float(dk[:, urow].abs().max()) == 0.0 and float(dv[:, urow].abs().max()) == 0.0
