"""GPU parity of the score modifiers (logit soft-capping and ALiBi) against
the float64 oracle (oracle/attention_ref.apply_score_mods and the backward
oracle's 1 - tanh^2 factor).

Bars as for the unmodified paths: forward output max abs error <= 1e-2 and
LSE <= 5e-3; gradients max abs error <= 1e-2 * max |ref| per tensor.  The
slopes are the geometric ALiBi set 2^(-8 (h + 1) / H); the soft cap (1.5 on
scores of unit spread) saturates tanh on a visible share of the pairs, so a
missing cap, a missing 1 - tanh^2 or a wrong distance sign fails the bars.
"""
import sys

import pytest
import torch

import seeded_inputs as si
import ulysses_sequence_attention_zigzag_amd as usp
from oracle import index_ref as ix
from oracle.attention_ref import attention_ref
from oracle.backward_ref import attention_bwd_ref, block_attention_bwd_ref

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 5e-3
GRAD_TOL = 1e-2
CAP = 1.5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a device"
    usp.lib()  # raises if libusp.so is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def slopes(H):
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def assert_parity(out, lse, O_ref, L_ref, what):
    o = out.detach().float().cpu().double()
    l = lse.detach().cpu().double()
    assert not torch.isnan(o).any() and not torch.isnan(l).any(), f"{what}: NaN"
    ref_empty = torch.isinf(L_ref) & (L_ref < 0)
    assert torch.equal(ref_empty, torch.isinf(l) & (l < 0)), f"{what}: -inf LSE rows differ"
    err_o = float((o - O_ref).abs().max())
    fin = ~ref_empty
    err_l = float((l[fin] - L_ref[fin]).abs().max()) if fin.any() else 0.0
    say(f"  {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= OUT_TOL, f"{what}: output error {err_o}"
    assert err_l <= LSE_TOL, f"{what}: LSE error {err_l}"


def assert_grad(got, ref, what):
    g = got.detach().cpu().double()
    assert not torch.isnan(g).any(), f"{what}: NaN"
    scale = float(ref.abs().max())
    err = float((g - ref).abs().max())
    say(f"  {what}: max|ref|={scale:.3e} max|err|={err:.3e}")
    assert err <= GRAD_TOL * scale, f"{what}: error {err} > {GRAD_TOL} * {scale}"


W = si.WORKLOADS
CASES = [
    W["zigzag_causal_small"],                                                       # D=64, every rank
    W["zigzag_causal_small"].scaled(causal=False, impl="basic"),                    # both distance signs
    W["zigzag_causal_small"].scaled(window=200, n_sink=2),                           # D=64 window kernel form
    W["ring_swa"].scaled(B=1, S=2048, Hq=4, Hkv=4, window=300),
    W["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=2, window=250, cu_seqlens=[0, 128, 1000, 2048],
                                 impl="zigzag"),
    W["usp_zigzag_gqa"].scaled(S=4096, Hq=8, Hkv=4, rank=3, ulysses_rank=1),         # slopes of head group 1
    W["stripe_mqa"].scaled(S=8192, Hq=4, Hkv=1, rank=7),                            # key step N
    W["stripe_mqa"].scaled(S=4096, Hq=2, Hkv=1, stripe_block=4, ring_degree=4, rank=-1),   # blocks of 4
]
MODS = [(CAP, False), (0.0, True), (CAP, True)]


def _share_kw(w):
    kw = dict(softmax_scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens)
    if w.rank < 0:
        return kw, None, None
    pos = ix.rank_positions(w.impl, w.S, w.ring_degree, w.rank, w.stripe_block)
    Hl = w.Hq // w.ulysses_degree
    heads = list(range(w.ulysses_rank * Hl, (w.ulysses_rank + 1) * Hl))
    return kw, pos, heads


def _ring(w, q, k, v, softcap, al):
    return usp.RingCall(q.cuda(), k.cuda(), v.cuda(), impl=w.impl, ring_degree=w.ring_degree,
                        ulysses_degree=w.ulysses_degree, stripe_block=w.stripe_block, causal=w.causal,
                        window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens,
                        softmax_scale=w.softmax_scale or 0.0, rank=w.rank, ulysses_rank=w.ulysses_rank,
                        softcap=softcap, alibi_slopes=None if al is None else al.cuda())


@pytest.mark.parametrize("softcap,alibi", MODS, ids=lambda m: str(m))
@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-{w.impl}-b{w.stripe_block}-r{w.rank}-c{int(w.causal)}-w{w.window}")
def test_ring_forward_score_mods(w, softcap, alibi):
    say(f"mods fwd {w.name} {w.impl} r={w.rank} cap={softcap} alibi={alibi}")
    q, k, v = w.make_inputs()
    al = slopes(w.Hq) if alibi else None
    kw, pos, heads = _share_kw(w)
    O_ref, L_ref = attention_ref(q, k, v, rows=pos, heads=heads, softcap=softcap, alibi_slopes=al, **kw)
    out, lse = _ring(w, q, k, v, softcap, al).run()
    torch.cuda.synchronize()
    assert_parity(out, lse, O_ref, L_ref, "forward")
    if softcap > 0 or alibi:
        # the modifiers must matter at these sizes
        O0, _ = attention_ref(q, k, v, rows=pos, heads=heads, **kw)
        assert float((O0 - O_ref).abs().max()) > 10 * OUT_TOL


def test_block_forward_softcap_explicit_class():
    say("mods block fwd causal class, softcap")
    q = si.randn_bf16((2, 300, 4, 128), 41, 0)
    k = si.randn_bf16((2, 300, 2, 128), 41, 1)
    v = si.randn_bf16((2, 300, 2, 128), 41, 2)
    scale = 128 ** -0.5
    O_ref, L_ref = attention_ref(q, k, v, softmax_scale=scale, causal=True, softcap=CAP)
    out, lse = usp.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask="causal", softcap=CAP)
    torch.cuda.synchronize()
    assert_parity(out, lse, O_ref, L_ref, "block softcap")


def _bwd_expected(w, q, k, v, softcap, al):
    kw, pos, heads = _share_kw(w)
    if w.rank < 0:
        O, LSE = attention_ref(q, k, v, softcap=softcap, alibi_slopes=al, **kw)
        dout = si.randn_bf16(tuple(O.shape), w.seed, 3)
        dq, dk, dv, _, _ = attention_bwd_ref(q, k, v, dout, softcap=softcap, alibi_slopes=al, **kw)
        return O, LSE, dout, (dq, dk, dv)
    N, ud, u = w.ring_degree, w.ulysses_degree, w.ulysses_rank
    Hkl = w.Hkv // ud
    kvh = list(range(u * Hkl, (u + 1) * Hkl))
    O, LSE = attention_ref(q, k, v, rows=pos, heads=heads, softcap=softcap, alibi_slopes=al, **kw)
    dout = si.randn_bf16(tuple(O.shape), w.seed, 3)
    delta = (dout.double() * O).sum(-1).transpose(1, 2)
    qi = q[:, pos][:, :, heads].contiguous()
    ks, vs = k[:, :, kvh].contiguous(), v[:, :, kvh].contiguous()
    dq, dk, dv = block_attention_bwd_ref(qi, ks, vs, dout, LSE, delta, pos, list(range(w.S)), scale=w.scale,
                                         causal=w.causal, window=w.window, n_sink=w.n_sink,
                                         cu_seqlens=w.cu_seqlens, softcap=softcap,
                                         alibi_slopes=None if al is None else al[heads])
    allpos = [ix.rank_positions(w.impl, w.S, N, r, w.stripe_block) for r in range(N)]
    perm = [p for r in range(N) for p in allpos[r]]          # rank-major row order
    return O, LSE, dout, (dq, dk[:, perm], dv[:, perm])


BWD_CASES = [CASES[0], CASES[1], CASES[3], CASES[4], CASES[5], CASES[6]]


@pytest.mark.parametrize("softcap,alibi", MODS, ids=lambda m: str(m))
@pytest.mark.parametrize("w", BWD_CASES,
                         ids=lambda w: f"{w.name}-{w.impl}-b{w.stripe_block}-r{w.rank}-c{int(w.causal)}-w{w.window}")
def test_ring_backward_score_mods(w, softcap, alibi):
    """usp_ring_bwd with the oracle's forward output and LSE."""
    say(f"mods bwd {w.name} {w.impl} r={w.rank} cap={softcap} alibi={alibi}")
    q, k, v = w.make_inputs()
    al = slopes(w.Hq) if alibi else None
    O, LSE, dout, ref = _bwd_expected(w, q, k, v, softcap, al)
    fwd = _ring(w, q, k, v, softcap, al)
    fwd.out.copy_(O.float())
    fwd.lse.copy_(LSE.float())
    got = usp.RingBwdCall(fwd, dout.cuda()).run()
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        assert tuple(g.shape) == tuple(r.shape), (name, g.shape, r.shape)
        assert_grad(g, r, name)


def test_ring_forward_then_backward_score_mods():
    """usp_ring_fwd then usp_ring_bwd on the device, both modifiers."""
    w = CASES[4]
    say(f"mods fwd+bwd {w.name}")
    q, k, v = w.make_inputs()
    al = slopes(w.Hq)
    _, _, dout, ref = _bwd_expected(w, q, k, v, CAP, al)
    fwd = _ring(w, q, k, v, CAP, al)
    fwd.run()
    got = usp.RingBwdCall(fwd, dout.cuda()).run()
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        assert_grad(g, r, name)
