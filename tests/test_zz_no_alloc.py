"""GPU test of usp_ring_fwd_noalloc, the allocation-free variant of
usp_ring_fwd (workspace in the library's per-GPU scratch array): called
through the C ABI twice in a row, the second time on a smaller input, each
result must equal usp_ring_fwd's (caller workspace) bit for bit; arguments
beyond the scratch size are refused on the host."""
import ctypes
import sys

import pytest
import torch

import seeded_inputs as si
import ulysses_sequence_attention_zigzag_amd as usp

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _noalloc_matches_ring_fwd(w, out_dtype):
    q, k, v = w.make_inputs()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref = usp.RingCall(qd, kd, vd, impl=w.impl, ring_degree=w.ring_degree, ulysses_degree=w.ulysses_degree,
                       stripe_block=w.stripe_block, causal=w.causal, window=w.window, n_sink=w.n_sink,
                       cu_seqlens=w.cu_seqlens, softmax_scale=w.softmax_scale or 0.0, rank=w.rank,
                       ulysses_rank=w.ulysses_rank, out_dtype=out_dtype)
    ro, rl = ref.run()
    out = torch.full_like(ro, float("nan"))
    lse = torch.full_like(rl, float("nan"))
    a = usp.RingArgs.from_buffer_copy(ref.args)
    a.out, a.lse = out.data_ptr(), lse.data_ptr()
    st = usp.lib().usp_ring_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, usp.lib().usp_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ro)) and torch.equal(bits(lse), bits(rl))
    return ref.ws_bytes


def test_noalloc_two_calls_then_smaller():
    big = si.WORKLOADS["zigzag_causal_small"].scaled(S=4096, Hq=8, Hkv=4, D=128, seed=1101)
    small = si.WORKLOADS["zigzag_causal_small"].scaled(seed=1102)
    say("noalloc: first call")
    n1 = _noalloc_matches_ring_fwd(big, torch.bfloat16)
    say(f"  workspace {n1} bytes")
    say("noalloc: second call, smaller input")
    n2 = _noalloc_matches_ring_fwd(small, torch.float32)
    say(f"  workspace {n2} bytes")
    assert n2 < n1
    say("noalloc: window workload with sinks and cu_seqlens")
    _noalloc_matches_ring_fwd(si.WORKLOADS["varlen_streaming"].scaled(S=2048, Hq=4, Hkv=4, window=250,
                                                                       cu_seqlens=[0, 128, 1000, 2048]),
                              torch.float32)


def test_noalloc_refuses_more_than_its_scratch():
    """The USP share at full size needs far more than 64 MiB of workspace:
    refused on the host (the pointers are never touched)."""
    w = si.WORKLOADS["usp_zigzag_gqa"]
    a = usp.RingArgs()
    a.q = a.k = a.v = 0x10000
    a.out = a.lse = 0x20000
    a.B, a.S, a.Hq, a.Hkv, a.D = w.B, w.S, w.Hq, w.Hkv, w.D
    a.impl, a.ring_degree, a.ulysses_degree, a.stripe_block = 1, w.ring_degree, w.ulysses_degree, 1
    a.rank, a.ulysses_rank, a.causal = 0, 0, 1
    need = usp.lib().usp_ring_fwd_workspace_size(ctypes.byref(a))
    assert need > 64 << 20
    st = usp.lib().usp_ring_fwd_noalloc(ctypes.byref(a), None)
    assert st == 3 and "scratch" in usp.lib().usp_last_error().decode()
