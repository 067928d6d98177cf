"""GPU parity of the decode entry points against the float64 oracle
(oracle/decode_ref.py): the split partials piece by piece, and the merged
result.  Bars as for the forward: output max abs error <= 1e-2 and LSE <=
5e-3 against float64 (P is rounded to bf16 before the PV product), -inf
LSE (a piece with no visible key) matched exactly."""
import sys

import pytest
import torch

import seeded_inputs as si
import ulysses_sequence_attention_zigzag_amd as usp
from oracle.decode_ref import decode_ref, decode_split_ref

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a device"
    usp.lib()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(out, lse, O_ref, L_ref, what):
    o = out.detach().float().cpu().double()
    l = lse.detach().cpu().double()
    assert not torch.isnan(o).any() and not torch.isnan(l).any(), what
    ref_empty = torch.isinf(L_ref) & (L_ref < 0)
    assert torch.equal(ref_empty, torch.isinf(l) & (l < 0)), f"{what}: -inf LSE rows differ"
    err_o = float((o - O_ref).abs().max())
    fin = ~ref_empty
    err_l = float((l[fin] - L_ref[fin]).abs().max()) if fin.any() else 0.0
    say(f"  {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= OUT_TOL and err_l <= LSE_TOL, what


def _cache(B, S, Lq, Hq, Hkv, D, seed):
    q = si.randn_bf16((B, Lq, Hq, D), seed, 0)
    k = si.randn_bf16((B, S, Hkv, D), seed, 1)
    v = si.randn_bf16((B, S, Hkv, D), seed, 2)
    return q, k, v


CASES = [
    # B, S, Lq, Hq, Hkv, D, kv_lens, split_keys, window, n_sink
    (2, 1000, 1, 8, 1, 128, [1000, 77], 256, 0, 0),
    (1, 4096, 4, 32, 8, 128, None, 512, 500, 4),
    (3, 300, 2, 4, 4, 64, [300, 2, 150], 64, 0, 0),
    (2, 2048, 4, 8, 1, 128, [2048, 1500], 256, 0, 0),     # 32 queries per KV head
    (1, 96, 1, 2, 2, 64, None, 32, 40, 2),
    (2, 700, 3, 6, 2, 128, [700, 3], 96, 0, 0),           # pieces beyond a short row
    (1, 9000, 1, 8, 2, 64, None, 32, 0, 0),               # 282 pieces: two merge passes, ragged last chunk
]


@pytest.mark.parametrize("case", CASES)
def test_decode_split_and_merge(case):
    B, S, Lq, Hq, Hkv, D, lens, split, window, n_sink = case
    say(f"decode {case}")
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=41)
    scale = D ** -0.5
    Op_ref, Lp_ref = decode_split_ref(q, k, v, lens, split_keys=split, softmax_scale=scale, window=window,
                                      n_sink=n_sink)
    op, lp = usp.decode_split_fwd(q.cuda(), k.cuda(), v.cuda(), kv_lens=lens, split_keys=split, window=window,
                                  n_sink=n_sink)
    torch.cuda.synchronize()
    assert op.shape[0] == Op_ref.shape[0]
    for i in range(op.shape[0]):
        _check(op[i], lp[i], Op_ref[i], Lp_ref[i], f"piece {i}")
    O_ref, L_ref = decode_ref(q, k, v, lens, softmax_scale=scale, window=window, n_sink=n_sink)
    out, lse = usp.decode_merge(op.clone(), lp.clone())
    _check(out, lse, O_ref, L_ref, "merged")
    outb, lseb = usp.decode_fwd(q.cuda(), k.cuda(), v.cuda(), kv_lens=lens, split_keys=split, window=window,
                                n_sink=n_sink, out_dtype=torch.bfloat16)
    assert outb.dtype == torch.bfloat16
    _check(outb, lseb, O_ref, L_ref, "merged bf16")


def test_decode_large_cache_and_determinism():
    B, S, Lq, Hq, Hkv, D = 2, 65536, 1, 32, 8, 128
    say("decode large")
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=43)
    O_ref, L_ref = decode_ref(q, k, v, [S, 40000])
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, lse = usp.decode_fwd(qd, kd, vd, kv_lens=[S, 40000], split_keys=256)
    _check(out, lse, O_ref, L_ref, "large")
    for _ in range(3):
        o2, l2 = usp.decode_fwd(qd, kd, vd, kv_lens=[S, 40000], split_keys=256)
        assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("name", ["decode_gqa_128k", "decode_mqa_1m"])
def test_decode_workloads_full_size(name):
    """The two decode workloads at full size, with the piece size and inputs
    the benchmark uses: every piece's partial and the merged result against
    the oracle."""
    import bench
    cfg = bench.DECODE_WORKLOADS[name]
    B, S, Lq, Hq, Hkv, D = (cfg[x] for x in ("B", "S", "Lq", "Hq", "Hkv", "D"))
    say(f"decode full size {name}: generating inputs")
    q = si.randn_bf16((B, Lq, Hq, D), cfg["seed"], 0)
    k = si.randn_bf16((B, S, Hkv, D), cfg["seed"], 1)
    v = si.randn_bf16((B, S, Hkv, D), cfg["seed"], 2)
    split = usp.default_split_keys(B, S, Hkv)
    op, lp = usp.decode_split_fwd(q.cuda(), k.cuda(), v.cuda(), split_keys=split)
    out, lse = usp.decode_merge(op.clone(), lp.clone())
    torch.cuda.synchronize()
    say(f"decode full size {name}: oracle ({op.shape[0]} pieces of {split} keys)")
    Op_ref, Lp_ref = decode_split_ref(q, k, v, split_keys=split)
    for i in (0, 1, op.shape[0] // 2, op.shape[0] - 1):
        _check(op[i], lp[i], Op_ref[i], Lp_ref[i], f"piece {i}")
    O_ref, L_ref = decode_ref(q, k, v)
    _check(out, lse, O_ref, L_ref, "merged")


def _slopes(H):
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


@pytest.mark.parametrize("softcap,alibi", [(1.5, False), (0.0, True), (1.5, True)], ids=str)
@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[2], CASES[3]])
def test_decode_score_mods(case, softcap, alibi):
    """Softcap and ALiBi (per-row positions from 0) in the split kernel."""
    B, S, Lq, Hq, Hkv, D, lens, split, window, n_sink = case
    say(f"decode mods {case} cap={softcap} alibi={alibi}")
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=43)
    scale = D ** -0.5
    al = _slopes(Hq) if alibi else None
    kw = dict(softmax_scale=scale, window=window, n_sink=n_sink, softcap=softcap, alibi_slopes=al)
    Op_ref, Lp_ref = decode_split_ref(q, k, v, lens, split_keys=split, **kw)
    op, lp = usp.decode_split_fwd(q.cuda(), k.cuda(), v.cuda(), kv_lens=lens, split_keys=split, window=window,
                                  n_sink=n_sink, softcap=softcap, alibi_slopes=None if al is None else al.cuda())
    torch.cuda.synchronize()
    for i in range(op.shape[0]):
        _check(op[i], lp[i], Op_ref[i], Lp_ref[i], f"piece {i}")
    O_ref, L_ref = decode_ref(q, k, v, lens, **kw)
    out, lse = usp.decode_merge(op.clone(), lp.clone())
    _check(out, lse, O_ref, L_ref, "merged")
    O0, _ = decode_ref(q, k, v, lens, softmax_scale=scale, window=window, n_sink=n_sink)
    assert float((O0 - O_ref).abs().max()) > 10 * OUT_TOL   # the modifiers matter here


def test_decode_graph_replay():
    """A decode step (split kernel + merge) recorded into a HIP graph: every
    replay, with eager steps between, gives the eager bits."""
    say("decode graph replay")
    B, S, Lq, Hq, Hkv, D = 2, 8192, 1, 8, 2, 128
    q, k, v = _cache(B, S, Lq, Hq, Hkv, D, seed=47)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    split = 512
    n = S // split
    op = torch.empty((n, B, Lq, Hq, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((n, B, Hq, Lq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Lq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda")

    def step():
        usp.decode_split_fwd(qd, kd, vd, split_keys=split, out_part=op, lse_part=lp)
        usp.decode_merge(op, lp, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    O_ref, L_ref = decode_ref(q, k, v)
    _check(out, lse, O_ref, L_ref, "eager")
    eo, el = out.cpu().clone(), lse.cpu().clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        out.fill_(5.0)
        lse.fill_(5.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), eo) and torch.equal(lse.cpu(), el), f"replay {i}"
        step()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), eo) and torch.equal(lse.cpu(), el), f"eager {i}"
