"""Pins for oracle/attention_ref: the float64 masked-attention definition.

* brute force: pure-Python scalar loops (math.exp / math.fsum) with the
  visibility rule written again here from the page text, on tiny inputs
  covering every mask kind, GQA/MQA, batch and varlen;
* a library routine: torch's scaled_dot_product_attention on CPU float64 with
  an explicit boolean mask, and torch.logsumexp for the LSE;
* closed forms: window 1, zero queries, identical keys, window >= S;
* counts: each windowed query sees min(W, p+1) keys plus the sinks outside
  the window; the visible-pair totals of the five workloads in closed form;
* varlen: packed sequences never see each other and equal running alone.
"""
import json
import math
import os
import pytest
import torch
import torch.nn.functional as F

from oracle.attention_ref import attention_ref, visibility, visible_pair_count

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def vis_scalar(pq, pk, causal, W, n_sink, cu):
    """Visibility rule, restated from the page text (independent of the oracle)."""
    if cu is not None:
        sq = max(i for i in range(len(cu) - 1) if cu[i] <= pq)
        sk = max(i for i in range(len(cu) - 1) if cu[i] <= pk)
        if sq != sk:
            return False
        start = cu[sq]
    else:
        start = 0
    if (causal or W > 0) and pk > pq:
        return False
    if W > 0 and not (pq - pk < W or pk - start < n_sink):
        return False
    return True


def brute(q, k, v, scale, causal, W, n_sink, cu):
    """Scalar-loop attention over nested lists q[b][p][h][d]."""
    B, S, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    grp = Hq // Hkv
    O = [[[[0.0] * D for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    LSE = [[[-math.inf] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(S):
                keys = [j for j in range(S) if vis_scalar(i, j, causal, W, n_sink, cu)]
                if not keys:
                    continue
                sc = [scale * math.fsum(q[b][i][h][d] * k[b][j][g][d] for d in range(D)) for j in keys]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                l = math.fsum(e)
                for d in range(D):
                    O[b][i][h][d] = math.fsum(e[t] * v[b][keys[t]][g][d] for t in range(len(keys))) / l
                LSE[b][h][i] = m + math.log(l)
    return torch.tensor(O, dtype=torch.float64), torch.tensor(LSE, dtype=torch.float64)


def _inputs(B, S, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    return q, k, v


MASKS = [
    dict(causal=False, window=0, n_sink=0, cu=None),
    dict(causal=True, window=0, n_sink=0, cu=None),
    dict(causal=False, window=3, n_sink=0, cu=None),
    dict(causal=False, window=4, n_sink=2, cu=None),
    dict(causal=True, window=0, n_sink=0, cu=[0, 5, 6, 13]),
    dict(causal=False, window=0, n_sink=0, cu=[0, 7, 13]),
    dict(causal=False, window=3, n_sink=1, cu=[0, 2, 9, 13]),
]


@pytest.mark.parametrize("mk", MASKS)
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (3, 1)])
def test_oracle_matches_brute_force(mk, Hq, Hkv):
    cu = mk["cu"]
    S = 13
    B = 1 if cu else 2
    D = 8
    q, k, v = _inputs(B, S, Hq, Hkv, D, seed=7 + Hq)
    scale = 0.37
    O_b, L_b = brute(q.double().tolist(), k.double().tolist(), v.double().tolist(),
                     scale, mk["causal"], mk["window"], mk["n_sink"], cu)
    if cu:
        O, L = attention_ref(q[0], k[0], v[0], softmax_scale=scale, causal=mk["causal"],
                             window=mk["window"], n_sink=mk["n_sink"], cu_seqlens=cu)
        O, L = O.unsqueeze(0), L.unsqueeze(0)
    else:
        O, L = attention_ref(q, k, v, softmax_scale=scale, causal=mk["causal"],
                             window=mk["window"], n_sink=mk["n_sink"])
    assert torch.allclose(O, O_b, atol=1e-12, rtol=0)
    assert torch.equal(torch.isinf(L), torch.isinf(L_b))
    fin = torch.isfinite(L_b)
    assert torch.allclose(L[fin], L_b[fin], atol=1e-12, rtol=0)


def test_oracle_rows_and_heads_subset():
    q, k, v = _inputs(2, 40, 4, 2, 8, seed=3)
    O, L = attention_ref(q, k, v, causal=True, window=9, n_sink=2)
    rows = [39, 0, 17, 5]
    heads = [3, 1]
    Os, Ls = attention_ref(q, k, v, causal=True, window=9, n_sink=2, rows=rows, heads=heads)
    assert torch.allclose(Os, O[:, rows][:, :, heads], atol=1e-12, rtol=0)
    assert torch.allclose(Ls, L[:, heads][:, :, rows], atol=1e-12, rtol=0)


@pytest.mark.parametrize("mk", MASKS)
def test_oracle_matches_sdpa_float64(mk):
    cu = mk["cu"]
    S, Hq, Hkv, D = 13 * 9, 4, 2, 16
    if cu:
        cu = [x * 9 for x in cu]
    q, k, v = _inputs(1, S, Hq, Hkv, D, seed=11)
    scale = D ** -0.5
    mask = torch.tensor([[vis_scalar(i, j, mk["causal"], mk["window"] * 3, mk["n_sink"], cu)
                          for j in range(S)] for i in range(S)])
    assert mask.any(1).all()
    qh = q[0].double().permute(1, 0, 2)
    kh = k[0].double().repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    vh = v[0].double().repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    scores = (qh @ kh.transpose(1, 2)) * scale
    lse_ref = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
    if cu:
        O, L = attention_ref(q[0], k[0], v[0], softmax_scale=scale, causal=mk["causal"],
                             window=mk["window"] * 3, n_sink=mk["n_sink"], cu_seqlens=cu)
    else:
        O, L = attention_ref(q, k, v, softmax_scale=scale, causal=mk["causal"],
                             window=mk["window"] * 3, n_sink=mk["n_sink"])
        O, L = O[0], L[0]
    assert torch.allclose(O.permute(1, 0, 2), ref, atol=1e-10, rtol=0)
    assert torch.allclose(L, lse_ref, atol=1e-10, rtol=0)


def test_closed_form_window_one_is_self():
    q, k, v = _inputs(2, 30, 4, 2, 16, seed=5)
    scale = 0.25
    O, L = attention_ref(q, k, v, softmax_scale=scale, window=1)
    kv = (torch.arange(4) // 2)
    assert torch.equal(O, v[:, :, kv].double())
    self_score = scale * (q.double() * k[:, :, kv].double()).sum(-1)        # [B,S,H]
    assert torch.allclose(L, self_score.transpose(1, 2), atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal,window,n_sink", [(True, 0, 0), (False, 5, 0), (False, 6, 3), (False, 0, 0)])
def test_closed_form_zero_query_is_mean(causal, window, n_sink):
    B, S, H, D = 1, 25, 2, 8
    _, k, v = _inputs(B, S, H, H, D, seed=9)
    q = torch.zeros(B, S, H, D, dtype=torch.bfloat16)
    O, L = attention_ref(q, k, v, causal=causal, window=window, n_sink=n_sink)
    pos = torch.arange(S)
    mask = visibility(pos, pos, causal=causal, window=window, n_sink=n_sink)
    cnt = mask.sum(1).double()
    for p in range(S):
        keys = [j for j in range(S) if vis_scalar(p, j, causal, window, n_sink, None)]
        assert len(keys) == int(cnt[p])
        mean = v[0, keys].double().mean(0)
        assert torch.allclose(O[0, p], mean, atol=1e-12, rtol=0)
        assert abs(float(L[0, 0, p]) - math.log(len(keys))) < 1e-12


def test_closed_form_identical_keys():
    B, S, H, D = 1, 20, 2, 8
    q, k, v = _inputs(B, S, H, H, D, seed=13)
    k = k[:, :1].expand(B, S, H, D).contiguous()
    scale = 0.5
    O, L = attention_ref(q, k, v, softmax_scale=scale, causal=True)
    for p in range(S):
        for h in range(H):
            s = scale * float((q[0, p, h].double() * k[0, 0, h].double()).sum())
            assert torch.allclose(O[0, p, h], v[0, :p + 1, h].double().mean(0), atol=1e-12, rtol=0)
            assert abs(float(L[0, h, p]) - (s + math.log(p + 1))) < 1e-12


def test_window_at_least_S_is_causal():
    q, k, v = _inputs(1, 33, 2, 1, 8, seed=17)
    O1, L1 = attention_ref(q, k, v, causal=True)
    O2, L2 = attention_ref(q, k, v, window=33)
    O3, L3 = attention_ref(q, k, v, window=1000, n_sink=4)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert torch.equal(O1, O3) and torch.equal(L1, L3)


def test_window_count_matches_page_semantics():
    g = json.load(open(os.path.join(GOLDEN, "window_size_semantics.json")))
    W = g["window"]
    S = 8192
    pos = torch.arange(S)
    for case in g["cases"]:
        p = case["position"]
        m = visibility(torch.tensor([p]), pos, causal=False, window=W, n_sink=0)
        assert int(m.sum()) == case["visible"] == min(W, p + 1)


@pytest.mark.parametrize("W,n_sink", [(5, 1), (5, 4), (3, 6), (1, 2)])
def test_window_plus_sink_count(W, n_sink):
    S = 40
    pos = torch.arange(S)
    m = visibility(pos, pos, causal=False, window=W, n_sink=n_sink)
    for p in range(S):
        expect = min(W, p + 1) + max(0, min(n_sink, p - W + 1))
        assert int(m[p].sum()) == expect


def test_varlen_sequences_are_isolated():
    g = json.load(open(os.path.join(GOLDEN, "varlen_example.json")))
    cu = [x // 16 for x in g["cu_seqlens"]]          # same structure, 1/16 the size
    T = cu[-1]
    W = 20
    q, k, v = _inputs(1, T, 4, 4, 8, seed=19)
    O, L = attention_ref(q[0], k[0], v[0], window=W, n_sink=4, cu_seqlens=cu)
    pos = torch.arange(T)
    mask = visibility(pos, pos, causal=False, window=W, n_sink=4, cu_seqlens=cu)
    for a in range(len(cu) - 1):
        lo, hi = cu[a], cu[a + 1]
        assert not mask[lo:hi, :lo].any() and not mask[lo:hi, hi:].any()
        Oa, La = attention_ref(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], window=W, n_sink=4)
        assert torch.allclose(O[lo:hi], Oa[0], atol=1e-12, rtol=0)
        assert torch.allclose(L[:, lo:hi], La[0], atol=1e-12, rtol=0)


def _pairs_window_sink(n, W, n_sink):
    return sum(min(W, p + 1) + max(0, min(n_sink, p - W + 1)) for p in range(n))


def test_pair_count_closed_forms_small():
    # counting with the oracle's predicate agrees with the closed forms
    assert visible_pair_count(37, causal=True, window=0, n_sink=0) == 37 * 38 // 2
    assert visible_pair_count(50, causal=False, window=7, n_sink=0) == 7 * 8 // 2 + (50 - 7) * 7
    cu = [0, 5, 31, 52]
    total = sum(_pairs_window_sink(cu[i + 1] - cu[i], 9, 3) for i in range(3))
    assert visible_pair_count(52, causal=False, window=9, n_sink=3, cu_seqlens=cu) == total


def test_workload_pair_totals():
    # visible (query, key) pairs per (batch row, head) of the five workloads
    S = 1024
    assert S * (S + 1) // 2 == 524_800
    assert visible_pair_count(S, causal=True, window=0, n_sink=0) == 524_800
    W, S = 1000, 8192
    assert W * (W + 1) // 2 + (S - W) * W == 7_692_500
    assert visible_pair_count(S, causal=False, window=W, n_sink=0) == 7_692_500
    cu = [0, 512, 4000, 8192]
    tot = sum(_pairs_window_sink(cu[i + 1] - cu[i], 1000, 4) for i in range(3))
    assert tot == 6_835_036
    assert visible_pair_count(8192, causal=False, window=1000, n_sink=4, cu_seqlens=cu) == tot
    # zigzag rank share: 2 N c^2 + c with c = S / 2N (checked against masks in test_oracle_index)
    N, c = 4, 131072 // 8
    assert 2 * N * c * c + c == 2_147_500_032
    assert N * (2 * N * c * c + c) == 131072 * 131073 // 2
    # stripe rank 0 share: N L (L-1)/2 + L
    N, L = 8, 1048576 // 8
    assert N * L * (L - 1) // 2 + L == 68_719_083_520


def test_planted_mistakes_are_caught(monkeypatch):
    """The brute-force pin is sensitive to plausible predicate mistakes."""
    import oracle.attention_ref as ar
    q, k, v = _inputs(1, 13, 2, 2, 8, seed=29)
    O_b, L_b = brute(q.double().tolist(), k.double().tolist(), v.double().tolist(),
                     0.5, False, 4, 2, None)
    good = ar.visibility

    def off_by_one(pos_q, pos_k, *, causal, window, n_sink, cu_seqlens=None):
        return good(pos_q, pos_k, causal=causal, window=window + 1, n_sink=n_sink, cu_seqlens=cu_seqlens)

    def sink_dropped(pos_q, pos_k, *, causal, window, n_sink, cu_seqlens=None):
        return good(pos_q, pos_k, causal=causal, window=window, n_sink=0, cu_seqlens=cu_seqlens)

    for bad in (off_by_one, sink_dropped):
        monkeypatch.setattr(ar, "visibility", bad)
        O, L = ar.attention_ref(q, k, v, softmax_scale=0.5, window=4, n_sink=2)
        assert not torch.allclose(O, O_b, atol=1e-6)
    monkeypatch.setattr(ar, "visibility", good)
    O, L = ar.attention_ref(q, k, v, softmax_scale=0.5, window=4, n_sink=2)
    assert torch.allclose(O, O_b, atol=1e-12, rtol=0)
    # a transposed operand (k and v swapped) is caught too
    O, L = ar.attention_ref(q, v, k, softmax_scale=0.5, window=4, n_sink=2)
    assert not torch.allclose(O, O_b, atol=1e-6)
