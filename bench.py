"""Benchmark: one GPU's share of USP / ring attention on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one usp_ring_fwd call over the whole hot path of the workload:
the device tile planner, token permutation of q/k/v (natural -> ring layout)
with the Ulysses seq->head relayout (one strided gather per tensor when
ulysses_degree > 1), every ring step's block attention with the LSE merge,
and the output finalisation, including the Ulysses head->seq relayout of
the output for a Ulysses rank.  Inputs are seeded bf16 N(0,1), resident in
HBM before the timed region.  Prints one JSON line.

With no --workload the line's headline is the striped MQA share (one rank
of S = 2^20, the largest one-GPU workload), and "extra" carries the same
share's last rank and the USP zigzag GQA share, each with its own
roofline; --workload NAME times that workload alone.

value  = mask-adjusted attention TFLOP/s of the whole step
         (4 * D * Hq_local * B * visible pairs / step time);
roofline = the block-attention kernel alone: the same FLOPs over the summed
         duration of its launches, measured with HIP events on the launch
         stream, against the dense bf16 MFMA peak;
cpu_baseline = the float64 oracle on a bounded sample of the same
         workload's output rows, on this host's cores, in the same unit,
         with the full-output time extrapolated from the sampled rate.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0       # HBM3E
TRAFFIC_FILES = {
    "fwd": os.path.join(ROOT, "profiles", "attn_fwd_traffic.txt"),   # attn_fwd_kernel
    "bwd": os.path.join(ROOT, "profiles", "attn_bwd_traffic.txt"),   # bwd_dkdv_kernel
}


def measured_traffic(workload: str, kind: str = "fwd"):
    """HBM bytes per launch of the dominant kernel from the committed counter
    record (FETCH_SIZE / WRITE_SIZE scaled by the copy-kernel calibration), or
    None when there is no record for the workload or the kernel source changed
    since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILES[kind]):
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
        src = os.path.join(ROOT, kv["kernel_source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv["kernel_source_sha256"]:
            return None
        fetch = float(kv[workload + ".fetch_kib_per_launch"]) * 1024 * float(kv["fetch_factor"])
        write = float(kv[workload + ".write_kib_per_launch"]) * 1024 * float(kv["write_factor"])
        return int(round(fetch + write))
    except (OSError, KeyError, ValueError):
        return None


def visible_pairs_per_head(w, rank_rows=None) -> int:
    """Visible (query, key) pairs per (batch row, head) of the workload's
    output rows: closed forms of the causal / window / sink / varlen masks."""
    N, S = w.ring_degree, w.S
    L = S // N

    def window_count(n):  # pairs of one sequence of length n
        W, ns = w.window, w.n_sink
        if W <= 0:
            return n * (n + 1) // 2 if (w.causal) else n * n
        tot = 0
        full = min(n, W)
        tot += full * (full + 1) // 2
        if n > W:
            tot += (n - W) * W
            # sinks outside the window: p - W + 1 capped at ns, for p >= W
            for p in range(W, n):
                tot += min(ns, p - W + 1)
        return tot

    if w.rank < 0:
        if w.cu_seqlens is not None:
            cu = w.cu_seqlens
            return sum(window_count(cu[i + 1] - cu[i]) for i in range(len(cu) - 1))
        return window_count(S)
    # one rank's share under a causal mask (the two one-rank workloads)
    assert w.causal and w.window == 0 and w.cu_seqlens is None
    if w.impl == "zigzag":
        c = S // (2 * N)
        return 2 * N * c * c + c
    if w.impl == "stripe" and w.stripe_block == 1:
        return N * L * (L - 1) // 2 + (w.rank + 1) * L
    if w.impl == "stripe":
        # striped blocks of b tokens: local row t = j*b + o of rank r sits at
        # position p = (j*N + r)*b + o and sees the p + 1 keys 0..p; summed
        # over j < L/b and o < b
        b, r = w.stripe_block, w.rank
        nb = L // b
        sum_j = nb * (nb - 1) // 2
        return b * b * N * sum_j + nb * b * r * b + nb * (b * (b - 1) // 2) + L
    raise ValueError("no closed form for this workload")


def step_bytes(w):
    """Algorithmic HBM bytes (read + write) of the staging copies in one step,
    as (row gather, Ulysses relayout).  With ulysses_degree > 1 the ring
    library does both in one strided copy per tensor (ring-ordered rows of
    Ulysses rank u's head group): its bytes are the first entry and the
    second is 0."""
    N, ud, S, B, D = w.ring_degree, w.ulysses_degree, w.S, w.B, w.D
    L = S // N
    q_rows = L if w.rank >= 0 else S                              # q: rank extract or full
    if ud > 1:
        return (2 * B * q_rows * (w.Hq // ud) * D * 2              # q rows of head group u
                + 2 * 2 * B * S * (w.Hkv // ud) * D * 2), 0        # k and v, all pieces
    perm = 0
    if w.impl != "basic":
        perm += 2 * 2 * B * S * w.Hkv * D * 2                      # k and v, full permute
        perm += 2 * B * q_rows * w.Hq * D * 2
    return perm, 0


def time_lse_merge(w, merge_mode: int, merge_timing) -> dict:
    """GB/s of the LSE merge kernel (usp_lse_merge) over one step's
    accumulator: f32 O [B, rows, Hq_local, D] and LSE [B, Hq_local, rows],
    timed standalone on seeded accumulators of that shape, outside the timed
    steps (the ring merges inside the attention epilogue unless merge_mode
    is 1).  With merge_mode 1 the ring's own merge launches are reported
    too; they read a partial the attention kernel has just written, much of
    it still in the cache, so their rate is not an HBM rate."""
    import torch

    import ulysses_sequence_attention_zigzag_amd as usp

    Hl = w.Hq // w.ulysses_degree
    rows = w.S // w.ring_degree if w.rank >= 0 else w.S
    B = 1 if w.cu_seqlens is not None else w.B
    nbytes = 3 * B * rows * Hl * (w.D + 1) * 4       # read acc + part, write acc (O and LSE)
    g = torch.Generator(device="cuda").manual_seed(77)
    oa = torch.randn((B, rows, Hl, w.D), generator=g, device="cuda")
    op = torch.randn((B, rows, Hl, w.D), generator=g, device="cuda")
    la = torch.randn((B, Hl, rows), generator=g, device="cuda")
    lp = torch.randn((B, Hl, rows), generator=g, device="cuda")
    for _ in range(2):
        usp.lse_merge(oa, la, op, lp)
    torch.cuda.synchronize()
    reps = 5
    usp.timing_reset()
    usp.timing_enable(True)
    for _ in range(reps):
        usp.lse_merge(oa, la, op, lp)
    torch.cuda.synchronize()
    usp.timing_enable(False)
    ms, n = usp.timing_read("merge")
    usp.timing_reset()
    rec = {"bytes": nbytes, "ms": None, "GB/s": None, "pct_hbm": None,
           "source": "standalone usp_lse_merge on seeded accumulators of one step's shape"}
    if n > 0 and ms > 0:
        per = ms / n
        gbps = nbytes / (per * 1e-3) / 1e9
        rec.update({"ms": round(per, 4), "GB/s": round(gbps, 1), "pct_hbm": round(100 * gbps / PEAK_HBM_GBS, 1)})
    if merge_mode == 1 and merge_timing[1] > 0:
        rec["in_ring_ms"] = round(merge_timing[0] / merge_timing[1], 4)
    return rec


def oracle_threads() -> int:
    """Gives the oracle every CPU this process may run on (the machine's
    logical CPUs unless an affinity mask narrows them) and returns that
    count."""
    import torch

    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    torch.set_num_threads(max(1, n))
    return torch.get_num_threads()


def host_info() -> dict:
    """The host the oracle runs on: the threads torch uses (the process's CPU
    share, set through OMP_NUM_THREADS), the machine's logical CPU count, the
    CPUs this process may run on, and the CPU model."""
    import subprocess

    import torch

    info = {"threads": torch.get_num_threads(), "cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    info["model"] = model
    return info


def cpu_baseline(w, q, k, v, budget_s: float):
    """Times the float64 oracle on a seeded sample of the workload's output rows."""
    import torch
    from oracle import index_ref as ix
    from oracle.attention_ref import attention_ref

    threads = oracle_threads()
    if w.rank >= 0:
        pos = ix.rank_positions(w.impl, w.S, w.ring_degree, w.rank, w.stripe_block)
        Hl = w.Hq // w.ulysses_degree
        heads = list(range(w.ulysses_rank * Hl, (w.ulysses_rank + 1) * Hl))
    else:
        pos = list(range(w.S))
        heads = list(range(w.Hq))
    g = torch.Generator().manual_seed(4242)
    order = torch.randperm(len(pos), generator=g).tolist()
    kw = dict(softmax_scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink,
              cu_seqlens=w.cu_seqlens, heads=heads)

    def keys_seen(p):
        if w.window > 0:
            s = 0
            if w.cu_seqlens is not None:
                s = max(c for c in w.cu_seqlens[:-1] if c <= p)
            off = p - s
            return min(w.window, off + 1) + max(0, min(w.n_sink, off - w.window + 1))
        if w.causal:
            return p + 1
        return w.S

    done, flops, t_used, n = 0, 0.0, 0.0, 4
    while t_used < budget_s and done < len(order):
        rows = [pos[i] for i in order[done:done + n]]
        t0 = time.perf_counter()
        attention_ref(q, k, v, rows=rows, **kw)
        dt = time.perf_counter() - t0
        t_used += dt
        done += len(rows)
        bmul = 1 if w.cu_seqlens is not None else w.B
        flops += sum(4.0 * w.D * len(heads) * bmul * keys_seen(p) for p in rows)
        # grow the batch so the remaining budget is used in a few calls
        per_row = dt / max(1, len(rows))
        n = max(1, min(4096, int(0.3 * max(0.0, budget_s - t_used) / max(per_row, 1e-6))))
    rate = flops / t_used
    bmul = 1 if w.cu_seqlens is not None else w.B
    full_flops = 4.0 * w.D * len(heads) * bmul * visible_pairs_per_head(w)
    rec = {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(pos)} output rows x {len(heads)} heads"
                  f"{' x ' + str(w.B) + ' batch rows' if w.B > 1 and w.cu_seqlens is None else ''}, "
                  f"float64 torch CPU, {t_used:.1f} s",
        "host": host_info(),
    }
    if done < len(pos):
        # the whole output at the sampled rate (FLOP-weighted, so causal rows count by their keys)
        rec["extrapolated_full_s"] = round(full_flops / rate, 1)
        rec["extrapolated_note"] = "extrapolated: full-output oracle time = the workload's FLOPs / the sampled rate"
    else:
        rec["full_s"] = round(t_used, 2)
    return rec


def cpu_baseline_bwd(w, q, k, v, dout, budget_s: float):
    """Times the float64 oracle's backward on a seeded sample of the
    workload's query rows: their forward (O, LSE), delta, and their gradient
    terms against every key (dQ of the rows, their dK / dV contributions).
    Counted like the GPU value: 10 * D per visible pair."""
    import torch
    from oracle import index_ref as ix
    from oracle.attention_ref import attention_ref
    from oracle.backward_ref import block_attention_bwd_ref

    threads = oracle_threads()
    varlen = w.cu_seqlens is not None
    qb, kb, vb = (t.unsqueeze(0) if varlen else t for t in (q, k, v))
    db = dout.unsqueeze(0) if varlen else dout
    if w.rank >= 0:
        pos = ix.rank_positions(w.impl, w.S, w.ring_degree, w.rank, w.stripe_block)
        Hl, Hkl = w.Hq // w.ulysses_degree, w.Hkv // w.ulysses_degree
        heads = list(range(w.ulysses_rank * Hl, (w.ulysses_rank + 1) * Hl))
        kvh = list(range(w.ulysses_rank * Hkl, (w.ulysses_rank + 1) * Hkl))
        local = True
    else:
        pos = list(range(w.S))
        heads, kvh = list(range(w.Hq)), list(range(w.Hkv))
        local = False
    kh, vh = kb[:, :, kvh], vb[:, :, kvh]
    g = torch.Generator().manual_seed(4243)
    order = torch.randperm(len(pos), generator=g).tolist()
    kw = dict(softmax_scale=w.scale, causal=w.causal, window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens)
    done, flops, t_used, n = 0, 0.0, 0.0, 2
    all_pos = list(range(w.S))
    bmul = 1 if varlen else w.B
    while t_used < budget_s and done < len(order):
        idx = order[done:done + n]
        rows = [pos[i] for i in idx]
        t0 = time.perf_counter()
        O, LSE = attention_ref(q, k, v, rows=rows, heads=heads, **kw)
        if varlen:
            O, LSE = O.unsqueeze(0), LSE.unsqueeze(0)
        d_rows = db[:, idx] if local else db[:, rows][:, :, heads]
        delta = (d_rows.double() * O).sum(-1).transpose(1, 2)
        qr = qb[:, rows][:, :, heads]
        block_attention_bwd_ref(qr, kh, vh, d_rows, LSE, delta, rows, all_pos, scale=w.scale, causal=w.causal,
                                window=w.window, n_sink=w.n_sink, cu_seqlens=w.cu_seqlens)
        dt = time.perf_counter() - t0
        t_used += dt
        done += len(rows)
        flops += 10.0 * w.D * len(heads) * bmul * float(visible_pairs_for_rows(w, rows))
        per_row = dt / max(1, len(rows))
        n = max(1, min(1024, int(0.3 * max(0.0, budget_s - t_used) / max(per_row, 1e-6))))
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(pos)} query rows x {len(heads)} heads against every key: forward, delta "
                  f"and backward, float64 torch CPU, {t_used:.1f} s",
    }


def visible_pairs_for_rows(w, rows) -> int:
    """Visible keys summed over the given global query positions."""
    total = 0
    for p in rows:
        if w.window > 0:
            s = 0
            if w.cu_seqlens is not None:
                s = max(c for c in w.cu_seqlens[:-1] if c <= p)
            off = p - s
            total += min(w.window, off + 1) + max(0, min(w.n_sink, off - w.window + 1))
        elif w.causal:
            s = 0
            if w.cu_seqlens is not None:
                s = max(c for c in w.cu_seqlens[:-1] if c <= p)
            total += p - s + 1
        else:
            if w.cu_seqlens is not None:
                s = max(c for c in w.cu_seqlens[:-1] if c <= p)
                e = min(c for c in w.cu_seqlens[1:] if c > p)
                total += e - s
            else:
                total += w.S
    return total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="one workload (default: the striped MQA share as the headline, with the USP zigzag "
                         "GQA share and the striped share's last rank as extra records)")
    ap.add_argument("--rank", type=int, default=None, help="one-rank workloads: the ring rank to time")
    ap.add_argument("--merge-mode", type=int, default=0)
    ap.add_argument("--out-layout", choices=["seq", "heads"], default="seq",
                    help="Ulysses ranks: seq (head -> seq relayout of the output, the default) or heads")
    ap.add_argument("--graph", action="store_true",
                    help="forward / decode: also time the step replayed from a HIP graph (graph_replay in the "
                         "JSON; value stays the eager rate)")
    ap.add_argument("--stripe-block", type=int, default=0,
                    help="striped workload only: tokens per stripe block (0: the workload's own, 1); b > 1 runs "
                         "the kernel form for stepped masks")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "decode"], default="forward",
                    help="forward: usp_ring_fwd (default); backward: usp_ring_bwd of that forward; "
                         "decode: split-KV decode + merge over a KV cache (--workload decode_gqa_128k or "
                         "decode_mqa_1m)")
    ap.add_argument("--split-keys", type=int, default=0,
                    help="decode: keys per cache piece (0: the binding's default_split_keys)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy kernel (float32 negate) over MIB MiB, three times, "
                         "as the known-size reference for HBM byte counters, and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs one GPU's share only; --gpus {args.gpus} is not supported "
              "(the multi-GPU ring and Ulysses all-to-all are not part of this library)", file=sys.stderr)
        sys.exit(2)

    import torch

    import seeded_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"read_bytes": 4 * n, "write_bytes": 4 * n, "launches": 3}}))
        return
    if args.which == "decode":
        return bench_decode(args)
    if args.workload is None and args.which == "backward":
        args.workload = "usp_zigzag_gqa"
    if args.workload is not None:
        w = workload_of(si, args, args.workload)
        q, k, v = gen_inputs(w)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        if args.which == "backward":
            return bench_backward(args, w, q, k, v, qd, kd, vd)
        rec = forward_record(args, w, q, k, v, qd, kd, vd, with_cpu=not args.no_cpu_baseline,
                             cpu_budget=args.cpu_budget)
        print(json.dumps(rec), flush=True)
        return

    # default: the striped MQA share (the largest one-GPU workload) is the
    # headline; its last rank (the most work) and the USP zigzag GQA share
    # (with the Ulysses output relayout) are extra records
    w4 = workload_of(si, args, "stripe_mqa")
    q, k, v = gen_inputs(w4)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    rec = forward_record(args, w4, q, k, v, qd, kd, vd, with_cpu=not args.no_cpu_baseline,
                         cpu_budget=args.cpu_budget)
    w4r = w4.scaled(rank=w4.ring_degree - 1)
    extra = {"stripe_mqa_rank%d" % w4r.rank: forward_record(args, w4r, q, k, v, qd, kd, vd, with_cpu=False)}
    del q, k, v, qd, kd, vd
    torch.cuda.empty_cache()
    w3 = workload_of(si, args, "usp_zigzag_gqa")
    q, k, v = gen_inputs(w3)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    extra["usp_zigzag_gqa"] = forward_record(args, w3, q, k, v, qd, kd, vd, with_cpu=not args.no_cpu_baseline,
                                             cpu_budget=min(args.cpu_budget, 10.0))
    for r in extra.values():
        for key in ("n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "dtype", "data",
                    "metric"):
            r.pop(key, None)
    rec["extra"] = extra
    print(json.dumps(rec), flush=True)


def workload_of(si, args, name):
    w = si.WORKLOADS[name]
    if args.stripe_block:
        if w.impl != "stripe":
            print("--stripe-block applies to the striped workload only", file=sys.stderr)
            sys.exit(2)
        w = w.scaled(stripe_block=args.stripe_block)
    if args.rank is not None:
        if w.rank < 0:
            print("--rank applies to the one-rank workloads only", file=sys.stderr)
            sys.exit(2)
        w = w.scaled(rank=args.rank)
    return w


def gen_inputs(w):
    t0 = time.perf_counter()
    q, k, v = w.make_inputs()
    print(f"# {w.name}: inputs generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    return q, k, v


def forward_record(args, w, q, k, v, qd, kd, vd, with_cpu: bool, cpu_budget: float = 15.0) -> dict:
    """Times usp_ring_fwd over the workload: K steps after W warm-ups, the
    attention kernel's own launches bracketed by HIP events on its stream."""
    import torch

    import ulysses_sequence_attention_zigzag_amd as usp

    out_layout = args.out_layout if (w.rank >= 0 and w.ulysses_degree > 1) else "heads"
    call = usp.RingCall(qd, kd, vd, impl=w.impl, ring_degree=w.ring_degree, ulysses_degree=w.ulysses_degree,
                        stripe_block=w.stripe_block, causal=w.causal, window=w.window, n_sink=w.n_sink,
                        cu_seqlens=w.cu_seqlens, softmax_scale=w.softmax_scale or 0.0, rank=w.rank,
                        ulysses_rank=w.ulysses_rank, merge_mode=args.merge_mode, out_layout=out_layout)
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()
    print(f"# {w.name} rank {w.rank}: warmup done", file=sys.stderr, flush=True)

    usp.timing_reset()
    usp.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call.run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    usp.timing_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    kt = {c: usp.timing_read(c) for c in ("attn", "permute", "relayout", "merge", "plan")}
    usp.timing_reset()

    Hl = w.Hq // w.ulysses_degree
    bmul = 1 if w.cu_seqlens is not None else w.B
    pairs = visible_pairs_per_head(w)
    flops = 4.0 * w.D * Hl * bmul * pairs
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_ms, attn_n = kt["attn"]
    attn_ms_step = attn_ms / args.steps
    attn_tflops = flops / (attn_ms_step * 1e-3) / 1e12 if attn_ms > 0 else None
    perm_bytes, _ = step_bytes(w)
    perm_ms = kt["permute"][0] / args.steps
    merge_rec = time_lse_merge(w, args.merge_mode, kt["merge"])
    graph_rec = None
    if args.graph:
        graph = call.capture()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        graph_rec = {"ms_per_step": round(g_ms, 4), "TFLOP/s": round(flops / (g_ms * 1e-3) / 1e12, 2)}

    def gbs(b, ms):
        return round(b / (ms * 1e-3) / 1e9, 1) if ms > 0 and b > 0 else None

    copy_name = "permute+relayout" if w.ulysses_degree > 1 else "permute"
    rec = {
        "metric": "masked-attention TFLOPS (mask-adjusted, % of dense bf16 MFMA peak); permute/merge GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B, "S_global": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "ring_impl": w.impl, "ring_degree": w.ring_degree, "ulysses_degree": w.ulysses_degree,
            "stripe_block": w.stripe_block,
            "rank": w.rank, "ulysses_rank": w.ulysses_rank, "causal": w.causal, "window": w.window,
            "n_sink": w.n_sink, "cu_seqlens": w.cu_seqlens, "merge_mode": args.merge_mode,
            "out_layout": out_layout,
            "mask_adjusted_tflop_per_step": round(flops / 1e12, 4),
        },
        "pct_peak_end_to_end": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2) if attn_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4) if attn_tflops else None,
            # the counter record was taken on the workloads as defined (stripe block 1, rank 0)
            "traffic": (measured_traffic(w.name if w.rank <= 0 else "%s_rank%d" % (w.name, w.rank))
                        if w.stripe_block == 1 else None),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "attn_fwd_kernel<%d%s>" % (w.D, "" if w.stripe_block == 1 else ", stepped"),
            "launches_per_step": attn_n // max(1, args.steps),
            "kernel_ms_per_step": round(attn_ms_step, 4),
        },
        "copy_kernels": {
            # the layout's row gather (with Ulysses: fused with the head split)
            copy_name: {
                "bytes": perm_bytes, "ms": round(perm_ms, 4), "GB/s": gbs(perm_bytes, perm_ms),
                "pct_hbm": round(100 * perm_bytes / (perm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)
                if perm_ms > 0 and perm_bytes > 0 else None},
            "merge": merge_rec,
        },
        "planner_ms_per_step": round(kt["plan"][0] / args.steps, 4),
        "cpu_baseline": None,
    }
    if graph_rec is not None:
        rec["graph_replay"] = graph_rec
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, cpu_budget)
    del call
    return rec


def bench_backward(args, w, q, k, v, qd, kd, vd):
    """Times usp_ring_bwd over the workload: the forward runs once untimed;
    a step is the whole backward (staging of q, k, v, delta, every ring
    step's dQ and dK / dV kernels, output order)."""
    import torch

    import seeded_inputs as si
    import ulysses_sequence_attention_zigzag_amd as usp

    fwd = usp.RingCall(qd, kd, vd, impl=w.impl, ring_degree=w.ring_degree, ulysses_degree=w.ulysses_degree,
                       stripe_block=w.stripe_block, causal=w.causal, window=w.window, n_sink=w.n_sink,
                       cu_seqlens=w.cu_seqlens, softmax_scale=w.softmax_scale or 0.0, rank=w.rank,
                       ulysses_rank=w.ulysses_rank)
    fwd.run()
    dout = si.randn_bf16(tuple(fwd.out.shape), w.seed, 3)
    call = usp.RingBwdCall(fwd, dout.cuda())
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)
    classes = ("bwd_dq", "bwd_dkdv", "bwd_delta", "permute", "relayout")
    usp.timing_reset()
    usp.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call.run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    usp.timing_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    kt = {c: usp.timing_read(c) for c in classes}
    usp.timing_reset()

    Hl = w.Hq // w.ulysses_degree
    bmul = 1 if w.cu_seqlens is not None else w.B
    pairs = visible_pairs_per_head(w)
    unit_flops = w.D * Hl * bmul * pairs
    flops = 10.0 * unit_flops
    tflops = flops / (ms_step * 1e-3) / 1e12
    kernels = {}
    for name, cls, per_pair in (("bwd_dkdv_kernel<%d>" % w.D, "bwd_dkdv", 8), ("bwd_dq_kernel<%d>" % w.D,
                                                                            "bwd_dq", 6)):
        ms = kt[cls][0] / args.steps
        ach = per_pair * unit_flops / (ms * 1e-3) / 1e12 if ms > 0 else None
        kernels[name] = {"ms_per_step": round(ms, 4), "launches_per_step": kt[cls][1] // max(1, args.steps),
                         "flop_per_pair": per_pair * w.D, "TFLOP/s": round(ach, 2) if ach else None}
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    ach = kernels[dom]["TFLOP/s"]
    rec = {
        "metric": "masked-attention backward TFLOPS (10*D FLOP per visible pair, % of dense bf16 MFMA peak)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "pass": "backward",
            "B": w.B, "S_global": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "ring_impl": w.impl, "ring_degree": w.ring_degree, "ulysses_degree": w.ulysses_degree,
            "stripe_block": w.stripe_block,
            "rank": w.rank, "ulysses_rank": w.ulysses_rank, "causal": w.causal, "window": w.window,
            "n_sink": w.n_sink, "cu_seqlens": w.cu_seqlens,
            "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        },
        "pct_peak_end_to_end": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": ach,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4) if ach else None,
            "traffic": measured_traffic(w.name, "bwd") if dom.startswith("bwd_dkdv") else None,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": dom,
            "launches_per_step": kernels[dom]["launches_per_step"],
            "kernel_ms_per_step": kernels[dom]["ms_per_step"],
        },
        "kernels": kernels,
        "other_ms_per_step": {c: round(kt[c][0] / args.steps, 4) for c in ("bwd_delta", "permute", "relayout")},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, dout, args.cpu_budget)
    print(json.dumps(rec), flush=True)


# Decode workloads: one new token per sequence over a full KV cache, with
# the head counts of the two large ring workloads (global heads: decoding
# runs after the sequence-parallel prefill, on the gathered cache).
DECODE_WORKLOADS = {
    "decode_gqa_128k": dict(B=4, S=131072, Lq=1, Hq=32, Hkv=8, D=128, seed=2001),
    "decode_mqa_1m": dict(B=1, S=1048576, Lq=1, Hq=8, Hkv=1, D=128, seed=2002),
}


def cpu_baseline_decode(cfg, q, k, v, budget_s: float):
    """Times the float64 oracle's decode on whole (batch row, KV head) units
    of the workload: bytes of K / V attended per second."""
    import torch
    from oracle.decode_ref import decode_ref

    threads = oracle_threads()
    B, Hkv, group = cfg["B"], cfg["Hkv"], cfg["Hq"] // cfg["Hkv"]
    done, t_used, nbytes = 0, 0.0, 0
    units = [(b, g) for b in range(B) for g in range(Hkv)]
    while t_used < budget_s and done < len(units):
        b, g = units[done]
        qs = q[b:b + 1, :, g * group:(g + 1) * group]
        ks, vs = k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1]
        t0 = time.perf_counter()
        decode_ref(qs, ks, vs)
        t_used += time.perf_counter() - t0
        nbytes += 2 * ks.numel() * 2
        done += 1
    return {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(units)} (batch row, KV head) units, whole cache, float64 torch CPU, "
                      f"{t_used:.1f} s"}


def bench_decode(args):
    """Times one decode step (usp_decode_split_fwd + usp_decode_merge) over a
    KV cache resident in HBM; the split kernel is HBM-bound."""
    import torch

    import seeded_inputs as si
    import ulysses_sequence_attention_zigzag_amd as usp

    name = args.workload if args.workload in DECODE_WORKLOADS else "decode_gqa_128k"
    cfg = DECODE_WORKLOADS[name]
    B, S, Lq, Hq, Hkv, D = (cfg[x] for x in ("B", "S", "Lq", "Hq", "Hkv", "D"))
    q = si.randn_bf16((B, Lq, Hq, D), cfg["seed"], 0)
    k = si.randn_bf16((B, S, Hkv, D), cfg["seed"], 1)
    v = si.randn_bf16((B, S, Hkv, D), cfg["seed"], 2)
    print("# inputs generated", file=sys.stderr, flush=True)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    split = args.split_keys or usp.default_split_keys(B, S, Hkv)
    n = (S + split - 1) // split
    op = torch.empty((n, B, Lq, Hq, D), dtype=torch.float32, device="cuda")
    lp = torch.empty((n, B, Hq, Lq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Lq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda")

    def step():
        usp.decode_split_fwd(qd, kd, vd, split_keys=split, out_part=op, lse_part=lp)
        usp.decode_merge(op, lp, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    usp.timing_reset()
    usp.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    usp.timing_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    split_ms, split_n = usp.timing_read("decode")
    merge_ms, _ = usp.timing_read("decode_merge")
    usp.timing_reset()
    split_ms /= args.steps
    merge_ms /= args.steps
    graph_ms = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kv_bytes = 2 * B * S * Hkv * D * 2
    part_bytes = n * B * Lq * Hq * (D + 1) * 4
    split_bytes = kv_bytes + B * Lq * Hq * D * 2 + part_bytes          # read K, V, q; write partials
    step_bytes = split_bytes + part_bytes + B * Lq * Hq * (D + 1) * 4   # + merge reads partials, writes out / lse
    achieved = split_bytes / (split_ms * 1e-3) / 1e9
    rec = {
        "metric": "decode HBM GB/s (K/V cache read once per step, % of HBM peak)",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "pass": "decode", "B": B, "S_cache": S, "Lq": Lq, "Hq": Hq, "Hkv": Hkv, "D": D,
                   "split_keys": split, "pieces": n, "algorithmic_bytes_per_step": step_bytes},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None,
            "kernel": "decode_split_kernel<%d>" % D,
            "launches_per_step": split_n // max(1, args.steps),
            "kernel_ms_per_step": round(split_ms, 4),
        },
        "merge_ms_per_step": round(merge_ms, 4),
        "cpu_baseline": None,
    }
    if graph_ms is not None:
        rec["graph_replay"] = {"ms_per_step": round(graph_ms, 4),
                               "GB/s": round(step_bytes / (graph_ms * 1e-3) / 1e9, 1)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_decode(cfg, q, k, v, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
