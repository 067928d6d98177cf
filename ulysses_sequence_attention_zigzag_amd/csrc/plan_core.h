// Tile planner, per item: which key rows one tile of query rows must visit
// (or, transposed, which query rows see one tile of keys), and which of
// those runs need no per-element mask.  The same code runs on the host
// (inspection calls, workspace sizing) and in the device planner kernels,
// which write the tile lists into the caller's workspace on every call.
//
// For a tile of query rows inside one monotone piece of a rank's rows
// (positions increase with the row index), the visible keys are contained in
//   * the band  [max(seq_start, pq_min - W + 1), min(seq_end - 1, pq_max)]
//     (window / causal / same-sequence constraints, hull over the rows), and
//   * for each sequence the rows touch, its first n_sink positions
//     (attention sinks; only with a window),
// and a key is visible to every row of the tile when its position lies in
//   [max(seq_start, pq_max - W + 1), min(seq_end - 1, pq_min)]
// with all rows in one sequence.  Position intervals become local key
// intervals by binary search over each monotone piece of the KV rank's rows
// [LCA "Ring Attention": each ring step is one block of the attention matrix;
// SWA: window, sinks and cu_seqlens on global positions].  The kernels
// evaluate the exact predicate inside partial runs, so these hulls only need
// to be conservative.
//
// The intervals of one piece are produced in increasing position order (the
// sinks of consecutive sequences, with the band slotted in at its place), so
// their local images come in nondecreasing order and are merged on the fly:
// no interval list is stored, which is what lets one GPU thread plan one
// item.
#pragma once

#include "usp_internal.h"

namespace usp {

__host__ __device__ inline int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }
__host__ __device__ inline int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ inline int32_t imax32(int32_t a, int32_t b) { return a > b ? a : b; }
__host__ __device__ inline int32_t imin32(int32_t a, int32_t b) { return a < b ? a : b; }

// Sequences of the packed axis: cu_seqlens (global over all ranks), or one
// sequence [0, S).
struct SeqView {
  const int32_t* cu;  // nullptr: one sequence [0, S)
  int32_t nseq;
  int32_t S;
  // largest i with cu[i] <= p (the sequence holding p; empty sequences skipped)
  __host__ __device__ int32_t index(int64_t p) const {
    if (!cu) return 0;
    int32_t lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) / 2;
      if (cu[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __host__ __device__ int64_t start(int32_t i) const { return cu ? cu[i] : 0; }
  __host__ __device__ int64_t end(int32_t i) const { return cu ? cu[i + 1] : S; }
};

// First u in [lo, hi) with position(u) >= P (hi if none); positions increase
// on [lo, hi), a monotone piece.  Closed form (first_row_at_least) between
// the two end checks, which also keep P inside int32.
__host__ __device__ inline int32_t bsearch_at_least(const PosMap& m, int32_t lo, int32_t hi, int64_t P) {
  if (lo >= hi || P <= position(m, lo)) return lo;
  if (P > position(m, hi - 1)) return hi;
  const int32_t u = first_row_at_least(m, lo, (int32_t)P);
  return u < lo ? lo : (u > hi ? hi : u);
}

// First u in [lo, hi) with position(u) > P (hi if none).
__host__ __device__ inline int32_t bsearch_above(const PosMap& m, int32_t lo, int32_t hi, int64_t P) {
  return bsearch_at_least(m, lo, hi, P + 1);
}

// Items (tiles of `tile` rows inside the monotone pieces) of one rank's rows.
__host__ __device__ inline int32_t tile_count(const PosMap& m, int32_t tile) {
  int32_t lo[2], hi[2];
  const int n = monotone_segments(m, lo, hi);
  int32_t c = 0;
  for (int s = 0; s < n; ++s) c += (hi[s] - lo[s] + tile - 1) / tile;
  return c;
}

// First row and row count of tile c (pieces in order, tiles in row order).
__host__ __device__ inline void tile_rows(const PosMap& m, int32_t tile, int32_t c, int32_t* t0, int32_t* rows) {
  int32_t lo[2], hi[2];
  const int n = monotone_segments(m, lo, hi);
  for (int s = 0; s < n; ++s) {
    const int32_t k = (hi[s] - lo[s] + tile - 1) / tile;
    if (c < k || s == n - 1) {
      *t0 = lo[s] + c * tile;
      *rows = imin32(tile, hi[s] - *t0);
      return;
    }
    c -= k;
  }
}

// Merges local intervals arriving in nondecreasing start order (touching or
// overlapping ones join) and cuts each merged interval into runs: the part
// inside [f0, f1) (visible to every row of the item), in multiples of
// `gran`, is one full run, the rest partial runs.  Emit(k_begin, k_end, full).
template <class Emit>
struct RunMerger {
  Emit& emit;
  int32_t f0, f1, gran;
  int32_t a = 0, b = 0;
  bool have = false;
  __host__ __device__ RunMerger(Emit& e, int32_t f0_, int32_t f1_, int32_t g) : emit(e), f0(f0_), f1(f1_), gran(g) {}
  __host__ __device__ void add(int32_t u0, int32_t u1) {
    if (u0 >= u1) return;
    if (have && u0 <= b) {
      if (u1 > b) b = u1;
      return;
    }
    flush();
    a = u0;
    b = u1;
    have = true;
  }
  __host__ __device__ void flush() {
    if (!have) return;
    have = false;
    const int32_t x0 = imax32(a, f0), x1 = imin32(b, f1);
    if (x1 - x0 >= gran) {
      const int32_t nfull = (x1 - x0) / gran * gran;
      if (a < x0) emit(a, x0, 0);
      emit(x0, x0 + nfull, 1);
      if (x0 + nfull < b) emit(x0 + nfull, b, 0);
    } else {
      emit(a, b, 0);
    }
  }
};

// Runs of keys of kmap's rank visible to query rows [t0, t0 + rows) of
// qmap's rank (one monotone piece).  Full runs come in multiples of `gran`.
template <class Emit>
__host__ __device__ void plan_query_tile(const PosMap& qmap, const PosMap& kmap, const MaskSpec& ms, const SeqView& seq,
                                         int32_t t0, int32_t rows, int32_t gran, Emit& emit) {
  const bool cw = ms.causal || ms.window > 0;
  const int64_t W = ms.window;
  const int64_t pq_min = position(qmap, t0);
  const int64_t pq_max = position(qmap, t0 + rows - 1);
  const int32_t s_min = seq.index(pq_min);
  const int32_t s_max = seq.index(pq_max);
  int64_t band_lo = seq.start(s_min);
  if (W > 0) band_lo = imax64(band_lo, pq_min - W + 1);
  int64_t band_hi = seq.end(s_max) - 1;
  if (cw) band_hi = imin64(band_hi, pq_max);
  const int64_t INF = int64_t(1) << 62;
  int64_t full_lo = INF, full_hi = -INF;
  if (s_min == s_max) {
    full_lo = seq.start(s_min);
    if (W > 0) full_lo = imax64(full_lo, pq_max - W + 1);
    full_hi = seq.end(s_min) - 1;
    if (cw) full_hi = imin64(full_hi, pq_min);
  }
  const bool sinks = W > 0 && ms.n_sink > 0;
  int32_t klo[2], khi[2];
  const int nk = monotone_segments(kmap, klo, khi);
  for (int ks = 0; ks < nk; ++ks) {
    int32_t f0 = 0, f1 = 0;
    if (full_lo <= full_hi) {
      f0 = bsearch_at_least(kmap, klo[ks], khi[ks], full_lo);
      f1 = bsearch_above(kmap, klo[ks], khi[ks], full_hi);
    }
    RunMerger<Emit> mg(emit, f0, f1, gran);
    auto add_pos = [&](int64_t lo, int64_t hi) {
      mg.add(bsearch_at_least(kmap, klo[ks], khi[ks], lo), bsearch_above(kmap, klo[ks], khi[ks], hi));
    };
    bool band_pending = band_lo <= band_hi;
    if (sinks) {
      for (int32_t s = s_min; s <= s_max; ++s) {
        const int64_t lo = seq.start(s);
        const int64_t hi = imin64(imin64(lo + ms.n_sink - 1, seq.end(s) - 1), pq_max);
        if (lo > hi) continue;
        if (band_pending && band_lo <= lo) {
          add_pos(band_lo, band_hi);
          band_pending = false;
        }
        add_pos(lo, hi);
      }
    }
    if (band_pending) add_pos(band_lo, band_hi);
    mg.flush();
  }
}

// The transposed plan: runs of query rows of qmap's rank that see some key
// of keys [u0, u0 + keys) of kmap's rank (one monotone piece); a run is full
// when every key of the tile is visible to every row of it.  For keys with
// positions in [pk_min, pk_max] a query sees some key only inside
//   * the band [max(seq_start, pk_min), min(seq_end - 1, pk_max + W - 1)]
//     (causal / window / same-sequence constraints), and
//   * for a sequence whose first n_sink positions meet the tile,
//     [max(seq_start, pk_min), seq_end - 1] (sink keys are seen by every
//     later query of their sequence);
// and sees every key of the tile when its position lies in
//   [max(seq_start, pk_max), min(seq_end - 1, pk_min + W - 1)]
// with all keys in one sequence.
template <class Emit>
__host__ __device__ void plan_key_tile(const PosMap& qmap, const PosMap& kmap, const MaskSpec& ms, const SeqView& seq,
                                       int32_t u0, int32_t keys, int32_t gran, Emit& emit) {
  const bool cw = ms.causal || ms.window > 0;
  const int64_t W = ms.window;
  const int64_t pk_min = position(kmap, u0);
  const int64_t pk_max = position(kmap, u0 + keys - 1);
  const int32_t s_min = seq.index(pk_min);
  const int32_t s_max = seq.index(pk_max);
  int64_t band_lo = seq.start(s_min);
  if (cw) band_lo = imax64(band_lo, pk_min);
  int64_t band_hi = seq.end(s_max) - 1;
  if (W > 0) band_hi = imin64(band_hi, pk_max + W - 1);
  const int64_t INF = int64_t(1) << 62;
  int64_t full_lo = INF, full_hi = -INF;
  if (s_min == s_max) {
    full_lo = seq.start(s_min);
    if (cw) full_lo = imax64(full_lo, pk_max);
    full_hi = seq.end(s_min) - 1;
    if (W > 0) full_hi = imin64(full_hi, pk_min + W - 1);
  }
  const bool sinks = W > 0 && ms.n_sink > 0;
  int32_t qlo[2], qhi[2];
  const int nq = monotone_segments(qmap, qlo, qhi);
  for (int qs = 0; qs < nq; ++qs) {
    int32_t f0 = 0, f1 = 0;
    if (full_lo <= full_hi) {
      f0 = bsearch_at_least(qmap, qlo[qs], qhi[qs], full_lo);
      f1 = bsearch_above(qmap, qlo[qs], qhi[qs], full_hi);
    }
    RunMerger<Emit> mg(emit, f0, f1, gran);
    auto add_pos = [&](int64_t lo, int64_t hi) {
      mg.add(bsearch_at_least(qmap, qlo[qs], qhi[qs], lo), bsearch_above(qmap, qlo[qs], qhi[qs], hi));
    };
    bool band_pending = band_lo <= band_hi;
    if (sinks) {
      for (int32_t s = s_min; s <= s_max; ++s) {
        const int64_t lo = imax64(seq.start(s), pk_min);
        const int64_t sink_end = imin64(seq.start(s) + ms.n_sink - 1, seq.end(s) - 1);
        if (lo > imin64(sink_end, pk_max) || lo > seq.end(s) - 1) continue;
        if (band_pending && band_lo <= lo) {
          add_pos(band_lo, band_hi);
          band_pending = false;
        }
        add_pos(lo, seq.end(s) - 1);
      }
    }
    if (band_pending) add_pos(band_lo, band_hi);
    mg.flush();
  }
}

// One planned family of launches: n_steps plans, plan s covering n_ranks
// blocks (query rank i = rank_lo + ii against KV rank (i - s) mod N in ring
// mode; the one block of qmap / kmap otherwise), each block cut into cpb
// candidate items.  Candidate g = s * cpp + ii * cpb + c (cpp = n_ranks *
// cpb) owns run slots [g * cap, (g + 1) * cap).
struct PlanJob {
  PosMap qmap, kmap;       // rank fields overridden per block in ring mode
  MaskSpec mask;
  const int32_t* cu;       // cu_seqlens (device for the kernels, host for the host planner), or nullptr
  int32_t kind;            // 0: query tiles (forward, dQ); 1: key tiles (dK / dV)
  int32_t tile;            // rows (kind 0) or keys (kind 1) per item
  int32_t gran;            // granularity of full runs
  int32_t acc_from_step;   // items without runs are dropped at steps >= this
  int32_t empty;           // explicit EMPTY class: no keys at all
  int32_t ring;            // 1: ring blocks; 0: one block
  int32_t N, rank_lo, n_ranks, n_steps, one_rank;
  int32_t L;               // rows per rank (row bases of the ring buffers)
  int32_t cpb, cap;        // candidates per block, run slots per candidate
  // device buffers (inside the caller's workspace)
  WorkItem* items;         // n_steps * cpp, sorted per plan
  Run* runs;               // n_steps * cpp * cap
  WorkItem* tmp;           // n_steps * cpp, candidate order
  int64_t* cost;           // n_steps * cpp
  __host__ __device__ int64_t cpp() const { return (int64_t)n_ranks * cpb; }
  __host__ __device__ int64_t candidates() const { return (int64_t)n_steps * cpp(); }
};

// Plans above this many candidates keep candidate order: their launches
// have many more workgroups than the GPU runs at once, so the longest-first
// order no longer shortens the tail noticeably.
constexpr int64_t kMaxSortItems = 16384;

// Block of candidate g: ranks, row bases of the q / k buffers.
__host__ __device__ inline void job_block(const PlanJob& J, int64_t g, int32_t* step, int32_t* cand, PosMap* qm,
                                          PosMap* km, int32_t* qbase, int32_t* kbase) {
  const int64_t cpp = J.cpp();
  const int32_t s = (int32_t)(g / cpp);
  const int64_t r = g - (int64_t)s * cpp;
  const int32_t ii = (int32_t)(r / J.cpb);
  *cand = (int32_t)(r - (int64_t)ii * J.cpb);
  *step = s;
  *qm = J.qmap;
  *km = J.kmap;
  *qbase = 0;
  *kbase = 0;
  if (J.ring) {
    const int32_t i = J.rank_lo + ii;
    const int32_t j = ((i - s) % J.N + J.N) % J.N;
    qm->rank = i;
    km->rank = j;
    *qbase = J.one_rank ? 0 : i * J.L;
    *kbase = j * J.L;
  }
}

// Plans candidate g of job J: writes its runs through `put(index, run)` for
// index < J.cap and returns the item (q_rows = 0 when it is dropped) and its
// cost ((1 + keys visited) * rows; -1 when dropped).  *emitted (optional)
// receives the number of runs found, which job_cap bounds by J.cap.
template <class Put>
__host__ __device__ WorkItem plan_candidate(const PlanJob& J, const SeqView& seq, int64_t g, Put&& put, int64_t* cost,
                                            int32_t* emitted = nullptr) {
  int32_t s, c, qbase, kbase;
  PosMap qm, km;
  job_block(J, g, &s, &c, &qm, &km, &qbase, &kbase);
  int32_t t0 = 0, rows = 0;
  tile_rows(J.kind == 0 ? qm : km, J.tile, c, &t0, &rows);
  int32_t n = 0;
  int64_t visited = 0;
  auto emit = [&](int32_t a, int32_t b, int32_t full) {
    if (n < J.cap) put(n, Run{a, b, full, 0});
    ++n;
    visited += b - a;
  };
  if (!J.empty) {
    if (J.kind == 0)
      plan_query_tile(qm, km, J.mask, seq, t0, rows, J.gran, emit);
    else
      plan_key_tile(qm, km, J.mask, seq, t0, rows, J.gran, emit);
  }
  if (emitted) *emitted = n;
  const int32_t rb = (int32_t)(g * J.cap);
  WorkItem it;
  if (J.kind == 0)
    it = WorkItem{qbase + t0, t0, rows, qm.rank, kbase, km.rank, rb, rb + imin32(n, J.cap)};
  else
    it = WorkItem{kbase + t0, t0, rows, km.rank, qbase, qm.rank, rb, rb + imin32(n, J.cap)};
  const bool drop = n == 0 && s >= J.acc_from_step;
  if (drop) {
    it.q_rows = 0;
    it.run_end = it.run_begin;
    *cost = -1;
  } else {
    *cost = (1 + visited) * rows;
  }
  return it;
}

// Up to two jobs planned by one pair of planner launches (the backward plans
// its dQ and dK / dV tiles together).
struct PlanJobs {
  PlanJob j[2];
  int32_t n;
};

// Run slots per candidate that bound every item of job J (host; cu_host as
// the job's cu_seqlens on the host).
int32_t job_cap(const PlanJob& J, const int32_t* cu_host);
// Whether some key of kmap's rank is visible to some query of qmap's rank
// (conservative: false only when no pair is visible).
bool block_has_work(const PosMap& qmap, const PosMap& kmap, const MaskSpec& ms, const int32_t* cu_host);
// Whether any block of plan `step` of J may have a visible pair.
bool step_has_work(const PlanJob& J, int32_t step, const int32_t* cu_host);
// Host-built plan `step` of J, in the device planner's order, dropped items
// left out and runs compacted.
// Returns false (and builds nothing more) if an item needed more than J.cap
// run slots, which job_cap rules out.
bool plan_job_host(const PlanJob& J, const int32_t* cu_host, int32_t step, Plan& plan);
// Enqueues the device planner for jobs.j[0 .. n): items, runs and costs of
// every candidate, then the per-plan ordering.
usp_status launch_plan(const PlanJobs& jobs, hipStream_t stream);

}  // namespace usp
