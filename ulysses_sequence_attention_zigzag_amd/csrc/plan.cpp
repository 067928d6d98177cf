// Host side of the tile planner: sizing of the device plans (run slots per
// item), the coarse test that lets a ring skip steps with no visible pair,
// and the host-built plans returned by the inspection calls.  The per-item
// logic is plan_core.h, shared with the device planner kernels, so the
// inspection calls show exactly what the kernels run.

#include <algorithm>
#include <cstdint>
#include <vector>

#include "plan_core.h"

namespace usp {

namespace {

SeqView host_seq(const PlanJob& J, const int32_t* cu_host) {
  return SeqView{J.mask.nseq > 0 ? cu_host : nullptr, J.mask.nseq, J.mask.S};
}

// Largest number of sequences that one tile of `tile` rows of map m touches.
int32_t max_seqs_per_tile(const PosMap& m, int32_t tile, const SeqView& seq) {
  int32_t lo[2], hi[2];
  const int n = monotone_segments(m, lo, hi);
  int32_t best = 0;
  for (int s = 0; s < n; ++s)
    for (int32_t t0 = lo[s]; t0 < hi[s]; t0 += tile) {
      const int32_t t1 = std::min(hi[s], t0 + tile) - 1;
      best = std::max(best, seq.index(position(m, t1)) - seq.index(position(m, t0)) + 1);
    }
  return best;
}

}  // namespace

int32_t job_cap(const PlanJob& J, const int32_t* cu_host) {
  // runs of one item: per monotone piece of the other side's rows, each
  // merged interval gives at most 3 runs (partial, full, partial), and the
  // merged intervals are at most the band plus one sink interval per
  // sequence the tile touches
  int32_t lo[2], hi[2];
  const int nseg = monotone_segments(J.kind == 0 ? J.kmap : J.qmap, lo, hi);
  int32_t T = 0;
  if (J.mask.window > 0 && J.mask.n_sink > 0) {
    T = 1;
    if (J.mask.nseq > 1 && cu_host) {
      const SeqView seq = host_seq(J, cu_host);
      PosMap m = J.kind == 0 ? J.qmap : J.kmap;
      if (J.ring) {
        const int r0 = J.kind == 0 ? J.rank_lo : 0;
        const int r1 = J.kind == 0 ? J.rank_lo + J.n_ranks : J.N;
        for (int r = r0; r < r1; ++r) {
          m.rank = r;
          T = std::max(T, max_seqs_per_tile(m, J.tile, seq));
        }
      } else {
        T = std::max(T, max_seqs_per_tile(m, J.tile, seq));
      }
    }
  }
  return nseg * 3 * (1 + T);
}

bool block_has_work(const PosMap& qmap, const PosMap& kmap, const MaskSpec& ms, const int32_t* cu_host) {
  // the hull of a whole monotone piece contains the hulls of its tiles, so
  // no run here means no visible pair in any tile of the block
  const SeqView seq{ms.nseq > 0 ? cu_host : nullptr, ms.nseq, ms.S};
  int32_t lo[2], hi[2];
  const int n = monotone_segments(qmap, lo, hi);
  for (int s = 0; s < n; ++s) {
    if (hi[s] <= lo[s]) continue;
    int32_t runs = 0;
    auto emit = [&](int32_t, int32_t, int32_t) { ++runs; };
    plan_query_tile(qmap, kmap, ms, seq, lo[s], hi[s] - lo[s], kTileN, emit);
    if (runs > 0) return true;
  }
  return false;
}

bool step_has_work(const PlanJob& J, int32_t step, const int32_t* cu_host) {
  if (J.empty) return false;
  for (int32_t ii = 0; ii < J.n_ranks; ++ii) {
    int32_t s, c, qb, kb;
    PosMap qm, km;
    job_block(J, (int64_t)step * J.cpp() + (int64_t)ii * J.cpb, &s, &c, &qm, &km, &qb, &kb);
    if (block_has_work(qm, km, J.mask, cu_host)) return true;
  }
  return false;
}

bool plan_job_host(const PlanJob& J, const int32_t* cu_host, int32_t step, Plan& plan) {
  const SeqView seq = host_seq(J, cu_host);
  const int64_t cpp = J.cpp();
  std::vector<int64_t> cost;
  std::vector<Run> slot(J.cap);
  for (int64_t c = 0; c < cpp; ++c) {
    const int64_t g = (int64_t)step * cpp + c;
    int64_t k = 0;
    int32_t found = 0;
    WorkItem it = plan_candidate(J, seq, g, [&](int32_t i, const Run& r) { slot[i] = r; }, &k, &found);
    if (found > J.cap) return false;
    if (it.q_rows == 0) continue;
    const int32_t n = it.run_end - it.run_begin;
    it.run_begin = (int32_t)plan.runs.size();
    it.run_end = it.run_begin + n;
    plan.runs.insert(plan.runs.end(), slot.begin(), slot.begin() + n);
    plan.items.push_back(it);
    cost.push_back(k);
  }
  if (cpp > kMaxSortItems) return true;
  // longest first, ties in candidate order (the device planner's rank rule)
  std::vector<size_t> order(plan.items.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return cost[x] > cost[y]; });
  std::vector<WorkItem> sorted;
  sorted.reserve(order.size());
  for (size_t i : order) sorted.push_back(plan.items[i]);
  plan.items.swap(sorted);
  return true;
}

}  // namespace usp
