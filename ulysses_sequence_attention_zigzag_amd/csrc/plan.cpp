// Tile planner: which key rows each block of query rows must visit, and
// which of those key tiles need no per-element mask.
//
// For a tile of BM query rows inside one monotone piece of a rank's rows
// (positions increase with the row index), the visible keys are contained in
//   * the band  [max(seq_start, pq_min - W + 1), min(seq_end - 1, pq_max)]
//     (window / causal / same-sequence constraints, hull over the rows), and
//   * for each sequence the rows touch, its first n_sink positions
//     (attention sinks; only with a window),
// and a key is visible to every row of the tile when its position lies in
//   [max(seq_start, pq_max - W + 1), min(seq_end - 1, pq_min)]
// with all rows in one sequence.  Position intervals become local key
// intervals by binary search over each monotone piece of the KV rank's rows.
// The kernel evaluates the exact predicate inside partial runs, so these
// hulls only need to be conservative.

#include <algorithm>
#include <cstdint>
#include <vector>

#include "usp_internal.h"

namespace usp {
namespace {

struct SeqInfo {
  const int32_t* cu;  // nullptr: one sequence [0, S)
  int32_t nseq;
  int32_t S;
  int32_t index(int64_t p) const {
    if (!cu) return 0;
    int32_t lo = 0, hi = nseq - 1;  // largest i with cu[i] <= p
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) / 2;
      if (cu[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  int64_t start(int32_t i) const { return cu ? cu[i] : 0; }
  int64_t end(int32_t i) const { return cu ? cu[i + 1] : S; }
};

// First u in [lo, hi) with position(u) >= P (hi if none); positions increase on [lo, hi).
int32_t first_at_least(const PosMap& m, int32_t lo, int32_t hi, int64_t P) {
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo) / 2;
    if (position(m, mid) >= P) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// First u in [lo, hi) with position(u) > P (hi if none).
int32_t first_above(const PosMap& m, int32_t lo, int32_t hi, int64_t P) {
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo) / 2;
    if (position(m, mid) > P) hi = mid; else lo = mid + 1;
  }
  return lo;
}

}  // namespace

void plan_block(const BlockSpec& blk, const MaskSpec& ms, const int32_t* cu_host, int accumulate,
                Plan& plan) {
  const SeqInfo seq{ms.nseq > 0 ? cu_host : nullptr, ms.nseq, ms.S};
  const bool cw = ms.causal || ms.window > 0;
  const int64_t W = ms.window;
  const int64_t INF = int64_t(1) << 62;

  int32_t qlo[2], qhi[2], klo[2], khi[2];
  const int nq = monotone_segments(blk.qmap, qlo, qhi);
  const int nk = monotone_segments(blk.kmap, klo, khi);

  std::vector<std::pair<int64_t, int64_t>> pos_iv;
  std::vector<std::pair<int32_t, int32_t>> loc_iv;

  for (int qs = 0; qs < nq; ++qs) {
    for (int32_t t0 = qlo[qs]; t0 < qhi[qs]; t0 += blk.tile_m) {
      const int32_t rows = std::min<int32_t>(blk.tile_m, qhi[qs] - t0);
      const int64_t pq_min = position(blk.qmap, t0);
      const int64_t pq_max = position(blk.qmap, t0 + rows - 1);
      const int32_t s_min = seq.index(pq_min);
      const int32_t s_max = seq.index(pq_max);

      pos_iv.clear();
      int64_t band_lo = seq.start(s_min);
      if (W > 0) band_lo = std::max(band_lo, pq_min - W + 1);
      int64_t band_hi = seq.end(s_max) - 1;
      if (cw) band_hi = std::min(band_hi, pq_max);
      if (band_lo <= band_hi) pos_iv.push_back({band_lo, band_hi});
      if (W > 0 && ms.n_sink > 0) {
        for (int32_t s = s_min; s <= s_max; ++s) {
          const int64_t lo = seq.start(s);
          const int64_t hi = std::min({lo + ms.n_sink - 1, seq.end(s) - 1, pq_max});
          if (lo <= hi) pos_iv.push_back({lo, hi});
        }
      }
      int64_t full_lo = INF, full_hi = -INF;
      if (s_min == s_max) {
        full_lo = seq.start(s_min);
        if (W > 0) full_lo = std::max(full_lo, pq_max - W + 1);
        full_hi = seq.end(s_min) - 1;
        if (cw) full_hi = std::min(full_hi, pq_min);
      }

      const int32_t run_begin = static_cast<int32_t>(plan.runs.size());
      for (int ks = 0; ks < nk; ++ks) {
        loc_iv.clear();
        for (const auto& iv : pos_iv) {
          const int32_t u0 = first_at_least(blk.kmap, klo[ks], khi[ks], iv.first);
          const int32_t u1 = first_above(blk.kmap, klo[ks], khi[ks], iv.second);
          if (u0 < u1) loc_iv.push_back({u0, u1});
        }
        if (loc_iv.empty()) continue;
        std::sort(loc_iv.begin(), loc_iv.end());
        // merge overlapping / touching intervals so no key is visited twice
        std::vector<std::pair<int32_t, int32_t>> merged;
        for (const auto& iv : loc_iv) {
          if (!merged.empty() && iv.first <= merged.back().second)
            merged.back().second = std::max(merged.back().second, iv.second);
          else
            merged.push_back(iv);
        }
        int32_t f0 = 0, f1 = 0;
        if (full_lo <= full_hi) {
          f0 = first_at_least(blk.kmap, klo[ks], khi[ks], full_lo);
          f1 = first_above(blk.kmap, klo[ks], khi[ks], full_hi);
        }
        for (const auto& iv : merged) {
          const int32_t a = iv.first, b = iv.second;
          const int32_t x0 = std::max(a, f0), x1 = std::min(b, f1);
          if (x1 - x0 >= kTileN) {
            const int32_t nfull = (x1 - x0) / kTileN * kTileN;
            if (a < x0) plan.runs.push_back({a, x0, 0, 0});
            plan.runs.push_back({x0, x0 + nfull, 1, 0});
            if (x0 + nfull < b) plan.runs.push_back({x0 + nfull, b, 0, 0});
          } else {
            plan.runs.push_back({a, b, 0, 0});
          }
        }
      }
      const int32_t run_end = static_cast<int32_t>(plan.runs.size());
      if (run_end == run_begin && accumulate) continue;  // nothing to merge
      plan.items.push_back({blk.q_row_base + t0, t0, rows, blk.qmap.rank, blk.k_row_base,
                            blk.kmap.rank, run_begin, run_end});
    }
  }
}

void plan_block_kv(const BlockSpec& blk, const MaskSpec& ms, const int32_t* cu_host, int32_t tile_k,
                   int32_t q_gran, Plan& plan) {
  // The same hulls with the roles swapped: for a tile of keys with positions
  // in [pk_min, pk_max] (one monotone piece), a query sees some key of the
  // tile only inside
  //   * the band [max(seq_start, pk_min), min(seq_end - 1, pk_max + W - 1)]
  //     (causal / window / same-sequence constraints), and
  //   * for a sequence whose first n_sink positions meet the tile,
  //     [max(seq_start, pk_min), seq_end - 1] (sink keys are seen by every
  //     later query of their sequence);
  // and sees every key of the tile when its position lies in
  //   [max(seq_start, pk_max), min(seq_end - 1, pk_min + W - 1)]
  // with all keys in one sequence.
  const SeqInfo seq{ms.nseq > 0 ? cu_host : nullptr, ms.nseq, ms.S};
  const bool cw = ms.causal || ms.window > 0;
  const int64_t W = ms.window;
  const int64_t INF = int64_t(1) << 62;

  int32_t qlo[2], qhi[2], klo[2], khi[2];
  const int nq = monotone_segments(blk.qmap, qlo, qhi);
  const int nk = monotone_segments(blk.kmap, klo, khi);

  std::vector<std::pair<int64_t, int64_t>> pos_iv;
  std::vector<std::pair<int32_t, int32_t>> loc_iv;

  for (int ks = 0; ks < nk; ++ks) {
    for (int32_t u0 = klo[ks]; u0 < khi[ks]; u0 += tile_k) {
      const int32_t keys = std::min<int32_t>(tile_k, khi[ks] - u0);
      const int64_t pk_min = position(blk.kmap, u0);
      const int64_t pk_max = position(blk.kmap, u0 + keys - 1);
      const int32_t s_min = seq.index(pk_min);
      const int32_t s_max = seq.index(pk_max);

      pos_iv.clear();
      int64_t band_lo = seq.start(s_min);
      if (cw) band_lo = std::max(band_lo, pk_min);
      int64_t band_hi = seq.end(s_max) - 1;
      if (W > 0) band_hi = std::min(band_hi, pk_max + W - 1);
      if (band_lo <= band_hi) pos_iv.push_back({band_lo, band_hi});
      if (W > 0 && ms.n_sink > 0) {
        for (int32_t s = s_min; s <= s_max; ++s) {
          const int64_t lo = std::max(seq.start(s), pk_min);
          const int64_t sink_end = std::min(seq.start(s) + ms.n_sink - 1, seq.end(s) - 1);
          if (lo <= std::min(sink_end, pk_max) && lo <= seq.end(s) - 1) pos_iv.push_back({lo, seq.end(s) - 1});
        }
      }
      int64_t full_lo = INF, full_hi = -INF;
      if (s_min == s_max) {
        full_lo = seq.start(s_min);
        if (cw) full_lo = std::max(full_lo, pk_max);
        full_hi = seq.end(s_min) - 1;
        if (W > 0) full_hi = std::min(full_hi, pk_min + W - 1);
      }

      const int32_t run_begin = static_cast<int32_t>(plan.runs.size());
      for (int qs = 0; qs < nq; ++qs) {
        loc_iv.clear();
        for (const auto& iv : pos_iv) {
          const int32_t t0 = first_at_least(blk.qmap, qlo[qs], qhi[qs], iv.first);
          const int32_t t1 = first_above(blk.qmap, qlo[qs], qhi[qs], iv.second);
          if (t0 < t1) loc_iv.push_back({t0, t1});
        }
        if (loc_iv.empty()) continue;
        std::sort(loc_iv.begin(), loc_iv.end());
        std::vector<std::pair<int32_t, int32_t>> merged;
        for (const auto& iv : loc_iv) {
          if (!merged.empty() && iv.first <= merged.back().second)
            merged.back().second = std::max(merged.back().second, iv.second);
          else
            merged.push_back(iv);
        }
        int32_t f0 = 0, f1 = 0;
        if (full_lo <= full_hi) {
          f0 = first_at_least(blk.qmap, qlo[qs], qhi[qs], full_lo);
          f1 = first_above(blk.qmap, qlo[qs], qhi[qs], full_hi);
        }
        for (const auto& iv : merged) {
          const int32_t a = iv.first, b = iv.second;
          const int32_t x0 = std::max(a, f0), x1 = std::min(b, f1);
          if (x1 - x0 >= q_gran) {
            const int32_t nfull = (x1 - x0) / q_gran * q_gran;
            if (a < x0) plan.runs.push_back({a, x0, 0, 0});
            plan.runs.push_back({x0, x0 + nfull, 1, 0});
            if (x0 + nfull < b) plan.runs.push_back({x0 + nfull, b, 0, 0});
          } else {
            plan.runs.push_back({a, b, 0, 0});
          }
        }
      }
      const int32_t run_end = static_cast<int32_t>(plan.runs.size());
      if (run_end == run_begin) continue;  // no query sees these keys: nothing to add
      plan.items.push_back({blk.k_row_base + u0, u0, keys, blk.kmap.rank, blk.q_row_base,
                            blk.qmap.rank, run_begin, run_end});
    }
  }
}

void finalize_plan(Plan& plan) {
  std::vector<int64_t> cost(plan.items.size());
  for (size_t i = 0; i < plan.items.size(); ++i) {
    int64_t c = 1;
    for (int32_t r = plan.items[i].run_begin; r < plan.items[i].run_end; ++r)
      c += plan.runs[r].k_end - plan.runs[r].k_begin;
    cost[i] = c * plan.items[i].q_rows;
  }
  std::vector<size_t> order(plan.items.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return cost[x] > cost[y]; });
  std::vector<WorkItem> sorted;
  sorted.reserve(order.size());
  for (size_t i : order) sorted.push_back(plan.items[i]);
  plan.items.swap(sorted);
}

}  // namespace usp
