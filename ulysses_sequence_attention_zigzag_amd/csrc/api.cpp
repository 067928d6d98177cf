// C ABI of libusp: argument validation, workspace layout and the virtual
// ring driver.  Every entry point validates everything on the host before
// enqueueing anything; the tile plans are built on the device into the
// caller's workspace, so no call allocates, copies from the host or waits for
// the device.  See include/usp.h for the contract of each call.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "plan_core.h"

namespace usp {

namespace {
thread_local std::string g_err;
}

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
}

namespace {

#define USP_CHECK(cond, code, ...) \
  do {                             \
    if (!(cond)) {                 \
      set_error(__VA_ARGS__);      \
      return (code);               \
    }                              \
  } while (0)

constexpr int64_t kMaxI32 = 0x7fffffff;

// ------------------------------------------------------------ validation
usp_status check_layout(int impl, int64_t S, int N, int b) {
  USP_CHECK(impl >= USP_RING_BASIC && impl <= USP_RING_STRIPE, USP_ERR_INVALID_ARG,
            "impl must be 0 (basic), 1 (zigzag) or 2 (stripe), got %d", impl);
  USP_CHECK(N >= 1, USP_ERR_INVALID_ARG, "ring_degree must be >= 1, got %d", N);
  USP_CHECK(S >= 1 && S <= (int64_t)1 << 30, USP_ERR_INVALID_ARG,
            "sequence length %lld out of range [1, 2^30]", (long long)S);
  if (impl == USP_RING_BASIC)
    USP_CHECK(S % N == 0, USP_ERR_INVALID_ARG, "basic layout needs S %% N == 0 (S=%lld, N=%d)", (long long)S, N);
  if (impl == USP_RING_ZIGZAG)
    USP_CHECK(S % (2 * N) == 0, USP_ERR_INVALID_ARG, "zigzag layout needs S %% 2N == 0 (S=%lld, N=%d)", (long long)S, N);
  if (impl == USP_RING_STRIPE) {
    USP_CHECK(b >= 1, USP_ERR_INVALID_ARG, "stripe_block must be >= 1, got %d", b);
    USP_CHECK(S % ((int64_t)N * b) == 0, USP_ERR_INVALID_ARG,
              "stripe layout needs S %% (N*b) == 0 (S=%lld, N=%d, b=%d)", (long long)S, N, b);
  }
  return USP_OK;
}

usp_status check_cu(const int32_t* cu_host, int nseq, int64_t total) {
  USP_CHECK(nseq >= 1, USP_ERR_INVALID_ARG, "nseq must be >= 1 with cu_seqlens");
  USP_CHECK(cu_host[0] == 0, USP_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int i = 0; i < nseq; ++i)
    USP_CHECK(cu_host[i + 1] >= cu_host[i], USP_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
  USP_CHECK(cu_host[nseq] == total, USP_ERR_INVALID_ARG,
            "cu_seqlens[nseq] (%d) must equal the total length (%lld)", cu_host[nseq], (long long)total);
  return USP_OK;
}

PosMap make_map(const usp_posmap& m) {
  PosMap p;
  p.kind = m.impl;
  p.N = m.ring_degree;
  p.rank = m.rank;
  p.b = m.impl == USP_RING_STRIPE ? m.stripe_block : 1;
  p.L = (int32_t)(m.S_global / m.ring_degree);
  p.offset = 0;
  return p;
}

PosMap affine_map(int32_t L, int32_t offset) {
  PosMap p;
  p.kind = MAP_AFFINE;
  p.N = 1;
  p.rank = 0;
  p.b = 1;
  p.L = L;
  p.offset = offset;
  return p;
}

struct BlockMaskSetup {
  PosMap qmap, kmap;
  MaskSpec ms;
  bool empty = false;
};

usp_status setup_block_mask(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                            const usp_posmap* kmap, int causal, int window, int n_sink,
                            const int32_t* cu_host, int nseq, int64_t B, BlockMaskSetup* out) {
  BlockMaskSetup s;
  s.ms.causal = causal ? 1 : 0;
  s.ms.window = window;
  s.ms.n_sink = n_sink;
  s.ms.nseq = 0;
  USP_CHECK(window >= 0, USP_ERR_INVALID_ARG, "window must be >= 0, got %d", window);
  USP_CHECK(n_sink >= 0, USP_ERR_INVALID_ARG, "n_sink must be >= 0, got %d", n_sink);
  switch (mask) {
    case USP_MASK_EMPTY:
    case USP_MASK_FULL:
    case USP_MASK_CAUSAL:
    case USP_MASK_CAUSAL_STRICT:
      USP_CHECK(!causal && window == 0 && n_sink == 0 && !cu_host, USP_ERR_INVALID_ARG,
                "explicit mask classes take no causal/window/n_sink/cu_seqlens");
      s.qmap = affine_map((int32_t)Lq, 0);
      s.kmap = affine_map((int32_t)Lk, mask == USP_MASK_CAUSAL_STRICT ? 1 : 0);
      s.ms.causal = (mask == USP_MASK_CAUSAL || mask == USP_MASK_CAUSAL_STRICT) ? 1 : 0;
      s.ms.S = (int32_t)(std::max(Lq, Lk) + 1);
      s.empty = mask == USP_MASK_EMPTY;
      break;
    case USP_MASK_POSITIONAL: {
      USP_CHECK(qmap && kmap, USP_ERR_INVALID_ARG, "POSITIONAL mask needs qmap and kmap");
      usp_status st = check_layout(qmap->impl, qmap->S_global, qmap->ring_degree, qmap->stripe_block);
      if (st != USP_OK) return st;
      USP_CHECK(qmap->impl == kmap->impl && qmap->ring_degree == kmap->ring_degree &&
                    qmap->S_global == kmap->S_global &&
                    (qmap->impl != USP_RING_STRIPE || qmap->stripe_block == kmap->stripe_block),
                USP_ERR_INVALID_ARG, "qmap and kmap must describe the same layout");
      USP_CHECK(qmap->rank >= 0 && qmap->rank < qmap->ring_degree && kmap->rank >= 0 &&
                    kmap->rank < kmap->ring_degree,
                USP_ERR_INVALID_ARG, "posmap rank out of range");
      const int64_t L = qmap->S_global / qmap->ring_degree;
      USP_CHECK(Lq == L && Lk == L, USP_ERR_INVALID_ARG,
                "POSITIONAL mask needs Lq == Lk == S/N (%lld), got %lld, %lld", (long long)L,
                (long long)Lq, (long long)Lk);
      s.qmap = make_map(*qmap);
      s.kmap = make_map(*kmap);
      s.ms.S = (int32_t)qmap->S_global;
      if (cu_host) {
        USP_CHECK(B == 1, USP_ERR_INVALID_ARG, "varlen (cu_seqlens) needs B == 1");
        st = check_cu(cu_host, nseq, qmap->S_global);
        if (st != USP_OK) return st;
        s.ms.nseq = nseq;
      }
      break;
    }
    default:
      USP_CHECK(false, USP_ERR_INVALID_ARG, "unknown mask class %d", (int)mask);
  }
  *out = s;
  return USP_OK;
}

// ------------------------------------------------------------ tile plans
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Offsets (bytes, within a workspace) of one job's device buffers.
struct JobSlots {
  size_t items = 0, runs = 0, tmp = 0, cost = 0;
};

// Reserves J's buffers at `off` (advanced past them).
JobSlots reserve_job(const PlanJob& J, size_t& off) {
  const size_t C = (size_t)J.candidates();
  JobSlots s;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  s.items = take(C * sizeof(WorkItem));
  s.runs = take(C * (size_t)J.cap * sizeof(Run));
  s.tmp = take(C * sizeof(WorkItem));
  s.cost = take(C * sizeof(int64_t));
  return s;
}

void bind_job(PlanJob& J, const JobSlots& s, char* ws, const int32_t* cu_dev) {
  J.items = reinterpret_cast<WorkItem*>(ws + s.items);
  J.runs = reinterpret_cast<Run*>(ws + s.runs);
  J.tmp = reinterpret_cast<WorkItem*>(ws + s.tmp);
  J.cost = reinterpret_cast<int64_t*>(ws + s.cost);
  J.cu = J.mask.nseq > 0 ? cu_dev : nullptr;
}

// Sets J.cap (run slots per item) and checks that run indices fit in int32.
usp_status finish_job(PlanJob& J, const int32_t* cu_host) {
  J.cap = job_cap(J, cu_host);
  USP_CHECK(J.candidates() * J.cap <= kMaxI32, USP_ERR_UNSUPPORTED,
            "tile plan too large (%lld items x %d run slots)", (long long)J.candidates(), J.cap);
  return USP_OK;
}

// The job of one block call: query tiles (kind 0, forward and dQ) or key
// tiles (kind 1, dK / dV) of the one block.
PlanJob block_job(const BlockMaskSetup& su, int kind, int32_t tile, int32_t gran, int32_t acc_from_step) {
  PlanJob J{};
  J.qmap = su.qmap;
  J.kmap = su.kmap;
  J.mask = su.ms;
  J.kind = kind;
  J.tile = tile;
  J.gran = gran;
  J.acc_from_step = acc_from_step;
  J.empty = su.empty ? 1 : 0;
  J.ring = 0;
  J.N = 1;
  J.rank_lo = 0;
  J.n_ranks = 1;
  J.n_steps = 1;
  J.one_rank = 1;
  J.L = 0;
  J.cpb = tile_count(kind == 0 ? su.qmap : su.kmap, tile);
  return J;
}

// The two jobs of a backward block: dQ (query tiles) and dK / dV (key tiles).
void bwd_block_jobs(const BlockMaskSetup& su, PlanJob* jq, PlanJob* jk) {
  *jq = block_job(su, 0, kBwdTileM, kTileN, 0);
  *jk = block_job(su, 1, kBwdTileK, kBwdTileQ, 0);
}

// Score modifiers in the kernels' raw-score units (ScoreMods).
usp_status make_mods(float softcap, const float* alibi, usp_mask_class mask, int64_t S, float scale,
                     ScoreMods* out) {
  USP_CHECK(std::isfinite(softcap) && softcap >= 0.f, USP_ERR_INVALID_ARG, "softcap must be finite and >= 0");
  USP_CHECK(!alibi || mask == USP_MASK_POSITIONAL, USP_ERR_INVALID_ARG,
            "ALiBi needs the POSITIONAL mask class (global positions)");
  USP_CHECK(!alibi || S <= kMaxAlibiPositions, USP_ERR_UNSUPPORTED,
            "ALiBi distances are computed in f32: at most %lld positions, got %lld",
            (long long)kMaxAlibiPositions, (long long)S);
  ScoreMods m{};
  if (softcap > 0.f) {
    m.a = softcap / scale;
    m.b2 = 2.f * scale * 1.4426950408889634f / softcap;
  }
  m.inv_scale = 1.f / scale;
  m.alibi = alibi;
  *out = m;
  return USP_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace
}  // namespace usp

using namespace usp;

extern "C" {

const char* usp_last_error(void) { return g_err.c_str(); }

const char* usp_version(void) { return "usp-gfx950 0.2"; }

usp_status usp_permute(const void* in, void* out, int64_t outer, int64_t S, int64_t inner,
                       usp_dtype dt, usp_ring_impl impl, int ring_degree, int ulysses_degree,
                       int stripe_block, int rank, int inverse, void* stream) {
  USP_CHECK(outer >= 0 && inner >= 1, USP_ERR_INVALID_ARG, "bad outer/inner sizes");
  USP_CHECK((in && out) || outer == 0, USP_ERR_INVALID_ARG, "null tensor pointer");
  USP_CHECK(dt == USP_DT_BF16 || dt == USP_DT_F32, USP_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  usp_status st = check_layout(impl, S, ring_degree, stripe_block);
  if (st != USP_OK) return st;
  USP_CHECK(ulysses_degree >= 1, USP_ERR_INVALID_ARG, "ulysses_degree must be >= 1");
  const int64_t L = S / ring_degree;
  USP_CHECK(L % ulysses_degree == 0, USP_ERR_INVALID_ARG,
            "rows per ring rank (%lld) not divisible by ulysses_degree %d", (long long)L, ulysses_degree);
  USP_CHECK(rank >= -1 && rank < ring_degree * ulysses_degree, USP_ERR_INVALID_ARG,
            "rank %d out of range [-1, %d)", rank, ring_degree * ulysses_degree);
  USP_CHECK(outer * S <= kMaxI32 * 4, USP_ERR_UNSUPPORTED, "tensor too large");
  const int64_t eb = dt == USP_DT_BF16 ? 2 : 4;
  const char* ib = static_cast<const char*>(in);
  const char* ob = static_cast<const char*>(out);
  const int64_t Sout = rank < 0 ? S : (inverse ? S : L / ulysses_degree);
  const int64_t Sin = rank < 0 ? S : (inverse ? L / ulysses_degree : S);
  const int64_t in_bytes = outer * Sin * inner * eb, out_bytes = outer * Sout * inner * eb;
  USP_CHECK(ib + in_bytes <= ob || ob + out_bytes <= ib, USP_ERR_INVALID_ARG,
            "permute is out-of-place: in and out overlap");
  GatherSpec gs;
  gs.impl = impl;
  gs.N = ring_degree;
  gs.ud = ulysses_degree;
  gs.b = impl == USP_RING_STRIPE ? stripe_block : 1;
  gs.g = rank < 0 ? 0 : rank;
  gs.L = (int32_t)L;
  gs.S = (int32_t)S;
  gs.kind = rank < 0 ? (inverse ? G_UNPERMUTE : G_PERMUTE) : (inverse ? G_INSERT : G_EXTRACT);
  return launch_permute(in, out, outer, Sin, Sout, inner * eb, gs, as_stream(stream));
}

usp_status usp_ulysses_relayout(void* const* shards, void* local, int64_t B, int64_t S_shard,
                                int64_t H, int64_t D, usp_dtype dt, int ulysses_degree,
                                int ulysses_rank, int direction, void* stream) {
  USP_CHECK(shards && local, USP_ERR_INVALID_ARG, "null pointer");
  USP_CHECK(ulysses_degree >= 1 && ulysses_degree <= 8, USP_ERR_UNSUPPORTED,
            "ulysses_degree must be in [1, 8], got %d", ulysses_degree);
  for (int i = 0; i < ulysses_degree; ++i) USP_CHECK(shards[i], USP_ERR_INVALID_ARG, "null shard pointer %d", i);
  USP_CHECK(B >= 0 && S_shard >= 0 && H >= 1 && D >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK(H % ulysses_degree == 0, USP_ERR_INVALID_ARG,
            "ulysses_degree %d must divide the head count %lld", ulysses_degree, (long long)H);
  USP_CHECK(ulysses_rank >= 0 && ulysses_rank < ulysses_degree, USP_ERR_INVALID_ARG, "ulysses_rank out of range");
  USP_CHECK(direction == 0 || direction == 1, USP_ERR_INVALID_ARG, "direction must be 0 or 1");
  USP_CHECK(dt == USP_DT_BF16 || dt == USP_DT_F32, USP_ERR_INVALID_ARG, "bad dtype");
  USP_CHECK(B * S_shard * ulysses_degree <= kMaxI32, USP_ERR_UNSUPPORTED, "tensor too large");
  const int64_t eb = dt == USP_DT_BF16 ? 2 : 4;
  return launch_relayout(shards, local, B, S_shard, H, D, eb, ulysses_degree, ulysses_rank, direction,
                         as_stream(stream));
}

usp_status usp_lse_merge(float* out_acc, float* lse_acc, const float* out_part, const float* lse_part,
                         int64_t B, int64_t L, int64_t H, int64_t D, int64_t row_begin,
                         int64_t row_end, void* stream) {
  USP_CHECK(B >= 0 && L >= 0 && H >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK((out_acc && lse_acc && out_part && lse_part) || B * L == 0, USP_ERR_INVALID_ARG, "null pointer");
  USP_CHECK(D >= 4 && D % 4 == 0 && 64 % (D / 4) == 0, USP_ERR_UNSUPPORTED,
            "merge supports D with D/4 dividing 64 (D = 4, 8, ..., 256; got %lld)", (long long)D);
  USP_CHECK(0 <= row_begin && row_begin <= row_end && row_end <= L, USP_ERR_INVALID_ARG,
            "row range [%lld, %lld) outside [0, %lld)", (long long)row_begin, (long long)row_end, (long long)L);
  USP_CHECK(B * L * H <= kMaxI32, USP_ERR_UNSUPPORTED, "tensor too large");
  return launch_lse_merge(out_acc, lse_acc, out_part, lse_part, B, L, H, D, row_begin, row_end,
                          as_stream(stream));
}

// ------------------------------------------------------------ plan inspection
usp_status usp_plan_block(int64_t Lq, int64_t Lk, int64_t D, usp_mask_class mask,
                          const usp_posmap* qmap, const usp_posmap* kmap, int causal, int window,
                          int n_sink, const int32_t* cu_seqlens_host, int nseq, int accumulate,
                          int32_t* items, int64_t items_cap, int32_t* runs, int64_t runs_cap,
                          int64_t* n_items, int64_t* n_runs, int32_t* tile_m, int32_t* tile_n) {
  USP_CHECK(n_items && n_runs, USP_ERR_INVALID_ARG, "null count pointer");
  USP_CHECK(Lq >= 0 && Lk >= 0 && Lq <= kMaxI32 / 2 && Lk <= kMaxI32 / 2, USP_ERR_INVALID_ARG, "bad Lq/Lk");
  USP_CHECK(D == 64 || D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)D);
  BlockMaskSetup su;
  usp_status st = setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host,
                                   nseq, 1, &su);
  if (st != USP_OK) return st;
  const int32_t tm = choose_tile_m(su.ms.window);
  Plan plan;
  if (Lq > 0) {
    PlanJob J = block_job(su, 0, tm, kTileN, accumulate ? 0 : INT_MAX);
    st = finish_job(J, cu_seqlens_host);
    if (st != USP_OK) return st;
    USP_CHECK(plan_job_host(J, cu_seqlens_host, 0, plan), USP_ERR_UNSUPPORTED,
              "internal: an item needs more than %d run slots", J.cap);
  }
  *n_items = (int64_t)plan.items.size();
  *n_runs = (int64_t)plan.runs.size();
  if (tile_m) *tile_m = tm;
  if (tile_n) *tile_n = kTileN;
  if (items) {
    USP_CHECK(items_cap >= *n_items, USP_ERR_INVALID_ARG, "items buffer too small");
    std::memcpy(items, plan.items.data(), plan.items.size() * sizeof(WorkItem));
  }
  if (runs) {
    USP_CHECK(runs_cap >= *n_runs, USP_ERR_INVALID_ARG, "runs buffer too small");
    std::memcpy(runs, plan.runs.data(), plan.runs.size() * sizeof(Run));
  }
  return USP_OK;
}

usp_status usp_plan_block_kv(int64_t Lq, int64_t Lk, int64_t D, usp_mask_class mask, const usp_posmap* qmap,
                             const usp_posmap* kmap, int causal, int window, int n_sink,
                             const int32_t* cu_seqlens_host, int nseq, int32_t* items, int64_t items_cap,
                             int32_t* runs, int64_t runs_cap, int64_t* n_items, int64_t* n_runs,
                             int32_t* tile_k, int32_t* tile_q) {
  USP_CHECK(n_items && n_runs, USP_ERR_INVALID_ARG, "null count pointer");
  USP_CHECK(Lq >= 0 && Lk >= 0 && Lq <= kMaxI32 / 2 && Lk <= kMaxI32 / 2, USP_ERR_INVALID_ARG, "bad Lq/Lk");
  USP_CHECK(D == 64 || D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)D);
  BlockMaskSetup su;
  usp_status st = setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host,
                                   nseq, 1, &su);
  if (st != USP_OK) return st;
  Plan plan;
  if (Lk > 0 && Lq > 0 && !su.empty) {
    PlanJob J = block_job(su, 1, kBwdTileK, kBwdTileQ, 0);
    st = finish_job(J, cu_seqlens_host);
    if (st != USP_OK) return st;
    USP_CHECK(plan_job_host(J, cu_seqlens_host, 0, plan), USP_ERR_UNSUPPORTED,
              "internal: an item needs more than %d run slots", J.cap);
  }
  *n_items = (int64_t)plan.items.size();
  *n_runs = (int64_t)plan.runs.size();
  if (tile_k) *tile_k = kBwdTileK;
  if (tile_q) *tile_q = kBwdTileQ;
  if (items) {
    USP_CHECK(items_cap >= *n_items, USP_ERR_INVALID_ARG, "items buffer too small");
    std::memcpy(items, plan.items.data(), plan.items.size() * sizeof(WorkItem));
  }
  if (runs) {
    USP_CHECK(runs_cap >= *n_runs, USP_ERR_INVALID_ARG, "runs buffer too small");
    std::memcpy(runs, plan.runs.data(), plan.runs.size() * sizeof(Run));
  }
  return USP_OK;
}

usp_status usp_plan_block_device(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                                 const usp_posmap* kmap, int causal, int window, int n_sink,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int nseq,
                                 int accumulate, int kv_tiles, void* workspace, size_t ws_bytes,
                                 int64_t* n_candidates, int32_t* run_slots, size_t* ws_needed, void* stream) {
  USP_CHECK(n_candidates && run_slots && ws_needed, USP_ERR_INVALID_ARG, "null count pointer");
  USP_CHECK(Lq >= 1 && Lk >= 0 && Lq <= kMaxI32 / 2 && Lk <= kMaxI32 / 2, USP_ERR_INVALID_ARG, "bad Lq/Lk");
  USP_CHECK(kv_tiles == 0 || kv_tiles == 1, USP_ERR_INVALID_ARG, "kv_tiles must be 0 or 1");
  USP_CHECK((cu_seqlens_host == nullptr) == (cu_seqlens_dev == nullptr), USP_ERR_INVALID_ARG,
            "cu_seqlens must be given on both host and device, or neither");
  BlockMaskSetup su;
  usp_status st = setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host,
                                   nseq, 1, &su);
  if (st != USP_OK) return st;
  PlanJob J = kv_tiles ? block_job(su, 1, kBwdTileK, kBwdTileQ, 0)
                       : block_job(su, 0, choose_tile_m(su.ms.window), kTileN, accumulate ? 0 : INT_MAX);
  st = finish_job(J, cu_seqlens_host);
  if (st != USP_OK) return st;
  size_t need = 0;
  const JobSlots js = reserve_job(J, need);
  *n_candidates = J.candidates();
  *run_slots = J.cap;
  *ws_needed = need;
  if (!workspace) return USP_OK;
  USP_CHECK(ws_bytes >= need, USP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  bind_job(J, js, static_cast<char*>(workspace), cu_seqlens_dev);
  PlanJobs jobs{};
  jobs.j[0] = J;
  jobs.n = 1;
  return launch_plan(jobs, as_stream(stream));
}

// ------------------------------------------------------------ block attention
size_t usp_block_attn_fwd_workspace_size(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                                         const usp_posmap* kmap, int causal, int window, int n_sink,
                                         const int32_t* cu_seqlens_host, int nseq) {
  if (Lq <= 0 || Lk < 0 || Lq > kMaxI32 / 2 || Lk > kMaxI32 / 2) return 0;
  BlockMaskSetup su;
  if (setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host, nseq, 1, &su) != USP_OK)
    return 0;
  PlanJob J = block_job(su, 0, choose_tile_m(su.ms.window), kTileN, 0);
  if (finish_job(J, cu_seqlens_host) != USP_OK) return 0;
  size_t off = 0;
  reserve_job(J, off);
  return off;
}

usp_status usp_block_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                              float softmax_scale, usp_mask_class mask, const usp_posmap* qmap,
                              const usp_posmap* kmap, int causal, int window, int n_sink,
                              const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int nseq,
                              usp_dtype out_dt, int accumulate, float softcap, const float* alibi_slopes,
                              void* workspace, size_t ws_bytes, void* stream) {
  USP_CHECK(B >= 1 && Lq >= 0 && Lk >= 0 && Hq >= 1 && Hkv >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  // k / v are never read without keys, q / out / lse never touched without queries
  USP_CHECK((q && out && lse) || Lq == 0, USP_ERR_INVALID_ARG, "null q / out / lse pointer");
  USP_CHECK((k && v) || Lk == 0, USP_ERR_INVALID_ARG, "null k / v pointer");
  USP_CHECK(D == 64 || D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)D);
  USP_CHECK(Hq % Hkv == 0, USP_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  USP_CHECK(out_dt == USP_DT_BF16 || out_dt == USP_DT_F32, USP_ERR_INVALID_ARG, "bad out dtype");
  USP_CHECK(!accumulate || out_dt == USP_DT_F32, USP_ERR_INVALID_ARG, "accumulate needs an f32 output");
  USP_CHECK((cu_seqlens_host == nullptr) == (cu_seqlens_dev == nullptr), USP_ERR_INVALID_ARG,
            "cu_seqlens must be given on both host and device, or neither");
  USP_CHECK(B * Lq <= kMaxI32 && B * Lk <= kMaxI32 && Lq * Hq <= kMaxI32 * 8, USP_ERR_UNSUPPORTED, "tensor too large");
  USP_CHECK(std::isfinite(softmax_scale), USP_ERR_INVALID_ARG, "softmax_scale must be finite");
  USP_CHECK(Lk * Hkv * D * 2 < ((int64_t)1 << 31), USP_ERR_UNSUPPORTED,
            "one batch row of k/v must be under 2 GiB (32-bit tile offsets)");
  BlockMaskSetup su;
  usp_status st = setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host,
                                   nseq, B, &su);
  if (st != USP_OK) return st;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  st = make_mods(softcap, alibi_slopes, mask, su.ms.S, scale, &mods);
  if (st != USP_OK) return st;
  if (Lq == 0) return USP_OK;

  const int32_t tm = choose_tile_m(su.ms.window);
  PlanJob J = block_job(su, 0, tm, kTileN, accumulate ? 0 : INT_MAX);
  st = finish_job(J, cu_seqlens_host);
  if (st != USP_OK) return st;
  size_t need = 0;
  const JobSlots js = reserve_job(J, need);
  USP_CHECK(workspace && ws_bytes >= need, USP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
            workspace ? ws_bytes : (size_t)0);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  // a partial with no visible pair changes nothing when merged
  if (accumulate && (su.empty || !block_has_work(su.qmap, su.kmap, su.ms, cu_seqlens_host))) return USP_OK;
  bind_job(J, js, static_cast<char*>(workspace), cu_seqlens_dev);
  PlanJobs jobs{};
  jobs.j[0] = J;
  jobs.n = 1;
  const hipStream_t stream_h = as_stream(stream);
  st = launch_plan(jobs, stream_h);
  if (st != USP_OK) return st;

  AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = out;
  p.lse = lse;
  p.items = J.items;
  p.runs = J.runs;
  p.cu_seqlens = su.ms.nseq ? cu_seqlens_dev : nullptr;
  p.q_batch_stride = Lq * Hq * D;
  p.o_batch_stride = Lq * Hq * D;
  p.kv_batch_stride = Lk * Hkv * D;
  p.Lq_buf = (int32_t)Lq;
  p.o_heads = (int32_t)Hq;
  p.o_head0 = 0;
  p.n_items = (int32_t)J.cpp();
  p.B = (int32_t)B;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.out_f32 = out_dt == USP_DT_F32;
  p.accumulate = accumulate ? 1 : 0;
  p.tile_m = tm;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.qmap = su.qmap;
  p.kmap = su.kmap;
  p.mask = su.ms;
  p.mods = mods;
  return launch_attn_fwd(p, (int)D, stream_h);
}

usp_status usp_attn_bwd_preprocess(const void* out, usp_dtype out_dt, const void* dout, float* delta,
                                   int64_t B, int64_t L, int64_t H, int64_t D, void* stream) {
  USP_CHECK(out && dout && delta, USP_ERR_INVALID_ARG, "null tensor pointer");
  USP_CHECK(B >= 0 && L >= 0 && H >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK(D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256, USP_ERR_UNSUPPORTED,
            "head_dim must be 8, 16, 32, 64, 128 or 256");
  USP_CHECK(out_dt == USP_DT_BF16 || out_dt == USP_DT_F32, USP_ERR_INVALID_ARG, "bad out dtype");
  USP_CHECK(B * L * H <= kMaxI32 * 8, USP_ERR_UNSUPPORTED, "tensor too large");
  USP_CHECK(L <= kMaxI32, USP_ERR_UNSUPPORTED, "sequence too long");
  return launch_bwd_delta(out, out_dt == USP_DT_F32, static_cast<const uint16_t*>(dout), delta, B, L, H, D,
                          as_stream(stream));
}

size_t usp_block_attn_bwd_workspace_size(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                                         const usp_posmap* kmap, int causal, int window, int n_sink,
                                         const int32_t* cu_seqlens_host, int nseq) {
  if (Lq <= 0 || Lk <= 0 || Lq > kMaxI32 / 2 || Lk > kMaxI32 / 2) return 0;
  BlockMaskSetup su;
  if (setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host, nseq, 1, &su) != USP_OK)
    return 0;
  if (su.empty) return 0;
  PlanJob jq, jk;
  bwd_block_jobs(su, &jq, &jk);
  if (finish_job(jq, cu_seqlens_host) != USP_OK || finish_job(jk, cu_seqlens_host) != USP_OK) return 0;
  size_t off = 0;
  reserve_job(jq, off);
  reserve_job(jk, off);
  return off;
}

usp_status usp_block_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              const float* delta, float* dq, float* dk, float* dv, int64_t B, int64_t Lq,
                              int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D, float softmax_scale,
                              usp_mask_class mask, const usp_posmap* qmap, const usp_posmap* kmap, int causal,
                              int window, int n_sink, const int32_t* cu_seqlens_dev,
                              const int32_t* cu_seqlens_host, int nseq, float softcap,
                              const float* alibi_slopes, void* workspace, size_t ws_bytes, void* stream) {
  USP_CHECK(q && k && v && dout && lse && delta && dq && dk && dv, USP_ERR_INVALID_ARG, "null tensor pointer");
  USP_CHECK(B >= 1 && Lq >= 0 && Lk >= 0 && Hq >= 1 && Hkv >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK(D == 64 || D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)D);
  USP_CHECK(Hq % Hkv == 0, USP_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  USP_CHECK((cu_seqlens_host == nullptr) == (cu_seqlens_dev == nullptr), USP_ERR_INVALID_ARG,
            "cu_seqlens must be given on both host and device, or neither");
  USP_CHECK(B * Lq <= kMaxI32 && B * Lk <= kMaxI32 && Lq * Hq <= kMaxI32 * 8, USP_ERR_UNSUPPORTED, "tensor too large");
  USP_CHECK(std::isfinite(softmax_scale), USP_ERR_INVALID_ARG, "softmax_scale must be finite");
  USP_CHECK(Lk * Hkv * D * 2 < ((int64_t)1 << 31) && Lq * Hq * D * 2 < ((int64_t)1 << 31), USP_ERR_UNSUPPORTED,
            "one batch row of q or k/v must be under 2 GiB (32-bit tile offsets)");
  BlockMaskSetup su;
  usp_status st = setup_block_mask(Lq, Lk, mask, qmap, kmap, causal, window, n_sink, cu_seqlens_host,
                                   nseq, B, &su);
  if (st != USP_OK) return st;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  st = make_mods(softcap, alibi_slopes, mask, su.ms.S, scale, &mods);
  if (st != USP_OK) return st;
  if (Lq == 0 || Lk == 0 || su.empty) return USP_OK;

  PlanJob jq, jk;
  bwd_block_jobs(su, &jq, &jk);
  st = finish_job(jq, cu_seqlens_host);
  if (st == USP_OK) st = finish_job(jk, cu_seqlens_host);
  if (st != USP_OK) return st;
  size_t need = 0;
  const JobSlots sq = reserve_job(jq, need);
  const JobSlots sk = reserve_job(jk, need);
  USP_CHECK(workspace && ws_bytes >= need, USP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
            workspace ? ws_bytes : (size_t)0);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (!block_has_work(su.qmap, su.kmap, su.ms, cu_seqlens_host)) return USP_OK;
  bind_job(jq, sq, static_cast<char*>(workspace), cu_seqlens_dev);
  bind_job(jk, sk, static_cast<char*>(workspace), cu_seqlens_dev);
  PlanJobs jobs{};
  jobs.j[0] = jq;
  jobs.j[1] = jk;
  jobs.n = 2;
  const hipStream_t stream_h = as_stream(stream);
  st = launch_plan(jobs, stream_h);
  if (st != USP_OK) return st;

  BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.cu_seqlens = su.ms.nseq ? cu_seqlens_dev : nullptr;
  p.q_batch_stride = Lq * Hq * D;
  p.g_batch_stride = Lq * Hq * D;
  p.kv_batch_stride = Lk * Hkv * D;
  p.Lq_buf = (int32_t)Lq;
  p.B = (int32_t)B;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.qmap = su.qmap;
  p.kmap = su.kmap;
  p.mask = su.ms;
  p.mods = mods;
  BwdParams pq = p, pk = p;
  pq.items = jq.items;
  pq.runs = jq.runs;
  pq.n_items = (int32_t)jq.cpp();
  pk.items = jk.items;
  pk.runs = jk.runs;
  pk.n_items = (int32_t)jk.cpp();
  return launch_bwd(pq, pk, (int)D, stream_h);
}

usp_status usp_decode_split_fwd(const void* q, const void* k, const void* v, const int32_t* kv_lens_dev,
                                const int32_t* kv_lens_host, float* out_part, float* lse_part, int64_t B, int64_t Lq,
                                int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t split_keys,
                                float softmax_scale, int window, int n_sink, float softcap,
                                const float* alibi_slopes, void* stream) {
  USP_CHECK(q && k && v && out_part && lse_part, USP_ERR_INVALID_ARG, "null tensor pointer");
  USP_CHECK(B >= 1 && Lq >= 1 && S >= 1 && Hq >= 1 && Hkv >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK(D == 64 || D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)D);
  USP_CHECK(Hq % Hkv == 0, USP_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  USP_CHECK((Hq / Hkv) * Lq <= 32, USP_ERR_UNSUPPORTED,
            "decode serves at most 32 queries per KV head (Hq/Hkv = %lld times Lq = %lld)", (long long)(Hq / Hkv),
            (long long)Lq);
  USP_CHECK(Lq <= S, USP_ERR_INVALID_ARG, "Lq (%lld) exceeds the cache length %lld", (long long)Lq, (long long)S);
  USP_CHECK(split_keys >= 32 && split_keys % 32 == 0 && split_keys <= kMaxI32, USP_ERR_INVALID_ARG,
            "split_keys must be a positive multiple of 32, got %lld", (long long)split_keys);
  USP_CHECK(window >= 0 && n_sink >= 0, USP_ERR_INVALID_ARG, "window and n_sink must be >= 0");
  USP_CHECK(std::isfinite(softmax_scale), USP_ERR_INVALID_ARG, "softmax_scale must be finite");
  USP_CHECK((kv_lens_dev == nullptr) == (kv_lens_host == nullptr), USP_ERR_INVALID_ARG,
            "kv_lens must be given on both host and device, or neither");
  USP_CHECK(S * Hkv * D * 2 < ((int64_t)1 << 31), USP_ERR_UNSUPPORTED,
            "one batch row of the k/v cache must be under 2 GiB (32-bit tile offsets)");
  USP_CHECK(B <= 65535 && Hkv <= 65535 && B * Lq * Hq <= kMaxI32, USP_ERR_UNSUPPORTED, "too many rows or heads");
  if (kv_lens_host)
    for (int64_t b = 0; b < B; ++b)
      USP_CHECK(kv_lens_host[b] >= Lq && kv_lens_host[b] <= S, USP_ERR_INVALID_ARG,
                "kv_lens[%lld] = %d outside [Lq, S] = [%lld, %lld]", (long long)b, kv_lens_host[b], (long long)Lq,
                (long long)S);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  usp_status st = make_mods(softcap, alibi_slopes, USP_MASK_POSITIONAL, S, scale, &mods);
  if (st != USP_OK) return st;
  DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kv_lens = kv_lens_dev;
  p.out_part = out_part;
  p.lse_part = lse_part;
  p.B = (int32_t)B;
  p.Lq = (int32_t)Lq;
  p.S = (int32_t)S;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.n_split = (int32_t)((S + split_keys - 1) / split_keys);
  p.split_keys = (int32_t)split_keys;
  p.window = window;
  p.n_sink = n_sink;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.mods = mods;
  return launch_decode_split(p, (int)D, as_stream(stream));
}

usp_status usp_decode_merge(float* out_part, float* lse_part, int64_t n_split, int64_t B, int64_t Lq,
                            int64_t Hq, int64_t D, void* out, usp_dtype out_dt, float* lse, void* stream) {
  USP_CHECK(out_part && lse_part && out && lse, USP_ERR_INVALID_ARG, "null tensor pointer");
  USP_CHECK(n_split >= 1 && n_split <= kMaxI32 && B >= 1 && Lq >= 1 && Hq >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK(D == 64 || D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)D);
  USP_CHECK(out_dt == USP_DT_BF16 || out_dt == USP_DT_F32, USP_ERR_INVALID_ARG, "bad out dtype");
  USP_CHECK(B * Lq * Hq <= kMaxI32, USP_ERR_UNSUPPORTED, "too many rows");
  return launch_decode_merge(out_part, lse_part, (int32_t)n_split, (int32_t)B, (int32_t)Lq, (int32_t)Hq, (int)D, out,
                             out_dt == USP_DT_F32, lse, as_stream(stream));
}

// ------------------------------------------------------------ virtual ring
namespace {

constexpr size_t NONE = SIZE_MAX;

struct RingLayout {
  bool one;          // one rank's share
  bool need_perm;    // natural-order input with a non-basic layout
  bool copy_in;      // q, k, v copied into the workspace (permutation, packed input, head group)
  bool seq_out;      // out_layout 1 with ud > 1: output rows hold every head, this call writes group u
  int64_t L, Ls;     // rows per ring rank, per Ulysses piece
  int64_t Hq_l, Hkv_l;
  int64_t q_rows;    // rows of the q buffer the kernel reads (per batch)
  // workspace offsets (bytes), NONE if unused
  size_t off_q, off_k, off_v, off_oacc, off_lacc, off_opart, off_lpart;
  PlanJob job;       // the ring's tile plans (one per step)
  JobSlots slots;
  size_t total;
  bool out_is_acc;   // accumulate straight into out / lse
};

usp_status check_ring_args(const usp_ring_args* a) {
  USP_CHECK(a, USP_ERR_INVALID_ARG, "null args");
  USP_CHECK(a->qkv_packed == 0 || a->qkv_packed == 1, USP_ERR_INVALID_ARG, "qkv_packed must be 0 or 1");
  USP_CHECK(a->q && (a->qkv_packed || (a->k && a->v)) && a->out && a->lse, USP_ERR_INVALID_ARG,
            "null tensor pointer");
  USP_CHECK(a->B >= 1 && a->Hq >= 1 && a->Hkv >= 1, USP_ERR_INVALID_ARG, "bad sizes");
  USP_CHECK(!a->qkv_packed || a->Hq == a->Hkv, USP_ERR_INVALID_ARG,
            "packed qkv needs Hq == Hkv (GQA / MQA use separate q, k, v)");
  USP_CHECK(a->D == 64 || a->D == 128, USP_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got %lld", (long long)a->D);
  USP_CHECK(a->Hq % a->Hkv == 0, USP_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  usp_status st = check_layout(a->impl, a->S, a->ring_degree, a->stripe_block);
  if (st != USP_OK) return st;
  USP_CHECK(a->ring_degree <= 65535, USP_ERR_UNSUPPORTED, "ring_degree must be at most 65535");
  USP_CHECK(a->ulysses_degree >= 1 && a->ulysses_degree <= 8, USP_ERR_UNSUPPORTED, "ulysses_degree must be in [1, 8]");
  USP_CHECK(a->Hq % a->ulysses_degree == 0 && a->Hkv % a->ulysses_degree == 0, USP_ERR_INVALID_ARG,
            "ulysses_degree %d must divide Hq (%lld) and Hkv (%lld)", a->ulysses_degree, (long long)a->Hq,
            (long long)a->Hkv);
  const int64_t L = a->S / a->ring_degree;
  USP_CHECK(L % a->ulysses_degree == 0, USP_ERR_INVALID_ARG, "rows per ring rank not divisible by ulysses_degree");
  USP_CHECK(a->rank >= -1 && a->rank < a->ring_degree, USP_ERR_INVALID_ARG, "rank %d out of range", a->rank);
  USP_CHECK(a->ulysses_rank >= 0 && a->ulysses_rank < a->ulysses_degree, USP_ERR_INVALID_ARG, "ulysses_rank out of range");
  USP_CHECK(a->rank >= 0 || a->ulysses_degree == 1, USP_ERR_INVALID_ARG, "all-ranks mode (rank -1) needs ulysses_degree 1");
  USP_CHECK(a->window >= 0 && a->n_sink >= 0, USP_ERR_INVALID_ARG, "window and n_sink must be >= 0");
  USP_CHECK(a->input_order == 0 || a->input_order == 1, USP_ERR_INVALID_ARG, "input_order must be 0 or 1");
  USP_CHECK(a->out_dtype == USP_DT_BF16 || a->out_dtype == USP_DT_F32, USP_ERR_INVALID_ARG, "bad out dtype");
  USP_CHECK(a->merge_mode == 0 || a->merge_mode == 1, USP_ERR_INVALID_ARG, "merge_mode must be 0 or 1");
  USP_CHECK(a->out_layout == 0 || a->out_layout == 1, USP_ERR_INVALID_ARG, "out_layout must be 0 or 1");
  USP_CHECK(a->out_layout == 0 || a->rank >= 0, USP_ERR_INVALID_ARG,
            "out_layout 1 (Ulysses sequence shards) needs one rank's share (rank >= 0)");
  USP_CHECK(std::isfinite(a->softmax_scale), USP_ERR_INVALID_ARG, "softmax_scale must be finite");
  USP_CHECK(std::isfinite(a->softcap) && a->softcap >= 0.f, USP_ERR_INVALID_ARG, "softcap must be finite and >= 0");
  USP_CHECK(!a->alibi_slopes || a->S <= kMaxAlibiPositions, USP_ERR_UNSUPPORTED,
            "ALiBi distances are computed in f32: at most %lld positions, got %lld",
            (long long)kMaxAlibiPositions, (long long)a->S);
  USP_CHECK((a->cu_seqlens_host == nullptr) == (a->cu_seqlens_dev == nullptr), USP_ERR_INVALID_ARG,
            "cu_seqlens must be given on both host and device, or neither");
  if (a->cu_seqlens_host) {
    USP_CHECK(a->B == 1, USP_ERR_INVALID_ARG, "varlen needs B == 1");
    st = check_cu(a->cu_seqlens_host, a->nseq, a->S);
    if (st != USP_OK) return st;
  }
  USP_CHECK(a->B * a->S <= kMaxI32, USP_ERR_UNSUPPORTED, "B*S too large");
  USP_CHECK(L * (a->Hkv / a->ulysses_degree) * a->D * 2 < ((int64_t)1 << 31), USP_ERR_UNSUPPORTED,
            "one ring rank's k/v rows must be under 2 GiB (32-bit tile offsets)");
  return USP_OK;
}

// The ring's score modifiers: the slopes of this Ulysses rank's head group.
usp_status ring_mods(const usp_ring_args* a, int64_t Hq_l, float scale, ScoreMods* out) {
  const float* slopes = a->alibi_slopes ? a->alibi_slopes + (int64_t)a->ulysses_rank * Hq_l : nullptr;
  return make_mods(a->softcap, slopes, USP_MASK_POSITIONAL, a->S, scale, out);
}

MaskSpec ring_mask(const usp_ring_args* a) {
  MaskSpec ms;
  ms.causal = a->causal ? 1 : 0;
  ms.window = a->window;
  ms.n_sink = a->n_sink;
  ms.nseq = a->cu_seqlens_host ? a->nseq : 0;
  ms.S = (int32_t)a->S;
  return ms;
}

PosMap ring_base_map(const usp_ring_args* a) {
  usp_posmap pm{a->impl, a->ring_degree, 0, a->impl == USP_RING_STRIPE ? a->stripe_block : 1, a->S};
  return make_map(pm);
}

// The ring's plan job: plan s is ring step s, its blocks the hosts i (all,
// or the one rank) against KV piece (i - s) mod N.
PlanJob ring_job(const usp_ring_args* a, int kind, int32_t tile, int32_t gran, int32_t acc_from_step) {
  const int N = a->ring_degree;
  const bool one = a->rank >= 0;
  PlanJob J{};
  J.qmap = J.kmap = ring_base_map(a);
  J.mask = ring_mask(a);
  J.kind = kind;
  J.tile = tile;
  J.gran = gran;
  J.acc_from_step = acc_from_step;
  J.empty = 0;
  J.ring = 1;
  J.N = N;
  J.rank_lo = one ? a->rank : 0;
  J.n_ranks = one ? 1 : N;
  J.n_steps = N;
  J.one_rank = one ? 1 : 0;
  J.L = (int32_t)(a->S / N);
  J.cpb = tile_count(J.qmap, tile);
  return J;
}

// Staging regions of q, k, v (shared by the forward and backward layouts).
void reserve_staging(const usp_ring_args* a, RingLayout& r, size_t& off) {
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t D = (size_t)a->D, B = (size_t)a->B, S = (size_t)a->S;
  r.off_q = r.off_k = r.off_v = NONE;
  if (r.copy_in) {
    r.off_q = take(B * (size_t)r.q_rows * r.Hq_l * D * 2);
    r.off_k = take(B * S * r.Hkv_l * D * 2);
    r.off_v = take(B * S * r.Hkv_l * D * 2);
  }
}

void ring_shape(const usp_ring_args* a, RingLayout& r) {
  r.one = a->rank >= 0;
  r.need_perm = a->input_order == 0 && a->impl != USP_RING_BASIC;
  const int ud = a->ulysses_degree;
  r.copy_in = r.need_perm || a->qkv_packed || ud > 1;
  r.seq_out = a->out_layout == 1 && ud > 1;
  r.L = a->S / a->ring_degree;
  r.Ls = r.L / ud;
  r.Hq_l = a->Hq / ud;
  r.Hkv_l = a->Hkv / ud;
  r.q_rows = r.one ? r.L : a->S;
}

usp_status ring_layout(const usp_ring_args* a, RingLayout* out) {
  RingLayout r;
  ring_shape(a, r);
  r.off_oacc = r.off_lacc = r.off_opart = r.off_lpart = NONE;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  reserve_staging(a, r, off);
  const size_t D = (size_t)a->D, B = (size_t)a->B;
  // accumulate directly into out/lse when they are f32 and already in the
  // order the kernel computes in (the merge kernel works on dense rows, so a
  // sequence-shard output with merge_mode 1 goes through the accumulator)
  r.out_is_acc = a->out_dtype == USP_DT_F32 && (r.one || !r.need_perm) && !(r.seq_out && a->merge_mode == 1);
  if (!r.out_is_acc) {
    r.off_oacc = take(B * (size_t)r.q_rows * r.Hq_l * D * 4);
    r.off_lacc = take(B * (size_t)r.Hq_l * r.q_rows * 4);
  }
  if (a->merge_mode == 1) {
    r.off_opart = take(B * (size_t)r.q_rows * r.Hq_l * D * 4);
    r.off_lpart = take(B * (size_t)r.Hq_l * r.q_rows * 4);
  }
  r.job = ring_job(a, 0, choose_tile_m(a->window), kTileN, a->merge_mode == 0 ? 1 : INT_MAX);
  usp_status st = finish_job(r.job, a->cu_seqlens_host);
  if (st != USP_OK) return st;
  r.slots = reserve_job(r.job, off);
  r.total = off;
  *out = r;
  return USP_OK;
}

// Identity row map (row i -> row i) over rows of `rows` per outer slice.
GatherSpec identity_rows(int64_t rows, int kind) {
  GatherSpec gs{};
  gs.impl = USP_RING_BASIC;
  gs.N = 1;
  gs.ud = 1;
  gs.b = 1;
  gs.g = 0;
  gs.L = (int32_t)rows;
  gs.S = (int32_t)rows;
  gs.kind = kind;
  return gs;
}

// Steps 1-2 of the ring (shared by forward and backward): token order
// (rank-major q, or ring rank r's rows; k, v), then the Ulysses seq -> head
// relayout for Ulysses rank u, written to qd, kd, vd when the ring reads
// copies (R.copy_in).
//
// With ulysses_degree > 1 the two steps are one strided copy per tensor.
// Ulysses rank u gathers, for each ring rank, the ud sub-shards of that
// rank's rows in order and keeps head group u, so its relayouted tensor is
// the ring-ordered rows restricted to heads [u H/ud, (u+1) H/ud): a gather
// of rows (the layout's permutation or rank extract) of a head slice.
struct Staged {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t q_batch_rows;  // rows between batches in the q buffer
  int64_t q_row_off;     // first row of the rank's q rows
  int64_t Hq_l, Hkv_l;   // heads after the Ulysses split
};

usp_status stage_ring_inputs(const usp_ring_args* a, const RingLayout& R, uint16_t* qd, uint16_t* kd,
                             uint16_t* vd, hipStream_t stream, Staged* out) {
  const int N = a->ring_degree, u = a->ulysses_rank;
  const int64_t B = a->B, S = a->S, D = a->D, L = R.L;
  const int b = a->impl == USP_RING_STRIPE ? a->stripe_block : 1;
  if (!R.copy_in) {
    // the caller's rank-major (or basic-layout) tensors are read in place
    *out = Staged{static_cast<const uint16_t*>(a->q), static_cast<const uint16_t*>(a->k),
                  static_cast<const uint16_t*>(a->v), S, R.one ? (int64_t)a->rank * L : 0, a->Hq, a->Hkv};
    return USP_OK;
  }
  // rows in ring order (all pieces of k and v; every rank's rows of q, or
  // ring rank r's), heads of group u, from natural or rank-major order,
  // packed or not: one strided row gather per tensor
  const int64_t Hq_l = R.Hq_l, Hkv_l = R.Hkv_l;
  const int64_t q_row = a->Hq * D * 2, kv_row = a->Hkv * D * 2;  // source row bytes (one tensor)
  const int64_t src_stride_q = a->qkv_packed ? 3 * q_row : q_row;
  const int64_t src_stride_kv = a->qkv_packed ? 3 * kv_row : kv_row;
  const char* qb = static_cast<const char*>(a->q);
  const char* kb = a->qkv_packed ? qb + q_row : static_cast<const char*>(a->k);
  const char* vb = a->qkv_packed ? qb + 2 * q_row : static_cast<const char*>(a->v);
  auto spec = [&](bool extract) {
    GatherSpec gs{};
    gs.impl = R.need_perm ? a->impl : USP_RING_BASIC;
    gs.N = N;
    gs.ud = 1;
    gs.b = R.need_perm ? b : 1;
    gs.g = extract ? a->rank : 0;
    gs.L = (int32_t)L;
    gs.S = (int32_t)S;
    gs.kind = extract ? G_EXTRACT : G_PERMUTE;
    return gs;
  };
  usp_status st = launch_permute_strided(kb + u * Hkv_l * D * 2, kd, B, S, S, Hkv_l * D * 2, src_stride_kv,
                                         Hkv_l * D * 2, spec(false), stream);
  if (st == USP_OK)
    st = launch_permute_strided(vb + u * Hkv_l * D * 2, vd, B, S, S, Hkv_l * D * 2, src_stride_kv, Hkv_l * D * 2,
                                spec(false), stream);
  if (st == USP_OK)
    st = launch_permute_strided(qb + u * Hq_l * D * 2, qd, B, S, R.q_rows, Hq_l * D * 2, src_stride_q,
                                Hq_l * D * 2, spec(R.one), stream);
  if (st != USP_OK) return st;
  *out = Staged{qd, kd, vd, R.q_rows, 0, Hq_l, Hkv_l};
  return USP_OK;
}

uint16_t* ws_ptr(char* ws, size_t off) { return off == NONE ? nullptr : reinterpret_cast<uint16_t*>(ws + off); }

// Workspace of the backward ring: the forward's staging regions, delta, and
// -- when the caller's tensors are in natural order but the ring runs
// rank-major (all ranks, non-basic layout) -- rank-major copies of dout and
// LSE and rank-major f32 gradient accumulators that are un-permuted into the
// outputs at the end; with a sequence-shard forward output (out_layout 1),
// head group u of out, dout and LSE gathered into the head-split layout.
struct RingBwdLayout {
  RingLayout base;        // only the staging regions of the forward layout are used
  bool reorder;           // all ranks, natural-order tensors, non-basic layout
  size_t off_delta, off_delta_nat, off_dop, off_lsep, off_dq, off_dk, off_dv;
  size_t off_og, off_dog, off_lg;  // head group u of out / dout / LSE (sequence-shard output)
  PlanJob jq, jk;         // dQ and dK / dV plans, one per step
  JobSlots sq, sk;
  size_t total;
};

usp_status ring_bwd_layout(const usp_ring_args* a, RingBwdLayout* out) {
  RingBwdLayout r;
  RingLayout& R = r.base;
  ring_shape(a, R);
  R.off_oacc = R.off_lacc = R.off_opart = R.off_lpart = NONE;
  R.out_is_acc = false;
  const size_t D = (size_t)a->D, B = (size_t)a->B, S = (size_t)a->S;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  reserve_staging(a, R, off);
  r.reorder = R.need_perm && !R.one;
  r.off_delta = take(B * (size_t)R.Hq_l * R.q_rows * 4);
  r.off_delta_nat = r.off_dop = r.off_lsep = r.off_dq = r.off_dk = r.off_dv = NONE;
  r.off_og = r.off_dog = r.off_lg = NONE;
  if (r.reorder) {
    r.off_delta_nat = take(B * (size_t)a->Hq * S * 4);
    r.off_dop = take(B * S * a->Hq * D * 2);
    r.off_lsep = take(B * (size_t)a->Hq * S * 4);
    r.off_dq = take(B * S * a->Hq * D * 4);
    r.off_dk = take(B * S * a->Hkv * D * 4);
    r.off_dv = take(B * S * a->Hkv * D * 4);
  }
  if (R.seq_out) {
    const size_t eb = a->out_dtype == USP_DT_F32 ? 4 : 2;
    r.off_og = take(B * (size_t)R.L * R.Hq_l * D * eb);
    r.off_dog = take(B * (size_t)R.L * R.Hq_l * D * 2);
    r.off_lg = take(B * (size_t)R.Hq_l * R.L * 4);
  }
  // Step 0 stores dq (and, with every host in the call, dk / dv) instead of
  // adding to zeros, so its plans keep the tiles no query reaches; for one
  // rank each step owns the dk / dv piece it meets, and every step stores.
  const int N = a->ring_degree;
  r.jq = ring_job(a, 0, kBwdTileM, kTileN, 1);
  r.jk = ring_job(a, 1, kBwdTileK, kBwdTileQ, a->rank >= 0 ? N : 1);
  usp_status st = finish_job(r.jq, a->cu_seqlens_host);
  if (st == USP_OK) st = finish_job(r.jk, a->cu_seqlens_host);
  if (st != USP_OK) return st;
  r.sq = reserve_job(r.jq, off);
  r.sk = reserve_job(r.jk, off);
  R.total = off;
  r.total = off;
  *out = r;
  return USP_OK;
}

}  // namespace

size_t usp_ring_fwd_workspace_size(const usp_ring_args* a) {
  if (check_ring_args(a) != USP_OK) return 0;
  RingLayout R;
  if (ring_layout(a, &R) != USP_OK) return 0;
  return R.total;
}

usp_status usp_ring_stage(const usp_ring_args* a, void* q_staged, void* k_staged, void* v_staged, void* stream_) {
  usp_status st = check_ring_args(a);
  if (st != USP_OK) return st;
  USP_CHECK(q_staged && k_staged && v_staged, USP_ERR_INVALID_ARG, "null staging buffer");
  RingLayout R;
  ring_shape(a, R);
  hipStream_t stream = as_stream(stream_);
  uint16_t* qd = static_cast<uint16_t*>(q_staged);
  uint16_t* kd = static_cast<uint16_t*>(k_staged);
  uint16_t* vd = static_cast<uint16_t*>(v_staged);
  Staged stg;
  st = stage_ring_inputs(a, R, qd, kd, vd, stream, &stg);
  if (st != USP_OK || R.copy_in) return st;
  // the ring reads the caller's tensors in place: copy the rows it reads
  const int64_t B = a->B, S = a->S, D = a->D;
  st = launch_permute_strided(stg.q + stg.q_row_off * a->Hq * D, qd, B, stg.q_batch_rows, R.q_rows, a->Hq * D * 2,
                              a->Hq * D * 2, a->Hq * D * 2, identity_rows(R.q_rows, G_PERMUTE), stream);
  if (st == USP_OK)
    st = launch_permute(stg.k, kd, B, S, S, a->Hkv * D * 2, identity_rows(S, G_PERMUTE), stream);
  if (st == USP_OK)
    st = launch_permute(stg.v, vd, B, S, S, a->Hkv * D * 2, identity_rows(S, G_PERMUTE), stream);
  return st;
}

usp_status usp_ring_fwd(const usp_ring_args* a, void* workspace, size_t ws_bytes, void* stream_) {
  usp_status st = check_ring_args(a);
  if (st != USP_OK) return st;
  RingLayout R;
  st = ring_layout(a, &R);
  if (st != USP_OK) return st;
  USP_CHECK(workspace && ws_bytes >= R.total, USP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", R.total,
            workspace ? ws_bytes : (size_t)0);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const int N = a->ring_degree;
  const int64_t B = a->B, D = a->D;
  const int64_t Hq_l = R.Hq_l;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  st = ring_mods(a, Hq_l, scale, &mods);
  if (st != USP_OK) return st;
  // everything is validated: enqueue
  hipStream_t stream = as_stream(stream_);
  char* ws = static_cast<char*>(workspace);
  PlanJob J = R.job;
  bind_job(J, R.slots, ws, a->cu_seqlens_dev);
  PlanJobs jobs{};
  jobs.j[0] = J;
  jobs.n = 1;
  st = launch_plan(jobs, stream);
  if (st != USP_OK) return st;
  Staged stg;
  st = stage_ring_inputs(a, R, ws_ptr(ws, R.off_q), ws_ptr(ws, R.off_k), ws_ptr(ws, R.off_v), stream, &stg);
  if (st != USP_OK) return st;

  // 3. ring steps
  float* oacc = R.out_is_acc ? static_cast<float*>(a->out) : reinterpret_cast<float*>(ws + R.off_oacc);
  float* lacc = R.out_is_acc ? a->lse : reinterpret_cast<float*>(ws + R.off_lacc);
  float* opart = a->merge_mode ? reinterpret_cast<float*>(ws + R.off_opart) : nullptr;
  float* lpart = a->merge_mode ? reinterpret_cast<float*>(ws + R.off_lpart) : nullptr;
  const int64_t cpp = J.cpp();
  const int32_t o_heads_acc = R.out_is_acc && R.seq_out ? (int32_t)a->Hq : (int32_t)Hq_l;
  const int32_t o_head0_acc = R.out_is_acc && R.seq_out ? (int32_t)(a->ulysses_rank * Hq_l) : 0;
  for (int s = 0; s < N; ++s) {
    // steps without a visible pair are skipped (step 0 always runs: it
    // initialises every row); a host-only test on the step's position ranges
    if (s > 0 && !step_has_work(R.job, s, a->cu_seqlens_host)) continue;
    const int acc_flag = (s > 0 && a->merge_mode == 0) ? 1 : 0;
    AttnParams p{};
    p.q = stg.q + stg.q_row_off * Hq_l * D;
    p.k = stg.k;
    p.v = stg.v;
    const bool to_part = a->merge_mode == 1 && s > 0;
    p.out = to_part ? static_cast<void*>(opart) : static_cast<void*>(oacc);
    p.lse = to_part ? lpart : lacc;
    p.items = J.items + (int64_t)s * cpp;
    p.runs = J.runs;
    p.cu_seqlens = J.mask.nseq ? a->cu_seqlens_dev : nullptr;
    p.q_batch_stride = stg.q_batch_rows * Hq_l * D;
    p.o_heads = to_part ? (int32_t)Hq_l : o_heads_acc;
    p.o_head0 = to_part ? 0 : o_head0_acc;
    p.o_batch_stride = R.q_rows * p.o_heads * D;
    p.kv_batch_stride = a->S * stg.Hkv_l * D;
    p.Lq_buf = (int32_t)R.q_rows;
    p.n_items = (int32_t)cpp;
    p.B = (int32_t)B;
    p.Hq = (int32_t)Hq_l;
    p.Hkv = (int32_t)stg.Hkv_l;
    p.out_f32 = 1;
    p.accumulate = acc_flag;
    p.tile_m = J.tile;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.qmap = J.qmap;
    p.kmap = J.kmap;
    p.mask = J.mask;
    p.mods = mods;
    st = launch_attn_fwd(p, (int)D, stream);
    if (st != USP_OK) return st;
    if (to_part) {
      st = launch_lse_merge(oacc, lacc, opart, lpart, B, R.q_rows, Hq_l, D, 0, R.q_rows, stream);
      if (st != USP_OK) return st;
    }
  }

  // 4. finalize: dtype, order and head layout of the outputs
  if (!R.out_is_acc) {
    const bool perm = R.need_perm && !R.one;
    GatherSpec gs = identity_rows(R.q_rows, G_UNPERMUTE);
    if (perm) {
      gs.impl = a->impl;
      gs.N = N;
      gs.b = a->impl == USP_RING_STRIPE ? a->stripe_block : 1;
      gs.L = (int32_t)R.L;
    }
    const int64_t row = Hq_l * D;                         // elements of one accumulator row
    const int64_t orow = R.seq_out ? a->Hq * D : row;     // elements between output rows
    const int64_t ohead = R.seq_out ? a->ulysses_rank * row : 0;
    if (a->out_dtype == USP_DT_F32) {
      st = launch_permute_strided(oacc, static_cast<float*>(a->out) + ohead, B, R.q_rows, R.q_rows, row * 4, row * 4,
                                  orow * 4, gs, stream);
    } else {
      st = launch_permute_f32_to_bf16(oacc, static_cast<uint16_t*>(a->out) + ohead, B, R.q_rows, R.q_rows, row, orow,
                                      gs, stream);
    }
    if (st != USP_OK) return st;
    if (R.seq_out) {
      // one rank's rows in order: batch row b's [Hq/ud, L] block goes to heads of group u
      const int64_t blk = Hq_l * R.q_rows;
      st = launch_permute_strided(lacc, a->lse + a->ulysses_rank * blk, 1, B, B, blk * 4, blk * 4,
                                  a->Hq * R.q_rows * 4, identity_rows(B, G_PERMUTE), stream);
    } else {
      st = launch_permute(lacc, a->lse, B * Hq_l, R.q_rows, R.q_rows, 4, gs, stream);
    }
    if (st != USP_OK) return st;
  }
  return USP_OK;
}

size_t usp_ring_bwd_workspace_size(const usp_ring_bwd_args* a) {
  if (!a || check_ring_args(&a->fwd) != USP_OK) return 0;
  RingBwdLayout RB;
  if (ring_bwd_layout(&a->fwd, &RB) != USP_OK) return 0;
  return RB.total;
}

usp_status usp_ring_bwd(const usp_ring_bwd_args* ba, void* workspace, size_t ws_bytes, void* stream_) {
  USP_CHECK(ba, USP_ERR_INVALID_ARG, "null args");
  const usp_ring_args* a = &ba->fwd;
  usp_status st = check_ring_args(a);
  if (st != USP_OK) return st;
  USP_CHECK(ba->dout && ba->dq && ba->dk && ba->dv, USP_ERR_INVALID_ARG, "null gradient pointer");
  RingBwdLayout RB;
  st = ring_bwd_layout(a, &RB);
  if (st != USP_OK) return st;
  const RingLayout& R = RB.base;
  USP_CHECK(R.L * R.Hq_l * a->D * 2 < ((int64_t)1 << 31) && R.q_rows * R.Hq_l * 4 < ((int64_t)1 << 31),
            USP_ERR_UNSUPPORTED, "one ring rank's q rows and one batch row of LSE must be under 2 GiB "
            "(32-bit tile offsets)");
  USP_CHECK(workspace && ws_bytes >= RB.total, USP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
            RB.total, workspace ? ws_bytes : (size_t)0);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const int N = a->ring_degree;
  const int64_t B = a->B, S = a->S, D = a->D, L = R.L;
  const int b = a->impl == USP_RING_STRIPE ? a->stripe_block : 1;
  const int64_t Hq_l = R.Hq_l;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  st = ring_mods(a, Hq_l, scale, &mods);
  if (st != USP_OK) return st;
  // everything is validated: enqueue
  hipStream_t stream = as_stream(stream_);
  char* ws = static_cast<char*>(workspace);
  PlanJob jq = RB.jq, jk = RB.jk;
  bind_job(jq, RB.sq, ws, a->cu_seqlens_dev);
  bind_job(jk, RB.sk, ws, a->cu_seqlens_dev);
  PlanJobs jobs{};
  jobs.j[0] = jq;
  jobs.j[1] = jk;
  jobs.n = 2;
  st = launch_plan(jobs, stream);
  if (st != USP_OK) return st;

  // 1-2. the forward's staging of q, k, v
  Staged stg;
  st = stage_ring_inputs(a, R, ws_ptr(ws, R.off_q), ws_ptr(ws, R.off_k), ws_ptr(ws, R.off_v), stream, &stg);
  if (st != USP_OK) return st;

  // the forward's out / LSE and dout in the head-split layout the kernels read
  const usp_dtype odt = (usp_dtype)a->out_dtype;
  const void* fout = a->out;
  const float* lse = a->lse;
  const uint16_t* dout = static_cast<const uint16_t*>(ba->dout);
  if (R.seq_out) {
    const int64_t eb = odt == USP_DT_F32 ? 4 : 2;
    const int64_t u = a->ulysses_rank;
    char* og = ws + RB.off_og;
    char* dog = ws + RB.off_dog;
    float* lg = reinterpret_cast<float*>(ws + RB.off_lg);
    const GatherSpec id = identity_rows(L, G_PERMUTE);
    st = launch_permute_strided(static_cast<const char*>(a->out) + u * Hq_l * D * eb, og, B, L, L, Hq_l * D * eb,
                                a->Hq * D * eb, Hq_l * D * eb, id, stream);
    if (st == USP_OK)
      st = launch_permute_strided(static_cast<const char*>(ba->dout) + u * Hq_l * D * 2, dog, B, L, L, Hq_l * D * 2,
                                  a->Hq * D * 2, Hq_l * D * 2, id, stream);
    if (st == USP_OK)
      st = launch_permute_strided(a->lse + u * Hq_l * L, lg, 1, B, B, Hq_l * L * 4, a->Hq * L * 4, Hq_l * L * 4,
                                  identity_rows(B, G_PERMUTE), stream);
    if (st != USP_OK) return st;
    fout = og;
    dout = reinterpret_cast<const uint16_t*>(dog);
    lse = lg;
  }

  // delta = rowsum(dO * O) over the rows the ring visits, in their order;
  // dout and LSE in that order too
  float* delta = reinterpret_cast<float*>(ws + RB.off_delta);
  if (RB.reorder) {
    float* dn = reinterpret_cast<float*>(ws + RB.off_delta_nat);
    uint16_t* dop = reinterpret_cast<uint16_t*>(ws + RB.off_dop);
    float* lsep = reinterpret_cast<float*>(ws + RB.off_lsep);
    st = launch_bwd_delta(fout, odt == USP_DT_F32, dout, dn, B, S, a->Hq, D, stream);
    if (st == USP_OK)
      st = usp_permute(dn, delta, B * a->Hq, S, 1, USP_DT_F32, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st == USP_OK)
      st = usp_permute(lse, lsep, B * a->Hq, S, 1, USP_DT_F32, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st == USP_OK)
      st = usp_permute(dout, dop, B, S, a->Hq * D, USP_DT_BF16, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st != USP_OK) return st;
    dout = dop;
    lse = lsep;
  } else {
    st = launch_bwd_delta(fout, odt == USP_DT_F32, dout, delta, B, R.q_rows, Hq_l, D, stream);
    if (st != USP_OK) return st;
  }

  // gradient accumulators
  float* dq = RB.reorder ? reinterpret_cast<float*>(ws + RB.off_dq) : ba->dq;
  float* dk = RB.reorder ? reinterpret_cast<float*>(ws + RB.off_dk) : ba->dk;
  float* dv = RB.reorder ? reinterpret_cast<float*>(ws + RB.off_dv) : ba->dv;

  // 3. ring steps: host i meets KV piece j = (i - s) mod N; one launch per
  // kernel per step covers every host of the step (their dq rows and dk / dv
  // pieces are disjoint).  Step 0 always runs and stores dq; dk / dv are
  // stored by step 0 when every host is in the call (each piece meets its
  // own host there), and by every step for one rank (each step meets a
  // different piece), so a step without work still runs its dK / dV launch
  // then, with tiles that only store zeros.
  const bool one = a->rank >= 0;
  const int64_t cq = jq.cpp(), ck = jk.cpp();
  for (int s = 0; s < N; ++s) {
    const bool work = s == 0 || step_has_work(RB.jq, s, a->cu_seqlens_host);
    if (!work && !one) continue;
    BwdParams p{};
    p.q = stg.q + stg.q_row_off * Hq_l * D;
    p.k = stg.k;
    p.v = stg.v;
    p.dout = dout;
    p.lse = lse;
    p.delta = delta;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.cu_seqlens = jq.mask.nseq ? a->cu_seqlens_dev : nullptr;
    p.q_batch_stride = stg.q_batch_rows * Hq_l * D;
    p.g_batch_stride = R.q_rows * Hq_l * D;
    p.kv_batch_stride = S * stg.Hkv_l * D;
    p.Lq_buf = (int32_t)R.q_rows;
    p.B = (int32_t)B;
    p.Hq = (int32_t)Hq_l;
    p.Hkv = (int32_t)stg.Hkv_l;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.qmap = jq.qmap;
    p.kmap = jq.kmap;
    p.mask = jq.mask;
    p.mods = mods;
    BwdParams pq = p, pk = p;
    pq.items = jq.items + (int64_t)s * cq;
    pq.runs = jq.runs;
    pq.n_items = work ? (int32_t)cq : 0;
    pq.overwrite = s == 0;
    pk.items = jk.items + (int64_t)s * ck;
    pk.runs = jk.runs;
    pk.n_items = (int32_t)ck;
    pk.overwrite = s == 0 || one;
    st = launch_bwd(pq, pk, (int)D, stream);
    if (st != USP_OK) return st;
  }

  // 4. natural order for the caller's tensors
  if (RB.reorder) {
    GatherSpec gs{};
    gs.impl = a->impl;
    gs.N = N;
    gs.ud = 1;
    gs.b = b;
    gs.g = 0;
    gs.L = (int32_t)L;
    gs.S = (int32_t)S;
    gs.kind = G_UNPERMUTE;
    st = launch_permute(dq, ba->dq, B, S, S, a->Hq * D * 4, gs, stream);
    if (st == USP_OK) st = launch_permute(dk, ba->dk, B, S, S, a->Hkv * D * 4, gs, stream);
    if (st == USP_OK) st = launch_permute(dv, ba->dv, B, S, S, a->Hkv * D * 4, gs, stream);
    if (st != USP_OK) return st;
  }
  return USP_OK;
}

}  // extern "C"
