// C ABI of libusp: argument validation, tile-plan cache, and the virtual
// ring driver.  Every entry point validates everything on the host before
// enqueueing anything; see include/usp.h for the contract of each call.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "usp_internal.h"

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

// ------------------------------------------------------------ plan cache
std::mutex g_plan_mu;
std::unordered_map<std::string, DevicePlan> g_plans;

// Returns the device copy of the plan cached under `key`; builds it with
// `build` and uploads it on a miss (one synchronous copy).
template <typename F>
usp_status device_plan(const std::string& key_in, F&& build, DevicePlan* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("hipGetDevice failed");
    return USP_ERR_HIP;
  }
  const std::string key = std::to_string(dev) + "|" + key_in;
  std::lock_guard<std::mutex> lock(g_plan_mu);
  auto f = g_plans.find(key);
  if (f != g_plans.end()) {
    *out = f->second;
    return USP_OK;
  }
  Plan plan;
  build(plan);
  finalize_plan(plan);
  USP_CHECK(plan.items.size() <= (size_t)kMaxI32 && plan.runs.size() <= (size_t)kMaxI32,
            USP_ERR_UNSUPPORTED, "tile plan too large");
  DevicePlan dp;
  dp.n_items = (int32_t)plan.items.size();
  dp.n_runs = (int32_t)plan.runs.size();
  const size_t ib = std::max<size_t>(1, plan.items.size()) * sizeof(WorkItem);
  const size_t rb = std::max<size_t>(1, plan.runs.size()) * sizeof(Run);
  if (hipMalloc(reinterpret_cast<void**>(&dp.items), ib) != hipSuccess ||
      hipMalloc(reinterpret_cast<void**>(&dp.runs), rb) != hipSuccess) {
    if (dp.items) (void)hipFree(dp.items);
    set_error("hipMalloc of tile plan failed");
    return USP_ERR_HIP;
  }
  hipError_t e = hipSuccess;
  if (!plan.items.empty())
    e = hipMemcpy(dp.items, plan.items.data(), plan.items.size() * sizeof(WorkItem), hipMemcpyHostToDevice);
  if (e == hipSuccess && !plan.runs.empty())
    e = hipMemcpy(dp.runs, plan.runs.data(), plan.runs.size() * sizeof(Run), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dp.items);
    (void)hipFree(dp.runs);
    set_error("upload of tile plan failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  g_plans.emplace(key, dp);
  *out = dp;
  return USP_OK;
}

std::string cu_key(const int32_t* cu, int nseq) {
  std::string s;
  if (!cu) return "-";
  for (int i = 0; i <= nseq; ++i) s += std::to_string(cu[i]) + ",";
  return s;
}

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

// Items / runs of one block call (explicit class or positional).
void build_block_plan(const BlockMaskSetup& su, int32_t Lq, int32_t Lk, const int32_t* cu_host,
                      int accumulate, int32_t tile_m, Plan& plan) {
  if (!su.empty) {
    BlockSpec blk{su.qmap, su.kmap, Lq, Lk, 0, 0, tile_m};
    plan_block(blk, su.ms, cu_host, accumulate, plan);
  } else if (!accumulate) {
    // EMPTY without accumulate: items with no runs write O = 0, LSE = -inf
    for (int32_t t0 = 0; t0 < Lq; t0 += tile_m)
      plan.items.push_back({t0, t0, std::min<int32_t>(tile_m, Lq - t0), 0, 0, 0, 0, 0});
  }
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

std::string map_key(const PosMap& m) {
  char buf[96];
  snprintf(buf, sizeof(buf), "%d.%d.%d.%d.%d.%d", m.kind, m.N, m.rank, m.b, m.L, m.offset);
  return buf;
}

std::string mask_key(const MaskSpec& ms) {
  char buf[96];
  snprintf(buf, sizeof(buf), "c%d.w%d.s%d.n%d.S%d", ms.causal, ms.window, ms.n_sink, ms.nseq, ms.S);
  return buf;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace
}  // namespace usp

using namespace usp;

extern "C" {

const char* usp_last_error(void) { return g_err.c_str(); }

const char* usp_version(void) { return "usp-gfx950 0.1"; }

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

int64_t usp_plan_cache_size(void) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  return (int64_t)g_plans.size();
}

usp_status usp_plan_cache_clear(void) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  usp_status st = USP_OK;
  int cur = 0;
  const bool have_dev = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_plans) {
    // the key starts with the plan's device ordinal
    const int dev = std::atoi(kv.first.c_str());
    if (have_dev && dev != cur) (void)hipSetDevice(dev);
    if (hipFree(kv.second.items) != hipSuccess || hipFree(kv.second.runs) != hipSuccess) {
      set_error("hipFree of a cached tile plan failed");
      st = USP_ERR_HIP;
    }
  }
  if (have_dev) (void)hipSetDevice(cur);
  g_plans.clear();
  return st;
}

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
  Plan plan;
  const int32_t tm = choose_tile_m(su.qmap);
  build_block_plan(su, (int32_t)Lq, (int32_t)Lk, cu_seqlens_host, accumulate, tm, plan);
  finalize_plan(plan);
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
  if (!su.empty) {
    BlockSpec blk{su.qmap, su.kmap, (int32_t)Lq, (int32_t)Lk, 0, 0, kBwdTileM};
    plan_block_kv(blk, su.ms, cu_seqlens_host, kBwdTileK, kBwdTileQ, plan);
  }
  finalize_plan(plan);
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

usp_status usp_block_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                              float softmax_scale, usp_mask_class mask, const usp_posmap* qmap,
                              const usp_posmap* kmap, int causal, int window, int n_sink,
                              const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int nseq,
                              usp_dtype out_dt, int accumulate, float softcap, const float* alibi_slopes,
                              void* stream) {
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

  const int32_t tm = choose_tile_m(su.qmap);
  std::string key = "blk|" + std::to_string(Lq) + "|" + std::to_string(Lk) + "|" + map_key(su.qmap) + "|" +
                    map_key(su.kmap) + "|" + mask_key(su.ms) + "|" + cu_key(su.ms.nseq ? cu_seqlens_host : nullptr, nseq) +
                    "|a" + std::to_string(accumulate) + "|e" + std::to_string(su.empty) + "|m" + std::to_string(tm);
  DevicePlan dp;
  st = device_plan(key, [&](Plan& plan) {
    build_block_plan(su, (int32_t)Lq, (int32_t)Lk, cu_seqlens_host, accumulate, tm, plan);
  }, &dp);
  if (st != USP_OK) return st;

  AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = out;
  p.lse = lse;
  p.items = dp.items;
  p.runs = dp.runs;
  p.cu_seqlens = su.ms.nseq ? cu_seqlens_dev : nullptr;
  p.q_batch_stride = Lq * Hq * D;
  p.o_batch_stride = Lq * Hq * D;
  p.kv_batch_stride = Lk * Hkv * D;
  p.Lq_buf = (int32_t)Lq;
  p.n_items = dp.n_items;
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
  return launch_attn_fwd(p, (int)D, as_stream(stream));
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

usp_status usp_block_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              const float* delta, float* dq, float* dk, float* dv, int64_t B, int64_t Lq,
                              int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D, float softmax_scale,
                              usp_mask_class mask, const usp_posmap* qmap, const usp_posmap* kmap, int causal,
                              int window, int n_sink, const int32_t* cu_seqlens_dev,
                              const int32_t* cu_seqlens_host, int nseq, float softcap,
                              const float* alibi_slopes, void* stream) {
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

  const std::string base = std::to_string(Lq) + "|" + std::to_string(Lk) + "|" + map_key(su.qmap) + "|" +
                           map_key(su.kmap) + "|" + mask_key(su.ms) + "|" +
                           cu_key(su.ms.nseq ? cu_seqlens_host : nullptr, nseq);
  DevicePlan dpq, dpk;
  st = device_plan("bwdq|" + base, [&](Plan& plan) {
    build_block_plan(su, (int32_t)Lq, (int32_t)Lk, cu_seqlens_host, 1, kBwdTileM, plan);
  }, &dpq);
  if (st != USP_OK) return st;
  st = device_plan("bwdkv|" + base, [&](Plan& plan) {
    BlockSpec blk{su.qmap, su.kmap, (int32_t)Lq, (int32_t)Lk, 0, 0, kBwdTileM};
    plan_block_kv(blk, su.ms, cu_seqlens_host, kBwdTileK, kBwdTileQ, plan);
  }, &dpk);
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
  pq.items = dpq.items;
  pq.runs = dpq.runs;
  pq.n_items = dpq.n_items;
  pk.items = dpk.items;
  pk.runs = dpk.runs;
  pk.n_items = dpk.n_items;
  return launch_bwd(pq, pk, (int)D, as_stream(stream));
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

struct RingLayout {
  bool one;          // one rank's share
  bool need_perm;    // natural-order input with a non-basic layout
  bool copy_in;      // q, k, v copied into the workspace (permutation or packed input)
  int64_t L, Ls;     // rows per ring rank, per Ulysses piece
  int64_t Hq_l, Hkv_l;
  int64_t q_rows;    // rows of the q buffer the kernel reads (per batch)
  // workspace offsets (bytes), SIZE_MAX if unused
  size_t off_qp, off_kp, off_vp, off_ql, off_kl, off_vl, off_oacc, off_lacc, off_opart, off_lpart;
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

RingLayout ring_layout(const usp_ring_args* a) {
  RingLayout r;
  const size_t NONE = SIZE_MAX;
  r.one = a->rank >= 0;
  r.need_perm = a->input_order == 0 && a->impl != USP_RING_BASIC;
  r.copy_in = r.need_perm || a->qkv_packed;
  r.L = a->S / a->ring_degree;
  const int ud = a->ulysses_degree;
  r.Ls = r.L / ud;
  r.Hq_l = a->Hq / ud;
  r.Hkv_l = a->Hkv / ud;
  r.q_rows = r.one ? r.L : a->S;
  r.off_qp = r.off_kp = r.off_vp = r.off_ql = r.off_kl = r.off_vl = NONE;
  r.off_oacc = r.off_lacc = r.off_opart = r.off_lpart = NONE;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t D = (size_t)a->D, B = (size_t)a->B, S = (size_t)a->S;
  if (r.copy_in && ud == 1) {
    r.off_qp = take(B * (size_t)r.q_rows * a->Hq * D * 2);
    r.off_kp = take(B * S * a->Hkv * D * 2);
    r.off_vp = take(B * S * a->Hkv * D * 2);
  }
  if (ud > 1) {
    r.off_ql = take(B * (size_t)r.L * r.Hq_l * D * 2);
    r.off_kl = take(B * S * r.Hkv_l * D * 2);
    r.off_vl = take(B * S * r.Hkv_l * D * 2);
  }
  // accumulate directly into out/lse when they are f32 and already in the
  // order the kernel computes in
  r.out_is_acc = a->out_dtype == USP_DT_F32 && (r.one || !r.need_perm);
  if (!r.out_is_acc) {
    r.off_oacc = take(B * (size_t)r.q_rows * r.Hq_l * D * 4);
    r.off_lacc = take(B * (size_t)r.Hq_l * r.q_rows * 4);
  }
  if (a->merge_mode == 1) {
    r.off_opart = take(B * (size_t)r.q_rows * r.Hq_l * D * 4);
    r.off_lpart = take(B * (size_t)r.Hq_l * r.q_rows * 4);
  }
  r.total = off;
  return r;
}

// Steps 1-2 of the ring (shared by forward and backward): token order
// (rank-major q, or ring rank r's rows; k, v), then the Ulysses seq -> head
// relayout for Ulysses rank u.  Uses the workspace regions of `R`.
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

usp_status stage_ring_inputs(const usp_ring_args* a, const RingLayout& R, char* ws, hipStream_t stream,
                             Staged* out) {
  usp_status st = USP_OK;
  const int N = a->ring_degree, ud = a->ulysses_degree, u = a->ulysses_rank;
  const int64_t B = a->B, S = a->S, D = a->D, L = R.L;
  const int b = a->impl == USP_RING_STRIPE ? a->stripe_block : 1;
  if (ud > 1) {
    // rows in ring order (all pieces of k and v; ring rank r's rows of q),
    // heads of group u, from natural or rank-major order, packed or not
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
    uint16_t* ql = reinterpret_cast<uint16_t*>(ws + R.off_ql);
    uint16_t* kl = reinterpret_cast<uint16_t*>(ws + R.off_kl);
    uint16_t* vl = reinterpret_cast<uint16_t*>(ws + R.off_vl);
    st = launch_permute_strided(kb + u * Hkv_l * D * 2, kl, B, S, S, Hkv_l * D * 2, src_stride_kv,
                                Hkv_l * D * 2, spec(false), stream);
    if (st == USP_OK)
      st = launch_permute_strided(vb + u * Hkv_l * D * 2, vl, B, S, S, Hkv_l * D * 2, src_stride_kv,
                                  Hkv_l * D * 2, spec(false), stream);
    if (st == USP_OK)
      st = launch_permute_strided(qb + u * Hq_l * D * 2, ql, B, S, L, Hq_l * D * 2, src_stride_q,
                                  Hq_l * D * 2, spec(true), stream);
    if (st != USP_OK) return st;
    *out = Staged{ql, kl, vl, L, 0, Hq_l, Hkv_l};
    return USP_OK;
  }

  // 1. token order: rank-major q (or ring rank r's rows), k, v
  const uint16_t* qsrc = static_cast<const uint16_t*>(a->q);
  const uint16_t* ksrc = static_cast<const uint16_t*>(a->k);
  const uint16_t* vsrc = static_cast<const uint16_t*>(a->v);
  int64_t q_batch_rows = S;   // rows between batches in the q buffer
  int64_t q_row_off = 0;      // first row of the rank's q rows
  if (a->qkv_packed) {
    // rows of the packed [B,S,3,H,D] tensor hold q, k, v one after the other:
    // copy each slice out (and into rank-major order when the input is
    // natural-order with a non-basic layout; the rank's rows only for q in
    // one-rank mode)
    const int64_t H = a->Hq, slice = H * D * 2;
    const char* base = static_cast<const char*>(a->q);
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
    uint16_t* qp = reinterpret_cast<uint16_t*>(ws + R.off_qp);
    uint16_t* kp = reinterpret_cast<uint16_t*>(ws + R.off_kp);
    uint16_t* vp = reinterpret_cast<uint16_t*>(ws + R.off_vp);
    st = launch_permute_strided(base + slice, kp, B, S, S, slice, 3 * slice, slice, spec(false), stream);
    if (st == USP_OK)
      st = launch_permute_strided(base + 2 * slice, vp, B, S, S, slice, 3 * slice, slice, spec(false), stream);
    if (st == USP_OK)
      st = launch_permute_strided(base, qp, B, S, R.q_rows, slice, 3 * slice, slice, spec(R.one), stream);
    if (st != USP_OK) return st;
    qsrc = qp;
    ksrc = kp;
    vsrc = vp;
    q_batch_rows = R.q_rows;
  } else if (R.need_perm) {
    uint16_t* qp = reinterpret_cast<uint16_t*>(ws + R.off_qp);
    uint16_t* kp = reinterpret_cast<uint16_t*>(ws + R.off_kp);
    uint16_t* vp = reinterpret_cast<uint16_t*>(ws + R.off_vp);
    st = usp_permute(a->k, kp, B, S, a->Hkv * D, USP_DT_BF16, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st == USP_OK)
      st = usp_permute(a->v, vp, B, S, a->Hkv * D, USP_DT_BF16, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st == USP_OK)
      st = usp_permute(a->q, qp, B, S, a->Hq * D, USP_DT_BF16, (usp_ring_impl)a->impl, N, 1, b,
                       R.one ? a->rank : -1, 0, stream);
    if (st != USP_OK) return st;
    qsrc = qp;
    ksrc = kp;
    vsrc = vp;
    q_batch_rows = R.q_rows;
  } else if (R.one) {
    q_row_off = (int64_t)a->rank * L;
  }

  *out = Staged{qsrc, ksrc, vsrc, q_batch_rows, q_row_off, a->Hq, a->Hkv};
  return USP_OK;
}

// Workspace of the backward ring: the forward's staging regions (permuted /
// relayouted q, k, v), delta, and -- when the caller's tensors are in
// natural order but the ring runs rank-major (all ranks, non-basic layout)
// -- rank-major copies of dout and LSE and rank-major f32 gradient
// accumulators that are un-permuted into the outputs at the end.
struct RingBwdLayout {
  RingLayout base;        // only the staging offsets of the forward layout are used
  bool reorder;           // all ranks, natural-order tensors, non-basic layout
  size_t off_delta, off_delta_nat, off_dop, off_lsep, off_dq, off_dk, off_dv;
  size_t total;
};

RingBwdLayout ring_bwd_layout(const usp_ring_args* a) {
  RingBwdLayout r;
  const size_t NONE = SIZE_MAX;
  r.base = ring_layout(a);
  RingLayout& R = r.base;
  const size_t D = (size_t)a->D, B = (size_t)a->B, S = (size_t)a->S;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  // the staging regions, as the forward lays them out; no forward accumulators
  R.off_qp = R.off_kp = R.off_vp = R.off_ql = R.off_kl = R.off_vl = NONE;
  R.off_oacc = R.off_lacc = R.off_opart = R.off_lpart = NONE;
  if (R.copy_in && a->ulysses_degree == 1) {
    R.off_qp = take(B * (size_t)R.q_rows * a->Hq * D * 2);
    R.off_kp = take(B * S * a->Hkv * D * 2);
    R.off_vp = take(B * S * a->Hkv * D * 2);
  }
  if (a->ulysses_degree > 1) {
    R.off_ql = take(B * (size_t)R.L * R.Hq_l * D * 2);
    R.off_kl = take(B * S * R.Hkv_l * D * 2);
    R.off_vl = take(B * S * R.Hkv_l * D * 2);
  }
  r.reorder = R.need_perm && !R.one;
  r.off_delta = take(B * (size_t)R.Hq_l * R.q_rows * 4);
  r.off_delta_nat = r.off_dop = r.off_lsep = r.off_dq = r.off_dk = r.off_dv = NONE;
  if (r.reorder) {
    r.off_delta_nat = take(B * (size_t)a->Hq * S * 4);
    r.off_dop = take(B * S * a->Hq * D * 2);
    r.off_lsep = take(B * (size_t)a->Hq * S * 4);
    r.off_dq = take(B * S * a->Hq * D * 4);
    r.off_dk = take(B * S * a->Hkv * D * 4);
    r.off_dv = take(B * S * a->Hkv * D * 4);
  }
  R.total = off;
  r.total = off;
  return r;
}

}  // namespace

size_t usp_ring_fwd_workspace_size(const usp_ring_args* a) {
  if (check_ring_args(a) != USP_OK) return 0;
  return ring_layout(a).total;
}

usp_status usp_ring_fwd(const usp_ring_args* a, void* workspace, size_t ws_bytes, void* stream_) {
  usp_status st = check_ring_args(a);
  if (st != USP_OK) return st;
  const RingLayout R = ring_layout(a);
  USP_CHECK(R.total == 0 || (workspace && ws_bytes >= R.total), USP_ERR_WORKSPACE,
            "workspace of %zu bytes needed, %zu given", R.total, workspace ? ws_bytes : (size_t)0);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t stream = as_stream(stream_);
  char* ws = static_cast<char*>(workspace);
  const int N = a->ring_degree;
  const int64_t B = a->B, S = a->S, D = a->D, L = R.L;
  const int b = a->impl == USP_RING_STRIPE ? a->stripe_block : 1;

  Staged stg;
  st = stage_ring_inputs(a, R, ws, stream, &stg);
  if (st != USP_OK) return st;
  const uint16_t* qsrc = stg.q;
  const uint16_t* ksrc = stg.k;
  const uint16_t* vsrc = stg.v;
  const int64_t q_batch_rows = stg.q_batch_rows, q_row_off = stg.q_row_off;
  const int64_t Hq_l = stg.Hq_l, Hkv_l = stg.Hkv_l;

  // 3. ring steps
  float* oacc = R.out_is_acc ? static_cast<float*>(a->out) : reinterpret_cast<float*>(ws + R.off_oacc);
  float* lacc = R.out_is_acc ? a->lse : reinterpret_cast<float*>(ws + R.off_lacc);
  float* opart = a->merge_mode ? reinterpret_cast<float*>(ws + R.off_opart) : nullptr;
  float* lpart = a->merge_mode ? reinterpret_cast<float*>(ws + R.off_lpart) : nullptr;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  st = ring_mods(a, Hq_l, scale, &mods);
  if (st != USP_OK) return st;

  MaskSpec ms;
  ms.causal = a->causal ? 1 : 0;
  ms.window = a->window;
  ms.n_sink = a->n_sink;
  ms.nseq = a->cu_seqlens_host ? a->nseq : 0;
  ms.S = (int32_t)S;
  usp_posmap pm{a->impl, N, 0, b, S};
  const PosMap base_map = make_map(pm);

  const int32_t tm = choose_tile_m(base_map);
  for (int s = 0; s < N; ++s) {
    const int acc_flag = (s > 0 && a->merge_mode == 0) ? 1 : 0;
    const std::string key = "ring|" + map_key(base_map) + "|" + mask_key(ms) + "|" +
                            cu_key(ms.nseq ? a->cu_seqlens_host : nullptr, a->nseq) + "|r" +
                            std::to_string(a->rank) + "|s" + std::to_string(s) + "|a" + std::to_string(acc_flag) +
                            "|m" + std::to_string(tm);
    DevicePlan dp;
    st = device_plan(key, [&](Plan& plan) {
      const int i0 = R.one ? a->rank : 0, i1 = R.one ? a->rank + 1 : N;
      for (int i = i0; i < i1; ++i) {
        const int j = ((i - s) % N + N) % N;
        BlockSpec blk;
        blk.qmap = base_map;
        blk.qmap.rank = i;
        blk.kmap = base_map;
        blk.kmap.rank = j;
        blk.Lq = (int32_t)L;
        blk.Lk = (int32_t)L;
        blk.q_row_base = R.one ? 0 : (int32_t)(i * L);
        blk.k_row_base = (int32_t)(j * L);
        blk.tile_m = tm;
        plan_block(blk, ms, a->cu_seqlens_host, acc_flag, plan);
      }
    }, &dp);
    if (st != USP_OK) return st;

    AttnParams p{};
    p.q = qsrc + q_row_off * Hq_l * D;
    p.k = ksrc;
    p.v = vsrc;
    const bool to_part = a->merge_mode == 1 && s > 0;
    p.out = to_part ? static_cast<void*>(opart) : static_cast<void*>(oacc);
    p.lse = to_part ? lpart : lacc;
    p.items = dp.items;
    p.runs = dp.runs;
    p.cu_seqlens = ms.nseq ? a->cu_seqlens_dev : nullptr;
    p.q_batch_stride = q_batch_rows * Hq_l * D;
    p.o_batch_stride = R.q_rows * Hq_l * D;
    p.kv_batch_stride = S * Hkv_l * D;
    p.Lq_buf = (int32_t)R.q_rows;
    p.n_items = dp.n_items;
    p.B = (int32_t)B;
    p.Hq = (int32_t)Hq_l;
    p.Hkv = (int32_t)Hkv_l;
    p.out_f32 = 1;
    p.accumulate = acc_flag;
    p.tile_m = tm;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.qmap = base_map;
    p.kmap = base_map;
    p.mask = ms;
    p.mods = mods;
    st = launch_attn_fwd(p, (int)D, stream);
    if (st != USP_OK) return st;
    if (to_part) {
      st = launch_lse_merge(oacc, lacc, opart, lpart, B, R.q_rows, Hq_l, D, 0, R.q_rows, stream);
      if (st != USP_OK) return st;
    }
  }

  // 4. finalize: dtype and order of the outputs
  if (!R.out_is_acc) {
    GatherSpec gs{};
    gs.impl = R.need_perm && !R.one ? a->impl : USP_RING_BASIC;
    gs.N = R.need_perm && !R.one ? N : 1;
    gs.ud = 1;
    gs.b = R.need_perm && !R.one ? b : 1;
    gs.g = 0;
    gs.L = (int32_t)(R.need_perm && !R.one ? L : R.q_rows);
    gs.S = (int32_t)R.q_rows;
    gs.kind = G_UNPERMUTE;
    if (a->out_dtype == USP_DT_F32) {
      st = launch_permute(oacc, a->out, B, R.q_rows, R.q_rows, Hq_l * D * 4, gs, stream);
    } else {
      st = launch_permute_f32_to_bf16(oacc, static_cast<uint16_t*>(a->out), B, R.q_rows, R.q_rows,
                                      Hq_l * D, gs, stream);
    }
    if (st != USP_OK) return st;
    st = launch_permute(lacc, a->lse, B * Hq_l, R.q_rows, R.q_rows, 4, gs, stream);
    if (st != USP_OK) return st;
  }
  return USP_OK;
}

size_t usp_ring_bwd_workspace_size(const usp_ring_bwd_args* a) {
  if (!a || check_ring_args(&a->fwd) != USP_OK) return 0;
  return ring_bwd_layout(&a->fwd).total;
}

usp_status usp_ring_bwd(const usp_ring_bwd_args* ba, void* workspace, size_t ws_bytes, void* stream_) {
  USP_CHECK(ba, USP_ERR_INVALID_ARG, "null args");
  const usp_ring_args* a = &ba->fwd;
  usp_status st = check_ring_args(a);
  if (st != USP_OK) return st;
  USP_CHECK(ba->dout && ba->dq && ba->dk && ba->dv, USP_ERR_INVALID_ARG, "null gradient pointer");
  const RingBwdLayout RB = ring_bwd_layout(a);
  USP_CHECK(RB.base.L * RB.base.Hq_l * a->D * 2 < ((int64_t)1 << 31) &&
                RB.base.q_rows * RB.base.Hq_l * 4 < ((int64_t)1 << 31),
            USP_ERR_UNSUPPORTED, "one ring rank's q rows and one batch row of LSE must be under 2 GiB "
            "(32-bit tile offsets)");
  const RingLayout& R = RB.base;
  USP_CHECK(workspace && ws_bytes >= RB.total, USP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
            RB.total, workspace ? ws_bytes : (size_t)0);
  USP_CHECK(((uintptr_t)workspace & 255) == 0, USP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t stream = as_stream(stream_);
  char* ws = static_cast<char*>(workspace);
  const int N = a->ring_degree;
  const int64_t B = a->B, S = a->S, D = a->D, L = R.L;
  const int b = a->impl == USP_RING_STRIPE ? a->stripe_block : 1;

  // 1-2. the forward's staging of q, k, v
  Staged stg;
  st = stage_ring_inputs(a, R, ws, stream, &stg);
  if (st != USP_OK) return st;
  const int64_t Hq_l = stg.Hq_l, Hkv_l = stg.Hkv_l;

  // delta = rowsum(dO * O) over the rows the ring visits, in their order;
  // dout and LSE in that order too
  float* delta = reinterpret_cast<float*>(ws + RB.off_delta);
  const uint16_t* dout = static_cast<const uint16_t*>(ba->dout);
  const float* lse = a->lse;
  const usp_dtype odt = (usp_dtype)a->out_dtype;
  if (RB.reorder) {
    float* dn = reinterpret_cast<float*>(ws + RB.off_delta_nat);
    uint16_t* dop = reinterpret_cast<uint16_t*>(ws + RB.off_dop);
    float* lsep = reinterpret_cast<float*>(ws + RB.off_lsep);
    st = launch_bwd_delta(a->out, odt == USP_DT_F32, dout, dn, B, S, a->Hq, D, stream);
    if (st == USP_OK)
      st = usp_permute(dn, delta, B * a->Hq, S, 1, USP_DT_F32, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st == USP_OK)
      st = usp_permute(a->lse, lsep, B * a->Hq, S, 1, USP_DT_F32, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st == USP_OK)
      st = usp_permute(ba->dout, dop, B, S, a->Hq * D, USP_DT_BF16, (usp_ring_impl)a->impl, N, 1, b, -1, 0, stream);
    if (st != USP_OK) return st;
    dout = dop;
    lse = lsep;
  } else {
    st = launch_bwd_delta(a->out, odt == USP_DT_F32, dout, delta, B, R.q_rows, Hq_l, D, stream);
    if (st != USP_OK) return st;
  }

  // gradient accumulators
  float* dq = RB.reorder ? reinterpret_cast<float*>(ws + RB.off_dq) : ba->dq;
  float* dk = RB.reorder ? reinterpret_cast<float*>(ws + RB.off_dk) : ba->dk;
  float* dv = RB.reorder ? reinterpret_cast<float*>(ws + RB.off_dv) : ba->dv;
  st = launch_fill_zero(dq, B * R.q_rows * Hq_l * D, stream);
  if (st == USP_OK) st = launch_fill_zero(dk, B * S * Hkv_l * D, stream);
  if (st == USP_OK) st = launch_fill_zero(dv, B * S * Hkv_l * D, stream);
  if (st != USP_OK) return st;

  // 3. ring steps: host i meets KV piece j = (i - s) mod N; one launch per
  // kernel per step covers every host of the step (their dq rows and dk / dv
  // pieces are disjoint)
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)D);
  ScoreMods mods;
  st = ring_mods(a, Hq_l, scale, &mods);
  if (st != USP_OK) return st;
  MaskSpec ms;
  ms.causal = a->causal ? 1 : 0;
  ms.window = a->window;
  ms.n_sink = a->n_sink;
  ms.nseq = a->cu_seqlens_host ? a->nseq : 0;
  ms.S = (int32_t)S;
  usp_posmap pm{a->impl, N, 0, b, S};
  const PosMap base_map = make_map(pm);
  for (int s = 0; s < N; ++s) {
    const std::string key = map_key(base_map) + "|" + mask_key(ms) + "|" +
                            cu_key(ms.nseq ? a->cu_seqlens_host : nullptr, a->nseq) + "|r" +
                            std::to_string(a->rank) + "|s" + std::to_string(s);
    auto blocks = [&](auto&& add) {
      const int i0 = R.one ? a->rank : 0, i1 = R.one ? a->rank + 1 : N;
      for (int i = i0; i < i1; ++i) {
        const int j = ((i - s) % N + N) % N;
        BlockSpec blk;
        blk.qmap = base_map;
        blk.qmap.rank = i;
        blk.kmap = base_map;
        blk.kmap.rank = j;
        blk.Lq = (int32_t)L;
        blk.Lk = (int32_t)L;
        blk.q_row_base = R.one ? 0 : (int32_t)(i * L);
        blk.k_row_base = (int32_t)(j * L);
        blk.tile_m = kBwdTileM;
        add(blk);
      }
    };
    DevicePlan dpq, dpk;
    st = device_plan("rbq|" + key, [&](Plan& plan) {
      blocks([&](const BlockSpec& blk) { plan_block(blk, ms, a->cu_seqlens_host, 1, plan); });
    }, &dpq);
    if (st != USP_OK) return st;
    st = device_plan("rbk|" + key, [&](Plan& plan) {
      blocks([&](const BlockSpec& blk) {
        plan_block_kv(blk, ms, a->cu_seqlens_host, kBwdTileK, kBwdTileQ, plan);
      });
    }, &dpk);
    if (st != USP_OK) return st;

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
    p.cu_seqlens = ms.nseq ? a->cu_seqlens_dev : nullptr;
    p.q_batch_stride = stg.q_batch_rows * Hq_l * D;
    p.g_batch_stride = R.q_rows * Hq_l * D;
    p.kv_batch_stride = S * Hkv_l * D;
    p.Lq_buf = (int32_t)R.q_rows;
    p.B = (int32_t)B;
    p.Hq = (int32_t)Hq_l;
    p.Hkv = (int32_t)Hkv_l;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.qmap = base_map;
    p.kmap = base_map;
    p.mask = ms;
    p.mods = mods;
    BwdParams pq = p, pk = p;
    pq.items = dpq.items;
    pq.runs = dpq.runs;
    pq.n_items = dpq.n_items;
    pk.items = dpk.items;
    pk.runs = dpk.runs;
    pk.n_items = dpk.n_items;
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
