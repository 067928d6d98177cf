// Internal definitions shared by the host planner, the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "usp.h"  // include/ is on the include path

namespace usp {

// Internal position-map kind: the three ring layouts plus an affine map
// (p = t + offset) used for the explicit mask classes.
enum MapKind : int32_t { MAP_BASIC = 0, MAP_ZIGZAG = 1, MAP_STRIPE = 2, MAP_AFFINE = 3 };

// Global position of local row t of one virtual rank.
//   basic : rank*L + t
//   zigzag: chunk `rank` then chunk 2N-1-rank, c = L/2 rows each
//   stripe: ((t/b)*N + rank)*b + t%b
//   affine: t + offset
struct PosMap {
  int32_t kind;
  int32_t N;
  int32_t rank;
  int32_t b;
  int32_t L;       // rows per rank
  int32_t offset;  // affine only
};

__host__ __device__ inline int32_t position(const PosMap& m, int32_t t) {
  switch (m.kind) {
    case MAP_BASIC:
      return m.rank * m.L + t;
    case MAP_ZIGZAG: {
      const int32_t c = m.L >> 1;
      return t < c ? m.rank * c + t : (2 * m.N - 1 - m.rank) * c + (t - c);
    }
    case MAP_STRIPE:
      return ((t / m.b) * m.N + m.rank) * m.b + t % m.b;
    default:
      return t + m.offset;
  }
}

// Load with the non-temporal cache hint, for data a kernel reads exactly once
// and nothing reads again soon (row copies, the LSE merge, the row sums of O
// and dO: 0.068 against 0.094 ms on a 402 MB input).
template <class T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

// Smallest local row t with position(m, t) >= P, for a row t_ref of the
// same monotone piece (positions increase with t across a whole basic,
// stripe or affine rank, and within each chunk of a zigzag rank, where
// they are consecutive).  Stripe: the rank holds blocks j*N + rank (block
// j at rows j*b ..); P in one of them maps to its row, otherwise to the
// first row of the rank's next block.  Exact for every t of the piece;
// callers clamp to the rows they hold.
__host__ __device__ inline int32_t first_row_at_least(const PosMap& m, int32_t t_ref, int32_t P) {
  if (m.kind == MAP_STRIPE) {
    // floor divisions of possibly negative numerators by b, N >= 1
    auto fdiv = [](int32_t a, int32_t d) {
      const int32_t q = a / d;
      return (a % d != 0 && a < 0) ? q - 1 : q;
    };
    const int32_t beta = fdiv(P, m.b);
    const int32_t o = P - beta * m.b;
    const int32_t j = fdiv(beta - m.rank, m.N);
    return (j * m.N + m.rank == beta) ? j * m.b + o : (j + 1) * m.b;
  }
  return t_ref + (P - position(m, t_ref));
}

// Monotone pieces of a rank's local rows: positions increase with t inside
// each piece.  Zigzag has two (its two chunks); the others one.
__host__ __device__ inline int monotone_segments(const PosMap& m, int32_t seg_lo[2], int32_t seg_hi[2]) {
  if (m.kind == MAP_ZIGZAG) {
    seg_lo[0] = 0;
    seg_hi[0] = m.L / 2;
    seg_lo[1] = m.L / 2;
    seg_hi[1] = m.L;
    return 2;
  }
  seg_lo[0] = 0;
  seg_hi[0] = m.L;
  return 1;
}

// Mask parameters on global positions (shared by planner and kernel).
struct MaskSpec {
  int32_t causal;   // causal (implied when window > 0)
  int32_t window;   // <= 0: none
  int32_t n_sink;
  int32_t nseq;     // 0: not varlen (one sequence [0, S))
  int32_t S;        // total positions (non-varlen sequence end)
};

// One work item: BM query rows of one rank against one rank's KV rows.
struct WorkItem {
  int32_t q_row0;     // first query row in the q buffer
  int32_t t0;         // local row index of q_row0 within its rank
  int32_t q_rows;     // valid rows (<= BM)
  int32_t q_rank;
  int32_t k_row0;     // row of local key 0 of the KV rank in the k/v buffers
  int32_t k_rank;
  int32_t run_begin;  // runs [run_begin, run_end)
  int32_t run_end;
};
static_assert(sizeof(WorkItem) == 32, "WorkItem layout");

struct Run {
  int32_t k_begin;    // local key rows [k_begin, k_end)
  int32_t k_end;
  int32_t full;       // 1: every key visible to every row of the item
  int32_t pad;
};
static_assert(sizeof(Run) == 16, "Run layout");

// Key granularity of the planner's full runs (their lengths are multiples
// of it) and the largest key tile of the attention kernel (128 keys; 256
// query rows per workgroup, 8 waves of 32 rows).
constexpr int kTileN = 128;

// Query rows per forward workgroup: 256 (8 waves), or 128 (4 waves, two
// workgroups per CU) under a window mask, whose short items are dominated by
// per-item fixed costs that a second resident workgroup overlaps.
inline int32_t choose_tile_m(int32_t window) { return window > 0 ? 128 : 256; }

// Host-built plan of one launch (the inspection calls return it).
struct Plan {
  std::vector<WorkItem> items;
  std::vector<Run> runs;
};

// Score modifiers of the attention call, in the kernels' raw-score units
// (scores before softmax_scale): with softcap c > 0 the scaled score s*scale
// becomes c * tanh(s*scale / c), i.e. the raw score becomes
// a - 2a / (exp2(s * b2) + 1) with a = c / scale and b2 = 2 * scale *
// log2(e) / c; ALiBi subtracts slope_h * |p_q - p_k| / scale.
struct ScoreMods {
  float a;               // softcap / scale (0: no softcap)
  float b2;              // 2 * scale * log2(e) / softcap
  float inv_scale;       // 1 / scale
  const float* alibi;    // slope per query head of this call's heads, or nullptr
};

// ALiBi distances are formed in f32 from row indices, with the stripe
// layout's block index taken as floor((t + 0.5) / b): exact while positions
// stay below 2^22.
constexpr int64_t kMaxAlibiPositions = int64_t(1) << 22;

// Kernel variant of a call's score modifiers: bit 0 softcap, bit 1 ALiBi.
inline int mods_variant(const ScoreMods& m) { return (m.a > 0.f ? 1 : 0) | (m.alibi ? 2 : 0); }

// Attention kernel parameters (passed by value).
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  float* lse;
  const WorkItem* items;
  const Run* runs;
  const int32_t* cu_seqlens;
  int64_t q_batch_stride;   // elements between batch rows of q
  int64_t o_batch_stride;   // elements between batch rows of out
  int64_t kv_batch_stride;  // elements between batch rows of k / v
  int32_t Lq_buf;           // rows per batch of q / out / lse
  int32_t o_heads;          // heads per row of out and per batch row of lse (Hq, or
                            // all heads when this call writes one head group)
  int32_t o_head0;          // first head of this call's group in out / lse
  int32_t n_items;
  int32_t B;
  int32_t Hq;
  int32_t Hkv;
  int32_t out_f32;
  int32_t accumulate;
  int32_t tile_m;           // query rows per item (256)
  float scale_log2;         // softmax_scale * log2(e)
  PosMap qmap;              // rank field overridden per item
  PosMap kmap;
  MaskSpec mask;
  ScoreMods mods;
};

// Launchers (return USP_ERR_HIP on launch failure).
usp_status launch_attn_fwd(const AttnParams& p, int D, hipStream_t stream);
// Backward kernels' parameters (passed by value): the dQ kernel reads the
// forward plan (tile_m = kBwdTileM), the dK / dV kernel the transposed plan
// (tile_k = kBwdTileK, query granularity kBwdTileQ).
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;          // [B, Hq, Lq_buf]
  const float* delta;        // [B, Hq, Lq_buf]
  float* dq;                 // [B, Lq, Hq, D], accumulated into
  float* dk;                 // [B, Lk, Hkv, D], accumulated into
  float* dv;
  const WorkItem* items;
  const Run* runs;
  const int32_t* cu_seqlens;
  int64_t q_batch_stride;    // elements between batch rows of q
  int64_t g_batch_stride;    // elements between batch rows of dout / dq
  int64_t kv_batch_stride;   // elements between batch rows of k / v / dk / dv
  int32_t Lq_buf;
  int32_t n_items;
  int32_t B;
  int32_t Hq;
  int32_t Hkv;
  float scale;               // softmax_scale
  float scale_log2;          // softmax_scale * log2(e)
  int32_t overwrite;         // 1: the launch stores its gradient rows instead of adding to
                             // them (a planned item without runs stores zeros)
  PosMap qmap;
  PosMap kmap;
  MaskSpec mask;
  ScoreMods mods;
};
constexpr int kBwdTileM = 128;  // query rows per dQ workgroup
constexpr int kBwdTileK = 128;  // keys per dK / dV workgroup
constexpr int kBwdTileQ = 64;   // query rows per dK / dV iteration
usp_status launch_bwd(const BwdParams& pq, const BwdParams& pkv, int D, hipStream_t stream);
// Enqueues the dQ kernel alone (no error check; launch_bwd checks).
void launch_bwd_dq(const BwdParams& p, int D, unsigned grid, hipStream_t stream);

// Decode over a KV cache, split into pieces of split_keys keys (a multiple
// of 32); one wave per (piece, batch row, KV head).
struct DecodeParams {
  const uint16_t* q;       // [B, Lq, Hq, D]
  const uint16_t* k;       // [B, S, Hkv, D]
  const uint16_t* v;
  const int32_t* kv_lens;  // [B] valid cache length per row, or nullptr (all S)
  float* out_part;         // [n_split, B, Lq, Hq, D]
  float* lse_part;         // [n_split, B, Hq, Lq]
  int32_t B, Lq, S, Hq, Hkv;
  int32_t n_split, split_keys;
  int32_t window, n_sink;
  float scale_log2;        // softmax_scale * log2(e)
  ScoreMods mods;          // slopes indexed by query head
};
usp_status launch_decode_split(const DecodeParams& p, int D, hipStream_t stream);
usp_status launch_decode_merge(float* out_part, float* lse_part, int32_t n_split, int32_t B, int32_t Lq,
                               int32_t Hq, int D, void* out, int out_f32, float* lse, hipStream_t stream);
usp_status launch_bwd_delta(const void* out, int out_f32, const uint16_t* dout, float* delta, int64_t B,
                            int64_t L, int64_t H, int64_t D, hipStream_t stream);

// Generic row gather: out row i (of n_out rows per outer slice) copies
// row src(i) of `in`; see permute.hip for the index kinds.
struct GatherSpec {
  int32_t kind;           // GatherKind
  int32_t impl;
  int32_t N;
  int32_t ud;
  int32_t b;
  int32_t g;              // extract: global rank
  int32_t L;              // rows per ring rank
  int32_t S;              // rows of the natural tensor
};
enum GatherKind : int32_t { G_PERMUTE = 0, G_UNPERMUTE = 1, G_EXTRACT = 2, G_INSERT = 3 };
usp_status launch_permute(const void* in, void* out, int64_t outer, int64_t S_in, int64_t S_out,
                          int64_t row_bytes, const GatherSpec& gs, hipStream_t stream);
// Same with row strides (bytes between consecutive rows) of the input and
// the output: copies row_bytes of each row (a slice of a packed row when the
// stride is larger).
usp_status launch_permute_strided(const void* in, void* out, int64_t outer, int64_t S_in, int64_t S_out,
                                  int64_t row_bytes, int64_t in_row_stride, int64_t out_row_stride,
                                  const GatherSpec& gs, hipStream_t stream);
// Same as launch_permute with fp32 -> bf16 conversion (row_elems fp32 in, bf16
// out); output rows are out_row_stride bf16 apart (row_elems when dense).
usp_status launch_permute_f32_to_bf16(const float* in, uint16_t* out, int64_t outer, int64_t S_in,
                                      int64_t S_out, int64_t row_elems, int64_t out_row_stride,
                                      const GatherSpec& gs, hipStream_t stream);
usp_status launch_relayout(void* const* shards, void* local, int64_t B, int64_t Ls, int64_t H,
                           int64_t D, int64_t elem_bytes, int ud, int u, int direction,
                           hipStream_t stream);
// Same with explicit batch strides (in rows) of the shards and the local tensor.
usp_status launch_relayout_strided(void* const* shards, void* local, int64_t B, int64_t Ls,
                                   int64_t H, int64_t D, int64_t elem_bytes, int ud, int u,
                                   int direction, int64_t shard_batch_rows,
                                   int64_t local_batch_rows, hipStream_t stream);
usp_status launch_lse_merge(float* out_acc, float* lse_acc, const float* out_part,
                            const float* lse_part, int64_t B, int64_t L, int64_t H, int64_t D,
                            int64_t row_begin, int64_t row_end, hipStream_t stream);

void set_error(const char* fmt, ...);

// Kernel classes of the timing facility (usp_timing_*).
enum KernelClass : int {
  K_ATTN = 0,
  K_PERMUTE = 1,
  K_RELAYOUT = 2,
  K_MERGE = 3,
  K_BWD_DQ = 4,
  K_BWD_DKDV = 5,
  K_BWD_DELTA = 6,
  K_DECODE = 7,
  K_DECODE_MERGE = 8,
  K_PLAN = 9
};

// Brackets one launch with hipEvents on `stream` while timing is enabled.
class TimingScope {
 public:
  TimingScope(int cls, hipStream_t stream);
  ~TimingScope();
  TimingScope(const TimingScope&) = delete;
  TimingScope& operator=(const TimingScope&) = delete;

 private:
  int cls_;
  hipStream_t stream_;
  void* start_ = nullptr;
  void* stop_ = nullptr;
  bool active_ = false;
};

}  // namespace usp
