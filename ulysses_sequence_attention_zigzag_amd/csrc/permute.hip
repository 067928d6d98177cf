// Row-copy kernels: ring-layout token permutation (gather / scatter of whole
// rows along the sequence axis) and the Ulysses seq <-> head relayout.
//
// Both are pure data movement, bound by HBM bandwidth.  A row (all heads x
// head_dim of one token) is contiguous in source and destination, so each
// row is moved with 16-byte vector loads/stores by a group of TPR threads
// (a power of two, up to the 256 threads of the workgroup); the index
// arithmetic (one division per row) is paid per row, not per element.

#include <hip/hip_runtime.h>

#include "usp_internal.h"

namespace usp {
namespace {

template <int BYTES> struct UnitT;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <> struct UnitT<16> { using type = u32x4; };
template <> struct UnitT<8> { using type = u32x2; };
template <> struct UnitT<4> { using type = uint32_t; };
template <> struct UnitT<2> { using type = uint16_t; };

// Position of task row i under the gather spec: the natural-order row that
// rank-major index i (permute) or extract row i (extract) corresponds to.
__device__ __forceinline__ int32_t mapped_row(const GatherSpec& gs, int32_t i) {
  PosMap m;
  m.kind = gs.impl;
  m.N = gs.N;
  m.b = gs.b;
  m.L = gs.L;
  m.offset = 0;
  int32_t t;
  if (gs.kind == G_EXTRACT || gs.kind == G_INSERT) {
    const int32_t Ls = gs.L / gs.ud;
    m.rank = gs.g / gs.ud;
    t = (gs.g % gs.ud) * Ls + i;
  } else {
    m.rank = i / gs.L;
    t = i - m.rank * gs.L;
  }
  return position(m, t);
}

// Rows are processed by groups of (1 << log_tpr) threads; each block covers
// (256 >> log_tpr) task rows.  Gather kinds read row map(i) and write row i;
// scatter kinds read row i and write row map(i).
// A row is units_per_row units; consecutive rows sit in_stride / out_stride
// units apart (equal to units_per_row for dense tensors; larger to read one
// slice of each row of a packed tensor).
template <int UB>
__global__ __launch_bounds__(256) void permute_rows_kernel(const char* __restrict__ in,
                                                           char* __restrict__ out, int64_t n_task_rows,
                                                           int32_t S_task, int64_t S_in, int64_t S_out,
                                                           int32_t units_per_row, int64_t in_stride,
                                                           int64_t out_stride, int32_t log_tpr,
                                                           GatherSpec gs) {
  using U = typename UnitT<UB>::type;
  const int32_t tpr = 1 << log_tpr;
  const int64_t row = (int64_t)blockIdx.x * (256 >> log_tpr) + (threadIdx.x >> log_tpr);
  if (row >= n_task_rows) return;
  const int32_t lane = threadIdx.x & (tpr - 1);
  const int64_t o = row / S_task;
  const int32_t i = (int32_t)(row - o * S_task);
  const int32_t m = mapped_row(gs, i);
  const bool scatter = gs.kind == G_UNPERMUTE || gs.kind == G_INSERT;
  const int64_t src_row = o * S_in + (scatter ? i : m);
  const int64_t dst_row = o * S_out + (scatter ? m : i);
  const U* src = reinterpret_cast<const U*>(in) + src_row * in_stride;
  U* dst = reinterpret_cast<U*>(out) + dst_row * out_stride;
    // loads with the non-temporal hint, plain stores (the hint on the stores
  // too made the copies slower)
  for (int32_t c = lane; c < units_per_row; c += tpr) dst[c] = ld_nt(src + c);
}

// fp32 rows in, bf16 rows out (round to nearest even), same row mapping.
// Consecutive output rows sit out_stride_elems bf16 apart (the row length
// for a dense output; larger to write one head group of wider rows).
__global__ __launch_bounds__(256) void permute_rows_f32_bf16_kernel(
    const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n_task_rows, int32_t S_task,
    int64_t S_in, int64_t S_out, int32_t quads_per_row, int64_t out_stride_elems, int32_t log_tpr,
    GatherSpec gs) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int32_t tpr = 1 << log_tpr;
  const int64_t row = (int64_t)blockIdx.x * (256 >> log_tpr) + (threadIdx.x >> log_tpr);
  if (row >= n_task_rows) return;
  const int32_t lane = threadIdx.x & (tpr - 1);
  const int64_t o = row / S_task;
  const int32_t i = (int32_t)(row - o * S_task);
  const int32_t m = mapped_row(gs, i);
  const bool scatter = gs.kind == G_UNPERMUTE || gs.kind == G_INSERT;
  const int64_t src_row = o * S_in + (scatter ? i : m);
  const int64_t dst_row = o * S_out + (scatter ? m : i);
  const float4* src = reinterpret_cast<const float4*>(in + src_row * quads_per_row * 4);
  uint2* dst = reinterpret_cast<uint2*>(out + dst_row * out_stride_elems);
  for (int32_t c = lane; c < quads_per_row; c += tpr) {
    const float4 x = src[c];
    const bf16x2 lo = __builtin_convertvector((f32x2){x.x, x.y}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){x.z, x.w}, bf16x2);
    dst[c] = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  }
}

struct ShardPtrs {
  char* p[8];
};

// Ulysses relayout.  Task row = (b, u', s) of the local tensor; the row of
// Hg*D elements is contiguous on both sides.
template <int UB>
__global__ __launch_bounds__(256) void relayout_kernel(ShardPtrs shards, char* __restrict__ local,
                                                       int64_t n_task_rows, int32_t Ls, int32_t ud,
                                                       int32_t u, int64_t shard_row_bytes,
                                                       int64_t local_row_bytes, int32_t units_per_row,
                                                       int32_t log_tpr, int32_t direction) {
  using U = typename UnitT<UB>::type;
  const int32_t tpr = 1 << log_tpr;
  const int64_t row = (int64_t)blockIdx.x * (256 >> log_tpr) + (threadIdx.x >> log_tpr);
  if (row >= n_task_rows) return;
  const int32_t lane = threadIdx.x & (tpr - 1);
  const int64_t per_b = (int64_t)ud * Ls;
  const int64_t bi = row / per_b;
  const int32_t r = (int32_t)(row - bi * per_b);  // u' * Ls + s
  const int32_t up = r / Ls;
  const int32_t s = r - up * Ls;
  char* shard_row = shards.p[up] + (bi * Ls + s) * shard_row_bytes + (int64_t)u * units_per_row * UB;
  char* local_row = local + row * local_row_bytes;
  const U* src = reinterpret_cast<const U*>(direction == 0 ? shard_row : local_row);
  U* dst = reinterpret_cast<U*>(direction == 0 ? local_row : shard_row);
    // loads with the non-temporal hint, plain stores (the hint on the stores
  // too made the copies slower)
  for (int32_t c = lane; c < units_per_row; c += tpr) dst[c] = ld_nt(src + c);
}

int unit_bytes_for(int64_t row_bytes, uintptr_t a, uintptr_t b) {
  for (int ub = 16; ub >= 2; ub >>= 1)
    if (row_bytes % ub == 0 && a % ub == 0 && b % ub == 0) return ub;
  return 1;
}

int log_tpr_for(int64_t units) {
  int l = 0;
  while ((1 << l) < units && l < 8) ++l;
  return l;
}

usp_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s launch failed: %s", what, hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace

usp_status launch_permute(const void* in, void* out, int64_t outer, int64_t S_in, int64_t S_out,
                          int64_t row_bytes, const GatherSpec& gs, hipStream_t stream) {
  return launch_permute_strided(in, out, outer, S_in, S_out, row_bytes, row_bytes, row_bytes, gs, stream);
}

usp_status launch_permute_strided(const void* in, void* out, int64_t outer, int64_t S_in, int64_t S_out,
                                  int64_t row_bytes, int64_t in_row_stride, int64_t out_row_stride,
                                  const GatherSpec& gs, hipStream_t stream) {
  const bool extract_like = gs.kind == G_EXTRACT || gs.kind == G_INSERT;
  const int64_t S_task = extract_like ? (int64_t)gs.L / gs.ud : (gs.kind == G_PERMUTE ? S_out : S_in);
  const int64_t n_rows = outer * S_task;
  if (n_rows == 0 || row_bytes == 0) return USP_OK;
  int ub = unit_bytes_for(row_bytes, (uintptr_t)in, (uintptr_t)out);
  while (ub > 2 && ((in_row_stride | out_row_stride) % ub)) ub >>= 1;
  const int64_t upr = row_bytes / ub;
  const int64_t in_st = in_row_stride / ub, out_st = out_row_stride / ub;
  const int ltpr = log_tpr_for(upr);
  const int64_t rows_per_block = 256 >> ltpr;
  const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)blocks), block(256);
  const char* i8 = static_cast<const char*>(in);
  char* o8 = static_cast<char*>(out);
  TimingScope ts(K_PERMUTE, stream);
  switch (ub) {
    case 16: hipLaunchKernelGGL(permute_rows_kernel<16>, grid, block, 0, stream, i8, o8, n_rows, (int32_t)S_task, S_in, S_out, (int32_t)upr, in_st, out_st, ltpr, gs); break;
    case 8: hipLaunchKernelGGL(permute_rows_kernel<8>, grid, block, 0, stream, i8, o8, n_rows, (int32_t)S_task, S_in, S_out, (int32_t)upr, in_st, out_st, ltpr, gs); break;
    case 4: hipLaunchKernelGGL(permute_rows_kernel<4>, grid, block, 0, stream, i8, o8, n_rows, (int32_t)S_task, S_in, S_out, (int32_t)upr, in_st, out_st, ltpr, gs); break;
    default: hipLaunchKernelGGL(permute_rows_kernel<2>, grid, block, 0, stream, i8, o8, n_rows, (int32_t)S_task, S_in, S_out, (int32_t)upr, in_st, out_st, ltpr, gs); break;
  }
  return check_launch("permute");
}

usp_status launch_permute_f32_to_bf16(const float* in, uint16_t* out, int64_t outer, int64_t S_in,
                                      int64_t S_out, int64_t row_elems, int64_t out_row_stride,
                                      const GatherSpec& gs, hipStream_t stream) {
  const bool extract_like = gs.kind == G_EXTRACT || gs.kind == G_INSERT;
  const int64_t S_task = extract_like ? (int64_t)gs.L / gs.ud : (gs.kind == G_PERMUTE ? S_out : S_in);
  const int64_t n_rows = outer * S_task;
  if (n_rows == 0 || row_elems == 0) return USP_OK;
  const int64_t quads = row_elems / 4;  // callers guarantee row_elems % 4 == 0 and out_row_stride % 4 == 0
  const int ltpr = log_tpr_for(quads);
  const int64_t rows_per_block = 256 >> ltpr;
  const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  TimingScope ts(K_PERMUTE, stream);
  hipLaunchKernelGGL(permute_rows_f32_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in,
                     out, n_rows, (int32_t)S_task, S_in, S_out, (int32_t)quads, out_row_stride, ltpr, gs);
  return check_launch("permute_f32_bf16");
}

usp_status launch_relayout(void* const* shards, void* local, int64_t B, int64_t Ls, int64_t H,
                           int64_t D, int64_t elem_bytes, int ud, int u, int direction,
                           hipStream_t stream) {
  return launch_relayout_strided(shards, local, B, Ls, H, D, elem_bytes, ud, u, direction, Ls,
                                 (int64_t)ud * Ls, stream);
}

// Strided form used by the ring driver: batch b of shard u' starts
// shard_batch_rows rows after batch b-1, and likewise for the local tensor.
// Only shard_batch_rows == Ls and local_batch_rows == ud*Ls are contiguous;
// other strides are handled by launching once per batch row.
usp_status launch_relayout_strided(void* const* shards, void* local, int64_t B, int64_t Ls,
                                   int64_t H, int64_t D, int64_t elem_bytes, int ud, int u,
                                   int direction, int64_t shard_batch_rows,
                                   int64_t local_batch_rows, hipStream_t stream) {
  const int64_t Hg = H / ud;
  const int64_t seg_bytes = Hg * D * elem_bytes;
  const int64_t shard_row_bytes = H * D * elem_bytes;
  const int64_t local_row_bytes = Hg * D * elem_bytes;
  uintptr_t align_or = (uintptr_t)local | (uintptr_t)seg_bytes | (uintptr_t)shard_row_bytes;
  for (int i = 0; i < ud; ++i) align_or |= (uintptr_t)shards[i];
  int ub = 16;
  while (ub > 2 && (align_or % ub)) ub >>= 1;
  const int64_t upr = seg_bytes / ub;
  const int ltpr = log_tpr_for(upr);
  const int64_t rows_per_block = 256 >> ltpr;
  const bool contiguous = shard_batch_rows == Ls && local_batch_rows == (int64_t)ud * Ls;
  const int64_t nb = contiguous ? 1 : B;
  const int64_t rows_per_launch = (contiguous ? B : 1) * ud * Ls;
  for (int64_t bi = 0; bi < nb; ++bi) {
    ShardPtrs sp{};
    for (int i = 0; i < ud; ++i)
      sp.p[i] = static_cast<char*>(shards[i]) + bi * shard_batch_rows * shard_row_bytes;
    char* lp = static_cast<char*>(local) + bi * local_batch_rows * local_row_bytes;
    const int64_t blocks = (rows_per_launch + rows_per_block - 1) / rows_per_block;
    if (blocks == 0) continue;
    const dim3 grid((unsigned)blocks), block(256);
    TimingScope ts(K_RELAYOUT, stream);
    switch (ub) {
      case 16: hipLaunchKernelGGL(relayout_kernel<16>, grid, block, 0, stream, sp, lp, rows_per_launch, (int32_t)Ls, ud, u, shard_row_bytes, local_row_bytes, (int32_t)upr, ltpr, direction); break;
      case 8: hipLaunchKernelGGL(relayout_kernel<8>, grid, block, 0, stream, sp, lp, rows_per_launch, (int32_t)Ls, ud, u, shard_row_bytes, local_row_bytes, (int32_t)upr, ltpr, direction); break;
      case 4: hipLaunchKernelGGL(relayout_kernel<4>, grid, block, 0, stream, sp, lp, rows_per_launch, (int32_t)Ls, ud, u, shard_row_bytes, local_row_bytes, (int32_t)upr, ltpr, direction); break;
      default: hipLaunchKernelGGL(relayout_kernel<2>, grid, block, 0, stream, sp, lp, rows_per_launch, (int32_t)Ls, ud, u, shard_row_bytes, local_row_bytes, (int32_t)upr, ltpr, direction); break;
    }
    const usp_status st = check_launch("ulysses_relayout");
    if (st != USP_OK) return st;
  }
  return USP_OK;
}

}  // namespace usp
