// Associative merge of a partial (O_b, L_b) into a running (O_a, L_a):
//   M = max(L_a, L_b), L = M + ln(e^(L_a-M) + e^(L_b-M)),
//   O = e^(L_a-L) O_a + e^(L_b-L) O_b;  L_b = -inf leaves (O_a, L_a).
// Elementwise and HBM-bound: one float4 of O per thread, all four loads of a
// thread issued together.  The D/4 threads of one (row, head) lie inside one
// wave (D/4 divides 64), and the one store of the new LSE comes after
// the wave has consumed every lane's read of the old value, so the in-place
// update needs no barrier.

#include <hip/hip_runtime.h>

#include <cmath>

#include "usp_internal.h"

namespace usp {
namespace {

__global__ __launch_bounds__(256) void lse_merge_kernel(float* __restrict__ out_acc,
                                                        float* __restrict__ lse_acc,
                                                        const float* __restrict__ out_part,
                                                        const float* __restrict__ lse_part, int32_t B,
                                                        int32_t L, int32_t H, int32_t quads,
                                                        int32_t row_begin, int32_t n_rows,
                                                        int64_t n_groups) {
  // group = (b, row, h); quads threads per group, 256/quads groups per block
  // (row-fastest groups, which read neighbouring LSE entries, measured 4 %
  // slower: their O rows lie H*D*4 bytes apart)
  const int32_t gpb = 256 / quads;
  const int64_t grp = (int64_t)blockIdx.x * gpb + threadIdx.x / quads;
  const int32_t q = threadIdx.x % quads;
  if (grp >= n_groups) return;
  const int32_t h = (int32_t)(grp % H);
  const int64_t br = grp / H;
  const int32_t r = (int32_t)(br % n_rows) + row_begin;
  const int32_t b = (int32_t)(br / n_rows);
  const int64_t lse_idx = ((int64_t)b * H + h) * L + r;
  const int64_t o_idx = (((int64_t)b * L + r) * H + h) * quads + q;
  const float la = lse_acc[lse_idx];
  const float lb = lse_part[lse_idx];
  // non-temporal loads, plain stores: 0.124 against 0.143 ms on an 811 MB
  // step (the hint on the stores as well was slower than none)
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 a = ld_nt(reinterpret_cast<const f32x4*>(out_acc) + o_idx);
  const f32x4 p = ld_nt(reinterpret_cast<const f32x4*>(out_part) + o_idx);
  const float M = fmaxf(la, lb);
  if (lb == -INFINITY || M == -INFINITY) return;  // nothing to merge
  const float Lm = M + logf(expf(la - M) + expf(lb - M));
  const float wa = expf(la - Lm), wb = expf(lb - Lm);
  float4 o;
  o.x = wa * a.x + wb * p.x;
  o.y = wa * a.y + wb * p.y;
  o.z = wa * a.z + wb * p.z;
  o.w = wa * a.w + wb * p.w;
  reinterpret_cast<float4*>(out_acc)[o_idx] = o;
  if (q == 0) lse_acc[lse_idx] = Lm;
}

}  // namespace

usp_status launch_lse_merge(float* out_acc, float* lse_acc, const float* out_part,
                            const float* lse_part, int64_t B, int64_t L, int64_t H, int64_t D,
                            int64_t row_begin, int64_t row_end, hipStream_t stream) {
  const int64_t n_rows = row_end - row_begin;
  const int64_t quads = D / 4;
  if (quads > 64 || 64 % quads != 0) {
    set_error("lse_merge: head_dim %lld unsupported (one (row, head) must fit in one wave)", (long long)D);
    return USP_ERR_UNSUPPORTED;
  }
  const int64_t n_groups = B * n_rows * H;
  if (n_groups == 0) return USP_OK;
  const int64_t gpb = 256 / quads;
  const int64_t blocks = (n_groups + gpb - 1) / gpb;
  TimingScope ts(K_MERGE, stream);
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out_acc, lse_acc,
                     out_part, lse_part, (int32_t)B, (int32_t)L, (int32_t)H, (int32_t)quads,
                     (int32_t)row_begin, (int32_t)n_rows, n_groups);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("lse_merge launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
