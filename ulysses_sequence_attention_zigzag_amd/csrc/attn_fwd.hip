// Block attention forward for one ring step on gfx950 (CDNA4).
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
// owns 32 query rows.  Per key tile of 64 keys:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS (A operand),
//                    Q resident in VGPRs (B operand);
//   mask             only in partial runs (the planner marks fully visible
//                    tiles), evaluated on global positions;
//   online softmax   in the log2 domain (scale*log2(e) folded into one
//                    multiply, hardware exp2); because S is computed
//                    transposed, each lane holds 32 scores of ONE query, so
//                    the row max needs a single cross-lane swap (lane ^ 32)
//                    and the row sum stays lane-local until the epilogue;
//   O^T += V^T P^T   P^T comes straight out of the S^T accumulator layout as
//                    the B operand (rounded to bf16); V^T is read from an
//                    LDS copy of the V tile stored key-contiguous.
// The epilogue writes O and LSE, or merges them into a running result
// (accumulate) with the associative max / logsumexp rescale.
//
// MFMA 32x32x16 operand layout used below (lane l, 8 bf16 per operand):
//   A: row i = l % 32, 8 values along k for lane half l / 32;
//   B: col j = l % 32, the same 8 k values;
//   C: acc[r] = C[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15.
// Any k-order works as long as A and B use the same one; P^T's k-order is
// fixed by the C layout above, and V^T is loaded to match it.

#include <hip/hip_runtime.h>

#include <cmath>

#include "usp_internal.h"

namespace usp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const AttnParams p) {
  constexpr int BN = kTileN;
  constexpr int KS = D / 16;        // k-steps of the QK^T contraction
  constexpr int DB = D / 32;        // 32-wide blocks of the output's head dim
  constexpr int NB = BN / 32;       // 32-key blocks per tile
  constexpr int KPAD = D + 8;       // sK row stride (elements)
  constexpr int VPAD = BN + 4;      // sV row stride (elements), V stored [d][key]
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VPAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work decode: logical id -> (batch*head, item).  Workgroups are handed to
  // the 8 XCDs round-robin, so logical ids are regrouped to give each XCD a
  // contiguous range (whole heads, which share K/V in that XCD's L2).
  const int total = p.n_items * p.Hq * p.B;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int hb = bid / p.n_items;
  const int item_idx = bid - hb * p.n_items;
  const int h = hb % p.Hq;
  const int b = hb / p.Hq;
  const WorkItem it = p.items[item_idx];
  const int hk = h / (p.Hq / p.Hkv);

  const int qr = wid * 32 + l32;              // this lane's query row in the tile
  const bool qvalid = qr < it.q_rows;
  const int64_t qrow = (int64_t)it.q_row0 + qr;

  // Q fragments (B operand): Q[q][ks*16 + hi*8 .. +7]
  bf16x8 qf[KS];
  {
    const uint16_t* qp = p.q + (int64_t)b * p.q_batch_stride + (qrow * p.Hq + h) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qvalid) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.f;
      }
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m = -INFINITY;  // running max of scale*log2(e)*s
  float lsum = 0.f;     // this lane's share of the running sum

  // Positions for per-element masks.
  PosMap qm = p.qmap;
  qm.rank = it.q_rank;
  PosMap km = p.kmap;
  km.rank = it.k_rank;
  const int32_t pq = position(qm, it.t0 + (qvalid ? qr : 0));
  int32_t sstart = 0, send = p.mask.S;
  if (p.mask.nseq > 0) {
    for (int i = 0; i < p.mask.nseq; ++i) {
      const int32_t lo = p.cu_seqlens[i], up = p.cu_seqlens[i + 1];
      if (pq >= lo && pq < up) {
        sstart = lo;
        send = up;
      }
    }
  }
  const bool cw = p.mask.causal || p.mask.window > 0;
  const int32_t W = p.mask.window;
  const int32_t nsink = p.mask.n_sink;

  const int64_t kv_row_stride = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;

  for (int ri = it.run_begin; ri < it.run_end; ++ri) {
    const Run run = p.runs[ri];
    for (int k0 = run.k_begin; k0 < run.k_end; k0 += BN) {
      const int nk = min(BN, run.k_end - k0);
      __syncthreads();  // the previous tile is no longer read
      for (int e = tid; e < BN * D / 8; e += 256) {
        const int row = e / (D / 8);
        const int c8 = e - row * (D / 8);
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (row < nk) {
          kv = *reinterpret_cast<const uint4*>(kbase + (int64_t)(k0 + row) * kv_row_stride + c8 * 8);
          vv = *reinterpret_cast<const uint4*>(vbase + (int64_t)(k0 + row) * kv_row_stride + c8 * 8);
        }
        *reinterpret_cast<uint4*>(&sK[row * KPAD + c8 * 8]) = kv;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sV[(c8 * 8 + 2 * i) * VPAD + row] = (uint16_t)(w[i] & 0xffffu);
          sV[(c8 * 8 + 2 * i + 1) * VPAD + row] = (uint16_t)(w[i] >> 16);
        }
      }
      __syncthreads();

      // S^T[key][q] for the tile's NB blocks of 32 keys
      f32x16 s[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[(kb * 32 + l32) * KPAD + ks * 16 + hi * 8]);
          s[kb] = mfma32(a, qf[ks], s[kb]);
        }
      }

      if (!run.full) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int u = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const int32_t pk = position(km, u);
            const bool vis = u < run.k_end && pk >= sstart && pk < send && (!cw || pk <= pq) &&
                             (W <= 0 || pq - pk < W || pk - sstart < nsink);
            if (!vis) s[kb][r] = -INFINITY;
          }
        }
      }

      // online softmax (log2 domain)
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m, mt * p.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

      bf16x8 pb[NB][2];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = fast_exp2(s[kb][half * 8 + e] * p.scale_log2 - m_use);
            const float p1 = fast_exp2(s[kb][half * 8 + e + 1] * p.scale_log2 - m_use);
            lsum += p0 + p1;
            const bf16x2 pk2 = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
            pb[kb][half][e] = pk2[0];
            pb[kb][half][e + 1] = pk2[1];
          }
        }
      }

      // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint16_t* vr = &sV[(d * 32 + l32) * VPAD + kb * 32 + half * 16 + hi * 4];
            const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(vr);
            const bf16x4 a1 = *reinterpret_cast<const bf16x4*>(vr + 8);
            const bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            o[d] = mfma32(a, pb[kb][half], o[d]);
          }
        }
      }
    }
  }

  // epilogue
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!qvalid) return;
  const float lse_new = ltot > 0.f ? m * kLn2 + logf(ltot) : -INFINITY;
  float* lse_ptr = p.lse + ((int64_t)b * p.Hq + h) * p.Lq_buf + qrow;
  const int64_t obase = (int64_t)b * p.o_batch_stride + (qrow * p.Hq + h) * D;
  float wa = 0.f, wb = ltot > 0.f ? 1.f / ltot : 0.f;
  float lse_out = lse_new;
  if (p.accumulate) {
    const float la = *lse_ptr;
    const float M = fmaxf(la, lse_new);
    if (lse_new == -INFINITY || M == -INFINITY) return;  // nothing to merge
    const float Lm = M + logf(expf(la - M) + expf(lse_new - M));
    wa = expf(la - Lm);
    wb *= expf(lse_new - Lm);
    lse_out = Lm;
  }
  if (p.out_f32) {
    float* op = static_cast<float*>(p.out) + obase;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + 8 * g + 4 * hi;
        float4 v = make_float4(o[d][4 * g] * wb, o[d][4 * g + 1] * wb, o[d][4 * g + 2] * wb,
                               o[d][4 * g + 3] * wb);
        if (wa != 0.f) {
          const float4 a = *reinterpret_cast<const float4*>(op + dd);
          v.x += wa * a.x;
          v.y += wa * a.y;
          v.z += wa * a.z;
          v.w += wa * a.w;
        }
        *reinterpret_cast<float4*>(op + dd) = v;
      }
    }
  } else {
    uint16_t* op = static_cast<uint16_t*>(p.out) + obase;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + 8 * g + 4 * hi;
        const bf16x2 lo = __builtin_convertvector((f32x2){o[d][4 * g] * wb, o[d][4 * g + 1] * wb}, bf16x2);
        const bf16x2 up = __builtin_convertvector((f32x2){o[d][4 * g + 2] * wb, o[d][4 * g + 3] * wb}, bf16x2);
        *reinterpret_cast<uint2*>(op + dd) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, up));
      }
    }
  }
  if (hi == 0) *lse_ptr = lse_out;
}

}  // namespace

usp_status launch_attn_fwd(const AttnParams& p, int D, hipStream_t stream) {
  const int64_t total = (int64_t)p.n_items * p.Hq * p.B;
  if (total == 0) return USP_OK;
  if (total > 0x7fffffff) {
    set_error("attention grid too large (%lld workgroups)", (long long)total);
    return USP_ERR_UNSUPPORTED;
  }
  const dim3 grid((unsigned)total), block(256);
  TimingScope ts(K_ATTN, stream);
  if (D == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, block, 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
