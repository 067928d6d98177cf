// Backward of block attention (the gradient terms of one ring step) on
// gfx950 (CDNA4).
//
// With the final LSE and delta = rowsum(dO * O) of the query rows, a step's
// terms are (per (batch, head), visible pairs only)
//   P = exp(scale * Q K^T - LSE),  dP = dO V^T,  dS = P * (dP - delta),
//   dQ += scale * dS K,  dK += scale * dS^T Q,  dV += P^T dO,
// and they add up over the steps.  Two kernels share the work, each output
// element written by exactly one workgroup per launch (no atomics):
//   bwd_dq_kernel:   4 waves x 32 query rows; K and V tiles of 64 keys in
//                    LDS; S^T = K Q^T and dP^T = V dO^T with Q and dO
//                    resident in registers (each lane holds one query, as in
//                    the forward kernel), then dQ^T += K^T dS^T with dS^T
//                    taken straight from the accumulator layout;
//   bwd_dkdv_kernel: 4 waves x 32 keys; K and V of the tile resident in
//                    registers; Q, dO, LSE and delta of 64-row query tiles in
//                    LDS; S = Q K^T and dP = dO V^T (each lane holds one
//                    key), then dV^T += dO^T P and dK^T += Q^T dS.
// Both walk the visible pairs from host plans: the forward's (query tile ->
// key runs) for dQ, and its transpose (key tile -> query runs) for dK / dV,
// with per-element masks only in partial runs.
//
// MFMA 32x32x16 operand layout (lane l, 8 bf16 per operand):
//   A: row i = l % 32, 8 values along k for lane half l / 32;
//   B: col j = l % 32, the same 8 k values;
//   C: acc[r] = C[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15.

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
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBufferRsrcWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family)

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int32_t floor_div(int32_t a, int32_t b) {
  if (b == 1) return a;
  const int32_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}
__device__ __forceinline__ int32_t ceil_div(int32_t a, int32_t b) { return -floor_div(-a, b); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i supplies the
// address of 4 consecutive bf16 (row i/4 of a 4 x 16 block); lane j receives
// column j of the block.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// LDS tile of R rows x D bf16 with 16-byte chunk c of row r at slot
// c ^ swz(r), swz(r) = 4 * ((r / RPL) & (CPR / 4 - 1)): conflict-free for the
// transpose reads (4 rows x 2 chunks per 16 lanes); plain 16-byte reads of
// one chunk by 16 consecutive rows see some bank conflicts.
template <int D>
struct BwdTile {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 16 / CPR;
  static constexpr int ROWB = D * 2;
  __device__ static __forceinline__ int swz(int r) { return 4 * ((r / RPL) & (CPR / 4 - 1)); }
  // 16-byte fragment: row r, logical chunk c
  __device__ static __forceinline__ bf16x8 frag(const char* t, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(t + r * ROWB + ((c ^ swz(r)) * 16));
  }
};

// Transposed fragment of a tile (rows = the contraction index): for MFMA
// half `half` of 32-row block kb, head-dim block d, the 8 rows
// kb*32 + 16*half + {0..3, 8..11} + 4*(l/32) of column d*32 + l%32, in the
// k-order of a C-layout operand.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const char* t, int kb, int half, int d, int lane) {
  using T = BwdTile<D>;
  const int hi = lane >> 5;
  const int row0 = 4 * hi + ((lane & 15) >> 2);
  const int chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int h8 = (lane & 1) * 8;
  const int r0 = kb * 32 + half * 16 + row0;
  const int r1 = r0 + 8;
  const int c = 4 * d + chunk;
  const bf16x4 a0 = lds_read_tr(t + r0 * T::ROWB + ((c ^ T::swz(r0)) * 16) + h8);
  const bf16x4 a1 = lds_read_tr(t + r1 * T::ROWB + ((c ^ T::swz(r1)) * 16) + h8);
  return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ delta
// delta[b, h, t] = sum_d dO[b, t, h, d] * O[b, t, h, d]; one thread per row.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void* out, int out_f32, const uint16_t* dout,
                                                        float* delta, int64_t n_rows, int32_t L, int32_t H,
                                                        int32_t D) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_rows) return;
  const int64_t bt = idx / H;
  const int32_t h = (int32_t)(idx - bt * H);
  const int64_t b = bt / L;
  const int32_t t = (int32_t)(bt - b * L);
  const uint16_t* dp = dout + idx * D;
  float acc = 0.f;
  for (int d = 0; d < D; d += 8) {
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(dp + d);
    if (out_f32) {
      const float4 o0 = *reinterpret_cast<const float4*>(static_cast<const float*>(out) + idx * D + d);
      const float4 o1 = *reinterpret_cast<const float4*>(static_cast<const float*>(out) + idx * D + d + 4);
      acc += (float)g[0] * o0.x + (float)g[1] * o0.y + (float)g[2] * o0.z + (float)g[3] * o0.w;
      acc += (float)g[4] * o1.x + (float)g[5] * o1.y + (float)g[6] * o1.z + (float)g[7] * o1.w;
    } else {
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(out) + idx * D + d);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)g[e] * (float)o[e];
    }
  }
  delta[(b * H + h) * L + t] = acc;
}

// -------------------------------------------------------------------- dQ
template <int D, bool LINEAR>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(const BwdParams p) {
  using T = BwdTile<D>;
  constexpr int BN = 64;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NB = BN / 32;
  constexpr int TILEB = BN * D * 2;
  constexpr int LPW = TILEB / 4096;
  constexpr int RPI = 1024 / T::ROWB;
  static_assert(kTileN % BN == 0, "planner granularity");
  __shared__ __attribute__((aligned(1024))) char smem[2 * TILEB];  // K, V
  char* const tK = smem;
  char* const tV = smem + TILEB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int total = p.n_items * p.Hq * p.B;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int hb = bid / p.n_items;
  const int item_idx = bid - hb * p.n_items;
  const int h = hb % p.Hq;
  const int b = hb / p.Hq;
  const WorkItem it = p.items[item_idx];
  const int hk = h / (p.Hq / p.Hkv);

  const int qr = wid * 32 + l32;
  const bool qvalid = qr < it.q_rows;
  const int64_t qrow = (int64_t)it.q_row0 + qr;

  bf16x8 qf[KS], dof[KS];
  {
    const int64_t off = (int64_t)b * p.q_batch_stride + (qrow * p.Hq + h) * D + hi * 8;
    const int64_t goff = (int64_t)b * p.g_batch_stride + (qrow * p.Hq + h) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qvalid) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(p.q + off + ks * 16);
        dof[ks] = *reinterpret_cast<const bf16x8*>(p.dout + goff + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = dof[ks][e] = (__bf16)0.f;
      }
    }
  }
  // exp2 subtrahend (LSE in log2 units; +inf gives P = 0) and delta of this row
  float lse2 = INFINITY, dl = 0.f;
  if (qvalid) {
    const int64_t li = ((int64_t)b * p.Hq + h) * p.Lq_buf + qrow;
    const float l = p.lse[li];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dl = p.delta[li];
  }

  f32x16 dqt[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[d][r] = 0.f;

  PosMap qm = p.qmap;
  qm.rank = it.q_rank;
  PosMap km = p.kmap;
  km.rank = it.k_rank;
  const bool cw = p.mask.causal || p.mask.window > 0;
  int32_t sstart, vis_lo, vis_hi, sink_hi;
  {
    const int32_t pq = position(qm, it.t0 + (qvalid ? qr : 0));
    int32_t s0 = 0, s1 = p.mask.S;
    for (int i = 0; i < p.mask.nseq; ++i) {
      const int32_t lo = p.cu_seqlens[i], up = p.cu_seqlens[i + 1];
      if (pq >= lo && pq < up) {
        s0 = lo;
        s1 = up;
      }
    }
    sstart = s0;
    vis_hi = cw ? min(pq, s1 - 1) : s1 - 1;
    vis_lo = p.mask.window > 0 ? max(s0, pq - p.mask.window + 1) : s0;
    sink_hi = p.mask.window > 0 ? min(s0 + p.mask.n_sink - 1, vis_hi) : s0 - 1;
  }
  const int32_t kv_step = km.kind == MAP_STRIPE ? km.N : 1;

  const int64_t kv_row_stride = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;
  const uint32_t row_bytes = (uint32_t)kv_row_stride * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, 0x7fffffff, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, 0x7fffffff, kBufferRsrcWord3);
  const int lrow = lane / T::CPR;
  const int lslot = lane % T::CPR;

  const float c = p.scale_log2;
  for (int ri = it.run_begin; ri < it.run_end; ++ri) {
    const Run run = p.runs[ri];
    for (int k0 = run.k_begin; k0 < run.k_end; k0 += BN) {
      i32x4 kr[LPW], vr[LPW];
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int row = (wid * LPW + j) * RPI + lrow;
        const uint32_t off = (uint32_t)min(k0 + row, run.k_end - 1) * row_bytes + (uint32_t)((lslot ^ T::swz(row)) * 16);
        kr[j] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
        vr[j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
      }
      __syncthreads();  // the previous tile's reads are done
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        *reinterpret_cast<i32x4*>(tK + (wid * LPW + j) * 1024 + lane * 16) = kr[j];
        *reinterpret_cast<i32x4*>(tV + (wid * LPW + j) * 1024 + lane * 16) = vr[j];
      }
      __syncthreads();

      // S^T = K Q^T and dP^T = V dO^T (keys x queries)
      f32x16 st[NB], dpt[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = dpt[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
          st[kb] = mfma32(T::frag(tK, kb * 32 + l32, 2 * ks + hi), qf[ks], st[kb]);
          dpt[kb] = mfma32(T::frag(tV, kb * 32 + l32, 2 * ks + hi), dof[ks], dpt[kb]);
        }
      }
      if (!run.full) {
        const int32_t kend_du = run.k_end - 1 - k0;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int du = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            bool vis;
            if constexpr (LINEAR) {
              const int32_t pk = position(km, k0) + du * kv_step;
              vis = (du <= kend_du) & (pk <= vis_hi) & ((pk >= vis_lo) | ((pk >= sstart) & (pk <= sink_hi)));
            } else {
              const int32_t pk = position(km, k0 + du);
              vis = (du <= kend_du) & (pk <= vis_hi) & ((pk >= vis_lo) | ((pk >= sstart) & (pk <= sink_hi)));
            }
            st[kb][r] = vis ? st[kb][r] : -INFINITY;
          }
        }
      }
      // dS^T = P^T (dP^T - delta), bf16, in the k-order of a B operand
      bf16x8 dsb[NB][2];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(st[kb][half * 8 + e] * c - lse2);
            const float p1 = __builtin_amdgcn_exp2f(st[kb][half * 8 + e + 1] * c - lse2);
            const float d0 = p0 * (dpt[kb][half * 8 + e] - dl);
            const float d1 = p1 * (dpt[kb][half * 8 + e + 1] - dl);
            const bf16x2 pk2 = __builtin_convertvector((f32x2){d0, d1}, bf16x2);
            dsb[kb][half][e] = pk2[0];
            dsb[kb][half][e + 1] = pk2[1];
          }
        }
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int d = 0; d < DB; ++d) dqt[d] = mfma32(frag_tr<D>(tK, kb, half, d, lane), dsb[kb][half], dqt[d]);
    }
  }

  // dq[b, row, h, :] += scale * dQ (this lane: query qrow, head-dim rows of dQ^T)
  if (!qvalid || it.run_begin == it.run_end) return;
  float* op = p.dq + (int64_t)b * p.g_batch_stride + (qrow * p.Hq + h) * D;
  const float sc = p.scale;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * hi;
      float4 a = *reinterpret_cast<const float4*>(op + dd);
      a.x += sc * dqt[d][4 * g];
      a.y += sc * dqt[d][4 * g + 1];
      a.z += sc * dqt[d][4 * g + 2];
      a.w += sc * dqt[d][4 * g + 3];
      *reinterpret_cast<float4*>(op + dd) = a;
    }
  }
}

// ------------------------------------------------------------------ dK dV
// Work item fields (the transposed plan): q_row0 = first key row of the tile
// in the k/v buffers, t0 = its local key index, q_rows = keys in the tile,
// q_rank = KV rank, k_row0 = row of local query 0 of the query rank in the
// q/dout buffers, k_rank = query rank; runs: local query rows
// [k_begin, k_end) and whether every pair of the run is visible.
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using T = BwdTile<D>;
  constexpr int BQ = 64;            // query rows per iteration
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NQB = BQ / 32;
  constexpr int TILEB = BQ * D * 2;
  constexpr int LPW = TILEB / 4096;
  constexpr int RPI = 1024 / T::ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * TILEB + 2 * BQ * 4];  // Q, dO, LSE2, delta
  char* const tQ = smem;
  char* const tO = smem + TILEB;
  float* const sl = reinterpret_cast<float*>(smem + 2 * TILEB);
  float* const sd = sl + BQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int total = p.n_items * p.Hkv * p.B;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int hb = bid / p.n_items;
  const int item_idx = bid - hb * p.n_items;
  const int hk = hb % p.Hkv;
  const int b = hb / p.Hkv;
  const WorkItem it = p.items[item_idx];
  const int group = p.Hq / p.Hkv;

  const int kr_ = wid * 32 + l32;
  const bool kvalid = kr_ < it.q_rows;
  const int64_t krow = (int64_t)it.q_row0 + kr_;
  const int64_t kv_row_stride = (int64_t)p.Hkv * D;

  bf16x8 kf[KS], vf[KS];
  {
    const int64_t off = (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (kvalid) {
        kf[ks] = *reinterpret_cast<const bf16x8*>(p.k + off + ks * 16);
        vf[ks] = *reinterpret_cast<const bf16x8*>(p.v + off + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[ks][e] = vf[ks][e] = (__bf16)0.f;
      }
    }
  }
  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkt[d][r] = dvt[d][r] = 0.f;

  // this lane's key position and the sequence it belongs to
  PosMap qm = p.qmap;
  qm.rank = it.k_rank;
  PosMap km = p.kmap;
  km.rank = it.q_rank;
  const int32_t pk = position(km, it.t0 + (kvalid ? kr_ : 0));
  int32_t ks0 = 0, ks1 = p.mask.S;
  for (int i = 0; i < p.mask.nseq; ++i) {
    const int32_t lo = p.cu_seqlens[i], up = p.cu_seqlens[i + 1];
    if (pk >= lo && pk < up) {
      ks0 = lo;
      ks1 = up;
    }
  }
  const bool cw = p.mask.causal || p.mask.window > 0;

  const int lrow = lane / T::CPR;
  const int lslot = lane % T::CPR;
  const float c = p.scale_log2;

  for (int gi = 0; gi < group; ++gi) {
    const int h = hk * group + gi;
    const uint16_t* qbase = p.q + (int64_t)b * p.q_batch_stride + (int64_t)it.k_row0 * p.Hq * D + h * D;
    const uint16_t* obase = p.dout + (int64_t)b * p.g_batch_stride + (int64_t)it.k_row0 * p.Hq * D + h * D;
    const uint32_t qrow_bytes = (uint32_t)p.Hq * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, (short)0, 0x7fffffff, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)obase, (short)0, 0x7fffffff, kBufferRsrcWord3);
    const float* lse_h = p.lse + ((int64_t)b * p.Hq + h) * p.Lq_buf + it.k_row0;
    const float* del_h = p.delta + ((int64_t)b * p.Hq + h) * p.Lq_buf + it.k_row0;

    for (int ri = it.run_begin; ri < it.run_end; ++ri) {
      const Run run = p.runs[ri];
      for (int t0 = run.k_begin; t0 < run.k_end; t0 += BQ) {
        i32x4 qr4[LPW], or4[LPW];
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
          const int row = (wid * LPW + j) * RPI + lrow;
          const uint32_t roff = (uint32_t)min(t0 + row, run.k_end - 1) * qrow_bytes + (uint32_t)((lslot ^ T::swz(row)) * 16);
          qr4[j] = __builtin_amdgcn_raw_buffer_load_b128(qrs, roff, 0, 0);
          or4[j] = __builtin_amdgcn_raw_buffer_load_b128(ors, roff, 0, 0);
        }
        float lv = INFINITY, dv_ = 0.f;
        if (tid < BQ && t0 + tid < run.k_end) {
          const float l = lse_h[t0 + tid];
          lv = l == -INFINITY ? INFINITY : l * kLog2e;
          dv_ = del_h[t0 + tid];
        }
        __syncthreads();  // the previous query tile's reads are done
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
          *reinterpret_cast<i32x4*>(tQ + (wid * LPW + j) * 1024 + lane * 16) = qr4[j];
          *reinterpret_cast<i32x4*>(tO + (wid * LPW + j) * 1024 + lane * 16) = or4[j];
        }
        if (tid < BQ) {
          sl[tid] = lv;
          sd[tid] = dv_;
        }
        __syncthreads();

        // S = Q K^T and dP = dO V^T (queries x keys): lane = key, 16 queries
        f32x16 s[NQB], dp[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][r] = dp[qb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            s[qb] = mfma32(T::frag(tQ, qb * 32 + l32, 2 * ks + hi), kf[ks], s[qb]);
            dp[qb] = mfma32(T::frag(tO, qb * 32 + l32, 2 * ks + hi), vf[ks], dp[qb]);
          }
        }
        bf16x8 pb[NQB][2], dsb[NQB][2];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int q4 = qb * 32 + 8 * g + 4 * hi;  // 4 consecutive queries
            const float4 l4 = *reinterpret_cast<const float4*>(sl + q4);
            const float4 d4 = *reinterpret_cast<const float4*>(sd + q4);
            const float lq[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dq4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g + e;
              float x = s[qb][r];
              if (!run.full) {
                const int32_t pq = position(qm, t0 + q4 + e);
                const bool vis = (pq >= ks0) & (pq < ks1) & (!cw | (pk <= pq)) &
                                 ((p.mask.window <= 0) | (pq - pk < p.mask.window) |
                                  ((pk - ks0 < p.mask.n_sink) & (pk <= pq)));
                x = vis ? x : -INFINITY;
              }
              const float pr = __builtin_amdgcn_exp2f(x * c - lq[e]);
              const float ds = pr * (dp[qb][r] - dq4[e]);
              pb[qb][r >> 3][r & 7] = (__bf16)pr;
              dsb[qb][r >> 3][r & 7] = (__bf16)ds;
            }
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS (head dim x keys)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int d = 0; d < DB; ++d) {
              dvt[d] = mfma32(frag_tr<D>(tO, qb, half, d, lane), pb[qb][half], dvt[d]);
              dkt[d] = mfma32(frag_tr<D>(tQ, qb, half, d, lane), dsb[qb][half], dkt[d]);
            }
      }
    }
  }

  if (!kvalid || it.run_begin == it.run_end) return;
  float* kp = p.dk + (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D;
  float* vp = p.dv + (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D;
  const float sc = p.scale;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * hi;
      float4 a = *reinterpret_cast<const float4*>(kp + dd);
      a.x += sc * dkt[d][4 * g];
      a.y += sc * dkt[d][4 * g + 1];
      a.z += sc * dkt[d][4 * g + 2];
      a.w += sc * dkt[d][4 * g + 3];
      *reinterpret_cast<float4*>(kp + dd) = a;
      float4 v4 = *reinterpret_cast<const float4*>(vp + dd);
      v4.x += dvt[d][4 * g];
      v4.y += dvt[d][4 * g + 1];
      v4.z += dvt[d][4 * g + 2];
      v4.w += dvt[d][4 * g + 3];
      *reinterpret_cast<float4*>(vp + dd) = v4;
    }
  }
}

}  // namespace

usp_status launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  // n is a multiple of 4 and p 16-byte aligned (the callers' f32 tensors of D >= 64 columns)
  if (n <= 0) return USP_OK;
  const int64_t n4 = n / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<float4*>(p), n4);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("fill launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

usp_status launch_bwd_delta(const void* out, int out_f32, const uint16_t* dout, float* delta, int64_t B,
                            int64_t L, int64_t H, int64_t D, hipStream_t stream) {
  const int64_t n = B * L * H;
  if (n == 0) return USP_OK;
  {
    TimingScope ts(K_BWD_DELTA, stream);
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, out, out_f32,
                       dout, delta, n, (int32_t)L, (int32_t)H, (int32_t)D);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("delta launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

usp_status launch_bwd(const BwdParams& pq, const BwdParams& pkv, int D, hipStream_t stream) {
  const bool linear = !(pq.kmap.kind == MAP_STRIPE && pq.kmap.b > 1);
  const int64_t nq = (int64_t)pq.n_items * pq.Hq * pq.B;
  const int64_t nk = (int64_t)pkv.n_items * pkv.Hkv * pkv.B;
  if (nq > 0x7fffffff || nk > 0x7fffffff) {
    set_error("backward grid too large");
    return USP_ERR_UNSUPPORTED;
  }
  if (nq > 0) {
    TimingScope ts(K_BWD_DQ, stream);
    if (D == 128) {
      if (linear) hipLaunchKernelGGL((bwd_dq_kernel<128, true>), dim3((unsigned)nq), dim3(256), 0, stream, pq);
      else hipLaunchKernelGGL((bwd_dq_kernel<128, false>), dim3((unsigned)nq), dim3(256), 0, stream, pq);
    } else {
      if (linear) hipLaunchKernelGGL((bwd_dq_kernel<64, true>), dim3((unsigned)nq), dim3(256), 0, stream, pq);
      else hipLaunchKernelGGL((bwd_dq_kernel<64, false>), dim3((unsigned)nq), dim3(256), 0, stream, pq);
    }
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && nk > 0) {
    TimingScope ts(K_BWD_DKDV, stream);
    if (D == 128) hipLaunchKernelGGL((bwd_dkdv_kernel<128>), dim3((unsigned)nk), dim3(256), 0, stream, pkv);
    else hipLaunchKernelGGL((bwd_dkdv_kernel<64>), dim3((unsigned)nk), dim3(256), 0, stream, pkv);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    set_error("backward launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
