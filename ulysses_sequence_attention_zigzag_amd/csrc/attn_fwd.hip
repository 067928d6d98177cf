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

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i supplies the address of 4 consecutive bf16 (row i/4 of a
// 4 x 16 block, columns 4*(i%4)..+3); lane j receives column j of the block,
// i.e. the 4 values of one column from 4 consecutive rows.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Asynchronous 16-byte global -> LDS copy (gfx950 global_load_lds_dwordx4):
// lane i's 16 bytes land at lds_wave_base + 16 * i.
__device__ __forceinline__ void load_to_lds(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

// LDS tile layout: a K or V tile is BN rows of D bf16 (D*2 bytes), rows
// packed back to back, each row made of D/8 chunks of 16 bytes.  Chunk c of
// row r is stored at chunk slot c ^ swz(r).  The swizzles make the two read
// patterns hit 16 distinct 16-byte bank groups of the 256-byte LDS line:
//   K (ds_read_b128, 16 lanes read rows r..r+15 at one chunk):
//     swz_k(r) = (r / RPL) & (CPR - 1)
//   V (transpose reads, 16 lanes read 4 rows x 2 chunks, 32 lanes 4 x 4):
//     swz_v(r) = 4 * ((r / RPL) & (CPR / 4 - 1))
// with CPR = D/8 chunks per row and RPL = 16/CPR rows per 256-byte line.
template <int D>
struct TileLayout {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 16 / CPR;
  static constexpr int ROWB = D * 2;
  __device__ static __forceinline__ int swz_k(int r) { return (r / RPL) & (CPR - 1); }
  __device__ static __forceinline__ int swz_v(int r) { return 4 * ((r / RPL) & (CPR / 4 - 1)); }
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const AttnParams p) {
  using TL = TileLayout<D>;
  constexpr int BN = kTileN;
  constexpr int KS = D / 16;        // k-steps of the QK^T contraction
  constexpr int DB = D / 32;        // 32-wide blocks of the output's head dim
  constexpr int NB = BN / 32;       // 32-key blocks per tile
  constexpr int TILEB = BN * D * 2; // bytes of one K or V tile
  constexpr int LPW = TILEB / 1024 / 4;  // direct loads per wave per tensor and tile
  constexpr int RPI = 1024 / TL::ROWB;   // tile rows per 1 KB load instruction
  static_assert(TILEB % 4096 == 0, "tile must split into 4 waves x 1 KB loads");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILEB];  // K0 K1 V0 V1

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
  // Running max m (log2 domain, scale folded in) and this lane's share of the
  // running sum.  m is raised lazily: only when a tile's max exceeds it by
  // more than kRescale, so the exponentials stay <= 2^kRescale.
  constexpr float kRescale = 8.f;
  float m = -INFINITY;
  float lsum = 0.f;

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

  // Direct loads of one K and one V tile into LDS buffer `buf`.  Wave w fills
  // 1 KB slices w*LPW .. w*LPW+LPW-1 of each tile; lane i of a slice writes
  // physical (row, chunk slot) = (slice*RPI + i / CPR, i % CPR) and so loads
  // logical chunk slot ^ swz(row) of that row.  Rows past the run's end are
  // clamped to its last row (finite values; those keys are masked).
  const int lrow = lane / TL::CPR;
  const int lslot = lane % TL::CPR;
  auto issue_tile = [&](int buf, int k0, int kend) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int slice = wid * LPW + j;
      const int row = slice * RPI + lrow;
      const int grow = min(k0 + row, kend - 1);
      const int ck = lslot ^ TL::swz_k(row);
      const int cv = lslot ^ TL::swz_v(row);
      load_to_lds(kbase + (int64_t)grow * kv_row_stride + ck * 8, smem + buf * TILEB + slice * 1024);
      load_to_lds(vbase + (int64_t)grow * kv_row_stride + cv * 8, smem + (2 + buf) * TILEB + slice * 1024);
    }
  };

  // Per-lane LDS read offsets (bytes within a tile).
  //   K: row kb*32 + l32, logical chunk 2*ks + hi.
  //   V: transpose reads of rows kb*32 + 16*half + 4*hi + 8*second + (lane%16)/4,
  //      logical chunk 4*d + 2*((lane/16)%2) + (lane%4)/2, 8-byte half lane%2.
  const int trow = (lane & 15) >> 2;
  const int vrow0 = 4 * hi + trow;
  const int vchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vhalf8 = (lane & 1) * 8;

  int ri = it.run_begin;
  if (ri < it.run_end) {
    Run run = p.runs[ri];
    int k0 = run.k_begin;
    int buf = 0;
    issue_tile(0, k0, run.k_end);
    while (true) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // tile `buf` is in LDS; every wave is done with buffer buf^1

      // next tile (uniform across the workgroup); its loads overlap this tile's math
      int nk0 = k0 + BN;
      int nri = ri;
      Run nrun = run;
      if (nk0 >= run.k_end) {
        nri = ri + 1;
        if (nri < it.run_end) {
          nrun = p.runs[nri];
          nk0 = nrun.k_begin;
        }
      }
      const bool has_next = nri < it.run_end;
      if (has_next) issue_tile(buf ^ 1, nk0, nrun.k_end);

      const char* tK = smem + buf * TILEB;
      const char* tV = smem + (2 + buf) * TILEB;

      // S^T[key][q] for the tile's NB blocks of 32 keys
      f32x16 s[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const int row = kb * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int slot = (2 * ks + hi) ^ TL::swz_k(row);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(tK + row * TL::ROWB + slot * 16);
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

      // online softmax (log2 domain) with lazy rescaling
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * p.scale_log2;
      if (__builtin_amdgcn_readfirstlane((int)(__ballot(mt > m + kRescale) != 0ull))) {
        const float m_new = fmaxf(m, mt);
        // 0 when only m is -inf; lanes that have seen no visible key keep 1
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      const float m_use = (m == -INFINITY) ? 0.f : m;

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
            const int r0 = kb * 32 + half * 16 + vrow0;
            const int r1 = r0 + 8;
            const int c = 4 * d + vchunk;
            const bf16x4 a0 = lds_read_tr(tV + r0 * TL::ROWB + ((c ^ TL::swz_v(r0)) * 16) + vhalf8);
            const bf16x4 a1 = lds_read_tr(tV + r1 * TL::ROWB + ((c ^ TL::swz_v(r1)) * 16) + vhalf8);
            const bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            o[d] = mfma32(a, pb[kb][half], o[d]);
          }
        }
      }

      if (!has_next) break;
      ri = nri;
      run = nrun;
      k0 = nk0;
      buf ^= 1;
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
