// dQ kernel of the block-attention backward (see attn_bwd.hip for the
// terms and the plan it walks).  Built in a translation unit of its own so
// that its MFMAs take the VGPR accumulator form: the S^T / dP^T results
// feed VALU softmax work directly and the dQ accumulators stay put, where the
// AGPR form would copy them between register files every tile.

#include "mfma_common.h"

namespace usp {
namespace {

// -------------------------------------------------------------------- dQ
// Per 64-key tile and wave (32 query rows, one per lane):
//   A(kb): S^T and dP^T of key block kb (32 keys) = K Q^T, V dO^T;
//   B(kb): dS^T = exp2(S^T c - lse2) (dP^T - delta) -> bf16 (B-operand order);
//   C(kb): dQ^T += K^T dS^T.
// Issue order A0 A1 B0 C0 B1 C1, with B0's VALU work placed between A1's
// MFMAs and B1's between C0's, and every LDS fragment read issued kPF
// MFMAs ahead of its use.
template <int D, int MODS>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(const BwdParams p) {
  using T = SwzTile<D>;
  constexpr int BN = 64;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILEB = BN * D * 2;
  constexpr int LPW = TILEB / 4096;
  constexpr int RPI = 1024 / T::ROWB;
  constexpr int PF = kPF;
  static_assert(kTileN % BN == 0, "planner granularity");
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILEB];  // two buffers of (K, V)

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
  if (it.q_rows == 0) return;  // planner slot with nothing to do (whole workgroup)
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
  const int32_t pq_row = position(qm, it.t0 + (qvalid ? qr : 0));
  {
    const int32_t pq = pq_row;
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

  const int64_t kv_row_stride = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;
  const uint32_t row_bytes = (uint32_t)kv_row_stride * 2;
  const i32x4 krs = buffer_rsrc(kbase);
  const i32x4 vrs = buffer_rsrc(vbase);
  const int lrow = lane / T::CPR;
  const int lslot = lane % T::CPR;
  const float c = p.scale_log2;
  // ALiBi distances in f32 (positions below 2^22 are exact): a key t of the
  // key rank is at t + floor(t / b) (N - 1) b + rank b under the stripe
  // layout and at t + (p(k0) - k0) inside a run of the others (inv_b = 0
  // there), so p_k - p_q = floor((t + 0.5) inv_b) nb1 + t + rb.
  // rb of a tile: rb0, or rb1 for a tile in the second zigzag chunk.
  const bool kstripe = km.kind == MAP_STRIPE;
  const float inv_b = kstripe ? 1.f / (float)km.b : 0.f;
  const float nb1 = kstripe ? (float)((km.N - 1) * km.b) : 0.f;
  const int32_t khalf = km.kind == MAP_ZIGZAG ? km.L >> 1 : 0x7fffffff;
  const float rb0 = (float)((kstripe ? km.rank * km.b : position(km, 0)) - pq_row);
  const float rb1 = km.kind == MAP_ZIGZAG ? (float)(position(km, khalf) - khalf - pq_row) : rb0;
  const float slope = (MODS & 2) ? p.mods.alibi[h] * p.mods.inv_scale : 0.f;

  // The workgroup walks the key tiles of its runs with two LDS buffers: tile
  // n + 1 is copied global -> LDS directly (buffer loads to LDS) while tile
  // n is computed.  Thread (wave wid, lane i) copies slices wid*LPW + j of K
  // and V: physical (row, chunk slot) = (slice*RPI + i / CPR, i % CPR), i.e.
  // logical chunk slot ^ swz(row); rows past the run's end are clamped to its
  // last row (masked in partial runs; full runs are multiples of BN keys).
  auto dma = [&](char* buf, int k0, int kend) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int row = (wid * LPW + j) * RPI + lrow;
      const uint32_t off = (uint32_t)min(k0 + row, kend - 1) * row_bytes + (uint32_t)((lslot ^ T::swz(row)) * 16);
      copy16_to_lds(krs, lds_addr(buf + (wid * LPW + j) * 1024), off);
      copy16_to_lds(vrs, lds_addr(buf + TILEB + (wid * LPW + j) * 1024), off);
    }
  };

  // One tile.  FULL: every pair visible (no mask).  Otherwise element r of
  // key block kb is key k0 + du, du = kb*32 + 8*(r/4) + 4*hi + r%4; key
  // positions increase through the run, so this lane's visible keys (window
  // band, sinks) are at most two intervals of du, found once per tile.
  auto tile = [&](auto full_c, const char* tK, int k0, int kend) {
    constexpr bool FULL = decltype(full_c)::value;
    const char* tV = tK + TILEB;
    int32_t lo = 0, up = 0, slo = 0, sup = -1;
    if constexpr (!FULL) {
      const int32_t last = kend - 1 - k0;
      const int32_t sh = k0 + 4 * hi;
      lo = first_row_at_least(km, k0, vis_lo) - sh;
      up = min(first_row_at_least(km, k0, vis_hi + 1) - 1 - k0, last) - 4 * hi;
      slo = first_row_at_least(km, k0, sstart) - sh;
      sup = min(first_row_at_least(km, k0, sink_hi + 1) - 1 - k0, last) - 4 * hi;
    }
    auto visible = [&](int kb, int r) -> bool {
      if constexpr (FULL) {
        return true;
      } else {
        const int cc = kb * 32 + 8 * (r >> 2) + (r & 3);
        return ((cc >= lo) & (cc <= up)) | ((cc >= slo) & (cc <= sup));
      }
    };
    // fragment streams: A phase i -> (K or V row kb*32 + l32, chunk 2*(i/2)+hi);
    // C phase j -> K^T block (kb, half, d)
    auto read_a = [&](int i) {
      const int kb = i / (2 * KS), w = i % (2 * KS);
      return T::frag((w & 1) ? tV : tK, kb * 32 + l32, 2 * (w >> 1) + hi);
    };
    auto read_c = [&](int j) {
      const int kb = j / (2 * DB), half = (j / DB) & 1, d = j % DB;
      return frag_tr<D>(tK, kb, half, d, lane);
    };
    constexpr int NA = 2 * 2 * KS;   // A0 + A1 MFMAs
    constexpr int NC = 2 * 2 * DB;   // C0 + C1 MFMAs
    f32x16 st[2], dpt[2];
    bf16x8 fa[NA], fc[NC];
    bf16x8 dsb[2][2];
    const f32x16 zero = {};
#pragma unroll
    for (int i = 0; i < PF; ++i) fa[i] = read_a(i);
    // A0, A1 (B0 follows in program order; the groups below interleave it)
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i + PF < NA) fa[i + PF] = read_a(i + PF);
      else fc[i + PF - NA] = read_c(i + PF - NA);
      const int kb = i / (2 * KS), w = i % (2 * KS), ks = w >> 1;
      if (w & 1) dpt[kb] = mfma32(fa[i], dof[ks], ks == 0 ? zero : dpt[kb]);
      else st[kb] = mfma32(fa[i], qf[ks], ks == 0 ? zero : st[kb]);
    }
    // Score modifiers of element r of key block kb (raw units, as the
    // forward): softcap a - 2a rc with rc = 1 / (exp2(s b2) + 1), whose
    // derivative factor 1 - tanh^2 = 4 rc (1 - rc) scales dS; then ALiBi.
    float abase = 0.f, rb = 0.f;
    if constexpr ((MODS & 2) != 0) {
      abase = (float)(k0 + 4 * hi);
      rb = k0 >= khalf ? rb1 : rb0;
    }
    auto mods = [&](int kb, int r, float& sv, float& f, float ab) {
      if constexpr ((MODS & 1) != 0) {
        const float rc = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sv * p.mods.b2) + 1.f);
        sv = p.mods.a - 2.f * p.mods.a * rc;
        f = 4.f * rc * (1.f - rc);
      }
      if constexpr ((MODS & 2) != 0) {
        // key index t (the constant is added first so that it folds into one
        // instruction)
        const float t = ab + (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
        const float dd = __builtin_floorf((t + 0.5f) * inv_b) * nb1 + (t + rb);
        sv -= slope * __builtin_fabsf(dd);
      }
    };
    auto softmax = [&](int kb) {
      // The bias terms depend on nothing the MFMAs produce; the empty asm
      // keeps the compiler from hoisting all of them into live registers
      // ahead of the matrix products.
      float ab = abase;
      if constexpr ((MODS & 2) != 0) asm volatile("" : "+v"(ab));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r0 = half * 8 + e, r1 = r0 + 1;
          float s0 = st[kb][r0], s1 = st[kb][r1], f0 = 1.f, f1 = 1.f;
          if constexpr (MODS != 0) {
            mods(kb, r0, s0, f0, ab);
            mods(kb, r1, s1, f1, ab);
          }
          float p0 = __builtin_amdgcn_exp2f(s0 * c - lse2);
          float p1 = __builtin_amdgcn_exp2f(s1 * c - lse2);
          if constexpr (!FULL) {
            p0 = visible(kb, r0) ? p0 : 0.f;
            p1 = visible(kb, r1) ? p1 : 0.f;
          }
          float d0 = p0 * (dpt[kb][r0] - dl);
          float d1 = p1 * (dpt[kb][r1] - dl);
          if constexpr ((MODS & 1) != 0) {
            d0 *= f0;
            d1 *= f1;
          }
          const bf16x2 pk2 = __builtin_convertvector((f32x2){d0, d1}, bf16x2);
          dsb[kb][half][e] = pk2[0];
          dsb[kb][half][e + 1] = pk2[1];
        }
      }
    };
    softmax(0);
    softmax(1);
    // C0, C1
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (j + PF < NC) fc[j + PF] = read_c(j + PF);
      const int kb = j / (2 * DB), half = (j / DB) & 1, d = j % DB;
      dqt[d] = mfma32(fc[j], dsb[kb][half], dqt[d]);
    }
    // scheduling groups, in issue order: A0 (MFMA, read), A1 (MFMA, read,
    // B0's VALU), C0 (MFMA, reads, B1's VALU), C1 (MFMA, reads); a frag_tr
    // is two DS reads
    constexpr int NA0 = 2 * KS;
    constexpr int NC0 = 2 * DB;
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      sched_ds_read((i + PF < NA) ? 1 : 2);
      if (i >= NA0) __builtin_amdgcn_sched_group_barrier(0x002, kDqValuA, 0);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j + PF < NC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (j < NC0) __builtin_amdgcn_sched_group_barrier(0x002, kDqValuC, 0);
    }
  };

  int n_tiles = 0;
  for (int ri = it.run_begin; ri < it.run_end; ++ri) {
    const Run r = p.runs[ri];
    n_tiles += (r.k_end - r.k_begin + BN - 1) / BN;
  }
  int c_ri = it.run_begin;
  Run c_run = n_tiles > 0 ? p.runs[c_ri] : Run{0, 0, 0, 0};
  int c_k0 = c_run.k_begin;
  if (n_tiles > 0) dma(smem, c_k0, c_run.k_end);
  for (int n = 0; n < n_tiles; ++n) {
    const int k0 = c_k0;
    const Run run = c_run;
    const char* tK = smem + (n & 1) * 2 * TILEB;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile n are in LDS
    __syncthreads();                     // every wave's copies landed; tile n - 1's buffer is free
    if (n + 1 < n_tiles) {
      c_k0 += BN;
      if (c_k0 >= c_run.k_end) {
        c_run = p.runs[++c_ri];
        c_k0 = c_run.k_begin;
      }
      dma(smem + ((n + 1) & 1) * 2 * TILEB, c_k0, c_run.k_end);
    }
    if (run.full) tile(std::true_type{}, tK, k0, run.k_end);
    else tile(std::false_type{}, tK, k0, run.k_end);
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

}  // namespace

void launch_bwd_dq(const BwdParams& p, int D, unsigned grid, hipStream_t stream) {
  TimingScope ts(K_BWD_DQ, stream);
  const int mods = mods_variant(p.mods);
#define USP_LAUNCH_Q(DD, M) hipLaunchKernelGGL((bwd_dq_kernel<DD, M>), dim3(grid), dim3(256), 0, stream, p)
#define USP_LAUNCH_Q_M(DD)                  \
  switch (mods) {                           \
    case 0: USP_LAUNCH_Q(DD, 0); break;     \
    case 1: USP_LAUNCH_Q(DD, 1); break;     \
    case 2: USP_LAUNCH_Q(DD, 2); break;     \
    default: USP_LAUNCH_Q(DD, 3); break;    \
  }
  if (D == 128) { USP_LAUNCH_Q_M(128) } else { USP_LAUNCH_Q_M(64) }
#undef USP_LAUNCH_Q_M
#undef USP_LAUNCH_Q
}

}  // namespace usp
