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

#include "mfma_common.h"

namespace usp {
namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ delta
// delta[b, h, t] = sum_d dO[b, t, h, d] * O[b, t, h, d].  A group of D/8
// threads per (row, head) reads 8 consecutive elements each (16 bytes of
// dO, 32 or 16 of O), so a wave's loads are contiguous; the group (inside
// one wave: D/8 divides 64) sums with cross-lane adds in a fixed order.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void* out, int out_f32, const uint16_t* dout,
                                                        float* delta, int64_t n_rows, int32_t L, int32_t H,
                                                        int32_t D) {
  const int32_t tpr = D / 8;
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) / tpr;
  const int32_t j = threadIdx.x % tpr;
  const bool live = idx < n_rows;
  float acc = 0.f;
  if (live) {
    const int64_t e0 = idx * D + j * 8;
    const bf16x8 g = ld_nt(reinterpret_cast<const bf16x8*>(dout + e0));
    if (out_f32) {
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4 o0 = ld_nt(reinterpret_cast<const f32x4*>(static_cast<const float*>(out) + e0));
      const f32x4 o1 = ld_nt(reinterpret_cast<const f32x4*>(static_cast<const float*>(out) + e0 + 4));
      acc = (float)g[0] * o0.x + (float)g[1] * o0.y + (float)g[2] * o0.z + (float)g[3] * o0.w;
      acc += (float)g[4] * o1.x + (float)g[5] * o1.y + (float)g[6] * o1.z + (float)g[7] * o1.w;
    } else {
      const bf16x8 o = ld_nt(reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(out) + e0));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)g[e] * (float)o[e];
    }
  }
  for (int32_t off = tpr >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (!live || j != 0) return;
  const int64_t bt = idx / H;
  const int32_t h = (int32_t)(idx - bt * H);
  const int64_t b = bt / L;
  const int32_t t = (int32_t)(bt - b * L);
  delta[(b * H + h) * L + t] = acc;
}

// ------------------------------------------------------------------ dK dV
// Work item fields (the transposed plan): q_row0 = first key row of the tile
// in the k/v buffers, t0 = its local key index, q_rows = keys in the tile,
// q_rank = KV rank, k_row0 = row of local query 0 of the query rank in the
// q/dout buffers, k_rank = query rank; runs: local query rows
// [k_begin, k_end) and whether every pair of the run is visible.
//
// The workgroup walks one flat sequence of query tiles ((run, 64-row tile)
// backwards, query head of the KV group innermost) with two LDS buffers: tile n + 1 (Q, dO, LSE,
// delta) is copied global -> LDS directly (buffer loads to LDS) while tile
// n is computed.  Per tile and wave (32 keys, one per lane):
//   A(qb): S and dP of query block qb (32 rows) = Q K^T, dO V^T;
//   B(qb): P = exp2(S c - LSE log2 e), dS = P (dP - delta) -> bf16;
//   C(qb): dV^T += dO^T P, dK^T += Q^T dS.
// Issue order A0 A1 B0 B1 C0 C1, with B0's VALU work placed between A1's
// MFMAs and B1's between C0's, and LDS fragment reads kPF MFMAs ahead.
template <int D, int MODS>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using T = SwzTile<D>;
  constexpr int BQ = 64;            // query rows per tile
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILEB = BQ * D * 2;
  constexpr int LPW = TILEB / 4096;
  constexpr int RPI = 1024 / T::ROWB;
  constexpr int BUFB = 2 * TILEB + 2 * BQ * 4;  // Q, dO, LSE, delta
  constexpr int PF = kPF;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUFB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Items come sorted by decreasing work and the hardware deals consecutive
  // workgroups round-robin to the 8 XCDs, so the plain order gives every XCD
  // an even share of large and small items (with one KV head, a contiguous
  // block per XCD would hand one XCD all the largest).
  const int bid = blockIdx.x;
  const int hb = bid / p.n_items;
  const int item_idx = bid - hb * p.n_items;
  const int hk = hb % p.Hkv;
  const int b = hb / p.Hkv;
  const WorkItem it = p.items[item_idx];
  if (it.q_rows == 0) return;  // key tile no query sees (whole workgroup)
  const int group = p.Hq / p.Hkv;

  const int kr_ = wid * 32 + l32;
  const bool kvalid = kr_ < it.q_rows;
  const int64_t krow = (int64_t)it.q_row0 + kr_;
  const int64_t kv_row_stride = (int64_t)p.Hkv * D;

  // query tiles of this item: group heads x runs x ceil(run / BQ)
  int tiles_per_head = 0;
  for (int ri = it.run_begin; ri < it.run_end; ++ri) {
    const Run r = p.runs[ri];
    tiles_per_head += (r.k_end - r.k_begin + BQ - 1) / BQ;
  }
  const int n_tiles = tiles_per_head * group;

  // copy sources: heads hk*group .. hk*group+group-1 of the query rank's rows
  const int h0 = hk * group;
  const uint16_t* qbase = p.q + (int64_t)b * p.q_batch_stride + (int64_t)it.k_row0 * p.Hq * D + h0 * D;
  const uint16_t* obase = p.dout + (int64_t)b * p.g_batch_stride + (int64_t)it.k_row0 * p.Hq * D + h0 * D;
  const float* lbase = p.lse + ((int64_t)b * p.Hq + h0) * p.Lq_buf + it.k_row0;
  const float* dbase = p.delta + ((int64_t)b * p.Hq + h0) * p.Lq_buf + it.k_row0;
  const uint32_t qrow_bytes = (uint32_t)p.Hq * D * 2;
  const i32x4 qrs = buffer_rsrc(qbase);
  const i32x4 ors = buffer_rsrc(obase);
  const i32x4 lrs = buffer_rsrc(wid == 1 ? (const void*)dbase : (const void*)lbase);
  const int lrow = lane / T::CPR;
  const int lslot = lane % T::CPR;

  // Thread (wave wid, lane i) copies slices wid*LPW + j of Q and dO: physical
  // (row, chunk slot) = (slice*RPI + i / CPR, i % CPR), i.e. logical chunk
  // slot ^ swz(row) of that row; waves 0 and 1 copy the 64 LSE / delta
  // values.  Rows past the run's end are clamped to its last row (they are
  // masked in the partial runs that have them; full runs are multiples of
  // BQ rows).
  auto dma = [&](char* buf, int gi, int t0, int tend) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int row = (wid * LPW + j) * RPI + lrow;
      const uint32_t off = (uint32_t)min(t0 + row, tend - 1) * qrow_bytes + (uint32_t)(gi * D * 2) +
                           (uint32_t)((lslot ^ T::swz(row)) * 16);
      copy16_to_lds(qrs, lds_addr(buf + (wid * LPW + j) * 1024), off);
      copy16_to_lds(ors, lds_addr(buf + TILEB + (wid * LPW + j) * 1024), off);
    }
    if (wid < 2) {
      const uint32_t off = (uint32_t)(gi * p.Lq_buf + min(t0 + lane, tend - 1)) * 4u;
      copy4_to_lds(lrs, lds_addr(buf + 2 * TILEB + wid * BQ * 4), off);
    }
  };

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

  // This lane's key position pk; the query positions that see it form one
  // interval [lo_p, hi_p]: same sequence, p_q >= p_k under causal / window,
  // and p_q - p_k < W unless the key is one of its sequence's sinks.
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
  const bool sink = p.mask.window > 0 && pk - ks0 < p.mask.n_sink;
  const int32_t lo_p = cw ? max(ks0, pk) : ks0;
  const int32_t hi_p = (p.mask.window > 0 && !sink) ? min(ks1 - 1, pk + p.mask.window - 1) : ks1 - 1;
  const float c = p.scale_log2;
  // ALiBi distances in f32 (positions below 2^22 are exact): a row t of the
  // query rank is at t + floor(t / b) (N - 1) b + rank b under the stripe
  // layout and at t + (p(t0) - t0) inside a monotone piece of the others
  // (inv_b = 0 there), so p_q - p_k = floor((t + 0.5) inv_b) nb1 + t + rb.
  // rb of a tile: rb0, or rb1 for a tile in the second zigzag chunk.
  const bool qstripe = qm.kind == MAP_STRIPE;
  const float inv_b = qstripe ? 1.f / (float)qm.b : 0.f;
  const float nb1 = qstripe ? (float)((qm.N - 1) * qm.b) : 0.f;
  const int32_t qhalf = qm.kind == MAP_ZIGZAG ? qm.L >> 1 : 0x7fffffff;
  const float rb0 = (float)((qstripe ? qm.rank * qm.b : position(qm, 0)) - pk);
  const float rb1 = qm.kind == MAP_ZIGZAG ? (float)(position(qm, qhalf) - qhalf - pk) : rb0;

  // One tile.  FULL: every pair visible.  Otherwise element r of query
  // block qb is local row t0 + qb*32 + 8*(r/4) + 4*hi + r%4; query
  // positions increase through the run, so the rows that see this lane's
  // key are one interval, found once per tile.
  auto tile = [&](auto full_c, const char* buf, int t0, int tend, int gi) {
    constexpr bool FULL = decltype(full_c)::value;
    const char* tQ = buf;
    const char* tO = buf + TILEB;
    const float* sl = reinterpret_cast<const float*>(buf + 2 * TILEB);
    const float* sd = sl + BQ;
    int32_t lo = 0, up = 0;
    if constexpr (!FULL) {
      lo = first_row_at_least(qm, t0, lo_p) - t0 - 4 * hi;
      up = min(first_row_at_least(qm, t0, hi_p + 1) - 1, tend - 1) - t0 - 4 * hi;
    }
    auto visible = [&](int qb, int r) -> bool {
      if constexpr (FULL) {
        return true;
      } else {
        const int cc = qb * 32 + 8 * (r >> 2) + (r & 3);
        return (cc >= lo) & (cc <= up);
      }
    };
    auto read_a = [&](int i) {
      const int qb = i / (2 * KS), w = i % (2 * KS);
      return T::frag((w & 1) ? tO : tQ, qb * 32 + l32, 2 * (w >> 1) + hi);
    };
    // C stream j: (qb, half, d, which): which 0 -> dO^T for dV, 1 -> Q^T for dK
    auto read_c = [&](int j) {
      const int qb = j / (4 * DB), r = j % (4 * DB), half = r / (2 * DB), d = (r / 2) % DB;
      return frag_tr<D>((r & 1) ? tQ : tO, qb, half, d, lane);
    };
    constexpr int NA = 2 * 2 * KS;
    constexpr int NC = 2 * 4 * DB;
    f32x16 s[2], dp[2];
    bf16x8 fa[NA], fc[NC];
    bf16x8 pb[2][2], dsb[2][2];
    const f32x16 zero = {};
    // LSE and delta of this lane's 16 query rows per block (rows
    // qb*32 + 8*g + 4*hi + 0..3 for g = 0..3)
    float4 l4[2][4], d4[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        l4[qb][g] = *reinterpret_cast<const float4*>(sl + qb * 32 + 8 * g + 4 * hi);
        d4[qb][g] = *reinterpret_cast<const float4*>(sd + qb * 32 + 8 * g + 4 * hi);
      }
#pragma unroll
    for (int i = 0; i < PF; ++i) fa[i] = read_a(i);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i + PF < NA) fa[i + PF] = read_a(i + PF);
      else fc[i + PF - NA] = read_c(i + PF - NA);
      const int qb = i / (2 * KS), w = i % (2 * KS), ks = w >> 1;
      if (w & 1) dp[qb] = mfma32(fa[i], vf[ks], ks == 0 ? zero : dp[qb]);
      else s[qb] = mfma32(fa[i], kf[ks], ks == 0 ? zero : s[qb]);
    }
    // Score modifiers of element r of block qb (raw units, as the
    // forward): softcap a - 2a rc with rc = 1 / (exp2(s b2) + 1), whose
    // derivative factor 1 - tanh^2 = 4 rc (1 - rc) scales dS; then ALiBi.
    float slope = 0.f, abase = 0.f, rb = 0.f;
    if constexpr ((MODS & 2) != 0) {
      slope = p.mods.alibi[h0 + gi] * p.mods.inv_scale;
      abase = (float)(t0 + 4 * hi);
      rb = t0 >= qhalf ? rb1 : rb0;
    }
    auto mods = [&](int qb, int r, float& sv, float& f, float ab) {
      if constexpr ((MODS & 1) != 0) {
        const float rc = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sv * p.mods.b2) + 1.f);
        sv = p.mods.a - 2.f * p.mods.a * rc;
        f = 4.f * rc * (1.f - rc);
      }
      if constexpr ((MODS & 2) != 0) {
        // row index t (the constant is added first so that it folds into one
        // instruction)
        const float t = ab + (float)(qb * 32 + 8 * (r >> 2) + (r & 3));
        const float dd = __builtin_floorf((t + 0.5f) * inv_b) * nb1 + (t + rb);
        sv -= slope * __builtin_fabsf(dd);
      }
    };
    auto softmax = [&](int qb) {
      // The bias terms depend on nothing the MFMAs produce; the empty asm
      // keeps the compiler from hoisting all of them into live registers
      // ahead of the matrix products.
      float ab = abase;
      if constexpr ((MODS & 2) != 0) asm volatile("" : "+v"(ab));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float lq[4] = {l4[qb][g].x, l4[qb][g].y, l4[qb][g].z, l4[qb][g].w};
        const float dq4[4] = {d4[qb][g].x, d4[qb][g].y, d4[qb][g].z, d4[qb][g].w};
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const int r0 = 4 * g + e, r1 = r0 + 1;
          float s0 = s[qb][r0], s1 = s[qb][r1], f0 = 1.f, f1 = 1.f;
          if constexpr (MODS != 0) {
            mods(qb, r0, s0, f0, ab);
            mods(qb, r1, s1, f1, ab);
          }
          float p0 = __builtin_amdgcn_exp2f(s0 * c - lq[e] * kLog2e);
          float p1 = __builtin_amdgcn_exp2f(s1 * c - lq[e + 1] * kLog2e);
          if constexpr (!FULL) {
            p0 = visible(qb, r0) ? p0 : 0.f;
            p1 = visible(qb, r1) ? p1 : 0.f;
          }
          float d0 = p0 * (dp[qb][r0] - dq4[e]);
          float d1 = p1 * (dp[qb][r1] - dq4[e + 1]);
          if constexpr ((MODS & 1) != 0) {
            d0 *= f0;
            d1 *= f1;
          }
          const bf16x2 pp = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
          const bf16x2 dd = __builtin_convertvector((f32x2){d0, d1}, bf16x2);
          pb[qb][r0 >> 3][r0 & 7] = pp[0];
          pb[qb][r0 >> 3][r1 & 7] = pp[1];
          dsb[qb][r0 >> 3][r0 & 7] = dd[0];
          dsb[qb][r0 >> 3][r1 & 7] = dd[1];
        }
      }
    };
    softmax(0);
    softmax(1);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (j + PF < NC) fc[j + PF] = read_c(j + PF);
      const int qb = j / (4 * DB), r = j % (4 * DB), half = r / (2 * DB), d = (r / 2) % DB;
      if (r & 1) dkt[d] = mfma32(fc[j], dsb[qb][half], dkt[d]);
      else dvt[d] = mfma32(fc[j], pb[qb][half], dvt[d]);
    }
    // scheduling groups, in issue order: the LSE / delta reads, A0 (MFMA,
    // read), A1 (MFMA, read, B0's VALU), C0 (MFMA, reads, B1's VALU), C1
    // (MFMA, reads)
    constexpr int NA0 = 2 * KS;
    constexpr int NC0 = 4 * DB;
    __builtin_amdgcn_sched_group_barrier(0x100, 16 + PF, 0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      sched_ds_read((i + PF < NA) ? 1 : 2);
      if (i >= NA0) __builtin_amdgcn_sched_group_barrier(0x002, kKvValuA, 0);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j + PF < NC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (j < NC0) __builtin_amdgcn_sched_group_barrier(0x002, kKvValuC, 0);
    }
  };

  // Tile order: query tiles from the last run's last tile backwards, the
  // group's query heads innermost.  Under a causal mask every key tile's
  // query range ends at the rank's last row, so the workgroups resident at
  // one time start at the same rows and stream the same Q / dO tiles at
  // about the same time (shared through L2 instead of refetched).
  auto last_tile = [](const Run& r) { return r.k_begin + ((r.k_end - r.k_begin - 1) / BQ) * BQ; };
  int c_gi = 0, c_ri = it.run_end - 1;
  Run c_run = p.runs[c_ri];
  int c_t0 = last_tile(c_run);
  dma(smem, c_gi, c_t0, c_run.k_end);

  for (int n = 0; n < n_tiles; ++n) {
    const int gi = c_gi;
    const int t0 = c_t0;
    const int t_end = c_run.k_end;
    const bool full = c_run.full != 0;
    const char* buf = smem + (n & 1) * BUFB;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile n are in LDS
    __syncthreads();                     // every wave's copies landed; tile n - 1's buffer is free
    if (n + 1 < n_tiles) {
      if (++c_gi == group) {
        c_gi = 0;
        c_t0 -= BQ;
        if (c_t0 < c_run.k_begin) {
          c_run = p.runs[--c_ri];
          c_t0 = last_tile(c_run);
        }
      }
      dma(smem + ((n + 1) & 1) * BUFB, c_gi, c_t0, c_run.k_end);
    }
    if (full) tile(std::true_type{}, buf, t0, t_end, gi);
    else tile(std::false_type{}, buf, t0, t_end, gi);
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
    const int64_t threads = n * (D / 8);
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, out,
                       out_f32, dout, delta, n, (int32_t)L, (int32_t)H, (int32_t)D);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("delta launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

usp_status launch_bwd(const BwdParams& pq, const BwdParams& pkv, int D, hipStream_t stream) {
  const int64_t nq = (int64_t)pq.n_items * pq.Hq * pq.B;
  const int64_t nk = (int64_t)pkv.n_items * pkv.Hkv * pkv.B;
  if (nq > 0x7fffffff || nk > 0x7fffffff) {
    set_error("backward grid too large");
    return USP_ERR_UNSUPPORTED;
  }
  if (nq > 0) launch_bwd_dq(pq, D, (unsigned)nq, stream);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && nk > 0) {
    TimingScope ts(K_BWD_DKDV, stream);
    const int mods = mods_variant(pkv.mods);
#define USP_LAUNCH_KV(DD, M) hipLaunchKernelGGL((bwd_dkdv_kernel<DD, M>), dim3((unsigned)nk), dim3(256), 0, stream, pkv)
#define USP_LAUNCH_KV_M(DD)                  \
  switch (mods) {                            \
    case 0: USP_LAUNCH_KV(DD, 0); break;     \
    case 1: USP_LAUNCH_KV(DD, 1); break;     \
    case 2: USP_LAUNCH_KV(DD, 2); break;     \
    default: USP_LAUNCH_KV(DD, 3); break;    \
  }
    if (D == 128) { USP_LAUNCH_KV_M(128) } else { USP_LAUNCH_KV_M(64) }
#undef USP_LAUNCH_KV_M
#undef USP_LAUNCH_KV
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    set_error("backward launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
