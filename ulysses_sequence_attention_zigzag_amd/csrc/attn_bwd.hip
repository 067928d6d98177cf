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
//   bwd_dkdv_kernel: 8 waves in pairs over 32 keys each (one key per
//                    lane); Q, dO, LSE and delta of 64-row query tiles in
//                    LDS; in each pair one wave holds K, forms S = Q K^T and
//                    P and accumulates dV^T += dO^T P, the other holds V,
//                    forms dP = dO V^T and dS (P through LDS) and
//                    accumulates dK^T += Q^T dS, the two alternating
//                    between the matrix core and the vector ALU.
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
// Wave roles.  8 waves: wave wg (0-3) and wave wg + 4 share the 32 keys
// wg*32 .. +31 of the tile (one key per lane) and, by the hardware's
// placement, one SIMD.  Wave wg (the P wave) holds K and accumulates dV^T;
// wave wg + 4 (the dS wave) holds V and accumulates dK^T.  Per 64-row query
// tile n (Q, dO, LSE, delta), with S = Q K^T and dP = dO V^T in the C layout
// of the forward kernel (lane = key, 16 query rows per 32-row block):
//   P wave:  S(n)                  [matrix]
//            P = exp2(S c - LSE log2 e) -> bf16 P for dV, and to the LDS
//            exchange (times the softcap derivative)   [vector]
//            dV^T += dO^T P         [matrix]
//   dS wave: delta - dP(n)         [matrix: -V fragments, C = delta]
//            dS = -P (delta - dP) from the exchange   [vector]
//            dK^T += Q^T dS         [matrix]
// The two waves of a SIMD alternate: in phase 2n the P wave runs its
// softmax of tile n while the dS wave runs dK(n-1) and dP(n) on the matrix
// core; in phase 2n+1 the P wave runs dV(n) and S(n+1) while the dS wave
// forms dS(n).  Every phase ends with a workgroup barrier (no memory fence;
// each wave waits for its own LDS writes and tile loads explicitly first).
// Tile staging straight into LDS: the P waves load Q (3 buffers: Q(n) is
// read in phases 2n-1 .. 2n+2), issued two phases ahead of use; the dS
// waves load dO, LSE and delta (2 buffers, read in phases 2n, 2n+1); once
// a tile's LSE has landed, dS wave 0 rewrites it in place as -LSE log2 e,
// the exp2 argument's second term.
template <int D, int MODS>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using T = SwzTile<D>;
  constexpr int BQ = 64;                    // query rows per tile
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILEB = BQ * D * 2;         // one Q or dO tile
  constexpr int LPT = TILEB / 4096;         // 16-byte copies per thread of a 4-wave group
  constexpr int RPI = 1024 / T::ROWB;
  constexpr int OBUFB = TILEB + 2 * BQ * 4; // dO, LSE, delta
  constexpr int XB = BQ * 32 * 2;           // P exchange of one wave pair (bf16)
  static_assert(TILEB % 4096 == 0 && OBUFB % 512 == 0, "tile layout");
  __shared__ __attribute__((aligned(1024))) char smem[3 * TILEB + 2 * OBUFB + 4 * XB];
  char* const qbuf = smem;
  char* const obuf = smem + 3 * TILEB;
  char* const xbuf = obuf + 2 * OBUFB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2;   // 0: P wave, 1: dS wave
  const int wg = wid & 3;     // key slice
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Items come sorted by decreasing work and the hardware deals consecutive
  // workgroups round-robin to the 8 XCDs (and, inside one, to its shader
  // engines), so the plain order gives every XCD an even share of large and
  // small items (with one KV head, a contiguous block per XCD would hand one
  // XCD all the largest).  The heads of one item are adjacent: ordered
  // head-major, each head's largest item sat n_items workgroups from the
  // next one's, which with n_items a multiple of 32 put all of them on one
  // shader engine of one XCD (varlen steps whose work is a few long items
  // ran them 8 at a time).
  const int bid = blockIdx.x;
  const int n_hb = p.Hkv * p.B;
  const int item_idx = bid / n_hb;
  const int hb = bid - item_idx * n_hb;
  const int hk = hb % p.Hkv;
  const int b = hb / p.Hkv;
  const WorkItem it = p.items[item_idx];
  if (it.q_rows == 0) return;  // planner slot with nothing to do (whole workgroup)
  const int group = p.Hq / p.Hkv;

  const int kr_ = wg * 32 + l32;
  const bool kvalid = kr_ < it.q_rows;
  const int64_t krow = (int64_t)it.q_row0 + kr_;
  const int64_t kv_row_stride = (int64_t)p.Hkv * D;
  if (it.run_begin == it.run_end) {  // no query sees these keys (whole workgroup)
    // a storing launch still writes their gradient rows: dV (P waves), dK
    if (p.overwrite && kvalid) {
      float* dst = (grp ? p.dk : p.dv) + (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<float4*>(dst + d * 32 + 8 * g + 4 * hi) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }

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
  const i32x4 trs = buffer_rsrc(grp ? (const void*)obase : (const void*)qbase);
  const i32x4 lrs = buffer_rsrc(wg == 1 ? (const void*)dbase : (const void*)lbase);
  const int lrow = lane / T::CPR;
  const int lslot = lane % T::CPR;

  // Tile cursor: query tiles from the last run's last tile backwards, the
  // group's query heads innermost.  Under a causal mask every key tile's
  // query range ends at the rank's last row, so the workgroups resident at
  // one time start at the same rows and stream the same Q / dO tiles at
  // about the same time (shared through L2 instead of refetched).
  struct Cursor {
    int gi, ri, t0;
    Run run;
  };
  auto last_tile = [](const Run& r) { return r.k_begin + ((r.k_end - r.k_begin - 1) / BQ) * BQ; };
  Cursor c0;
  c0.gi = 0;
  c0.ri = it.run_end - 1;
  c0.run = p.runs[c0.ri];
  c0.t0 = last_tile(c0.run);
  auto advance = [&](Cursor& c) {  // only while another tile follows
    if (++c.gi == group) {
      c.gi = 0;
      c.t0 -= BQ;
      if (c.t0 < c.run.k_begin) {
        c.run = p.runs[--c.ri];
        c.t0 = last_tile(c.run);
      }
    }
  };

  // Tile copy by this wave's group (Q for the P waves; dO, LSE and delta for
  // the dS waves): thread (wave wg, lane i) copies slices wg*LPT + j, i.e.
  // physical (row, chunk slot) = (slice*RPI + i / CPR, i % CPR) = logical
  // chunk slot ^ swz(row) of that row; dS waves 0 and 1 copy the 64 LSE /
  // delta values.  Rows past the run's end are clamped to its last row
  // (masked in the partial runs that have them; full runs are multiples of
  // BQ rows).
  // The offsets' lane parts are loop-invariant: row s*RPI + lrow of slice
  // s = wg*LPT + j has a swizzle that depends on s only through j (s*RPI/RPL
  // = 4s, and wg*LPT is a multiple of the swizzle's period in s), and the
  // clamp distributes over the row stride, so a slice costs an add and a
  // min besides the copy.  (Named scalars, not an array: the copy lambdas
  // run inside the matrix phase's unrolled loop.)
  const uint32_t lrb = (uint32_t)lrow * qrow_bytes;
  const uint32_t lsw0 = (uint32_t)((lslot ^ T::swz(lrow)) * 16);
  const uint32_t lsw1 = (uint32_t)((lslot ^ T::swz(RPI + lrow)) * 16);
  const uint32_t lsw2 = (uint32_t)((lslot ^ T::swz(2 * RPI + lrow)) * 16);
  const uint32_t lsw3 = (uint32_t)((lslot ^ T::swz(3 * RPI + lrow)) * 16);
  static_assert(LPT <= 4, "four lane swizzles");
  auto dma_slice = [&](char* buf, const Cursor& c, int j) {
    const uint32_t rows = min(lrb + (uint32_t)(c.t0 + (wg * LPT + j) * RPI) * qrow_bytes,
                              (uint32_t)(c.run.k_end - 1) * qrow_bytes);
    const uint32_t off = rows + (uint32_t)(c.gi * D * 2) + (j == 0 ? lsw0 : j == 1 ? lsw1 : j == 2 ? lsw2 : lsw3);
    copy16_to_lds(trs, lds_addr(buf + (wg * LPT + j) * 1024), off);
  };

  auto dma_side = [&](char* buf, const Cursor& c) {
    if (grp == 1 && wg < 2) {
      const uint32_t off = (uint32_t)(c.gi * p.Lq_buf + min(c.t0 + lane, c.run.k_end - 1)) * 4u;
      copy4_to_lds(lrs, lds_addr(buf + TILEB + wg * BQ * 4), off);
    }
  };
  auto dma = [&](char* buf, const Cursor& c) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma_slice(buf, c, j);
    dma_side(buf, c);
  };
  // Inside a matrix phase of NM MFMAs: slice j after MFMA FIRST + j*STRIDE
  // (mfma_common.h's placement; the copies then overlap the matrix work
  // instead of delaying the barrier).  Past the last tile the copy repeats
  // the last one into the free buffer, which nothing reads again: the phase
  // keeps a single straight-line body.
  auto copy_in = [&](char* buf, const Cursor* c, auto nm_c) {
    constexpr int STRIDE = kCopyStride > 0 ? kCopyStride : decltype(nm_c)::value / LPT;
    constexpr int FIRST = kCopyFirst >= 0 ? kCopyFirst : STRIDE - 1;
    static_assert(FIRST + (LPT - 1) * STRIDE < decltype(nm_c)::value, "copy positions");
    return [&dma_slice, buf, c](int m) {
      if (m >= FIRST && (m - FIRST) % STRIDE == 0 && (m - FIRST) / STRIDE < LPT) dma_slice(buf, *c, (m - FIRST) / STRIDE);
    };
  };

  // K (P waves) or -V (dS waves, sign bits flipped: exact) fragments of this
  // lane's key: B operand
  bf16x8 kv[KS];
  {
    const uint16_t* src = (grp ? p.v : p.k) + (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D + hi * 8;
    const uint32_t flip = grp ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (kvalid) {
        uint4 u = *reinterpret_cast<const uint4*>(src + ks * 16);
        u.x ^= flip;
        u.y ^= flip;
        u.z ^= flip;
        u.w ^= flip;
        kv[ks] = __builtin_bit_cast(bf16x8, u);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[ks][e] = (__bf16)0.f;
      }
    }
  }
  // acc: dV^T (P waves) or dK^T (dS waves); sc: S or delta - dP of the two
  // 32-row blocks; bb: bf16 P or dS (B operand of the accumulating products)
  f32x16 acc[DB], sc[2];
  bf16x8 bb[2][2];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;

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
  float cap_a = p.mods.a, cap_2a = 2.f * p.mods.a, cap_b2 = p.mods.b2;
  if constexpr ((MODS & 1) != 0) asm("" : "+v"(cap_a), "+v"(cap_2a), "+v"(cap_b2));

  // Matrix phases: acc += X^T bb (X = dO for dV, Q for dK), then sc = Y kv
  // (Y = Q for S, dO for dP).
  int tro[2][DB], rro[KS];
  pp_offsets<D>(lane, tro, rro);
  auto m_phase = [&](auto do_t_c, auto do_r_c, uint32_t tT, uint32_t tR, const f32x16(&c0)[2], auto&& hook) {
    pp_matrix_phase<D, decltype(do_t_c)::value, decltype(do_r_c)::value>(acc, sc, bb, kv, tro, rro, tT, tR, c0, hook);
  };
  const auto no_copy = [](int) {};
  // C operands of the first S MFMA (0) and of the first dP MFMA (delta of
  // the tile's rows, element r of block qb for row qb*32 + 8*(r/4) + 4*hi +
  // r%4, read from the tile's side buffer)
  f32x16 c_zero[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) c_zero[0][r] = c_zero[1][r] = 0.f;
  auto delta_c = [&](f32x16 (&cd)[2], const char* ob) {
    const float* sd = reinterpret_cast<const float*>(ob + TILEB + BQ * 4);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4*>(sd + qb * 32 + 8 * g + 4 * hi);
        cd[qb][4 * g] = d4.x;
        cd[qb][4 * g + 1] = d4.y;
        cd[qb][4 * g + 2] = d4.z;
        cd[qb][4 * g + 3] = d4.w;
      }
  };
  // dS wave 0, once its tile's LSE has landed: LSE -> -LSE log2 e in place
  // (its own copy, so the wait on its own loads covers it); the write is
  // complete before the barrier that follows.
  auto fix_lse = [&](char* ob) {
    if (wg == 0) {
      asm volatile("" ::: "memory");
      float* sl = reinterpret_cast<float*>(ob + TILEB);
      sl[lane] = -sl[lane] * kLog2e;
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    }
  };

  // P exchange slot of this wave pair: the 8 bf16 of (block qb, half) of
  // lane l at ((qb * 2 + half) * 64 + l) * 16, in the B-operand order
  char* const xw = xbuf + wg * XB;

  // Vector phase of the P wave: P of tile `cur` (S in sc), element r of
  // block qb is local row t0 + qb*32 + 8*(r/4) + 4*hi + r%4 of head gi.
  // FULL: every pair visible; otherwise the rows that see this lane's key
  // are one interval (query positions increase through a run), found once.
  auto softmax = [&](auto full_c, const Cursor& cur, const char* ob) {
    constexpr bool FULL = decltype(full_c)::value;
    const float* sl = reinterpret_cast<const float*>(ob + TILEB);
    const int t0 = cur.t0;
    int32_t lo = 0, up = 0;
    if constexpr (!FULL) {
      lo = first_row_at_least(qm, t0, lo_p) - t0 - 4 * hi;
      up = min(first_row_at_least(qm, t0, hi_p + 1) - 1, cur.run.k_end - 1) - t0 - 4 * hi;
    }
    // Score modifiers (raw units, as the forward): softcap a - 2a rc with
    // rc = 1 / (exp2(s b2) + 1), whose derivative factor 1 - tanh^2 =
    // 4 rc (1 - rc) scales dS (the exchange carries P times it); then ALiBi.
    float slope = 0.f, ab = 0.f, rb = 0.f;
    if constexpr ((MODS & 2) != 0) {
      slope = p.mods.alibi[h0 + cur.gi] * p.mods.inv_scale;
      ab = (float)(t0 + 4 * hi);
      rb = t0 >= qhalf ? rb1 : rb0;
    }
    bf16x8 xf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *reinterpret_cast<const float4*>(sl + qb * 32 + 8 * g + 4 * hi);
        const float lq[4] = {l4.x, l4.y, l4.z, l4.w};
        float px[4], pf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float sv = sc[qb][r], f = 1.f;
          if constexpr ((MODS & 1) != 0) {
            const float rc = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sv * cap_b2) + 1.f);
            sv = cap_a - cap_2a * rc;
            f = 4.f * rc * (1.f - rc);
          }
          if constexpr ((MODS & 2) != 0) {
            const float t = ab + (float)(qb * 32 + 8 * g + e);
            const float dd = __builtin_floorf((t + 0.5f) * inv_b) * nb1 + (t + rb);
            sv -= slope * __builtin_fabsf(dd);
          }
          float pe = __builtin_amdgcn_exp2f(fmaf(sv, c, lq[e]));
          if constexpr (!FULL) {
            const int cc = qb * 32 + 8 * g + e;
            pe = ((cc >= lo) & (cc <= up)) ? pe : 0.f;
          }
          px[e] = pe;
          pf[e] = ((MODS & 1) != 0) ? pe * f : pe;
        }
        const bf16x2 p01 = __builtin_convertvector((f32x2){px[0], px[1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector((f32x2){px[2], px[3]}, bf16x2);
        const int half = g >> 1, e0 = (g & 1) * 4;
        bb[qb][half][e0] = p01[0];
        bb[qb][half][e0 + 1] = p01[1];
        bb[qb][half][e0 + 2] = p23[0];
        bb[qb][half][e0 + 3] = p23[1];
        if constexpr ((MODS & 1) != 0) {
          const bf16x2 f01 = __builtin_convertvector((f32x2){pf[0], pf[1]}, bf16x2);
          const bf16x2 f23 = __builtin_convertvector((f32x2){pf[2], pf[3]}, bf16x2);
          xf[qb][half][e0] = f01[0];
          xf[qb][half][e0 + 1] = f01[1];
          xf[qb][half][e0 + 2] = f23[0];
          xf[qb][half][e0 + 3] = f23[1];
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        *reinterpret_cast<bf16x8*>(xw + ((qb * 2 + half) * 64 + lane) * 16) =
            ((MODS & 1) != 0) ? xf[qb][half] : bb[qb][half];
      if constexpr (!FULL) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Vector phase of the dS wave: dS = -P (delta - dP), the latter in sc.
  auto form_ds = [&]() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bf16x8 xh[2] = {*reinterpret_cast<const bf16x8*>(xw + (qb * 2 * 64 + lane) * 16),
                            *reinterpret_cast<const bf16x8*>(xw + ((qb * 2 + 1) * 64 + lane) * 16)};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int hh = g >> 1, o = (g & 1) * 4;
        const float4 px = make_float4((float)xh[hh][o], (float)xh[hh][o + 1], (float)xh[hh][o + 2], (float)xh[hh][o + 3]);
        const float d0 = -(px.x * sc[qb][4 * g]);
        const float d1 = -(px.y * sc[qb][4 * g + 1]);
        const float d2 = -(px.z * sc[qb][4 * g + 2]);
        const float d3 = -(px.w * sc[qb][4 * g + 3]);
        const bf16x2 a01 = __builtin_convertvector((f32x2){d0, d1}, bf16x2);
        const bf16x2 a23 = __builtin_convertvector((f32x2){d2, d3}, bf16x2);
        const int half = g >> 1, e0 = (g & 1) * 4;
        bb[qb][half][e0] = a01[0];
        bb[qb][half][e0 + 1] = a01[1];
        bb[qb][half][e0 + 2] = a23[0];
        bb[qb][half][e0 + 3] = a23[1];
      }
    }
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  auto barrier = []() { pp_barrier(); };
  auto prio_hi = []() { __builtin_amdgcn_s_setprio(1); };
  auto prio_lo = []() { __builtin_amdgcn_s_setprio(0); };
  auto qb_at = [&](int n) { return qbuf + (n % 3) * TILEB; };
  auto ob_at = [&](int n) { return obuf + (n & 1) * OBUFB; };
  auto ql_at = [&](int n) { return lds_addr(qb_at(n)); };
  auto ol_at = [&](int n) { return lds_addr(ob_at(n)); };

  // Epilogue: dV (P waves) or scale * dK (dS waves) added into the f32
  // gradients of this lane's key (stored alone by a storing launch).
  // The gradient this call adds to is loaded before the role's last matrix
  // phase (K or V and the S / dP results are dead by then), which covers
  // part of the load's latency: the store is a fifth to a quarter of a
  // short (window) item's time.
  float4 prev[DB][4];
  auto load_prev = [&](const float* base) {
    if (!kvalid) return;
    if (p.overwrite) {  // storing launch: nothing to add to
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) prev[d][g] = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    const float* src = base + (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) prev[d][g] = *reinterpret_cast<const float4*>(src + d * 32 + 8 * g + 4 * hi);
  };
  auto store = [&](float* base, float w) {
    if (!kvalid) return;
    float* dst = base + (int64_t)b * p.kv_batch_stride + krow * kv_row_stride + hk * D;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + 8 * g + 4 * hi;
        float4 a = prev[d][g];
        a.x += w * acc[d][4 * g];
        a.y += w * acc[d][4 * g + 1];
        a.z += w * acc[d][4 * g + 2];
        a.w += w * acc[d][4 * g + 3];
        *reinterpret_cast<float4*>(dst + dd) = a;
      }
    }
  };

  // The two roles run separate programs that pass the same barriers:
  // prologue (tile 0 lands; the P waves compute S(0)), two phases per tile,
  // and the dS waves' last dK after the final barrier.  Each loop body holds
  // one copy of its matrix phase (the first and last tiles' phases are
  // peeled), so the accumulators keep their registers across iterations.
  if (grp == 0) {
    Cursor cs = c0;  // tile of S / softmax
    Cursor cq = c0;  // tile of the last Q copy
    dma(qb_at(0), cq);
    if (n_tiles > 1) {
      advance(cq);
      dma(qb_at(1), cq);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    barrier();
    prio_hi();
    m_phase(F_{}, T_{}, 0u, ql_at(0), c_zero, no_copy);
    prio_lo();
    barrier();
    // phase 0: softmax of tile 0
    if (cs.run.full) softmax(T_{}, cs, ob_at(0));
    else softmax(F_{}, cs, ob_at(0));
    // the exchange writes, and Q(1) complete
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    barrier();
    for (int n = 0; n + 1 < n_tiles; ++n) {
      // phase 2n+1: dV(n), S(n+1); Q(n+2) copied meanwhile
      if (n + 2 < n_tiles) advance(cq);
      prio_hi();
      m_phase(T_{}, T_{}, ol_at(n), ql_at(n + 1), c_zero, copy_in(qb_at(n + 2), &cq, std::integral_constant<int, 4 * KS>{}));
      prio_lo();
      advance(cs);
      barrier();
      // phase 2n+2: softmax of tile n+1
      if (cs.run.full) softmax(T_{}, cs, ob_at(n + 1));
      else softmax(F_{}, cs, ob_at(n + 1));
      // the exchange writes, and Q(n+2) (copied since phase 2n+1), complete
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      barrier();
    }
    // phase 2N-1: dV(N-1)
    prio_hi();
    load_prev(p.dv);
    m_phase(T_{}, F_{}, ol_at(n_tiles - 1), 0u, c_zero, no_copy);
    prio_lo();
    barrier();
    store(p.dv, 1.f);
  } else {
    Cursor co = c0;  // tile of the last dO copy
    f32x16 cd[2];    // delta of the next dP's rows
    dma(ob_at(0), co);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    fix_lse(ob_at(0));
    barrier();
    barrier();
    // phase 0: dP(0)
    delta_c(cd, ob_at(0));
    prio_hi();
    m_phase(F_{}, T_{}, 0u, ol_at(0), cd, no_copy);
    prio_lo();
    if (n_tiles > 1) {
      advance(co);
      dma(ob_at(1), co);
    }
    barrier();
    // phase 1: dS(0)
    form_ds();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): dO(1) landed
    if (n_tiles > 1) fix_lse(ob_at(1));
    barrier();
    for (int n = 0; n + 1 < n_tiles; ++n) {
      // phase 2n+2: dK(n), dP(n+1); dO(n+2) copied meanwhile
      if (n + 2 < n_tiles) advance(co);
      delta_c(cd, ob_at(n + 1));
      prio_hi();
      m_phase(T_{}, T_{}, ql_at(n), ol_at(n + 1), cd, copy_in(ob_at(n + 2), &co, std::integral_constant<int, 4 * KS>{}));
      prio_lo();
      if (n + 2 < n_tiles) dma_side(ob_at(n + 2), co);
      barrier();
      // phase 2n+3: dS(n+1)
      form_ds();
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): dO(n+2) landed
      if (n + 2 < n_tiles) fix_lse(ob_at(n + 2));
      barrier();
    }
    // phase 2N: dK(N-1)
    prio_hi();
    load_prev(p.dk);
    m_phase(T_{}, F_{}, ql_at(n_tiles - 1), 0u, c_zero, no_copy);
    prio_lo();
    store(p.dk, p.scale);
  }
}

}  // namespace

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
#define USP_LAUNCH_KV(DD, M) hipLaunchKernelGGL((bwd_dkdv_kernel<DD, M>), dim3((unsigned)nk), dim3(512), 0, stream, pkv)
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
