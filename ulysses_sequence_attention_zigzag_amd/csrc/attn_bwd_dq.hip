// dQ kernel of the block-attention backward (see attn_bwd.hip for the
// terms and the plan it walks).  Built with VGPR-form MFMAs: the S^T / dP^T
// results feed the vector phases directly.

#include "mfma_common.h"

namespace usp {
namespace {

// -------------------------------------------------------------------- dQ
// Wave roles.  8 waves: wave wg (0-3) and wave wg + 4 share the 32 query
// rows wg*32 .. +31 of the item (one row per lane) and, by the hardware's
// placement, one SIMD.  Wave wg (the P wave) holds Q; wave wg + 4 (the dS
// wave) holds dO and accumulates dQ^T.  Per 64-key tile n (K, V), with
// S^T = K Q^T and dP^T = V dO^T in the C layout (lane = query, 16 keys per
// 32-key block):
//   P wave:  S^T(n)                 [matrix]
//            P^T = exp2(S^T c - LSE log2 e) -> LDS exchange (bf16, times
//            the softcap derivative)    [vector]
//   dS wave: delta - dP^T(n)        [matrix: -dO fragments, C = delta]
//            dS^T = -P^T (delta - dP^T) from the exchange   [vector]
//            dQ^T += K^T dS^T       [matrix]
// Phases: in phase 2n the P wave forms P(n) while the dS wave runs dQ(n-1)
// and dP(n); in phase 2n+1 the P wave runs S(n+1) while the dS wave forms
// dS(n).  Every phase ends with a workgroup barrier.  Tile staging straight
// into LDS: the P waves load K (3 buffers: K(n) is read in phases
// 2n-1 .. 2n+2), the dS waves V (2 buffers), each two phases ahead of use.
// OW: a storing launch (p.overwrite), built apart so that the adding form
// keeps its own code.
template <int D, int MODS, bool OW>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const BwdParams p) {
  using T = SwzTile<D>;
  constexpr int BN = 64;                   // keys per tile
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILEB = BN * D * 2;
  constexpr int LPT = TILEB / 4096;        // 16-byte copies per thread of a 4-wave group
  constexpr int RPI = 1024 / T::ROWB;
  constexpr int XB = BN * 32 * 2;          // P exchange of one wave pair (bf16)
  static_assert(kTileN % BN == 0, "planner granularity");
  static_assert(TILEB % 4096 == 0, "tile layout");
  __shared__ __attribute__((aligned(1024))) char smem[3 * TILEB + 2 * TILEB + 4 * XB];
  char* const kbuf = smem;
  char* const vbuf = smem + 3 * TILEB;
  char* const xbuf = vbuf + 2 * TILEB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2;   // 0: P wave, 1: dS wave
  const int wg = wid & 3;     // query slice
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
  // nothing to do (whole workgroup); a storing launch still writes the dq
  // rows of a tile that sees no key
  if (it.q_rows == 0 || (!OW && it.run_begin == it.run_end)) return;
  const int hk = h / (p.Hq / p.Hkv);

  const int qr = wg * 32 + l32;
  const bool qvalid = qr < it.q_rows;
  const int64_t qrow = (int64_t)it.q_row0 + qr;
  if constexpr (OW) {
    if (it.run_begin == it.run_end) {  // the dS waves own dq
      if (grp == 1 && qvalid) {
        float* op = p.dq + (int64_t)b * p.g_batch_stride + (qrow * p.Hq + h) * D;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(op + d * 32 + 8 * g + 4 * hi) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      return;
    }
  }

  // Q (P waves) or -dO (dS waves, sign bits flipped: exact) fragments of
  // this lane's row: B operand
  bf16x8 kv[KS];
  {
    const uint16_t* src = grp ? p.dout + (int64_t)b * p.g_batch_stride : p.q + (int64_t)b * p.q_batch_stride;
    src += (qrow * p.Hq + h) * D + hi * 8;
    const uint32_t flip = grp ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qvalid) {
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
  // exp2 subtrahend (LSE in log2 units; +inf gives P = 0) and delta of this row
  float lse2 = INFINITY, dl = 0.f;
  if (qvalid) {
    const int64_t li = ((int64_t)b * p.Hq + h) * p.Lq_buf + qrow;
    const float l = p.lse[li];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dl = p.delta[li];
  }
  // acc: dQ^T (dS waves); sc: S^T or delta - dP^T of the two 32-key blocks;
  // bb: dS^T; c_s / c_dp: C operands of the first S / dP MFMA (0 / delta)
  f32x16 acc[DB], sc[2];
  bf16x8 bb[2][2];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  f32x16 c_s[2], c_dp[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    c_s[0][r] = c_s[1][r] = 0.f;
    c_dp[0][r] = c_dp[1][r] = dl;
  }

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
  const uint16_t* tbase = (grp ? p.v : p.k) + (int64_t)b * p.kv_batch_stride + (int64_t)it.k_row0 * kv_row_stride + hk * D;
  const uint32_t row_bytes = (uint32_t)kv_row_stride * 2;
  const i32x4 trs = buffer_rsrc(tbase);
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
  float cap_a = p.mods.a, cap_2a = 2.f * p.mods.a, cap_b2 = p.mods.b2;
  if constexpr ((MODS & 1) != 0) asm("" : "+v"(cap_a), "+v"(cap_2a), "+v"(cap_b2));
  // Key rows and positions differ by a constant per monotone piece (per
  // zigzag chunk) except under the stripe layout, whose first key row at or
  // past a position does not depend on the tile: those bounds are found once.
  const int32_t dpos0 = kstripe ? 0 : -position(km, 0);
  const int32_t dpos1 = km.kind == MAP_ZIGZAG ? khalf - position(km, khalf) : dpos0;
  int32_t fs_lo = 0, fs_hi = 0, fs_slo = 0, fs_shi = 0;
  if (kstripe) {
    fs_lo = first_row_at_least(km, 0, vis_lo);
    fs_hi = first_row_at_least(km, 0, vis_hi + 1);
    fs_slo = first_row_at_least(km, 0, sstart);
    fs_shi = first_row_at_least(km, 0, sink_hi + 1);
  }

  // Tile cursor: the key tiles of the item's runs in order.
  struct Cursor {
    int ri, k0;
    Run run;
  };
  Cursor c0;
  c0.ri = it.run_begin;
  c0.run = p.runs[c0.ri];
  c0.k0 = c0.run.k_begin;
  auto advance = [&](Cursor& cu) {  // only while another tile follows
    cu.k0 += BN;
    if (cu.k0 >= cu.run.k_end) {
      cu.run = p.runs[++cu.ri];
      cu.k0 = cu.run.k_begin;
    }
  };
  int n_tiles = 0;
  for (int ri = it.run_begin; ri < it.run_end; ++ri) {
    const Run r = p.runs[ri];
    n_tiles += (r.k_end - r.k_begin + BN - 1) / BN;
  }

  // Tile copy by this wave's group (K for the P waves, V for the dS waves):
  // thread (wave wg, lane i) copies slices wg*LPT + j, physical (row, chunk
  // slot) = (slice*RPI + i / CPR, i % CPR) = logical chunk slot ^ swz(row);
  // rows past the run's end are clamped to its last row (masked in partial
  // runs; full runs are multiples of BN keys).
  // Loop-invariant lane parts of the offsets (as in the dK/dV kernel: the
  // swizzle of row s*RPI + lrow depends on s only through j, and the clamp
  // distributes over the row stride).
  const uint32_t lrb = (uint32_t)lrow * row_bytes;
  const uint32_t lsw0 = (uint32_t)((lslot ^ T::swz(lrow)) * 16);
  const uint32_t lsw1 = (uint32_t)((lslot ^ T::swz(RPI + lrow)) * 16);
  const uint32_t lsw2 = (uint32_t)((lslot ^ T::swz(2 * RPI + lrow)) * 16);
  const uint32_t lsw3 = (uint32_t)((lslot ^ T::swz(3 * RPI + lrow)) * 16);
  static_assert(LPT <= 4, "four lane swizzles");
  auto dma_slice = [&](char* buf, const Cursor& cu, int j) {
    const uint32_t rows = min(lrb + (uint32_t)(cu.k0 + (wg * LPT + j) * RPI) * row_bytes,
                              (uint32_t)(cu.run.k_end - 1) * row_bytes);
    const uint32_t off = rows + (j == 0 ? lsw0 : j == 1 ? lsw1 : j == 2 ? lsw2 : lsw3);
    copy16_to_lds(trs, lds_addr(buf + (wg * LPT + j) * 1024), off);
  };

  auto dma = [&](char* buf, const Cursor& cu) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma_slice(buf, cu, j);
  };
  // Inside a matrix phase of NM MFMAs: slice j after MFMA FIRST + j*STRIDE
  // (mfma_common.h's placement; the copies then overlap the matrix work
  // instead of delaying the barrier).  Past the last tile the copy repeats
  // the last one into the free buffer, which nothing reads again: the phase
  // keeps a single straight-line body.
  auto copy_in = [&](char* buf, const Cursor* cu, auto nm_c) {
    constexpr int STRIDE = kCopyStride > 0 ? kCopyStride : decltype(nm_c)::value / LPT;
    constexpr int FIRST = kCopyFirst >= 0 ? kCopyFirst : STRIDE - 1;
    static_assert(FIRST + (LPT - 1) * STRIDE < decltype(nm_c)::value, "copy positions");
    return [&dma_slice, buf, cu](int m) {
      if (m >= FIRST && (m - FIRST) % STRIDE == 0 && (m - FIRST) / STRIDE < LPT) dma_slice(buf, *cu, (m - FIRST) / STRIDE);
    };
  };

  int tro[2][DB], rro[KS];
  pp_offsets<D>(lane, tro, rro);
  auto m_phase = [&](auto do_t_c, auto do_r_c, uint32_t tT, uint32_t tR, const f32x16(&c0)[2], auto&& hook) {
    pp_matrix_phase<D, decltype(do_t_c)::value, decltype(do_r_c)::value>(acc, sc, bb, kv, tro, rro, tT, tR, c0, hook);
  };
  const auto no_copy = [](int) {};

  // P exchange slot of this wave pair: the 8 bf16 of (block kb, half) of
  // lane l at ((kb * 2 + half) * 64 + l) * 16, in the B-operand order
  char* const xw = xbuf + wg * XB;

  // Vector phase of the P wave: P^T of the tile at cu (S^T in sc); element
  // r of key block kb is key k0 + du, du = kb*32 + 8*(r/4) + 4*hi + r%4.
  // FULL: every pair visible; otherwise key positions increase through the
  // run, so this lane's visible keys (window band, sinks) are at most two
  // intervals of du, found once per tile.
  auto softmax = [&](auto full_c, const Cursor& cu) {
    constexpr bool FULL = decltype(full_c)::value;
    const int k0 = cu.k0;
    int32_t lo = 0, up = 0, slo = 0, sup = -1;
    if constexpr (!FULL) {
      const int32_t last = cu.run.k_end - 1 - k0;
      const int32_t sh = k0 + 4 * hi;
      const int32_t dpos = k0 >= khalf ? dpos1 : dpos0;
      lo = (kstripe ? fs_lo : vis_lo + dpos) - sh;
      up = min((kstripe ? fs_hi : vis_hi + 1 + dpos) - 1 - k0, last) - 4 * hi;
      slo = (kstripe ? fs_slo : sstart + dpos) - sh;
      sup = min((kstripe ? fs_shi : sink_hi + 1 + dpos) - 1 - k0, last) - 4 * hi;
    }
    // Score modifiers (raw units, as the forward): softcap a - 2a rc with
    // rc = 1 / (exp2(s b2) + 1), whose derivative factor 1 - tanh^2 =
    // 4 rc (1 - rc) scales dS (the exchange carries P times it); then ALiBi.
    float ab = 0.f, rb = 0.f;
    if constexpr ((MODS & 2) != 0) {
      ab = (float)(k0 + 4 * hi);
      rb = k0 >= khalf ? rb1 : rb0;
    }
    bf16x8 xq[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float pf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float sv = sc[kb][r], f = 1.f;
          if constexpr ((MODS & 1) != 0) {
            const float rc = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sv * cap_b2) + 1.f);
            sv = cap_a - cap_2a * rc;
            f = 4.f * rc * (1.f - rc);
          }
          if constexpr ((MODS & 2) != 0) {
            const float t = ab + (float)(kb * 32 + 8 * g + e);
            const float dd = __builtin_floorf((t + 0.5f) * inv_b) * nb1 + (t + rb);
            sv -= slope * __builtin_fabsf(dd);
          }
          float pe = __builtin_amdgcn_exp2f(sv * c - lse2);
          if constexpr (!FULL) {
            const int cc = kb * 32 + 8 * g + e;
            pe = (((cc >= lo) & (cc <= up)) | ((cc >= slo) & (cc <= sup))) ? pe : 0.f;
          }
          pf[e] = ((MODS & 1) != 0) ? pe * f : pe;
        }
        const bf16x2 p01 = __builtin_convertvector((f32x2){pf[0], pf[1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector((f32x2){pf[2], pf[3]}, bf16x2);
        const int half = g >> 1, e0 = (g & 1) * 4;
        xq[kb][half][e0] = p01[0];
        xq[kb][half][e0 + 1] = p01[1];
        xq[kb][half][e0 + 2] = p23[0];
        xq[kb][half][e0 + 3] = p23[1];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        *reinterpret_cast<bf16x8*>(xw + ((kb * 2 + half) * 64 + lane) * 16) = xq[kb][half];
      if constexpr (!FULL) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Vector phase of the dS wave: dS^T = -P^T (delta - dP^T), the latter in sc.
  auto form_ds = [&]() {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 xh[2] = {*reinterpret_cast<const bf16x8*>(xw + (kb * 2 * 64 + lane) * 16),
                            *reinterpret_cast<const bf16x8*>(xw + ((kb * 2 + 1) * 64 + lane) * 16)};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int hh = g >> 1, o = (g & 1) * 4;
        const float4 px = make_float4((float)xh[hh][o], (float)xh[hh][o + 1], (float)xh[hh][o + 2], (float)xh[hh][o + 3]);
        const float d0 = -(px.x * sc[kb][4 * g]);
        const float d1 = -(px.y * sc[kb][4 * g + 1]);
        const float d2 = -(px.z * sc[kb][4 * g + 2]);
        const float d3 = -(px.w * sc[kb][4 * g + 3]);
        const bf16x2 a01 = __builtin_convertvector((f32x2){d0, d1}, bf16x2);
        const bf16x2 a23 = __builtin_convertvector((f32x2){d2, d3}, bf16x2);
        const int half = g >> 1, e0 = (g & 1) * 4;
        bb[kb][half][e0] = a01[0];
        bb[kb][half][e0 + 1] = a01[1];
        bb[kb][half][e0 + 2] = a23[0];
        bb[kb][half][e0 + 3] = a23[1];
      }
    }
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  auto prio_hi = []() { __builtin_amdgcn_s_setprio(1); };
  auto prio_lo = []() { __builtin_amdgcn_s_setprio(0); };
  auto kb_at = [&](int n) { return kbuf + (n % 3) * TILEB; };
  auto vb_at = [&](int n) { return vbuf + (n & 1) * TILEB; };
  auto kl_at = [&](int n) { return lds_addr(kb_at(n)); };
  auto vl_at = [&](int n) { return lds_addr(vb_at(n)); };

  // The two roles run separate programs that pass the same barriers:
  // prologue (tile 0 lands; the P waves compute S(0)), two phases per tile,
  // and the dS waves' last dQ after the final barrier.  Each loop body holds
  // one copy of its matrix phase and exits at the bottom, so the
  // accumulators keep their registers across iterations.
  if (grp == 0) {
    Cursor cs = c0;  // tile of S / softmax
    Cursor ck = c0;  // tile of the last K copy
    dma(kb_at(0), ck);
    if (n_tiles > 1) {
      advance(ck);
      dma(kb_at(1), ck);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    pp_barrier();
    prio_hi();
    m_phase(F_{}, T_{}, 0u, kl_at(0), c_s, no_copy);
    prio_lo();
    pp_barrier();
    // phase 0: P of tile 0
    if (cs.run.full) softmax(T_{}, cs);
    else softmax(F_{}, cs);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the exchange writes, K(1)
    pp_barrier();
    for (int n = 0; n + 1 < n_tiles; ++n) {
      // phase 2n+1: S(n+1); K(n+2) copied meanwhile
      if (n + 2 < n_tiles) advance(ck);
      prio_hi();
      m_phase(F_{}, T_{}, 0u, kl_at(n + 1), c_s, copy_in(kb_at(n + 2), &ck, std::integral_constant<int, 2 * KS>{}));
      prio_lo();
      advance(cs);
      pp_barrier();
      // phase 2n+2: P of tile n+1
      if (cs.run.full) softmax(T_{}, cs);
      else softmax(F_{}, cs);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the exchange writes, K(n+2)
      pp_barrier();
    }
    // phase 2N-1: the dS waves form dS(N-1)
    pp_barrier();
  } else {
    Cursor cv = c0;  // tile of the last V copy
    dma(vb_at(0), cv);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    pp_barrier();
    pp_barrier();
    // phase 0: dP(0)
    prio_hi();
    m_phase(F_{}, T_{}, 0u, vl_at(0), c_dp, no_copy);
    prio_lo();
    if (n_tiles > 1) {
      advance(cv);
      dma(vb_at(1), cv);
    }
    pp_barrier();
    // phase 1: dS(0)
    form_ds();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): V(1) landed
    pp_barrier();
    for (int n = 0; n + 1 < n_tiles; ++n) {
      // phase 2n+2: dQ(n), dP(n+1); V(n+2) copied meanwhile
      if (n + 2 < n_tiles) advance(cv);
      prio_hi();
      m_phase(T_{}, T_{}, kl_at(n), vl_at(n + 1), c_dp, copy_in(vb_at(n + 2), &cv, std::integral_constant<int, 4 * KS>{}));
      prio_lo();
      pp_barrier();
      // phase 2n+3: dS(n+1)
      form_ds();
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): V(n+2) landed
      pp_barrier();
    }
    // phase 2N: dQ(N-1).  The dq rows this call adds to are loaded before
    // it (V and the dP results are dead by then), which covers part of the
    // load's latency; a storing launch adds to nothing.
    float4 prev[DB][4];
    float* op = p.dq + (int64_t)b * p.g_batch_stride + (qrow * p.Hq + h) * D;
    if constexpr (OW) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) prev[d][g] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else if (qvalid) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) prev[d][g] = *reinterpret_cast<const float4*>(op + d * 32 + 8 * g + 4 * hi);
    }
    prio_hi();
    m_phase(T_{}, F_{}, kl_at(n_tiles - 1), 0u, c_dp, no_copy);
    prio_lo();

    // dq[b, row, h, :] += scale * dQ (this lane: query qrow, head-dim rows of
    // dQ^T), or = for a storing launch
    if (!qvalid) return;
    const float w = p.scale;
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
        *reinterpret_cast<float4*>(op + dd) = a;
      }
    }
  }
}

}  // namespace

void launch_bwd_dq(const BwdParams& p, int D, unsigned grid, hipStream_t stream) {
  TimingScope ts(K_BWD_DQ, stream);
  const int mods = mods_variant(p.mods);
#define USP_LAUNCH_Q(DD, M)                                                                                 \
  do {                                                                                                      \
    if (p.overwrite)                                                                                        \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, M, true>), dim3(grid), dim3(512), 0, stream, p);                \
    else                                                                                                    \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, M, false>), dim3(grid), dim3(512), 0, stream, p);               \
  } while (0)
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
