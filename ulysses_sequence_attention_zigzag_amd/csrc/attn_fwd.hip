// Block attention forward for one ring step on gfx950 (CDNA4).
//
// One workgroup = 8 waves = 256 query rows of one (batch, head); each wave
// owns 32 rows (under a window mask: 4 waves, 128 rows, two workgroups per
// CU; see the kernel).  Per key tile (128 keys; 64 in the window form at
// D = 128):
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
#include <type_traits>

#include "usp_internal.h"

namespace usp {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

// MFMAs by which LDS operand reads run ahead in the matrix phase (2, 4, 6
// and 8 measured on MI355X: 6 is best by ~1.5%, 8 no better).
constexpr int kPrefetch = 6;

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


// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferRsrcWord3 = 0x00020000;

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

// Masks.  Key positions increase through every run of the plan for every
// layout (striped blocks of any size included), so the keys a query sees in a
// partial tile form at most two intervals (window band, sinks), found once
// per tile through the inverse of the position map.
//
// Wave roles.  The workgroup is 8 waves in two groups of 4 (waves 0-3 and
// 4-7); the hardware places wave w and wave w + 4 on the same SIMD.  Each
// wave owns 32 query rows.  The groups run the same per-tile program
//   M(t): PV(t-1), QK(t)        (matrix cores + LDS reads)
//   V(t): mask + softmax(t)     (vector ALU)
// shifted by one phase, with a workgroup barrier between phases, so that on
// every SIMD one wave feeds the matrix core while the other does its softmax:
//   phase 2t  : group 0 in M(t), group 1 in V(t-1)
//   phase 2t+1: group 0 in V(t), group 1 in M(t)
// Group 0 stages the K tiles and group 1 the V tiles: at the start of its
// V(t), past the barrier that ends its M(t), a group issues the loads of
// tile t+1 straight into LDS, into the buffer whose previous tile both
// groups have finished reading, and waits for them at the end of its V(t),
// before the barrier that hands the phase over.  (Issued at the end of M(t)
// instead, the copies lengthened the matrix phases, the longer side of
// each phase.)  Phase barriers carry no memory fence: every LDS read of a
// matrix phase is consumed by its MFMAs before the phase ends.
//
// Window masks (WIN) make short work items: a query tile sees a band of a few
// key tiles, and the item's fixed costs (loading q, the first tile, reading
// and writing the f32 accumulator) take half of its time.  Those launches run
// the 4-wave form (W4): 128-row items, 64-key tiles at D = 128 (64 KB of
// LDS), so that two workgroups share a CU and one's prologue and epilogue
// overlap the other's tiles.  Its waves stage K and V together and run
// M(t), V(t) in turn, with a barrier before each tile copy (all waves are
// done with the buffer) and after each V(t) (the copy landed).
template <int D, int MODS, bool WIN, bool W4>
__global__ __launch_bounds__(W4 ? 256 : 512, 2) void attn_fwd_kernel(const AttnParams p) {
  using TL = TileLayout<D>;
  // Keys per tile; the planner's full runs come in multiples of kTileN.
  constexpr int BN = (W4 && D == 128) ? 64 : 128;
  static_assert(kTileN % BN == 0, "planner granularity");
  constexpr int KS = D / 16;        // k-steps of the QK^T contraction
  constexpr int DB = D / 32;        // 32-wide blocks of the output's head dim
  constexpr int NB = BN / 32;       // 32-key blocks per tile
  constexpr int TILEB = BN * D * 2; // bytes of one K or V tile
  constexpr int LPT = TILEB / 4096; // 16-byte loads per thread of the staging group
  constexpr int RPI = 1024 / TL::ROWB;  // tile rows per 1 KB slice
  static_assert(TILEB % 4096 == 0, "tile must split into 4 waves x 1 KB slices");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILEB];  // K0 K1 V0 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = W4 ? 0 : wid >> 2;
  const int wg = wid & 3;
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
  if (it.q_rows == 0) return;  // planner slot with nothing to do (whole workgroup)
  const int hk = h / (p.Hq / p.Hkv);

  // This lane's query row: wid*32 + l32.
  const int qr = wid * 32 + l32;
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
  // The row sum is accumulated from the bf16-rounded probabilities with
  // v_dot2 (one instruction per pair instead of two adds; numerator and
  // denominator then use the same rounded P), in two partial sums that
  // halve the dependency chain.  1.2-1.5 % faster on both large shares.
  float m = -INFINITY, lsum = 0.f, lsum2 = 0.f;
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  // Visible key positions of this query: [vis_lo, vis_hi], plus the sinks
  // [sstart, sink_hi] when a window is set (same sequence, causal band,
  // window p_q - p_k < W, first n_sink positions of the sequence).
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

  // Tile staging by this wave's group (K for group 0, V for group 1): buffer
  // loads straight into LDS (16 bytes per lane, 32-bit offsets from a buffer
  // resource; lane i of a load lands at 16*i past the wave-uniform LDS
  // address).  The group's 256 threads cover the tile as 1 KB slices:
  // thread (wave wg, lane i) handles slices wg*LPT + j, physical (row, chunk
  // slot) = (slice*RPI + i / CPR, i % CPR), and so loads the logical chunk
  // slot ^ swz(row) of that row.  Rows past the run's end are clamped to its
  // last row (finite values; those keys are masked), so no load leaves the
  // run.
  const int lrow = lane / TL::CPR;
  const int lslot = lane % TL::CPR;
  const uint32_t row_bytes = (uint32_t)kv_row_stride * 2;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(grp ? vbase : kbase), (short)0, 0x7fffffff, kBufferRsrcWord3);
  char* const stage_tiles = smem + grp * 2 * TILEB;
  // A tile that lies inside its run needs no clamp, and the lane's part of
  // each offset is loop-invariant: slice s = wg*LPT + j starts at row s*RPI,
  // which the swizzles see only through s % NSW (s*RPI/RPL = 4s), and
  // wg*LPT is a multiple of NSW.  So NSW per-lane offsets (one for V, whose
  // swizzle ignores the slice) serve every slice, and the tile's first key
  // plus the slice's row go into the scalar offset of the load.  (Named
  // scalars rather than an array: an array indexed inside the copy lambda
  // made the host pass drop the kernels' launch stubs.)
  constexpr int NSW = TL::CPR / 4;
  static_assert(LPT % NSW == 0 && RPI == 4 * TL::RPL && NSW <= 4, "slice / swizzle period");
  const uint32_t lrb = (uint32_t)lrow * row_bytes;
  const uint32_t lofs_k0 = lrb + (uint32_t)((lslot ^ TL::swz_k(lrow)) * 16);
  const uint32_t lofs_k1 = lrb + (uint32_t)((lslot ^ TL::swz_k(RPI + lrow)) * 16);
  const uint32_t lofs_k2 = lrb + (uint32_t)((lslot ^ TL::swz_k(2 * RPI + lrow)) * 16);
  const uint32_t lofs_k3 = lrb + (uint32_t)((lslot ^ TL::swz_k(3 * RPI + lrow)) * 16);
  const uint32_t lofs_v = lrb + (uint32_t)((lslot ^ TL::swz_v(lrow)) * 16);
  // one tile (V when is_v) into `tile` (the D = 64 window kernels keep the
  // clamped form: the scalar offsets would take them past the SGPR budget)
  constexpr bool kFastCopy = !(W4 && D == 64);
  auto dma_one = [&](const __amdgpu_buffer_rsrc_t& rs, bool is_v, char* tile, int k0, int kend) {
    if (kFastCopy && k0 + BN <= kend) {
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const uint32_t soff = (uint32_t)(k0 + (wg * LPT + j) * RPI) * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (wg * LPT + j) * 1024), 16,
                                                 is_v ? lofs_v
                                                      : (j % NSW == 0 ? lofs_k0 : j % NSW == 1 ? lofs_k1 : j % NSW == 2 ? lofs_k2 : lofs_k3),
                                                 soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int row = (wg * LPT + j) * RPI + lrow;
        const int sw = is_v ? TL::swz_v(row) : TL::swz_k(row);
        const uint32_t off = (uint32_t)min(k0 + row, kend - 1) * row_bytes + (uint32_t)((lslot ^ sw) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (wg * LPT + j) * 1024), 16, off, 0, 0, 0);
      }
    }
  };
  // this group's tile (8 waves: K for group 0, V for group 1), or both (W4:
  // K into `tile`, V two tiles further)
  auto dma_tile = [&](char* tile, int k0, int kend) {
    if constexpr (W4) {
      const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, 0x7fffffff,
                                                                           kBufferRsrcWord3);
      dma_one(srs, false, tile, k0, kend);
      dma_one(vrs, true, tile + 2 * TILEB, k0, kend);
    } else {
      dma_one(srs, grp != 0, tile, k0, kend);
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

  // Fragment reads.  QK op j = (ks, kb) = (j / NB, j % NB) reads the K
  // fragment of key block kb, k-step ks; PV op j = (kb, half, d) with d
  // fastest reads the V^T fragment of head-dim block d, keys
  // kb*32 + 16*half + (8 keys in the P^T k-order) with two transpose reads.
  auto read_k = [&](const char* tK, int j) -> bf16x8 {
    const int ks = j / NB, kb = j % NB;
    const int row = kb * 32 + l32;
    const int slot = (2 * ks + hi) ^ TL::swz_k(row);
    return *reinterpret_cast<const bf16x8*>(tK + row * TL::ROWB + slot * 16);
  };
  auto read_v = [&](const char* tV, int j) -> bf16x8 {
    const int d = j % DB, half = (j / DB) & 1, kb = j / (2 * DB);
    const int r0 = kb * 32 + half * 16 + vrow0;
    const int r1 = r0 + 8;
    const int c = 4 * d + vchunk;
    const bf16x4 a0 = lds_read_tr(tV + r0 * TL::ROWB + ((c ^ TL::swz_v(r0)) * 16) + vhalf8);
    const bf16x4 a1 = lds_read_tr(tV + r1 * TL::ROWB + ((c ^ TL::swz_v(r1)) * 16) + vhalf8);
    return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  };

  // Matrix phase: O^T += V^T P^T for the previous tile (DO_PV), then
  // S^T = K Q^T for the current one (DO_QK).  Only one wave per SIMD is in
  // this phase at a time, so LDS latency is hidden inside the wave: operand
  // fragments are read kPrefetch MFMAs ahead, across the PV -> QK boundary,
  // and the order is pinned with scheduling groups (DS read 0x100, MFMA 0x8).
  constexpr int NPV = NB * 2 * DB;  // PV MFMAs per tile
  constexpr int NQK = KS * NB;      // QK MFMAs per tile
  constexpr int PF = kPrefetch;
  static_assert(PF <= NPV && PF <= NQK, "prefetch depth");
  auto m_phase = [&](auto do_pv_c, auto do_qk_c, const char* tV, const char* tK, f32x16 (&sc)[NB],
                     const bf16x8 (&pb)[NB][2]) {
    constexpr bool DO_PV = decltype(do_pv_c)::value;
    constexpr bool DO_QK = decltype(do_qk_c)::value;
    bf16x8 fv[NPV], fk[NQK];
    if constexpr (DO_PV) {
#pragma unroll
      for (int i = 0; i < PF; ++i) fv[i] = read_v(tV, i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + PF < NPV) fv[i + PF] = read_v(tV, i + PF);
        else if (DO_QK) fk[i + PF - NPV] = read_k(tK, i + PF - NPV);
        const int d = i % DB, half = (i / DB) & 1, kb = i / (2 * DB);
        o[d] = mfma32(fv[i], pb[kb][half], o[d]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PF; ++i) fk[i] = read_k(tK, i);
    }
    if constexpr (DO_QK) {
      const f32x16 zero = {};
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        if (i + PF < NQK) fk[i + PF] = read_k(tK, i + PF);
        const int ks = i / NB, kb = i % NB;
        sc[kb] = mfma32(fk[i], qf[ks], ks == 0 ? zero : sc[kb]);
      }
    }
    // scheduling groups, in issue order
    if constexpr (DO_PV) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
      for (int i = 0; i < NPV - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (DO_QK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
    }
    if constexpr (DO_QK) {
#pragma unroll
      for (int i = 0; i < NQK - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < PF; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // Score modifiers (MODS bit 0: softcap, bit 1: ALiBi) on the raw scores of
  // the tile at key k0, before the mask: softcap a - 2a / (exp2(s b2) + 1)
  // (= c tanh(s scale / c) / scale), then minus slope_h |p_q - p_k| / scale.
  // ALiBi distances in f32 (positions below 2^22 are exact): key t of the
  // key rank is at t + floor(t / b) (N - 1) b + rank b under the stripe
  // layout and at t + (p(k0) - k0) inside a run of the others (inv_b = 0
  // there), so p_k - p_q = floor((t + 0.5) inv_b) nb1 + t + rb.
  const float slope_raw = (MODS & 2) ? p.mods.alibi[h] * p.mods.inv_scale : 0.f;
  // softcap constants held in VGPRs (the window kernels use every SGPR)
  float cap_a = p.mods.a, cap_2a = 2.f * p.mods.a, cap_b2 = p.mods.b2;
  if constexpr ((MODS & 1) != 0) asm("" : "+v"(cap_a), "+v"(cap_2a), "+v"(cap_b2));
  // rb of a tile: rb0, or rb1 for a tile in the second zigzag chunk.
  const bool kstripe = km.kind == MAP_STRIPE;
  const float inv_b = kstripe ? 1.f / (float)km.b : 0.f;
  const float nb1 = kstripe ? (float)((km.N - 1) * km.b) : 0.f;
  const int32_t khalf = km.kind == MAP_ZIGZAG ? km.L >> 1 : 0x7fffffff;
  const float rb0 = (float)((kstripe ? km.rank * km.b : position(km, 0)) - pq_row);
  const float rb1 = km.kind == MAP_ZIGZAG ? (float)(position(km, khalf) - khalf - pq_row) : rb0;
  auto apply_mods = [&](f32x16 (&sc)[NB], int k0) {
    if constexpr ((MODS & 1) != 0) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(sc[kb][r] * cap_b2);
          sc[kb][r] = cap_a - cap_2a * __builtin_amdgcn_rcpf(e + 1.f);
        }
    }
    if constexpr ((MODS & 2) != 0) {
      // element (kb, r) is key t = k0 + 4*hi + kb*32 + 8*(r/4) + r%4 (the
      // constant is added first so that it folds into one instruction); the
      // empty asm keeps the compiler from hoisting the bias terms ahead of
      // the matrix products.
      float ab = (float)(k0 + 4 * hi);
      const float rb = k0 >= khalf ? rb1 : rb0;
      asm volatile("" : "+v"(ab));
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = ab + (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
          const float dd = __builtin_floorf((t + 0.5f) * inv_b) * nb1 + (t + rb);
          sc[kb][r] -= slope_raw * __builtin_fabsf(dd);
        }
    }
  };

  // Per-element mask of a partial tile starting at key k0.  Element (kb, r)
  // of this lane is key k0 + du with du = c + 4*hi, c = kb*32 + 8*(r/4) + r%4.
  // Key positions increase with du, so the visible du form at most two
  // intervals (window band, sinks); their bounds come from the inverse of
  // the position map once per tile, shifted by 4*hi, and are compared with
  // the compile-time c.
  // Under the stripe layout the first key row at or past a position does
  // not depend on the tile: the four bounds are found once (per-lane
  // divisions kept out of the tile loop).  Under the others key rows and
  // positions differ by a constant per monotone piece (per zigzag chunk).
  const int32_t dpos0 = kstripe ? 0 : -position(km, 0);
  const int32_t dpos1 = km.kind == MAP_ZIGZAG ? khalf - position(km, khalf) : dpos0;
  int32_t fs_lo = 0, fs_hi = 0, fs_slo = 0, fs_shi = 0;
  if (kstripe) {
    fs_lo = first_row_at_least(km, 0, vis_lo);
    fs_hi = first_row_at_least(km, 0, vis_hi + 1);
    fs_slo = first_row_at_least(km, 0, sstart);
    fs_shi = first_row_at_least(km, 0, sink_hi + 1);
  }
  auto apply_mask = [&](f32x16 (&sc)[NB], int k0, int kend) {
    const int32_t kend_du = kend - 1 - k0;
    const int32_t sh = k0 + 4 * hi;
    const int32_t dpos = k0 >= khalf ? dpos1 : dpos0;
    const int32_t lo = (kstripe ? fs_lo : vis_lo + dpos) - sh;
    const int32_t up = min((kstripe ? fs_hi : vis_hi + 1 + dpos) - 1 - k0, kend_du) - 4 * hi;
    const int32_t slo = (kstripe ? fs_slo : sstart + dpos) - sh;
    const int32_t sup = min((kstripe ? fs_shi : sink_hi + 1 + dpos) - 1 - k0, kend_du) - 4 * hi;
    // With a window (WIN) most of a partial tile's 32-key blocks are
    // visible or hidden as a whole for every lane of the wave: such a block
    // takes no per-element mask (wave-uniform branches).  Without one the
    // partial tiles are the few along a causal diagonal, and the plain mask
    // keeps the kernel's code as it is.
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      if constexpr (WIN) {
        const int cmin = kb * 32, cmax = kb * 32 + 27;  // this lane's keys of the block
        const bool all_vis = ((lo <= cmin) & (cmax <= up)) | ((slo <= cmin) & (cmax <= sup));
        const bool none_vis = ((up < cmin) | (lo > cmax)) & ((sup < cmin) | (slo > cmax));
        if (__builtin_amdgcn_readfirstlane((int)(__ballot(!all_vis) == 0ull))) continue;
        if (__builtin_amdgcn_readfirstlane((int)(__ballot(!none_vis) == 0ull))) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][r] = -INFINITY;
          continue;
        }
      }
      if constexpr (WIN) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          const bool vis = ((c >= lo) & (c <= up)) | ((c >= slo) & (c <= sup));
          sc[kb][r] = vis ? sc[kb][r] : -INFINITY;
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // no window: no sinks either, one interval [lo, up], tested with
        // one unsigned compare per element (an empty interval becomes one
        // that starts past every key of the tile).  The scheduling barrier
        // per 32-key block keeps the compiler from computing all the blocks'
        // lane masks ahead of their selects (which spilled hundreds of SGPRs).
        const bool empty = up < lo;
        const int32_t lo1 = empty ? (1 << 30) : lo;
        const uint32_t w1 = empty ? 0u : (uint32_t)(up - lo);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          const bool vis = (uint32_t)(c - lo1) <= w1;
          sc[kb][r] = vis ? sc[kb][r] : -INFINITY;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Tiles of this item: the runs' key ranges cut into BN-key tiles.
  int n_tiles = 0;
  for (int r = it.run_begin; r < it.run_end; ++r) {
    const Run rr = p.runs[r];
    n_tiles += (rr.k_end - rr.k_begin + BN - 1) / BN;
  }

  // W4, accumulating into an f32 result: the previous partial of this lane's
  // row is loaded before the last matrix phase, which then covers part of
  // the load's latency (the epilogue is a third of a window item's time).
  float4 oprev[W4 ? DB : 1][4];
  float la_pre = 0.f;
  bool have_pre = false;
  auto load_prev = [&]() {
    if constexpr (W4) {
      if (p.accumulate && p.out_f32 && qvalid) {
        la_pre = p.lse[((int64_t)b * p.o_heads + p.o_head0 + h) * p.Lq_buf + qrow];
        const float* op = static_cast<const float*>(p.out) + (int64_t)b * p.o_batch_stride +
                          (qrow * p.o_heads + p.o_head0 + h) * D;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) oprev[d][g] = *reinterpret_cast<const float4*>(op + d * 32 + 8 * g + 4 * hi);
        have_pre = true;
      }
    }
  };

  if (n_tiles > 0) {
    // This wave's tile cursor (tile t of its current step).
    int ri = it.run_begin;
    Run run = p.runs[ri];
    int k0 = run.k_begin;
    dma_tile(stage_tiles, k0, run.k_end);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    f32x16 s[NB];
    bf16x8 pb[NB][2];
    int nri = ri, nk0 = k0;
    Run nrun = run;
    // Cursor of tile t+1.
    auto prefetch_next = [&]() {
      nk0 = k0 + BN;
      nri = ri;
      nrun = run;
      if (nk0 >= run.k_end) {
        nri = ri + 1;
        nrun = p.runs[nri];
        nk0 = nrun.k_begin;
      }
    };
    // V(t): mask, online softmax (log2 domain, lazy rescale); tile t+1 lands.
    auto v_phase = [&](int t) {
      if constexpr (MODS != 0) apply_mods(s, k0);
      if (!run.full) apply_mask(s, k0, run.k_end);
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mt),
                                                         __builtin_bit_cast(unsigned, mt), false, false);
        mt = fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
      }
      mt *= p.scale_log2;
      const float m_new = (mt > m + kRescale) ? mt : m;
      const float alpha = (m_new == m || m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
      lsum2 *= alpha;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = fast_exp2(s[kb][half * 8 + e] * p.scale_log2 - m_use);
            const float p1 = fast_exp2(s[kb][half * 8 + e + 1] * p.scale_log2 - m_use);
            const bf16x2 pk2 = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
            if (half == 0)
              lsum = __builtin_amdgcn_fdot2_f32_bf16(pk2, ones2, lsum, false);
            else
              lsum2 = __builtin_amdgcn_fdot2_f32_bf16(pk2, ones2, lsum2, false);
            pb[kb][half][e] = pk2[0];
            pb[kb][half][e + 1] = pk2[1];
          }
        }
      }
      if (__builtin_amdgcn_readfirstlane((int)(__ballot(alpha != 1.f) != 0ull))) {
        asm volatile("" ::: "memory");  // keep this a branch (rarely taken)
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      if (t + 1 < n_tiles) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this group's tile t+1 is in LDS
        ri = nri;
        run = nrun;
        k0 = nk0;
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;

    // Phase barrier: no memory fence (the matrix phase's LDS reads are all
    // consumed by its MFMAs before it ends, and tile loads are waited for
    // explicitly), only a compiler ordering point.
    auto phase_barrier = [&]() { asm volatile("s_barrier" ::: "memory"); };
    // A wave runs its matrix phase at raised priority, so the SIMD's other
    // wave (in its softmax) does not delay its MFMA and LDS issue: 0.6-1.5 %
    // faster on both large shares.
    auto prio_hi = []() { __builtin_amdgcn_s_setprio(1); };
    auto prio_lo = []() { __builtin_amdgcn_s_setprio(0); };
    if constexpr (W4) {
      // M(t) then V(t) in every wave; tile t+1 is copied into the buffers of
      // tile t-1 once every wave has finished M(t) (its last reads of them).
      if (n_tiles > 1) prefetch_next();
      prio_hi();
      m_phase(F_{}, T_{}, nullptr, smem, s, pb);
      prio_lo();
      if (n_tiles > 1) dma_tile(smem + TILEB, nk0, nrun.k_end);
      v_phase(0);
      phase_barrier();
      for (int t = 1; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) prefetch_next();
        prio_hi();
        m_phase(T_{}, T_{}, smem + (2 + ((t - 1) & 1)) * TILEB, smem + (t & 1) * TILEB, s, pb);
        prio_lo();
        phase_barrier();
        if (t + 1 < n_tiles) dma_tile(smem + ((t + 1) & 1) * TILEB, nk0, nrun.k_end);
        v_phase(t);
        phase_barrier();
      }
      load_prev();
      prio_hi();
      m_phase(T_{}, F_{}, smem + (2 + ((n_tiles - 1) & 1)) * TILEB, nullptr, s, pb);
      prio_lo();
    } else {
      // Group 1 starts one phase late (group 0 runs M(0) meanwhile) and group
      // 0 ends one phase early, so both pass the same number of barriers.
      if (grp == 1) phase_barrier();
      if (n_tiles > 1) prefetch_next();
      prio_hi();
      m_phase(F_{}, T_{}, nullptr, smem, s, pb);
      prio_lo();
      phase_barrier();
      if (n_tiles > 1) dma_tile(stage_tiles + TILEB, nk0, nrun.k_end);
      v_phase(0);
      phase_barrier();
      for (int t = 1; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) prefetch_next();
        prio_hi();
        m_phase(T_{}, T_{}, smem + (2 + ((t - 1) & 1)) * TILEB, smem + (t & 1) * TILEB, s, pb);
        prio_lo();
        phase_barrier();
        if (t + 1 < n_tiles) dma_tile(stage_tiles + ((t + 1) & 1) * TILEB, nk0, nrun.k_end);
        v_phase(t);
        phase_barrier();
      }
      prio_hi();
      m_phase(T_{}, F_{}, smem + (2 + ((n_tiles - 1) & 1)) * TILEB, nullptr, s, pb);
      prio_lo();
      if (grp == 0) phase_barrier();
    }
  }

  // epilogue: O = O_acc / l, LSE = m ln 2 + ln l; or merge into (out, lse)
  lsum += lsum2;
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!qvalid) return;
  const float lse_new = ltot > 0.f ? m * kLn2 + logf(ltot) : -INFINITY;
  // out rows and lse batch rows hold o_heads heads; this call's are o_head0 ..
  float* lse_ptr = p.lse + ((int64_t)b * p.o_heads + p.o_head0 + h) * p.Lq_buf + qrow;
  const int64_t obase = (int64_t)b * p.o_batch_stride + (qrow * p.o_heads + p.o_head0 + h) * D;
  float wa = 0.f, wb = ltot > 0.f ? 1.f / ltot : 0.f;
  float lse_out = lse_new;
  if (p.accumulate) {
    const float la = have_pre ? la_pre : *lse_ptr;
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
        float4 v = make_float4(o[d][4 * g] * wb, o[d][4 * g + 1] * wb, o[d][4 * g + 2] * wb, o[d][4 * g + 3] * wb);
        if (wa != 0.f) {
          const float4 a = have_pre ? oprev[d][g] : *reinterpret_cast<const float4*>(op + dd);
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
  const bool win = p.mask.window > 0;
  if (p.tile_m != (win ? 128 : 256)) {
    set_error("internal: unsupported query tile %d", p.tile_m);
    return USP_ERR_UNSUPPORTED;
  }
  const dim3 grid((unsigned)total), block(win ? 256 : 512);
  TimingScope ts(K_ATTN, stream);
  const int mods = mods_variant(p.mods);
#define USP_LAUNCH(DD, M, W) hipLaunchKernelGGL((attn_fwd_kernel<DD, M, W, W>), grid, block, 0, stream, p)
#define USP_LAUNCH_M(DD, W)                     \
  switch (mods) {                                \
    case 0: USP_LAUNCH(DD, 0, W); break;         \
    case 1: USP_LAUNCH(DD, 1, W); break;         \
    case 2: USP_LAUNCH(DD, 2, W); break;         \
    default: USP_LAUNCH(DD, 3, W); break;        \
  }
  if (D == 128) {
    if (win) { USP_LAUNCH_M(128, true) } else { USP_LAUNCH_M(128, false) }
  } else {
    if (win) { USP_LAUNCH_M(64, true) } else { USP_LAUNCH_M(64, false) }
  }
#undef USP_LAUNCH_M
#undef USP_LAUNCH
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
