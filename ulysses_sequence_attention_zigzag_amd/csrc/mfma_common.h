// Device helpers shared by the MFMA kernels that stage tiles through LDS
// (backward: attn_bwd.hip, attn_bwd_dq.hip; decode: decode.hip).  Everything
// here has internal linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

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
// LDS fragment reads in flight ahead of the MFMAs that use them
// (build-time overridable for tuning sweeps)
#ifndef USP_BWD_PF
#define USP_BWD_PF 4
#endif
constexpr int kPF = USP_BWD_PF;
// Positions of the tile-copy slices inside a matrix phase: slice j after MFMA
// kCopyFirst + j * kCopyStride (0 / -1: spread evenly over the phase).  Early
// in the phase, every other MFMA, measured best (0.5-0.9 % over spread
// evenly; every fourth from the second MFMA lost 2-3 %): the copies then have
// the rest of the phase and the next one to land.
#ifndef USP_BWD_COPY_STRIDE
#define USP_BWD_COPY_STRIDE 2
#endif
#ifndef USP_BWD_COPY_FIRST
#define USP_BWD_COPY_FIRST 0
#endif
constexpr int kCopyStride = USP_BWD_COPY_STRIDE;
constexpr int kCopyFirst = USP_BWD_COPY_FIRST;
constexpr int kBufferRsrcWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family)

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer resource of `base` (no stride, 2^31 - 1 bytes, no swizzle),
// wave-uniform so it lives in SGPRs.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = 0x7fffffff;
  r[3] = kBufferRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Global -> LDS copies (buffer loads to LDS): lane i's 16 (or 4) bytes at
// byte offset voff of the buffer land at LDS address lds + 16*i (4*i).
// They are issued through inline assembly so that the compiler does not
// order later LDS reads of other addresses behind them; the kernels wait
// for them explicitly (s_waitcnt vmcnt(0), then a barrier) before reading
// their destination, and never read a destination while a copy into it may
// be in flight.
// M0 (the LDS destination) is saved and restored around each copy.
__device__ __forceinline__ void copy16_to_lds(const i32x4& rsrc, uint32_t lds, uint32_t voff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(rsrc));
}
// the same copy with the non-temporal hint (data read once)
__device__ __forceinline__ void copy16_to_lds_nt(const i32x4& rsrc, uint32_t lds, uint32_t voff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(rsrc));
}
__device__ __forceinline__ void copy4_to_lds(const i32x4& rsrc, uint32_t lds, uint32_t voff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(rsrc));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i supplies the
// address of 4 consecutive bf16 (row i/4 of a 4 x 16 block); lane j receives
// column j of the block.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}
// The two reads at LDS byte addresses.
__device__ __forceinline__ bf16x4 lds_read_tr_at(uint32_t a) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(a));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 lds_read_b128_at(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(a);
}

// LDS tile of R rows x D bf16 (CPR 16-byte chunks per row, RPL rows per
// 256-byte bank line) with chunk c of row r at slot c ^ swz(r),
//   swz(r) = 4 * ((r / RPL) % (CPR / 4)) + (r / (RPL * CPR / 4)) % 4.
// Both read patterns hit distinct bank slots: a plain 16-byte read of one
// chunk by 16 consecutive rows (swz takes 16 distinct values over the rows
// of each bank-line position), and a transpose read of 4 consecutive rows x
// 4 aligned chunks (swz / 4 differs between the rows sharing a line
// position).
template <int D>
struct SwzTile {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 16 / CPR;
  static constexpr int ROWB = D * 2;
  __device__ static __forceinline__ int swz(int r) {
    return 4 * ((r / RPL) & (CPR / 4 - 1)) + ((r / (RPL * CPR / 4)) & 3);
  }
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
  using T = SwzTile<D>;
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


// ---------------------------------------------------------------- ping-pong
// Helpers of the 8-wave backward kernels, whose waves work on 64-row tiles
// (two 32-row blocks) of a staged operand with one lane per row of their
// own 32-row slice.

// Per-lane LDS byte offsets of the fragments of a 64-row SwzTile.  The
// swizzle of a row depends on its low 4 bits only, which the 16-row steps of
// the blocks leave alone, so one offset per (row, chunk) of block 0 serves
// all blocks (their distance is an immediate).  Transposed reads (as
// frag_tr): rows trow and trow + 8 of each 16-row half, chunk 4d + tchunk,
// 8-byte half (lane & 1).  Row reads: row lane % 32, chunk 2ks + lane / 32.
template <int D>
__device__ __forceinline__ void pp_offsets(int lane, int (&tro)[2][D / 32], int (&rro)[D / 16]) {
  using T = SwzTile<D>;
  const int hi = lane >> 5, l32 = lane & 31;
  const int trow = 4 * hi + ((lane & 15) >> 2);
  const int tchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
      const int r = trow + 8 * x;
      tro[x][d] = r * T::ROWB + (((4 * d + tchunk) ^ T::swz(r)) * 16) + (lane & 1) * 8;
    }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) rro[ks] = l32 * T::ROWB + (((2 * ks + hi) ^ T::swz(l32)) * 16);
}

// Matrix phase: the transposed-operand products acc[d] += X^T bb (X the
// 64-row tile at LDS address tT; 2 blocks x 2 halves x D/32 MFMAs) if DT,
// then the row-operand products sc[blk] = Y kv + c0[blk] (Y the tile at
// tR; 2 blocks x D/16 MFMAs, the two blocks alternating) if DR.  Fragments are read kPF MFMAs
// ahead, across the boundary, in an order pinned with scheduling groups.
// hook(m) runs after the phase's m-th MFMA (m a constant once unrolled): the
// kernels issue their tile copies from it, spread over the phase.
template <int D, bool DT, bool DR, typename Hook>
__device__ __forceinline__ void pp_matrix_phase(f32x16 (&acc)[D / 32], f32x16 (&sc)[2], const bf16x8 (&bb)[2][2],
                                                const bf16x8 (&kv)[D / 16], const int (&tro)[2][D / 32],
                                                const int (&rro)[D / 16], uint32_t tT, uint32_t tR,
                                                const f32x16 (&c0)[2], Hook&& hook) {
  using T = SwzTile<D>;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int NT = 2 * 2 * DB;
  constexpr int NR = 2 * KS;
  constexpr int PF = kPF;
  static_assert(PF <= NT && PF <= NR, "prefetch depth");
  // Per-phase lane bases (tile + lane offset), made opaque: otherwise the
  // loop-invariant sums lane offset + fragment constant are hoisted out of
  // the tile loop (one register each) and every read pays an add; from an
  // opaque base each fragment's constant goes in the read's offset field.
  uint32_t bt0[D / 32], bt1[D / 32], br[D / 16];
  if constexpr (DT) {
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      bt0[d] = tT + (uint32_t)tro[0][d];
      bt1[d] = tT + (uint32_t)tro[1][d];
      asm volatile("" : "+v"(bt0[d]), "+v"(bt1[d]));
    }
  }
  if constexpr (DR) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      br[ks] = tR + (uint32_t)rro[ks];
      asm volatile("" : "+v"(br[ks]));
    }
  }
  auto rd_t = [&](int j) {
    const int blk = j / (2 * DB), half = (j / DB) & 1, d = j % DB;
    const uint32_t cst = (uint32_t)((blk * 32 + half * 16) * T::ROWB);
    const bf16x4 a0 = lds_read_tr_at(bt0[d] + cst);
    const bf16x4 a1 = lds_read_tr_at(bt1[d] + cst);
    return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  };
  auto rd_r = [&](int i) {
    const int ks = i >> 1, blk = i & 1;
    return lds_read_b128_at(br[ks] + (uint32_t)(blk * 32 * T::ROWB));
  };
  bf16x8 ft[NT], fr[NR];
  if constexpr (DT) {
#pragma unroll
    for (int j = 0; j < PF; ++j) ft[j] = rd_t(j);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j + PF < NT) ft[j + PF] = rd_t(j + PF);
      else if (DR) fr[j + PF - NT] = rd_r(j + PF - NT);
      const int blk = j / (2 * DB), half = (j / DB) & 1, d = j % DB;
      acc[d] = mfma32(ft[j], bb[blk][half], acc[d]);
      hook(j);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PF; ++i) fr[i] = rd_r(i);
  }
  if constexpr (DR) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (i + PF < NR) fr[i + PF] = rd_r(i + PF);
      const int ks = i >> 1, blk = i & 1;
      sc[blk] = mfma32(fr[i], kv[ks], ks == 0 ? c0[blk] : sc[blk]);
      hook((DT ? NT : 0) + i);
    }
  }
  // scheduling groups, in issue order (a transposed fragment is 2 reads)
  if constexpr (DT) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
    for (int j = 0; j < NT - PF; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (DR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  } else {
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
  }
  if constexpr (DR) {
#pragma unroll
    for (int i = 0; i < NR - PF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// Workgroup barrier of the phase programs: no memory fence (each wave waits
// for its own LDS writes and tile copies explicitly before it), only a
// compiler ordering point.
__device__ __forceinline__ void pp_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace
}  // namespace usp
