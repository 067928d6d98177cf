// Decode-time attention over a KV cache on gfx950: the cache is cut into
// pieces whose partial (O, LSE) are computed independently and then
// combined (flash decoding read as ring attention at inference; the
// combine is associative, so it can run as a tree reduction).
//
// decode_split_kernel: one wave per (cache piece, batch row, KV head).  The
//   wave's B operand is Q^T of the KV head's whole query group (group heads
//   x Lq new tokens, at most 32 columns; each lane owns one query), resident
//   in registers.  32-key K and V tiles are copied global -> LDS into the
//   wave's own LDS buffer; per tile S^T = K Q^T (8 MFMAs at D = 128),
//   mask, online softmax in the log2 domain, O^T += V^T P^T (8 MFMAs, V^T
//   by LDS transpose reads).  The work is HBM-bound: every K / V byte of the
//   cache is read once per decode step, so the copies carry the
//   non-temporal hint (76-79 % of 8 TB/s against 68-69 % without it).
// decode_merge_kernel: per (batch row, query, head), the piece partials are
//   folded by groups of threads (pieces g, g + G, ...) and the G group
//   results combined pairwise in log2(G) rounds; many pieces go through a
//   first pass over chunks of 64 pieces (in place) and a final pass.

#include "mfma_common.h"

namespace usp {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

// Waves per workgroup, LDS stages (K + V tile buffers) per wave and the
// minimum waves per SIMD the register budget must allow, for the split
// kernel; a workgroup's LDS is waves x stages x 16 KB at D = 128.  With one
// stage a wave copies a tile, waits for it and computes on it, and the other
// waves of its SIMD cover the wait; with more, a wave keeps stages - 1 tiles
// in flight (their copies must fit the 6-bit vmcnt).  Measured on MI355X
// (kernel GB/s): the rate follows the waves per CU, not the tiles in flight
// per wave -- 4 waves x 2 stages (one workgroup per CU) 4.7-5.0 TB/s; one
// stage with 8-10 waves per CU (2 x 1, 4 x 1, 8 x 1, 1 x 1) 5.4-5.5 TB/s.
#ifndef USP_DEC_WAVES
#define USP_DEC_WAVES 2
#endif
#ifndef USP_DEC_STAGES
#define USP_DEC_STAGES 1
#endif
#ifndef USP_DEC_MINW
#define USP_DEC_MINW 2
#endif
constexpr int kDecWaves = USP_DEC_WAVES;
constexpr int kDecStages = USP_DEC_STAGES;

// s_waitcnt vmcnt(n) for the counts the split kernel uses (any other count
// waits for everything, which is only slower).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

template <int D, int MODS>
__global__ __launch_bounds__(64 * kDecWaves, USP_DEC_MINW) void decode_split_kernel(const DecodeParams p) {
  using T = SwzTile<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TK = 32;                 // keys per tile
  constexpr int TILEB = TK * D * 2;
  constexpr int NLD = TILEB / 1024;      // 1 KB copies per tile and tensor
  constexpr int RPI = 1024 / T::ROWB;
  constexpr int NST = kDecStages;
  static_assert(NST >= 1 && (NST - 2) * 2 * NLD <= 63, "tiles in flight must fit vmcnt");
  __shared__ __attribute__((aligned(1024))) char smem[kDecWaves * NST * 2 * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int split = blockIdx.x * kDecWaves + wid;
  if (split >= p.n_split) return;  // the whole wave leaves; the kernel has no barrier
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int group = p.Hq / p.Hkv;
  const int R = group * p.Lq;
  const int kv_len = p.kv_lens ? p.kv_lens[b] : p.S;
  const int k_lo = split * p.split_keys;
  const int k_hi = min(k_lo + p.split_keys, kv_len);

  // this lane's query: column r = gi * Lq + t of the group (r < R)
  const int r = l32;
  const bool valid = r < R;
  const int gi = valid ? r / p.Lq : 0;
  const int t = valid ? r - gi * p.Lq : 0;
  const int h = hk * group + gi;
  const int pq = kv_len - p.Lq + t;
  // visible keys: [lo_k, hi_k] (causal band, window) and [0, sink_hi] (sinks)
  int hi_k = valid ? pq : -1;
  const int lo_k = p.window > 0 ? max(0, pq - p.window + 1) : 0;
  const int sink_hi = (valid && p.window > 0) ? min(p.n_sink - 1, pq) : -1;

  float* const opart = p.out_part + (((int64_t)split * p.B + b) * p.Lq + t) * p.Hq * D + (int64_t)h * D;
  float* const lpart = p.lse_part + (((int64_t)split * p.B + b) * p.Hq + h) * p.Lq + t;
  if (k_lo >= k_hi) {  // the piece lies beyond this row's cache
    if (valid) {
      for (int d = hi * 4; d < D; d += 8) *reinterpret_cast<float4*>(opart + d) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (hi == 0) *lpart = -INFINITY;
    }
    return;
  }

  bf16x8 qf[KS];
  {
    const uint16_t* qrow = p.q + (((int64_t)b * p.Lq + t) * p.Hq + h) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (valid) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.f;
      }
    }
  }

  const int64_t row_elems = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)b * p.S * row_elems + hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * p.S * row_elems + hk * D;
  const i32x4 krs = buffer_rsrc(kbase);
  const i32x4 vrs = buffer_rsrc(vbase);
  const uint32_t row_bytes = (uint32_t)row_elems * 2;
  const int lrow = lane / T::CPR;
  const int lslot = lane % T::CPR;
  char* const wbuf = smem + wid * NST * 2 * TILEB;  // this wave's NST (K, V) buffers

  // copy of the tile at key k0: lane i of copy j moves physical (row, slot) =
  // (j*RPI + i / CPR, i % CPR), i.e. logical chunk slot ^ swz(row); rows past
  // the piece are clamped to its last key (masked below)
  auto copy_tile = [&](char* buf, int k0) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int row = j * RPI + lrow;
      const uint32_t off = (uint32_t)min(k0 + row, k_hi - 1) * row_bytes + (uint32_t)((lslot ^ T::swz(row)) * 16);
      copy16_to_lds_nt(krs, lds_addr(buf + j * 1024), off);
      copy16_to_lds_nt(vrs, lds_addr(buf + TILEB + j * 1024), off);
    }
  };

  f32x16 ot[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) ot[d][e] = 0.f;
  float m = -INFINITY;  // running max of s * scale * log2(e)
  float lsum = 0.f;     // this lane's share of the running sum
  const float c = p.scale_log2;
  const int n_tiles = (k_hi - k_lo + TK - 1) / TK;
  // score modifiers (MODS bit 0 softcap, bit 1 ALiBi; raw-score units as in
  // the attention kernels): distance p_q - p_k of element e of the tile at
  // k0 is (pq - k0 - 4*hi) - cc, formed in f32 (exact below 2^22 keys)
  const float slope = ((MODS & 2) && valid) ? p.mods.alibi[h] * p.mods.inv_scale : 0.f;

  // tile n lives in buffer n % NST.  With NST > 1, tiles n + 1 .. n + NST - 1
  // are copied while tile n computes, into the buffers of tiles
  // n + 1 - NST .. n - 1, whose reads the MFMAs of earlier iterations have
  // consumed; with NST = 1 the next copy starts after tile n's last MFMA.
  for (int i = 0; i < max(NST - 1, 1) && i < n_tiles; ++i) copy_tile(wbuf + i * 2 * TILEB, k_lo + i * TK);
  for (int n = 0; n < n_tiles; ++n) {
    const int k0 = k_lo + n * TK;
    const char* tK = wbuf + (n % NST) * 2 * TILEB;
    const char* tV = tK + TILEB;
    // tile n's copies are in LDS once at most the copies of the tiles issued
    // after it (n + 1 .. n + NST - 2) are outstanding (loads complete in
    // order); no memory access moves across the wait
    wait_vmcnt(NST >= 2 ? min(NST - 2, n_tiles - 1 - n) * 2 * NLD : 0);
    if (NST >= 2 && n + NST - 1 < n_tiles)
      copy_tile(wbuf + ((n + NST - 1) % NST) * 2 * TILEB, k0 + (NST - 1) * TK);

    f32x16 st = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) st = mfma32(T::frag(tK, l32, 2 * ks + hi), qf[ks], st);
    // element e is key k0 + 4*hi + cc, cc = 8*(e/4) + e%4
    const int sh = k0 + 4 * hi;
    const int lo = lo_k - sh, up = min(hi_k, k_hi - 1) - sh, sup = min(sink_hi, k_hi - 1) - sh;
    const float ab = (float)(pq - sh);
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int cc = 8 * (e >> 2) + (e & 3);
      const bool vis = ((cc >= lo) & (cc <= up)) | (cc <= sup);
      float sv = st[e];
      if constexpr ((MODS & 1) != 0)
        sv = p.mods.a - 2.f * p.mods.a * __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sv * p.mods.b2) + 1.f);
      if constexpr ((MODS & 2) != 0) sv -= slope * __builtin_fabsf(ab - (float)cc);
      x[e] = vis ? sv * c : -INFINITY;
      tmax = fmaxf(tmax, x[e]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);  // 0 while nothing was visible
    bf16x8 pb[2];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(x[e] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(x[e + 1] - m_use);
      ps += p0 + p1;
      const bf16x2 pk = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
      pb[e >> 3][e & 7] = pk[0];
      pb[e >> 3][(e & 7) + 1] = pk[1];
    }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) ot[d][e] *= alpha;
    m = m_new;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int d = 0; d < DB; ++d) ot[d] = mfma32(frag_tr<D>(tV, 0, half, d, lane), pb[half], ot[d]);
    if (NST == 1 && n + 1 < n_tiles) {
      // every fragment read of the buffer has returned (the MFMAs above
      // consumed them) before the next tile's copy is issued into it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      copy_tile(wbuf, k0 + TK);
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!valid) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = d * 32 + 8 * g + 4 * hi;
      *reinterpret_cast<float4*>(opart + dd) =
          make_float4(ot[d][4 * g] * inv, ot[d][4 * g + 1] * inv, ot[d][4 * g + 2] * inv, ot[d][4 * g + 3] * inv);
    }
  }
  if (hi == 0) *lpart = ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
}

// Folds (o_b, l_b) into (o, l): l' = M + ln(e^(l - M) + e^(l_b - M)),
// o' = e^(l - l') o + e^(l_b - l') o_b; an empty side (-inf) changes nothing.
__device__ __forceinline__ void merge_into(float4& o, float& l, const float4& ob, float lb) {
  const float M = fmaxf(l, lb);
  if (M == -INFINITY) return;
  const float L = M + __logf(__expf(l - M) + __expf(lb - M));
  const float wa = __expf(l - L), wb = __expf(lb - L);
  o = make_float4(wa * o.x + wb * ob.x, wa * o.y + wb * ob.y, wa * o.z + wb * ob.z, wa * o.w + wb * ob.w);
  l = L;
}

// One workgroup per (batch row, query, head) and chunk of pieces: pieces
// first + stride * i for i < count.  TPR = D/4 threads hold one float4 of a
// row; G = 256 / TPR groups fold pieces g, g + G, ... and the G results are
// combined pairwise in log2(G) rounds through LDS.  FINAL writes out / lse;
// otherwise the result replaces the chunk's first piece (only this
// workgroup reads that slot, and it has read its pieces before it writes).
template <int D, bool FINAL>
__global__ __launch_bounds__(256) void decode_merge_kernel(float* out_part, float* lse_part, int32_t n_split,
                                                           int32_t chunk, int32_t stride, int32_t B, int32_t Lq,
                                                           int32_t Hq, void* out, int32_t out_f32, float* lse) {
  constexpr int TPR = D / 4;
  constexpr int G = 256 / TPR;
  __shared__ float4 so[256];
  __shared__ float sl[G];
  const int row = blockIdx.x;  // (b * Lq + t) * Hq + h
  const int first = blockIdx.y * chunk * stride;
  const int h = row % Hq;
  const int bt = row / Hq;
  const int t = bt % Lq;
  const int b = bt / Lq;
  const int tid = threadIdx.x;
  const int g = tid / TPR;
  const int j = tid % TPR;
  const int64_t piece_o = (int64_t)B * Lq * Hq * D;
  const int64_t piece_l = (int64_t)B * Hq * Lq;
  const int64_t lidx = ((int64_t)b * Hq + h) * Lq + t;

  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = -INFINITY;
  for (int i = g; i < chunk; i += G) {
    const int64_t piece = first + (int64_t)i * stride;
    if (piece >= n_split) break;
    const float li = lse_part[piece * piece_l + lidx];
    const float4 oi = *reinterpret_cast<const float4*>(out_part + piece * piece_o + (int64_t)row * D + 4 * j);
    merge_into(o, l, oi, li);
  }
  so[tid] = o;
  if (j == 0) sl[g] = l;
  __syncthreads();
  // pairwise rounds; every thread passes both barriers of every round (reads
  // before the first, writes after it)
#pragma unroll
  for (int s = 1; s < G; s *= 2) {
    const bool act = (g % (2 * s)) == 0 && g + s < G;
    float4 a = o;
    float la = l;
    if (act) {
      a = so[tid];
      la = sl[g];
      merge_into(a, la, so[tid + s * TPR], sl[g + s]);
    }
    __syncthreads();
    if (act) {
      so[tid] = a;
      if (j == 0) sl[g] = la;
    }
    __syncthreads();
  }
  if (g != 0) return;
  const float4 r = so[j];
  const float lt = sl[0];
  if constexpr (FINAL) {
    if (out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + (int64_t)row * D + 4 * j) = r;
    } else {
      const bf16x2 a = __builtin_convertvector((f32x2){r.x, r.y}, bf16x2);
      const bf16x2 c2 = __builtin_convertvector((f32x2){r.z, r.w}, bf16x2);
      bf16x4 v4 = {a[0], a[1], c2[0], c2[1]};
      *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(out) + (int64_t)row * D + 4 * j) = v4;
    }
    if (j == 0) lse[lidx] = lt;
  } else {
    *reinterpret_cast<float4*>(out_part + (int64_t)first * piece_o + (int64_t)row * D + 4 * j) = r;
    if (j == 0) lse_part[(int64_t)first * piece_l + lidx] = lt;
  }
}

}  // namespace

usp_status launch_decode_split(const DecodeParams& p, int D, hipStream_t stream) {
  const dim3 grid((unsigned)((p.n_split + kDecWaves - 1) / kDecWaves), (unsigned)p.Hkv, (unsigned)p.B);
  {
    TimingScope ts(K_DECODE, stream);
    const int mods = mods_variant(p.mods);
#define USP_LAUNCH_DEC(DD, M) hipLaunchKernelGGL((decode_split_kernel<DD, M>), grid, dim3(64 * kDecWaves), 0, stream, p)
#define USP_LAUNCH_DEC_M(DD)                \
  switch (mods) {                           \
    case 0: USP_LAUNCH_DEC(DD, 0); break;   \
    case 1: USP_LAUNCH_DEC(DD, 1); break;   \
    case 2: USP_LAUNCH_DEC(DD, 2); break;   \
    default: USP_LAUNCH_DEC(DD, 3); break;  \
  }
    if (D == 128) { USP_LAUNCH_DEC_M(128) } else { USP_LAUNCH_DEC_M(64) }
#undef USP_LAUNCH_DEC_M
#undef USP_LAUNCH_DEC
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("decode launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

usp_status launch_decode_merge(float* out_part, float* lse_part, int32_t n_split, int32_t B, int32_t Lq, int32_t Hq,
                               int D, void* out, int out_f32, float* lse, hipStream_t stream) {
  const unsigned rows = (unsigned)((int64_t)B * Lq * Hq);
  if (rows == 0) return USP_OK;
  // above kMergeChunk pieces, a first pass folds chunks of kMergeChunk pieces
  // in place (rows x chunks workgroups), then the final pass merges the
  // chunk results (stride kMergeChunk)
  constexpr int kMergeChunk = 64;
  {
    TimingScope ts(K_DECODE_MERGE, stream);
    int32_t count = n_split, stride = 1;
    if (n_split > kMergeChunk) {
      const unsigned chunks = (unsigned)((n_split + kMergeChunk - 1) / kMergeChunk);
      if (D == 128)
        hipLaunchKernelGGL((decode_merge_kernel<128, false>), dim3(rows, chunks), dim3(256), 0, stream, out_part,
                           lse_part, n_split, kMergeChunk, 1, B, Lq, Hq, nullptr, 0, nullptr);
      else
        hipLaunchKernelGGL((decode_merge_kernel<64, false>), dim3(rows, chunks), dim3(256), 0, stream, out_part,
                           lse_part, n_split, kMergeChunk, 1, B, Lq, Hq, nullptr, 0, nullptr);
      count = (int32_t)chunks;
      stride = kMergeChunk;
    }
    if (D == 128)
      hipLaunchKernelGGL((decode_merge_kernel<128, true>), dim3(rows, 1), dim3(256), 0, stream, out_part, lse_part,
                         n_split, count, stride, B, Lq, Hq, out, out_f32, lse);
    else
      hipLaunchKernelGGL((decode_merge_kernel<64, true>), dim3(rows, 1), dim3(256), 0, stream, out_part, lse_part,
                         n_split, count, stride, B, Lq, Hq, out, out_f32, lse);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("decode merge launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
