/*
 * usp.h -- C ABI of libusp: one GPU's share of ring / zigzag / striped /
 * Ulysses-hybrid sequence-parallel attention, as HIP kernels for gfx950.
 *
 * Sources for what each call computes (cited by page title and section):
 *   [YC]  YunChang (USP) README: "2. Usage" (extract the local shard with the
 *         ring layout, then run LongContextAttention with a ring_impl_type of
 *         basic / zigzag / stripe; ulysses x ring degrees), "Why not apply
 *         Ulysses and Ring Attention Individually?" (Ulysses all-to-all splits
 *         heads; its degree cannot exceed the head count).
 *   [SWA] ring sliding-window attention README: argument list (q/k/v shapes,
 *         window_size, cu_seqlens global over all ranks, softmax_scale default
 *         1/sqrt(head_dim), cp_group None = single-GPU mode), varlen example,
 *         streaming-LLM (attention sink) section.
 *   [LCA] Long Context Attention notes: "Ring Attention" (N hosts on a ring
 *         pass KV pieces; block order is free), "Solution" (striped
 *         permutation), "Zig-Zag Attention" (fold the mask), "Tree Attention"
 *         (max / logsumexp are associative), "Motivation" (keep the LSE).
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, contiguous, in device memory owned by
 *     the caller.  bf16 is IEEE bfloat16; f32 is IEEE binary32.
 *   - q is [B,S,Hq,D]; k and v are [B,S,Hkv,D] (varlen: B = 1, [T,H,D]).
 *     Hq must be a multiple of Hkv; query head h reads kv head h / (Hq/Hkv).
 *   - LSE is the natural-log log-sum-exp of the scaled scores over the
 *     visible keys, f32, laid out [B,Hq,S]; a row with no visible key has
 *     LSE = -inf and output 0.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; no call synchronises, allocates device memory or copies from
 *     the host, so every call can be recorded into a HIP graph.  Scratch
 *     (tile lists, staged copies, accumulators) lives in caller-owned
 *     workspace sized by the matching *_workspace_size call; the tile lists
 *     are built on the device at the start of each call.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On a status other than USP_OK and USP_ERR_HIP nothing was enqueued
 *     and outputs are untouched; usp_last_error() returns a message for the
 *     calling thread.  USP_ERR_HIP reports a failed kernel launch, after
 *     which the launches before it stay enqueued.
 *   - Results are deterministic: no atomics in any reduction.
 */
#ifndef USP_H_
#define USP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  USP_OK = 0,
  USP_ERR_INVALID_ARG = 1,   /* bad pointer, shape, divisibility, range    */
  USP_ERR_UNSUPPORTED = 2,   /* valid request this library does not serve  */
  USP_ERR_WORKSPACE = 3,     /* workspace missing or too small             */
  USP_ERR_HIP = 4            /* HIP runtime error                          */
} usp_status;

/* Ring layouts of the sequence over N virtual ranks, L = S/N rows each.
 *   BASIC  : rank r holds positions [r*L, (r+1)*L)                    [LCA "Ring Attention"]
 *   ZIGZAG : 2N chunks of c = S/(2N); rank r holds chunk r then chunk 2N-1-r
 *                                                                    [LCA "Zig-Zag Attention"]
 *   STRIPE : blocks of b tokens; block beta goes to rank beta mod N, so
 *            local row t of rank r is position ((t/b)*N + r)*b + t%b [LCA "Solution"] */
typedef enum { USP_RING_BASIC = 0, USP_RING_ZIGZAG = 1, USP_RING_STRIPE = 2 } usp_ring_impl;

/* Mask of one block-attention call.  POSITIONAL derives visibility from the
 * global positions of the rows (qmap/kmap) and causal / window / n_sink /
 * cu_seqlens.  The explicit classes use local indices t (query) and u (key):
 *   FULL: every key;  CAUSAL: u <= t;  CAUSAL_STRICT: u < t (the striped
 *   round that drops the first query and the last key, [LCA "Solution"]);
 *   EMPTY: no key (the call writes O = 0, LSE = -inf, or with accumulate=1
 *   changes nothing). */
typedef enum {
  USP_MASK_EMPTY = 0,
  USP_MASK_FULL = 1,
  USP_MASK_CAUSAL = 2,
  USP_MASK_CAUSAL_STRICT = 3,
  USP_MASK_POSITIONAL = 4
} usp_mask_class;

typedef enum { USP_DT_BF16 = 0, USP_DT_F32 = 1 } usp_dtype;

/* Which global positions the rows of one virtual rank hold. */
typedef struct usp_posmap {
  int32_t impl;          /* usp_ring_impl                        */
  int32_t ring_degree;   /* N >= 1                               */
  int32_t rank;          /* 0 <= rank < N                        */
  int32_t stripe_block;  /* b >= 1 (STRIPE only)                 */
  int64_t S_global;      /* total sequence length S              */
} usp_posmap;

/* Message for the last non-OK status of the calling thread ("" if none). */
const char* usp_last_error(void);

/* Library version string. */
const char* usp_version(void);

/* ------------------------------------------------------------------ permute
 * Token reorder along the sequence axis of a tensor viewed as
 * [outer, S, inner] (inner elements of dtype dt per row), [YC "2. Usage":
 * the extract function reorders inputs for the load-balanced ring].
 *   rank == -1, inverse == 0: out[o, r*L + t, :] = in[o, pos_r(t), :]
 *        (natural order -> rank-major order, all ranks);
 *   rank == -1, inverse == 1: the inverse (rank-major -> natural);
 *   rank >= 0 : global USP rank g = rank = r*ud + u (ring rank r, Ulysses
 *        rank u) holding the u-th contiguous piece of L/ud rows of ring rank
 *        r's shard; inverse == 0 extracts it: out is [outer, L/ud, inner];
 *        inverse == 1 scatters such a shard back into the natural-order out
 *        (only that shard's rows are written).
 * Out-of-place only (in and out must not overlap).  S must be divisible by N
 * (BASIC), 2N (ZIGZAG) or N*b (STRIPE), and L by ulysses_degree.  Bit-exact
 * copy; HBM-bound.  outer may be 0 (nothing is enqueued; in and out may then
 * be NULL). */
usp_status usp_permute(const void* in, void* out, int64_t outer, int64_t S, int64_t inner,
                       usp_dtype dt, usp_ring_impl impl, int ring_degree, int ulysses_degree,
                       int stripe_block, int rank, int inverse, void* stream);

/* ------------------------------------------------------- Ulysses relayout
 * The local pack / unpack around the Ulysses all-to-all for Ulysses rank u
 * of ud, with the all-to-all itself replaced by reading every peer's piece
 * from this device [YC "Why not apply Ulysses and Ring Attention
 * Individually?": Ulysses trades sequence for heads].  Hg = H/ud.
 *   direction 0 (seq -> head): shards[u'] is [B, Ls, H, D] for u' < ud;
 *       local is [B, ud*Ls, Hg, D];
 *       local[b, u'*Ls + s, h', :] = shards[u'][b, s, u*Hg + h', :].
 *   direction 1 (head -> seq): the inverse; writes only head group u of
 *       each shards[u'] and nothing else.
 * `shards` is a host array of ud device pointers; 1 <= ud <= 8, ud divides
 * H.  Bit-exact copy. */
usp_status usp_ulysses_relayout(void* const* shards, void* local, int64_t B, int64_t S_shard,
                                int64_t H, int64_t D, usp_dtype dt, int ulysses_degree,
                                int ulysses_rank, int direction, void* stream);

/* ------------------------------------------------------ block attention
 * One ring step: softmax attention of q [B,Lq,Hq,D] (bf16) against k, v
 * [B,Lk,Hkv,D] (bf16) under `mask`, emitting the partial output and LSE
 * [LCA "Ring Attention", "Motivation"].  For every visible (query t, key u):
 * s = softmax_scale * <q_t, k_u> (bf16 products, f32 accumulation); the
 * partial is O_t = sum_u exp(s - m) v_u / sum_u exp(s - m), LSE_t = m +
 * ln sum_u exp(s - m).  softmax_scale <= 0 selects 1/sqrt(D) [SWA args].
 *
 * POSITIONAL masks: qmap/kmap give the global positions of the q and k rows
 * (same impl, N, b and S; Lq and Lk equal S/N).  A key is visible when it is
 * in the query's sequence (cu_seqlens, global over all ranks [SWA varlen];
 * B must then be 1), and, if causal or window > 0, p_k <= p_q, and, if
 * window > 0, p_q - p_k < window [SWA window_size: the number of keys each
 * query attends to, itself included] or the key is one of the first n_sink
 * tokens of that sequence [SWA streaming-LLM attention sink].
 * Explicit classes require causal = window = n_sink = 0 and no cu_seqlens.
 *
 * out is [B,Lq,Hq,D] in out_dt, lse is [B,Hq,Lq] f32.  accumulate = 0
 * overwrites them with this call's partial; accumulate = 1 (out_dt must be
 * F32) merges this partial into the running (out, lse) with the associative
 * rescale of usp_lse_merge.  D must be 64 or 128.  cu_seqlens_host (nseq+1
 * int32, host) sizes the tile plan; cu_seqlens_dev (same values, device) is
 * read by the device planner and the kernel.  workspace: caller-owned device
 * memory, 256-byte aligned, of at least usp_block_attn_fwd_workspace_size
 * bytes for the same mask arguments (USP_ERR_WORKSPACE otherwise); it holds
 * the call's tile plan, built on the device.
 * Lq or Lk may be 0.  With Lk = 0 no row has a visible key: out = 0 and
 * lse = -inf (accumulate = 1 leaves them unchanged); k and v may then be
 * NULL.  With Lq = 0 nothing is enqueued and q, out, lse may be NULL.
 *
 * Score modifiers, applied to s in this order before the mask and softmax
 * (both off with softcap = 0 and alibi_slopes = NULL):
 *   softcap > 0: s = softcap * tanh(s / softcap) (logit soft-capping: the
 *     softcap argument of [YC] "2. Usage", read with flash-attention's
 *     meaning);
 *   alibi_slopes (device, Hq f32, one per query head of this call): s -=
 *     slope_h * |p_q - p_k| on global positions (the alibi_slopes
 *     argument of [YC] "2. Usage", same reading); POSITIONAL mask only.
 * The returned LSE is that of the modified scores.  A negative or non-finite
 * softcap is USP_ERR_INVALID_ARG; ALiBi over more than 2^22 positions
 * (S, or the varlen token count) is USP_ERR_UNSUPPORTED. */
size_t usp_block_attn_fwd_workspace_size(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                                         const usp_posmap* kmap, int causal, int window, int n_sink,
                                         const int32_t* cu_seqlens_host, int nseq);

usp_status usp_block_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                              float softmax_scale, usp_mask_class mask,
                              const usp_posmap* qmap, const usp_posmap* kmap,
                              int causal, int window, int n_sink,
                              const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int nseq,
                              usp_dtype out_dt, int accumulate, float softcap, const float* alibi_slopes,
                              void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- backward
 * The backward of block attention, as the ring runs it [LCA "Ring
 * Attention": the backward passes the same KV pieces, and their gradients,
 * around the ring, from the saved output and log-sum-exp].  With the final
 * (merged over all steps) output O and LSE of the query rows, one step's
 * gradient terms for every visible (query t, key u) of one (batch, head) are
 *   P = exp(s - LSE_t),  dP = <dO_t, v_u>,  dS = P (dP - delta_t),
 *   dQ_t += softmax_scale * sum_u dS k_u,
 *   dK_u += softmax_scale * sum_t dS q_t,   dV_u += sum_t P dO_t,
 * with s as in usp_block_attn_fwd (bf16 products, f32 accumulation) and
 * delta_t = <dO_t, O_t>.  Because P uses the final LSE, the terms of the
 * ring steps add up to the gradients of the whole attention.
 *
 * usp_attn_bwd_preprocess: delta [B,H,L] f32 = rowsum(dout * out), with out
 *   [B,L,H,D] in out_dt (bf16 or f32) and dout [B,L,H,D] bf16; D one of
 *   8, 16, 32, 64, 128, 256 (D/8 threads share a row inside one wave).
 * usp_block_attn_bwd: q, dout [B,Lq,Hq,D] and k, v [B,Lk,Hkv,D] bf16; lse
 *   and delta [B,Hq,Lq] f32 (a row with LSE = -inf contributes nothing);
 *   dq [B,Lq,Hq,D], dk, dv [B,Lk,Hkv,D] f32 are ACCUMULATED into (+=): the
 *   caller zeroes them once and calls once per ring step.  dK / dV of a KV
 *   head sum over the query heads sharing it (GQA / MQA).  Mask arguments,
 *   softmax_scale, cu_seqlens and D are as in usp_block_attn_fwd; EMPTY
 *   leaves the gradients unchanged.  dq must not alias dk or dv.  Each
 *   gradient element is written by one workgroup (deterministic, no
 *   atomics).  workspace (caller-owned, 256-byte aligned, at least
 *   usp_block_attn_bwd_workspace_size bytes; may be NULL when that is 0)
 *   holds the call's two tile plans, built on the device.  softcap and
 *   alibi_slopes are those of the forward (s above is the modified score,
 *   and with softcap dS is multiplied by the derivative 1 - tanh^2 of the
 *   cap before it reaches dQ and dK). */
usp_status usp_attn_bwd_preprocess(const void* out, usp_dtype out_dt, const void* dout, float* delta,
                                   int64_t B, int64_t L, int64_t H, int64_t D, void* stream);

size_t usp_block_attn_bwd_workspace_size(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                                         const usp_posmap* kmap, int causal, int window, int n_sink,
                                         const int32_t* cu_seqlens_host, int nseq);

usp_status usp_block_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, const float* delta, float* dq, float* dk, float* dv,
                              int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                              float softmax_scale, usp_mask_class mask,
                              const usp_posmap* qmap, const usp_posmap* kmap,
                              int causal, int window, int n_sink,
                              const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int nseq,
                              float softcap, const float* alibi_slopes, void* workspace, size_t ws_bytes,
                              void* stream);

/* --------------------------------------------------------------- decode
 * Decode-time attention over a KV cache, as flash decoding: the cache is cut
 * into pieces of split_keys keys whose partial (O, LSE) are computed
 * independently, then combined [LCA "Ring Attention": flash decoding as
 * ring attention at inference; "Tree Attention": the combine is associative
 * and can run as a tree reduction].
 *
 * q [B,Lq,Hq,D] bf16: Lq new queries per batch row, sitting at the last Lq
 * positions of that row's cache (query t at kv_len - Lq + t); k, v
 * [B,S,Hkv,D] bf16: the cache, row b valid for keys 0 .. kv_len[b]-1
 * (kv_lens NULL: every row holds S keys; otherwise given on device and on
 * host, values in [Lq, S]).  Visibility: causal, and with window > 0 the
 * window / n_sink rule of usp_block_attn_fwd (positions from 0 per row).
 * (Hq/Hkv)*Lq must not exceed 32; D is 64 or 128; split_keys is a positive
 * multiple of 32.  softmax_scale <= 0 selects 1/sqrt(D).  softcap and
 * alibi_slopes (device, Hq f32) are the score modifiers of
 * usp_block_attn_fwd, with the same per-row positions (ALiBi needs S <=
 * 2^22).
 *
 * usp_decode_split_fwd writes, for n = ceil(S / split_keys) pieces, the
 *   partials out_part [n,B,Lq,Hq,D] and lse_part [n,B,Hq,Lq] (f32) of keys
 *   [i*split_keys, (i+1)*split_keys) of each row (LSE = -inf, O = 0 for a
 *   piece with no visible key).  Reads every valid K / V byte once.
 * usp_decode_merge combines the n partials of every (row, query, head):
 *   groups of threads fold interleaved pieces, then pairwise rounds combine
 *   the groups; out [B,Lq,Hq,D] (out_dt) and lse [B,Hq,Lq] f32.  With more
 *   than 64 pieces a first pass folds chunks of 64 pieces into each chunk's
 *   first piece, so out_part / lse_part are scratch: their contents are
 *   undefined after the call. */
usp_status usp_decode_split_fwd(const void* q, const void* k, const void* v,
                                const int32_t* kv_lens_dev, const int32_t* kv_lens_host,
                                float* out_part, float* lse_part,
                                int64_t B, int64_t Lq, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                int64_t split_keys, float softmax_scale, int window, int n_sink,
                                float softcap, const float* alibi_slopes, void* stream);

usp_status usp_decode_merge(float* out_part, float* lse_part, int64_t n_split,
                            int64_t B, int64_t Lq, int64_t Hq, int64_t D,
                            void* out, usp_dtype out_dt, float* lse, void* stream);

/* ---------------------------------------------------------------- merge
 * In-place associative combine of a partial into a running result, rows
 * [row_begin, row_end) of the sequence axis [LCA "Tree Attention": max and
 * logsumexp are associative]:
 *   M = max(L_a, L_b); L = M + ln(e^(L_a - M) + e^(L_b - M));
 *   O = e^(L_a - L) O_a + e^(L_b - L) O_b;   (L_b = -inf leaves (O_a, L_a)).
 * out_acc/out_part are f32 [B,L,H,D]; lse_acc/lse_part f32 [B,H,L].
 * D/4 must divide 64 (D = 4, 8, 16, ..., 256), else USP_ERR_UNSUPPORTED;
 * a row range outside [0, L] is USP_ERR_INVALID_ARG.  An empty row range
 * changes nothing; with B or L = 0 the pointers may be NULL. */
usp_status usp_lse_merge(float* out_acc, float* lse_acc, const float* out_part, const float* lse_part,
                         int64_t B, int64_t L, int64_t H, int64_t D, int64_t row_begin,
                         int64_t row_end, void* stream);

/* ------------------------------------------------------- virtual ring
 * All ring_degree steps of ring attention on one device [LCA "Ring
 * Attention"; SWA single-GPU mode]: host i holds query piece i and at step s
 * the KV piece of j = (i - s) mod N; each step runs block attention with the
 * mask its positions imply and merges its partial into the running result.
 * The KV "send" is a pointer offset; every step is enqueued in order on one
 * stream.  With ulysses_degree ud > 1 the Ulysses seq -> head relayout of
 * q, k, v runs first for Ulysses rank `ulysses_rank` [YC "2. Usage"]; its
 * result is the ring-ordered rows restricted to head group u, so the token
 * permutation and the relayout are one strided copy per tensor.
 *
 * Inputs q [B,S,Hq,D], k/v [B,S,Hkv,D] bf16 hold the whole sequence, in
 * natural order (input_order 0; permuted on the device first) or already
 * rank-major (input_order 1).  Varlen (cu_seqlens set) requires B = 1;
 * the ring layout (basic, zigzag or stripe) then applies to the packed token
 * axis, as the basic layout's contiguous split does [SWA varlen example],
 * with every mask taken from global positions and cu_seqlens.
 * Outputs:
 *   rank == -1: every rank; out [B,S,Hq,D] (out_dtype) and lse [B,Hq,S] in
 *     the input's order (ud must be 1: the head split does not change the
 *     result of all ranks together);
 *   rank >= 0, out_layout 0: ring rank `rank`'s share for Ulysses rank
 *     `ulysses_rank` as attention leaves it, heads split: out [B,L,Hq/ud,D]
 *     and lse [B,Hq/ud,L] in that rank's local row order;
 *   rank >= 0, out_layout 1: the same share after the Ulysses head -> seq
 *     relayout that follows attention [YC "Why not apply Ulysses and Ring
 *     Attention Individually?": the all-to-all before and after attention]:
 *     out [B,L,Hq,D] and lse [B,Hq,L] hold ring rank r's rows in local order
 *     with every head, i.e. the ud Ulysses sequence shards one after another
 *     (shard u' = rows [u' L/ud, (u'+1) L/ud) of each batch row, the rows
 *     usp_permute extracts for global rank r*ud + u'); this call writes head
 *     group u = ulysses_rank of every row and nothing else, so the ud
 *     Ulysses ranks' calls together fill the tensors.  The relayout is part
 *     of the attention epilogue (f32 output) or of the final copy.
 * merge_mode 0 merges in the attention kernel's epilogue; 1 writes each
 * step's partial to the workspace and runs usp_lse_merge.
 * qkv_packed = 1 takes q, k, v from one packed [B,S,3,H,D] tensor (varlen
 * [T,3,H,D]) in the same order convention, as [YC]'s QKV-packed attention
 * (multi-head only: [YC] "Some Conclusions" 2); the slices are copied into
 * the workspace while they are put in ring order.  With usp_ring_bwd the
 * gradients are still returned as separate dq, dk, dv.  softcap and
 * alibi_slopes are the score modifiers of usp_block_attn_fwd, positions
 * global. */
typedef struct usp_ring_args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t B, S, Hq, Hkv, D;
  float softmax_scale;               /* <= 0: 1/sqrt(D)                   */
  int32_t causal, window, n_sink;
  const int32_t* cu_seqlens_dev;     /* NULL unless varlen                 */
  const int32_t* cu_seqlens_host;
  int32_t nseq;
  int32_t impl;                      /* usp_ring_impl                      */
  int32_t ring_degree, ulysses_degree, stripe_block;
  int32_t rank, ulysses_rank;
  int32_t input_order;               /* 0 natural, 1 rank-major            */
  int32_t out_dtype;                 /* usp_dtype                          */
  int32_t merge_mode;                /* 0 fused epilogue, 1 separate merge */
  int32_t qkv_packed;                /* 1: q points to a packed [B,S,3,H,D]
                                        tensor (q, k, v of a token stored
                                        one after the other; Hq == Hkv == H;
                                        k and v are ignored)               */
  float softcap;                     /* score soft-cap, 0: off             */
  const float* alibi_slopes;         /* device, Hq f32 over ALL heads (the
                                        Ulysses rank reads its own group),
                                        or NULL                            */
  int32_t out_layout;                /* rank >= 0: 0 heads split, 1 Ulysses
                                        sequence shards (see Outputs)      */
} usp_ring_args;

/* Bytes of device workspace usp_ring_fwd needs for these arguments. */
size_t usp_ring_fwd_workspace_size(const usp_ring_args* a);

/* Runs the virtual ring.  workspace: device memory of at least
 * usp_ring_fwd_workspace_size(a) bytes, owned by the caller, 256-byte
 * aligned; it holds the tile plans of every step (built on the device by the
 * call), the staged q / k / v and the accumulators. */
usp_status usp_ring_fwd(const usp_ring_args* a, void* workspace, size_t ws_bytes, void* stream);

/* usp_ring_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call with its workspace in a 64 MiB array the library holds on
 * each GPU it runs on, from the first call on that GPU until the process
 * ends.  No allocation of any kind happens in the call.  Arguments whose
 * usp_ring_fwd_workspace_size exceeds 64 MiB are rejected with
 * USP_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * that GPU's one array: calls that overlap on a GPU (other streams or
 * threads, or a recorded graph replayed while another call runs) race on it
 * and must be ordered by the caller.  Nothing in it needs to start at zero:
 * each call rewrites what it reads. */
usp_status usp_ring_fwd_noalloc(const usp_ring_args* a, void* stream);

/* The ring's input staging on its own: writes q, k, v exactly as the
 * attention kernels of usp_ring_fwd / usp_ring_bwd read them for arguments
 * `a`, i.e. the layout's token order [YC "2. Usage": the extract function;
 * LCA "Solution", "Zig-Zag Attention"] restricted to Ulysses head group u:
 *   q_staged [B, Lq_rows, Hq/ud, D]: every rank's rows rank-major (rank -1,
 *     Lq_rows = S) or ring rank r's rows in local order (Lq_rows = L);
 *   k_staged, v_staged [B, S, Hkv/ud, D]: all ranks' rows, rank-major.
 * From natural or rank-major input, packed or not; bf16, bit-exact copies.
 * Where the ring reads the caller's tensors in place (rank-major or basic
 * input, ud = 1, not packed) the same rows are copied with the same gather
 * kernel.  Buffers are caller-owned and must not overlap the inputs. */
usp_status usp_ring_stage(const usp_ring_args* a, void* q_staged, void* k_staged, void* v_staged, void* stream);

/* ------------------------------------------------ virtual ring backward
 * The backward of usp_ring_fwd on one device [LCA "Ring Attention": the
 * backward runs the same ring from the saved output and LSE, dK / dV of a
 * KV piece accumulating as it travels].  `fwd` holds the forward call's
 * arguments unchanged (merge_mode is ignored); its out and lse are now
 * INPUTS: the forward's results, in the order and dtype it wrote them.
 * dout (bf16) has the shape and order of fwd.out.  Outputs, f32,
 * overwritten:
 *   rank == -1: dq [B,S,Hq,D], dk / dv [B,S,Hkv,D], the full gradients, in
 *     the input's order;
 *   rank >= 0 : dq [B,L,Hq/ud,D] of the rank's rows in its local order
 *     (complete: the rank meets every KV piece), and dk / dv
 *     [B,S,Hkv/ud,D] in rank-major order (piece j at rows j*L): the
 *     contributions of this rank's queries to every piece, which a real ring
 *     would sum over the hosts.
 * With fwd.out_layout 1, out, lse and dout are in the sequence-shard layout
 * and their head group u is read; dq stays [B,L,Hq/ud,D].
 * Steps: staging of q, k, v as in usp_ring_fwd; delta =
 * usp_attn_bwd_preprocess(out, dout); N steps of usp_block_attn_bwd (every
 * host of a step in one launch per kernel); natural-order outputs are
 * un-permuted at the end.  The outputs need no initial value: the first
 * launch that reaches a gradient row stores it (step 0 for dq, and for
 * dk / dv with every host; each step for one rank's dk / dv pieces), and
 * rows that no query or key reaches are stored as zeros.  The workspace holds the dQ and dK / dV tile plans
 * of every step (built on the device by the call) and the staged tensors. */
typedef struct usp_ring_bwd_args {
  usp_ring_args fwd;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
} usp_ring_bwd_args;

/* Bytes of device workspace usp_ring_bwd needs (0 for invalid arguments). */
size_t usp_ring_bwd_workspace_size(const usp_ring_bwd_args* a);

/* Runs the backward ring.  workspace: caller-owned device memory of at least
 * usp_ring_bwd_workspace_size(a) bytes, 256-byte aligned. */
usp_status usp_ring_bwd(const usp_ring_bwd_args* a, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ tile scheduler
 * Host-only inspection of the tile plan usp_block_attn_fwd would run (no
 * device work).  Items are 8 int32 each: {q_row0, t0, q_rows, q_rank, k_row0,
 * k_rank, run_begin, run_end}; runs are 4 int32 each: {k_begin, k_end, full,
 * 0}: keys [k_begin, k_end) of the item's KV rows, `full` = 1 when every key
 * of the run is visible to every query row of the item (no per-element
 * mask; length a multiple of *tile_n).  Keys outside every run are visible
 * to no row of the item.  Items come ordered by decreasing work (ties in
 * tile order) when the plan has at most 16384 candidate tiles, in tile
 * order otherwise.  Pass NULL buffers to query the counts only. */
usp_status usp_plan_block(int64_t Lq, int64_t Lk, int64_t D, usp_mask_class mask,
                          const usp_posmap* qmap, const usp_posmap* kmap,
                          int causal, int window, int n_sink,
                          const int32_t* cu_seqlens_host, int nseq, int accumulate,
                          int32_t* items, int64_t items_cap, int32_t* runs, int64_t runs_cap,
                          int64_t* n_items, int64_t* n_runs, int32_t* tile_m, int32_t* tile_n);

/* The transposed plan usp_block_attn_bwd's dK / dV kernel runs (host only,
 * no device work): one item per tile of *tile_k keys of the KV rank, 8 int32
 * each: {first key row, its local key index, keys in the tile, KV rank,
 * first query row (0), query rank, run_begin, run_end}; runs {t_begin,
 * t_end, full, 0} of local query rows, `full` = 1 when every key of the item
 * is visible to every query row of the run (length a multiple of *tile_q).
 * Query rows outside every run see no key of the item; tiles no query sees
 * get no item.  Items come ordered as in usp_plan_block. */
usp_status usp_plan_block_kv(int64_t Lq, int64_t Lk, int64_t D, usp_mask_class mask,
                             const usp_posmap* qmap, const usp_posmap* kmap,
                             int causal, int window, int n_sink,
                             const int32_t* cu_seqlens_host, int nseq,
                             int32_t* items, int64_t items_cap, int32_t* runs, int64_t runs_cap,
                             int64_t* n_items, int64_t* n_runs, int32_t* tile_k, int32_t* tile_q);

/* The device planner on one block, for inspection: the plan the calls above
 * run, built by the GPU into `workspace` exactly as the attention calls
 * build theirs (kv_tiles 0: usp_block_attn_fwd's plan, kv_tiles 1: the dK /
 * dV plan).  Outputs: *n_candidates tiles, *run_slots runs per tile, and
 * *ws_needed bytes; with workspace NULL only these are returned.  Layout:
 * items (8 int32 each, as in usp_plan_block) at byte 0, ordered as there,
 * with the tiles that have nothing to do last (or in place, above 16384
 * candidates) and marked by q_rows = 0; runs (4 int32 each) at byte
 * ((n_candidates * 32 + 255) / 256) * 256, tile g's in slots [g * run_slots,
 * ...), addressed by run_begin / run_end as the kernels read them. */
usp_status usp_plan_block_device(int64_t Lq, int64_t Lk, usp_mask_class mask, const usp_posmap* qmap,
                                 const usp_posmap* kmap, int causal, int window, int n_sink,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int nseq,
                                 int accumulate, int kv_tiles, void* workspace, size_t ws_bytes,
                                 int64_t* n_candidates, int32_t* run_slots, size_t* ws_needed, void* stream);

/* ---------------------------------------------------- kernel timing
 * Instrumentation for benchmarks.  While enabled, every kernel launch of the
 * library is bracketed by two hipEvents recorded on its stream; read sums
 * the elapsed times of the recorded launches of one kernel class (waiting on
 * their events).  Off by default; enabling adds two event records per
 * launch.  Not thread-safe with respect to concurrent reset. */
typedef enum {
  USP_KERNEL_ATTN = 0,      /* block attention (usp_block_attn_fwd and ring steps) */
  USP_KERNEL_PERMUTE = 1,   /* token permutation, output reorder / conversion      */
  USP_KERNEL_RELAYOUT = 2,  /* Ulysses relayout                                     */
  USP_KERNEL_MERGE = 3,     /* separate LSE merge                                   */
  USP_KERNEL_BWD_DQ = 4,    /* backward: dQ kernel of usp_block_attn_bwd            */
  USP_KERNEL_BWD_DKDV = 5,  /* backward: dK / dV kernel of usp_block_attn_bwd       */
  USP_KERNEL_BWD_DELTA = 6, /* backward: usp_attn_bwd_preprocess                    */
  USP_KERNEL_DECODE = 7,    /* decode: usp_decode_split_fwd                         */
  USP_KERNEL_DECODE_MERGE = 8, /* decode: usp_decode_merge                          */
  USP_KERNEL_PLAN = 9       /* device tile planner (both of its kernels)            */
} usp_kernel_class;

usp_status usp_timing_enable(int enable);
usp_status usp_timing_reset(void);
usp_status usp_timing_read(int kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* USP_H_ */
