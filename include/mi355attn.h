/*
 * mi355attn: flash (tiled online-softmax) scaled-dot-product attention and a
 * residual + LayerNorm for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer that the caller allocates, owns
 *    and keeps alive until the enqueued work has finished.  The library never
 *    allocates or frees memory, never synchronizes, and enqueues all of its work on `stream` (0 = the null
 *    stream).  Calls are asynchronous: a return of ATTN_OK means the work was
 *    enqueued.
 *  - Calls enqueue kernel launches only (no memset, copy or event), so they
 *    can be captured into a HIP graph and replayed; every replay recomputes
 *    from the inputs (workspace contents on entry are never read as state).
 *  - Arguments are validated on the host before anything is launched.  A
 *    failed check returns an error code and leaves every output untouched.
 *  - Device DATA is not inspected on the host: a block-table entry outside
 *    [0, num_blocks) is undefined behaviour.
 *  - Results are bitwise deterministic: the same inputs give the same bits,
 *    and a query row's output does not depend on any other query row, head
 *    or batch entry (every online-softmax decision is taken per row).
 *  - Softmax runs in fp32 (row max and row sum in fp32 registers), the
 *    contractions run on bf16 MFMA with fp32 accumulation.  Inference only:
 *    there is no backward pass.
 *  - Masks are additive fp32: 0 keeps a key, -inf removes it (any finite
 *    value is added to the scaled score).  A query row whose keys are all
 *    removed produces an all-zero output and lse = -inf.
 */
#ifndef MI355ATTN_H
#define MI355ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null required pointer, bad size, misaligned or non-unit-stride tensor */
  ATTN_ERR_UNSUPPORTED = 2, /* a head_dim, dtype or shape that is not compiled in */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returns */
  ATTN_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_FP8_E4M3FN = 2 } attn_dtype_t;

/* Rotary position embedding pairing of the encoder's fused RoPE prologue. */
typedef enum {
  ATTN_ROPE_NONE = 0,
  ATTN_ROPE_HALF = 1,        /* lane k pairs with lane k + D/2 (rotate-half) */
  ATTN_ROPE_INTERLEAVED = 2  /* lane 2k pairs with lane 2k + 1 */
} attn_rope_t;

/* Static, human-readable text for a status code (never NULL). */
ATTN_API const char *attn_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
ATTN_API int attn_version(void);

/*
 * Non-causal encoder attention with an optional fused residual add and
 * LayerNorm epilogue.
 *
 * Follows: vit-encoder-neuron-kernels, "Supported shapes and limits"
 * (bidirectional self-attention, standard LayerNorm, residual stream in
 * fp32) and "Repository layout" (attention followed by residual + LayerNorm);
 * V-JEPA2 ViT-L Encoder NKI Kernels for AWS Trainium2, "Repository layout"
 * (residual + LayerNorm kernels around the attention inner); gte-encoder-
 * neuron-kernels, "Constraints" (right padding expressed as an additive key
 * mask).
 *
 *   o[b,h,i,:] = softmax_j(softmax_scale * q[b,h,i,:].k[b,h,j,:] + mask[b,j]) v[b,h,j,:]
 *
 * Layout: q [B,H,S_q,D], k/v [B,H,S_kv,D] addressed by element strides
 * {b,h,s,d}; the d stride must be 1, the others multiples of 8 elements, and
 * the base pointers 16-byte aligned.  in_dtype is ATTN_BF16 or ATTN_F32 (fp32
 * inputs are rounded to bf16, round-to-nearest-even, as they are loaded).
 * D must be 64.
 *
 * Outputs (each optional, but at least one of out / residual_out required):
 *   out          attention output, out_dtype BF16 or F32, [B,H,S_q,D] by
 *                element strides (use strides {S*H*D, D, H*D, 1} for the
 *                token-major [B,S_q,H*D] layout); same alignment rules.
 *   lse          fp32 [B,H,S_q], natural-log log-sum-exp of the scaled scores.
 *   residual_out fp32 [B,S_q,H*D] contiguous: residual + o (head h owns
 *                columns h*D..h*D+D-1); requires residual.  May alias residual.
 *   ln_out       LayerNorm(residual_out) over H*D, ln_dtype BF16 or F32,
 *                contiguous [B,S_q,H*D]; requires residual_out.
 *   ln_mean/ln_rstd  fp32 [B*S_q] statistics of that LayerNorm (nullable).
 * gamma/beta are fp32 [H*D] and nullable (affine-free LayerNorm).
 * mask is nullable fp32 [B,1,1,S_kv], 4-byte aligned, row b at mask + b *
 * mask_stride_b: a stride of at least S_kv (rows do not overlap), or 0 for one
 * row [1,1,1,S_kv] shared by the whole batch; a negative stride, or one in
 * 1..S_kv-1 with B > 1, is ATTN_ERR_INVALID_ARG.
 * key_len is nullable int32 [B] in device memory, 4-byte aligned: the right
 * padding of gte-encoder-neuron-kernels, "Constraints" (a 0/1 attention
 * mask over right-padded rows) and vit-encoder-neuron-kernels, "Attribution
 * and license" (padded-key skipping) as lengths.  Batch row b attends keys
 * 0 .. key_len[b]-1 (clamped to [0, S_kv]); the result is that of an
 * additive mask of 0 on those keys and -inf on the rest, but key tiles past
 * the length are never read.  A row with no key gets o = 0 and lse = -inf.
 * key_len together with mask is ATTN_ERR_INVALID_ARG.
 *
 * Fused RoPE prologue (rope != ATTN_ROPE_NONE; vit-encoder-neuron-kernels,
 * "Kernels": the rotate-half and interleaved pairings; V-JEPA2 ViT-L Encoder
 * NKI Kernels, "Repository layout": host-side RoPE tables).  q and k are
 * rotated before the contraction, in fp32, then rounded to bf16: for each
 * pair (a, b) of lanes of token s (q row s, key s), with k the pair index,
 *     a' = a cos[s,k] - b sin[s,k],   b' = b cos[s,k] + a sin[s,k].
 * rope_cos/rope_sin are fp32 [rows, D/2] contiguous (rows >= max(S_q, S_kv)),
 * 16-byte aligned, the tables of batch entry b at + b * rope_stride_b floats
 * (0: one table for the whole batch; otherwise a multiple of 4).  Any
 * positional layout (1D, 2D or 3D grids, extra unrotated tokens with
 * cos = 1, sin = 0, scaled frequencies) is a matter of the tables.
 * q rows are rotated as the attention kernel loads them; K is rotated once,
 * by a pass on the same stream before it, into rope_workspace (at least
 * attn_encoder_rope_workspace_size() bytes, 256-byte aligned, owned by the
 * caller, contents on entry ignored): every query tile streams all keys, so
 * rotating K inside the key loop would repeat the rotation per query tile.
 * Without rope the workspace fields are ignored.
 */
typedef struct {
  const void *q, *k, *v;
  attn_dtype_t in_dtype;
  int B, H, S_q, S_kv, D;
  int64_t q_stride[4], k_stride[4], v_stride[4];
  const float *mask;
  int64_t mask_stride_b;
  float softmax_scale;
  void *out;
  attn_dtype_t out_dtype;
  int64_t out_stride[4];
  float *lse;
  const float *residual;
  float *residual_out;
  const float *gamma, *beta;
  float eps;
  void *ln_out;
  attn_dtype_t ln_dtype;
  float *ln_mean, *ln_rstd;
  const float *rope_cos, *rope_sin;
  int64_t rope_stride_b;
  attn_rope_t rope;
  void *rope_workspace;
  size_t rope_workspace_bytes;
  const int32_t *key_len;
} attn_encoder_args_t;

ATTN_API int attn_encoder_fwd(const attn_encoder_args_t *args, hipStream_t stream);
/* Bytes of the rotated-K workspace: B * H * S_kv * D elements of in_dtype
 * (0 for invalid arguments). */
ATTN_API size_t attn_encoder_rope_workspace_size(int B, int H, int S_kv, int D, attn_dtype_t in_dtype);

/*
 * GQA single-token decode (split-K "flash-decode" plus a combine pass).
 *
 * Follows: head_dim>128 (256/512) GQA Flash-Decode NKI Kernel for AWS
 * Trainium, "Input contract" (shapes, additive 0/-inf mask, softmax_scale,
 * num_kv_groups) and "Supported shapes (the eligibility gate)" (turned into
 * argument checks here, never into a fallback); its "Future performance
 * follow-on" (sharding the KV stream across many programs) is the split-K.
 *
 *   q [B,Hq,1,D] bf16, k/v [B,Hkv,S_ctx,D] bf16, attn_mask [B,1,1,S_ctx] fp32
 *   (nullable = no mask), out [B,Hq,1,D] bf16, all contiguous and 16-byte
 *   aligned.  Query head h reads KV head h / num_kv_groups; Hq must equal
 *   Hkv * num_kv_groups, num_kv_groups in {1, 2, 4, 8}, D in {256, 512} (the
 *   page's introduction: 256 on sliding-window layers, 512 on global ones).
 *   Key chunks whose mask entries are all -inf are skipped without reading K/V.
 *   A query row whose keys are all masked gets o = 0.
 *   workspace: device scratch of at least attn_decode_gqa_workspace_size()
 *   bytes, 256-byte aligned, owned by the caller; its contents on entry are
 *   ignored.
 */
ATTN_API size_t attn_decode_gqa_workspace_size(int B, int Hq, int S_ctx, int D);
ATTN_API int attn_decode_gqa(const void *q, const void *k, const void *v, const float *attn_mask,
                    float softmax_scale, int num_kv_groups, int B, int Hq, int Hkv, int S_ctx, int D,
                    void *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_gqa without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same operation, operands,
 * requirements and result bits as attn_decode_gqa; the chunk partials go to
 * a device array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends.  The call allocates nothing.
 *   - A problem whose attn_decode_gqa_workspace_size() exceeds
 *     ATTN_DECODE_NOALLOC_SCRATCH_BYTES returns ATTN_ERR_WORKSPACE (use
 *     attn_decode_gqa with a workspace of that size instead).
 *   - Every call on one GPU uses that GPU's one array: calls that can overlap
 *     on the same GPU (two streams, or two host threads) race on it and must
 *     be serialised by the caller.  The array's contents on entry are never
 *     read as state.
 *   - The first call on each device looks the array up (hipGetSymbolAddress);
 *     a failure there returns ATTN_ERR_HIP.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ATTN_API int attn_decode_gqa_noalloc(const void *q, const void *k, const void *v, const float *attn_mask,
                                     float softmax_scale, int num_kv_groups, int B, int Hq, int Hkv, int S_ctx,
                                     int D, void *out, hipStream_t stream);

/*
 * GQA single-token decode over a per-sequence key range (sliding-window
 * layers).
 *
 * Follows: the same page, "Future performance follow-on" (a windowed-KV
 * gather for sliding-window layers: only the most recent window of keys is
 * needed).  Sequence b attends the keys j with
 *     e_b = clamp(key_end[b], 0, S_ctx)              (S_ctx if key_end is null)
 *     s_b = max(clamp(key_begin[b], 0, e_b), e_b - max_keys)   (0 if key_begin is null)
 *     s_b <= j < e_b  and  attn_mask[b, j] != -inf,
 * i.e. the range is cut to its last max_keys keys (the window).  The other
 * operands, their layouts and the requirements are those of attn_decode_gqa;
 * key_begin/key_end are device int32 [B] (each nullable, 4-byte aligned),
 * read by the kernels, so the range may change between calls without a host
 * round trip.  The grid covers only min(ceil(min(max_keys, S_ctx)/64) + 1,
 * ceil(S_ctx/64)) chunks of 64 keys per sequence, counted from s_b rounded
 * down to a multiple of 64: keys before the window are neither fetched nor
 * given work.  A sequence with an empty range gets o = 0.
 *   workspace: at least attn_decode_gqa_window_workspace_size(B, Hq, S_ctx,
 *   max_keys, D) bytes, 256-byte aligned, owned by the caller; contents on
 *   entry ignored.  max_keys >= 1, else ATTN_ERR_INVALID_ARG.
 */
ATTN_API size_t attn_decode_gqa_window_workspace_size(int B, int Hq, int S_ctx, int max_keys, int D);
ATTN_API int attn_decode_gqa_window(const void *q, const void *k, const void *v, const float *attn_mask,
                           const int32_t *key_begin, const int32_t *key_end, int max_keys,
                           float softmax_scale, int num_kv_groups, int B, int Hq, int Hkv, int S_ctx,
                           int D, void *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * History-only GQA prefill over a paged FP8 KV cache.
 *
 * Follows: Prefill Context-Parallel Attention POC for Trainium2, "Layout"
 * (Q [Hq,Lq,D], K/V [blocks,Hkv,block_size,D], O [Hq,Lq,D]; Q heads sharing
 * a KV head packed together; online max/sum in fp32; runtime additive score
 * bias derived from actual_history_len) and "Current POC constraints" (BF16
 * Q, FP8 E4M3FN K/V, head_dim a multiple of 128, block_size <= 512).  Only
 * history keys participate; query tokens do not attend to one another.
 *
 *   q [Hq,Lq,D] bf16; k_cache/v_cache [num_blocks,Hkv,block_size,D] e4m3fn
 *   codes with one fp32 dequantisation scale each (k = code * k_scale);
 *   block_table int32 [max_blocks] maps logical block i to a physical block;
 *   logical key j lives at block_table[j / block_size], row j % block_size.
 *   Keys j >= actual_history_len get an additive -inf (blocks wholly past
 *   it are never read).  out [Hq,Lq,D] bf16, lse fp32 [Hq,Lq] (nullable).
 *   Requirements: D == 256, block_size a multiple of 64, 1 <= actual_history_len
 *   <= max_blocks*block_size, Hq == Hkv*num_kv_groups, all pointers 16-byte
 *   aligned.
 */
ATTN_API int attn_prefill_paged(const void *q, const void *k_cache, const void *v_cache, float k_scale,
                       float v_scale, const int32_t *block_table, int max_blocks, int num_blocks,
                       int block_size, int actual_history_len, float softmax_scale, int num_kv_groups,
                       int Hq, int Hkv, int Lq, int D, void *out, float *lse, hipStream_t stream);

/*
 * The history-only GQA prefill of attn_prefill_paged, computed through a
 * workspace: the same operation, arguments and requirements, the same
 * result (the fp8 codes expand to bf16 exactly either way).
 *
 * Follows: the same page, "Layout" and "Current POC constraints"; its FP8
 * K/V is consumed by bf16 matmuls.  Here the live history
 * (actual_history_len keys of every KV head) is first expanded once per call
 * into bf16 tiles of 32 keys laid out as the attention kernel's on-chip
 * buffers hold them; the attention kernel then copies each tile from memory
 * into on-chip storage directly, with no per-tile conversion.  Faster at long
 * histories; costs one pass over the live history (fp8 read, bf16 written).
 *   workspace: at least attn_prefill_paged_expanded_workspace_size(Hkv,
 *   actual_history_len, D) bytes (Hkv * ceil(actual_history_len / 32) *
 *   32768 at D = 256), 256-byte aligned, owned by the caller; contents on
 *   entry ignored, overwritten.  Missing or too small: ATTN_ERR_WORKSPACE.
 *   The size function returns 0 for invalid or unsupported arguments.
 */
ATTN_API size_t attn_prefill_paged_expanded_workspace_size(int Hkv, int actual_history_len, int D);
ATTN_API int attn_prefill_paged_expanded(const void *q, const void *k_cache, const void *v_cache, float k_scale,
                                float v_scale, const int32_t *block_table, int max_blocks, int num_blocks,
                                int block_size, int actual_history_len, float softmax_scale, int num_kv_groups,
                                int Hq, int Hkv, int Lq, int D, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Paged history plus causal current-token GQA prefill.
 *
 * Follows: Prefill Context-Parallel Attention POC for Trainium2, introduction
 * (its first version leaves attention among the current tokens out) and
 * "Layout".  Query token t of head h attends the history keys
 * 0..actual_history_len-1 of the paged cache exactly as attn_prefill_paged,
 * and then the current tokens' keys 0..t of KV head h / num_kv_groups: one
 * softmax over the joined key list, which is the log-sum-exp merge of the
 * history result and the current-token result.  Two kernels on the stream:
 * the history one hands its fp32 result and lse to the current-token one,
 * which continues the same online softmax (the merge is exact up to fp32
 * rounding).
 *
 *   Arguments as attn_prefill_paged, plus k_cur/v_cur [Hkv,Lq,D] bf16
 *   (contiguous, 16-byte aligned, non-null; no scale: the current tokens'
 *   K/V in model units).  actual_history_len may be 0 (no history; the block
 *   table is then not read).  lse (nullable) is the joined log-sum-exp.
 *   workspace: device scratch of at least
 *   attn_prefill_paged_causal_workspace_size(Hq, Hkv, Lq, D) bytes (about
 *   Hq*Lq*(4D+4) bytes), 256-byte aligned, owned by the caller, contents on
 *   entry ignored: the history kernel leaves its normalised output in fp32
 *   and its lse there, and the current-token kernel continues the softmax
 *   from that state (running max = lse, sum = 1).
 *   Current V rows after a query's token contribute p = 0 exactly, which
 *   keeps every finite value out; a non-finite current V value also reaches
 *   the earlier rows of its 32-key tile (0 * inf), so current K/V must be
 *   finite, as they are for real tokens.
 */
ATTN_API int attn_prefill_paged_causal(const void *q, const void *k_cache, const void *v_cache, float k_scale,
                              float v_scale, const int32_t *block_table, int max_blocks, int num_blocks,
                              int block_size, int actual_history_len, const void *k_cur, const void *v_cur,
                              float softmax_scale, int num_kv_groups, int Hq, int Hkv, int Lq, int D,
                              void *out, float *lse, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * attn_prefill_paged_causal with the history taken through expanded bf16
 * tile images, as attn_prefill_paged_expanded does for the history-only
 * prefill: the same operation, arguments, requirements and result.
 *
 * Follows: the passages of attn_prefill_paged_causal and of
 * attn_prefill_paged_expanded.
 *   workspace: at least attn_prefill_paged_causal_expanded_workspace_size(Hq,
 *   Hkv, Lq, actual_history_len, D) bytes, 256-byte aligned, owned by the
 *   caller: the hand-off state of attn_prefill_paged_causal (rounded up to 256
 *   bytes), then the history's tile images (none for an empty history), then
 *   the current tokens' K/V as tile images of their own (Hkv * ceil(Lq / 32)
 *   * 32768 bytes at D = 256).  Contents on entry ignored.  Missing or too
 *   small: ATTN_ERR_WORKSPACE.  The size function returns 0 for invalid or
 *   unsupported arguments.
 */
ATTN_API size_t attn_prefill_paged_causal_expanded_workspace_size(int Hq, int Hkv, int Lq, int actual_history_len,
                                                                  int D);
ATTN_API int attn_prefill_paged_causal_expanded(const void *q, const void *k_cache, const void *v_cache,
                                       float k_scale, float v_scale, const int32_t *block_table, int max_blocks,
                                       int num_blocks, int block_size, int actual_history_len, const void *k_cur,
                                       const void *v_cur, float softmax_scale, int num_kv_groups, int Hq, int Hkv,
                                       int Lq, int D, void *out, float *lse, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream);
ATTN_API size_t attn_prefill_paged_causal_workspace_size(int Hq, int Hkv, int Lq, int D);

/*
 * (Residual +) LayerNorm over the last dimension.
 *
 * Follows: gte-encoder-neuron-kernels, "Repository layout" ((residual +)
 * LayerNorm kernel) and vit-encoder-neuron-kernels, "Supported shapes and
 * limits" (standard LayerNorm, fp32 residual stream and statistics).
 *
 *   residual_out = residual + x          (x nullable: then residual_out = residual)
 *   y = (residual_out - mean) * rstd * gamma + beta,  rstd = 1/sqrt(var + eps),
 *   var the biased variance; statistics in fp32.
 *   residual fp32 [rows,hidden]; x [rows,hidden] in x_dtype (BF16 or F32);
 *   residual_out fp32 (nullable, may alias residual); y in y_dtype (BF16 or
 *   F32); gamma/beta fp32 [hidden] nullable; mean/rstd fp32 [rows] nullable.
 *   hidden must be a multiple of 8 and at most 8192; pointers 16-byte aligned.
 */
ATTN_API int res_ln(const float *residual, const void *x, attn_dtype_t x_dtype, const float *gamma,
           const float *beta, float eps, int rows, int hidden, float *residual_out, void *y,
           attn_dtype_t y_dtype, float *mean, float *rstd, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355ATTN_H */
