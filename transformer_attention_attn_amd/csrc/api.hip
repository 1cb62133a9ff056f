// C-ABI entry points: host-side validation, then kernel launches on the
// caller's stream.  No allocation, no synchronisation.
#include <math.h>
#include <string.h>

#include "../../include/mi355attn.h"
#include "launch.h"

using namespace mi355;

static_assert(kDecodeScratchBytes == ATTN_DECODE_NOALLOC_SCRATCH_BYTES, "scratch size stated in the header");

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// finite by bit pattern (exponent field not all ones), immune to fast-math folding
bool finite(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return (u & 0x7f800000u) != 0x7f800000u;
}

// Kernels take the exp2 scale c > 0: a negative scale becomes a positive one on
// -q (exact), and a zero scale a positive one so small that every exponent
// rounds to 2^0 exactly (|c * s| < 2^-40 for any finite bf16 score), which is
// what a zero scale gives.
void exp2_scale(float scale, float *c, int *q_neg) {
  float x = scale * 1.4426950408889634f;
  *q_neg = x < 0.0f;
  x = fabsf(x);
  *c = x > 0.0f ? x : 1e-30f;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Chunks of keys per sequence the decode grid spans.  Without a range: the
// whole cache.  With one: a range of at most w = min(max_keys, S_ctx) keys
// starting anywhere touches at most ceil(w / chunk) + 1 chunks, and never
// more than the cache holds.
int64_t decode_chunks(int S_ctx, int max_keys, bool ranged) {
  const int64_t C = decode_chunk_keys();
  const int64_t all = (S_ctx + C - 1) / C;
  if (!ranged) return all;
  const int64_t w = max_keys < S_ctx ? max_keys : S_ctx;
  const int64_t n = (w + C - 1) / C + 1;
  return n < all ? n : all;
}

// Checks of the decode's operands (everything but the workspace).
int decode_check(const void *q, const void *k, const void *v, const float *attn_mask, float softmax_scale,
                 int num_kv_groups, int B, int Hq, int Hkv, int S_ctx, int D, const void *out) {
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_ctx <= 0 || D <= 0 || num_kv_groups <= 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)Hkv * num_kv_groups != Hq) return ATTN_ERR_INVALID_ARG;
  if (D != 256 && D != 512) return ATTN_ERR_UNSUPPORTED;
  if (num_kv_groups > decode_max_groups() || (num_kv_groups & (num_kv_groups - 1)))
    return ATTN_ERR_UNSUPPORTED;
  if (!finite(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_INVALID_ARG;
  if (attn_mask && !aligned16(attn_mask)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

int decode_common(const void *q, const void *k, const void *v, const float *attn_mask, const int32_t *key_begin,
                  const int32_t *key_end, int max_keys, bool ranged, float softmax_scale, int num_kv_groups, int B,
                  int Hq, int Hkv, int S_ctx, int D, void *out, void *workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  const int rc = decode_check(q, k, v, attn_mask, softmax_scale, num_kv_groups, B, Hq, Hkv, S_ctx, D, out);
  if (rc != ATTN_OK) return rc;
  const int64_t n_chunks = decode_chunks(S_ctx, max_keys, ranged);
  const size_t need = ranged ? attn_decode_gqa_window_workspace_size(B, Hq, S_ctx, max_keys, D)
                             : attn_decode_gqa_workspace_size(B, Hq, S_ctx, D);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_INVALID_ARG;
  if (n_chunks * Hkv * B > 0x7fffffffLL || Hq > 65535) return ATTN_ERR_UNSUPPORTED;  // one-dimensional grid

  DecodeLaunch L;
  memset(&L, 0, sizeof L);
  L.q = static_cast<const __bf16 *>(q);
  L.k = static_cast<const __bf16 *>(k);
  L.v = static_cast<const __bf16 *>(v);
  L.mask = attn_mask;
  L.key_begin = key_begin;
  L.key_end = key_end;
  L.max_keys = max_keys;
  L.B = B;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.G = num_kv_groups;
  L.S_ctx = S_ctx;
  L.D = D;
  L.n_chunks = (int)n_chunks;
  L.c = softmax_scale * 1.4426950408889634f;
  const int64_t parts = (int64_t)B * Hq * n_chunks;
  L.ws_o = static_cast<float *>(workspace);
  L.ws_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + ((parts * D * 4) + 255) / 256 * 256);
  L.out = static_cast<__bf16 *>(out);
  return hip_status(launch_decode(L, stream));
}

}  // namespace
extern "C" size_t attn_prefill_paged_causal_workspace_size(int Hq, int Hkv, int Lq, int D);
extern "C" size_t attn_prefill_paged_expanded_workspace_size(int Hkv, int actual_history_len, int D);
extern "C" size_t attn_prefill_paged_causal_expanded_workspace_size(int Hq, int Hkv, int Lq, int actual_history_len,
                                                                      int D);
namespace {

// Bytes of the history -> current-token handoff's O part: the normalised
// history output [Hq*Lq, D] in fp32, rounded up to 256 bytes (the lse
// [Hq*Lq] follows).
int64_t prefill_handoff_o_bytes(int Hq, int, int Lq, int D) {
  return ((int64_t)Hq * Lq * D * 4 + 255) / 256 * 256;
}

// Shared validation and launch of the paged prefill; k_cur/v_cur non-null
// adds the causal current-token part (then an empty history is allowed and
// the workspace carries the history's state).
int prefill_common(const void *q, const void *k_cache, const void *v_cache, float k_scale, float v_scale,
                   const int32_t *block_table, int max_blocks, int num_blocks, int block_size, int actual_history_len,
                   const void *k_cur, const void *v_cur, float softmax_scale, int num_kv_groups, int Hq, int Hkv,
                   int Lq, int D, void *out, float *lse, void *workspace, size_t workspace_bytes,
                   void *img_ws, size_t img_bytes, void *img_cur, hipStream_t stream) {
  const bool cur = k_cur != nullptr;
  if (!q || !k_cache || !v_cache || !block_table || !out) return ATTN_ERR_INVALID_ARG;
  if (max_blocks <= 0 || num_blocks <= 0 || block_size <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || D <= 0 ||
      num_kv_groups <= 0)
    return ATTN_ERR_INVALID_ARG;
  if ((int64_t)Hkv * num_kv_groups != Hq) return ATTN_ERR_INVALID_ARG;
  if (actual_history_len < (cur ? 0 : 1) || (int64_t)actual_history_len > (int64_t)max_blocks * block_size)
    return ATTN_ERR_INVALID_ARG;
  if (D != 256) return ATTN_ERR_UNSUPPORTED;
  if (block_size % 64 != 0 || block_size % prefill_key_tile() != 0) return ATTN_ERR_UNSUPPORTED;
  if (!finite(k_scale) || !finite(v_scale) || !(k_scale > 0.0f) || !(v_scale > 0.0f)) return ATTN_ERR_INVALID_ARG;
  if (!finite(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return ATTN_ERR_INVALID_ARG;
  if (cur && (!aligned16(k_cur) || !aligned16(v_cur))) return ATTN_ERR_INVALID_ARG;
  if (cur) {
    if (!workspace || workspace_bytes < attn_prefill_paged_causal_workspace_size(Hq, Hkv, Lq, D))
      return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_INVALID_ARG;
  }
  if (img_ws) {
    if (img_bytes < attn_prefill_paged_expanded_workspace_size(Hkv, actual_history_len, D)) return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(img_ws) & 255u) != 0) return ATTN_ERR_INVALID_ARG;
  }
  if (((int64_t)num_blocks * Hkv * block_size * D) > ((int64_t)1 << 40)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)num_kv_groups * Lq > 0x7fffffffLL - 256) return ATTN_ERR_UNSUPPORTED;
  // a 32-key tile of current K/V is addressed with 32-bit offsets from its own base
  if (cur && (int64_t)Lq * D * 2 > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;

  PrefillLaunch L;
  memset(&L, 0, sizeof L);
  L.q = static_cast<const __bf16 *>(q);
  L.kc = static_cast<const uint8_t *>(k_cache);
  L.vc = static_cast<const uint8_t *>(v_cache);
  L.bt = block_table;
  L.bs = block_size;
  L.L_act = actual_history_len;
  L.Hkv = Hkv;
  L.G = num_kv_groups;
  L.Lq = Lq;
  exp2_scale(softmax_scale * k_scale, &L.c, &L.q_neg);
  L.v_scale = v_scale;
  if (cur) {
    int neg;
    L.kcur = static_cast<const __bf16 *>(k_cur);
    L.vcur = static_cast<const __bf16 *>(v_cur);
    exp2_scale(softmax_scale, &L.c_cur, &neg);
    // One q sign for both loops: the sign of softmax_scale (k_scale > 0; if
    // softmax_scale * k_scale underflowed to zero the history part is
    // sign-blind anyway).
    L.q_neg = neg;
    L.ws_o = static_cast<float *>(workspace);
    L.ws_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + prefill_handoff_o_bytes(Hq, Hkv, Lq, D));
  }
  if (img_ws) {
    L.img = static_cast<char *>(img_ws);
    L.n_tiles = (actual_history_len + prefill_key_tile() - 1) / prefill_key_tile();
  }
  if (img_cur) {
    L.img_cur = static_cast<char *>(img_cur);
    L.n_tiles_cur = (Lq + prefill_key_tile() - 1) / prefill_key_tile();
  }
  L.out = static_cast<__bf16 *>(out);
  L.lse = lse;
  return hip_status(launch_prefill(L, stream));
}

}  // namespace

extern "C" {

const char *attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument (null pointer, size, stride or alignment)";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: head_dim, dtype or shape not compiled in";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
    default: return "unknown attn status";
  }
}

int attn_version(void) { return 10400; }

size_t attn_encoder_rope_workspace_size(int B, int H, int S_kv, int D, attn_dtype_t in_dtype) {
  if (B <= 0 || H <= 0 || S_kv <= 0 || D <= 0) return 0;
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F32) return 0;
  return (size_t)B * H * S_kv * D * (in_dtype == ATTN_F32 ? 4 : 2);
}

int attn_encoder_fwd(const attn_encoder_args_t *a, hipStream_t stream) {
  if (!a) return ATTN_ERR_INVALID_ARG;
  if (!a->q || !a->k || !a->v) return ATTN_ERR_INVALID_ARG;
  if (a->B <= 0 || a->H <= 0 || a->S_q <= 0 || a->S_kv <= 0 || a->D <= 0) return ATTN_ERR_INVALID_ARG;
  if (a->in_dtype != ATTN_BF16 && a->in_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (a->D != 64) return ATTN_ERR_UNSUPPORTED;
  if (!finite(a->softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!a->out && !a->residual_out) return ATTN_ERR_INVALID_ARG;
  if ((a->residual == nullptr) != (a->residual_out == nullptr)) return ATTN_ERR_INVALID_ARG;
  if (a->ln_out && !a->residual_out) return ATTN_ERR_INVALID_ARG;
  if ((a->ln_mean || a->ln_rstd) && !a->ln_out) return ATTN_ERR_INVALID_ARG;
  if (a->ln_out && !(finite(a->eps) && a->eps >= 0.0f)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v)) return ATTN_ERR_INVALID_ARG;
  const int64_t *st[3] = {a->q_stride, a->k_stride, a->v_stride};
  for (int t = 0; t < 3; ++t) {
    if (st[t][3] != 1) return ATTN_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i)
      if (st[t][i] < 0 || st[t][i] % 8) return ATTN_ERR_INVALID_ARG;
    if (st[t][2] >= ((int64_t)1 << 22)) return ATTN_ERR_UNSUPPORTED;  // per-tile offsets are 32-bit
  }
  if (a->out) {
    if (a->out_dtype != ATTN_BF16 && a->out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(a->out) || a->out_stride[3] != 1) return ATTN_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i)
      if (a->out_stride[i] < 0 || a->out_stride[i] % 8) return ATTN_ERR_INVALID_ARG;
  }
  if (a->residual && (!aligned16(a->residual) || !aligned16(a->residual_out))) return ATTN_ERR_INVALID_ARG;
  // per-batch mask rows must not overlap; stride 0 shares one row across the batch
  if (a->mask && (a->mask_stride_b < 0 || (a->B > 1 && a->mask_stride_b != 0 && a->mask_stride_b < a->S_kv)))
    return ATTN_ERR_INVALID_ARG;
  if (a->mask && (reinterpret_cast<uintptr_t>(a->mask) & 3u)) return ATTN_ERR_INVALID_ARG;
  if (a->key_len && (a->mask || (reinterpret_cast<uintptr_t>(a->key_len) & 3u))) return ATTN_ERR_INVALID_ARG;
  const int64_t hidden = (int64_t)a->H * a->D;
  if (a->ln_out) {
    if (a->ln_dtype != ATTN_BF16 && a->ln_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (hidden > res_ln_max_hidden()) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(a->ln_out) || (a->gamma && !aligned16(a->gamma)) || (a->beta && !aligned16(a->beta)))
      return ATTN_ERR_INVALID_ARG;
  }
  if ((int64_t)a->B * a->H * ((a->S_q + encoder_rows_per_block() - 1) / encoder_rows_per_block()) > 0x7fffffffLL)
    return ATTN_ERR_UNSUPPORTED;
  if (a->rope != ATTN_ROPE_NONE) {
    if (a->rope != ATTN_ROPE_HALF && a->rope != ATTN_ROPE_INTERLEAVED) return ATTN_ERR_UNSUPPORTED;
    if (!a->rope_cos || !a->rope_sin || !aligned16(a->rope_cos) || !aligned16(a->rope_sin)) return ATTN_ERR_INVALID_ARG;
    if (a->rope_stride_b < 0 || a->rope_stride_b % 4) return ATTN_ERR_INVALID_ARG;
    if (!a->rope_workspace ||
        a->rope_workspace_bytes < attn_encoder_rope_workspace_size(a->B, a->H, a->S_kv, a->D, a->in_dtype))
      return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->rope_workspace) & 255u) != 0) return ATTN_ERR_INVALID_ARG;
  }

  EncoderLaunch L;
  memset(&L, 0, sizeof L);
  L.q = a->q;
  L.k = a->k;
  L.v = a->v;
  for (int i = 0; i < 4; ++i) {
    L.qs[i] = a->q_stride[i];
    L.ks[i] = a->k_stride[i];
    L.vs[i] = a->v_stride[i];
    L.os[i] = a->out_stride[i];
  }
  L.mask = a->mask;
  L.mask_sb = a->mask_stride_b;
  L.key_len = a->key_len;
  L.B = a->B;
  L.H = a->H;
  L.Sq = a->S_q;
  L.Skv = a->S_kv;
  exp2_scale(a->softmax_scale, &L.c, &L.q_neg);
  L.out = a->out;
  L.out_f32 = a->out_dtype == ATTN_F32;
  L.lse = a->lse;
  L.res = a->residual;
  L.res_out = a->residual_out;
  L.rope = (int)a->rope;
  L.rope_cos = a->rope_cos;
  L.rope_sin = a->rope_sin;
  L.rope_sb = a->rope_stride_b;
  if (a->rope != ATTN_ROPE_NONE) {
    // K rotated once into the workspace (contiguous [B,H,S_kv,D]), read from there
    RopeLaunch R;
    memset(&R, 0, sizeof R);
    R.k = a->k;
    for (int i = 0; i < 4; ++i) R.ks[i] = a->k_stride[i];
    R.out = a->rope_workspace;
    R.B = a->B;
    R.H = a->H;
    R.S = a->S_kv;
    R.D = a->D;
    R.f32 = a->in_dtype == ATTN_F32;
    R.rope = (int)a->rope;
    R.cos = a->rope_cos;
    R.sin = a->rope_sin;
    R.sb = a->rope_stride_b;
    const int rc0 = hip_status(launch_rope_k(R, stream));
    if (rc0 != ATTN_OK) return rc0;
    L.k = a->rope_workspace;
    L.ks[0] = (int64_t)a->H * a->S_kv * a->D;
    L.ks[1] = (int64_t)a->S_kv * a->D;
    L.ks[2] = a->D;
    L.ks[3] = 1;
  }
  int rc = hip_status(launch_encoder(L, a->in_dtype == ATTN_F32, stream));
  if (rc != ATTN_OK || !a->ln_out) return rc;

  ResLnLaunch R;
  memset(&R, 0, sizeof R);
  R.res = a->residual_out;
  R.x = nullptr;
  R.gamma = a->gamma;
  R.beta = a->beta;
  R.eps = a->eps;
  R.rows = a->B * a->S_q;
  R.hidden = (int)hidden;
  R.res_out = nullptr;
  R.y = a->ln_out;
  R.y_bf16 = a->ln_dtype == ATTN_BF16;
  R.mean = a->ln_mean;
  R.rstd = a->ln_rstd;
  return hip_status(launch_res_ln(R, stream));
}

size_t attn_decode_gqa_window_workspace_size(int B, int Hq, int S_ctx, int max_keys, int D) {
  if (B <= 0 || Hq <= 0 || S_ctx <= 0 || max_keys <= 0 || D <= 0) return 0;
  const int64_t n_chunks = decode_chunks(S_ctx, max_keys, true);
  const int64_t parts = (int64_t)B * Hq * n_chunks;
  const int64_t o_bytes = ((parts * D * 4) + 255) / 256 * 256;
  return (size_t)(o_bytes + parts * 2 * 4);
}

size_t attn_decode_gqa_workspace_size(int B, int Hq, int S_ctx, int D) {
  if (B <= 0 || Hq <= 0 || S_ctx <= 0 || D <= 0) return 0;
  const int64_t n_chunks = decode_chunks(S_ctx, S_ctx, false);
  const int64_t parts = (int64_t)B * Hq * n_chunks;
  const int64_t o_bytes = ((parts * D * 4) + 255) / 256 * 256;
  return (size_t)(o_bytes + parts * 2 * 4);
}

int attn_decode_gqa(const void *q, const void *k, const void *v, const float *attn_mask, float softmax_scale,
                    int num_kv_groups, int B, int Hq, int Hkv, int S_ctx, int D, void *out, void *workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return decode_common(q, k, v, attn_mask, nullptr, nullptr, S_ctx, false, softmax_scale, num_kv_groups, B, Hq,
                       Hkv, S_ctx, D, out, workspace, workspace_bytes, stream);
}

int attn_decode_gqa_noalloc(const void *q, const void *k, const void *v, const float *attn_mask,
                            float softmax_scale, int num_kv_groups, int B, int Hq, int Hkv, int S_ctx, int D,
                            void *out, hipStream_t stream) {
  // every argument is checked before the device is touched
  const int rc = decode_check(q, k, v, attn_mask, softmax_scale, num_kv_groups, B, Hq, Hkv, S_ctx, D, out);
  if (rc != ATTN_OK) return rc;
  const size_t need = attn_decode_gqa_workspace_size(B, Hq, S_ctx, D);
  if (need == 0 || need > kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
  void *scratch = nullptr;
  if (decode_scratch(stream, &scratch) != hipSuccess) return ATTN_ERR_HIP;
  return decode_common(q, k, v, attn_mask, nullptr, nullptr, S_ctx, false, softmax_scale, num_kv_groups, B, Hq,
                       Hkv, S_ctx, D, out, scratch, kDecodeScratchBytes, stream);
}

int attn_decode_gqa_window(const void *q, const void *k, const void *v, const float *attn_mask,
                           const int32_t *key_begin, const int32_t *key_end, int max_keys, float softmax_scale,
                           int num_kv_groups, int B, int Hq, int Hkv, int S_ctx, int D, void *out, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (max_keys <= 0) return ATTN_ERR_INVALID_ARG;
  if ((key_begin && (reinterpret_cast<uintptr_t>(key_begin) & 3u)) ||
      (key_end && (reinterpret_cast<uintptr_t>(key_end) & 3u)))
    return ATTN_ERR_INVALID_ARG;
  return decode_common(q, k, v, attn_mask, key_begin, key_end, max_keys, true, softmax_scale, num_kv_groups, B,
                       Hq, Hkv, S_ctx, D, out, workspace, workspace_bytes, stream);
}

int attn_prefill_paged(const void *q, const void *k_cache, const void *v_cache, float k_scale, float v_scale,
                       const int32_t *block_table, int max_blocks, int num_blocks, int block_size,
                       int actual_history_len, float softmax_scale, int num_kv_groups, int Hq, int Hkv, int Lq,
                       int D, void *out, float *lse, hipStream_t stream) {
  return prefill_common(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, num_blocks, block_size,
                        actual_history_len, nullptr, nullptr, softmax_scale, num_kv_groups, Hq, Hkv, Lq, D, out, lse,
                        nullptr, 0, nullptr, 0, nullptr, stream);
}

size_t attn_prefill_paged_expanded_workspace_size(int Hkv, int actual_history_len, int D) {
  if (Hkv <= 0 || actual_history_len <= 0 || D != 256) return 0;
  const int64_t tiles = (actual_history_len + prefill_key_tile() - 1) / prefill_key_tile();
  return (size_t)((int64_t)Hkv * tiles * prefill_tile_image_bytes());
}

int attn_prefill_paged_expanded(const void *q, const void *k_cache, const void *v_cache, float k_scale,
                                float v_scale, const int32_t *block_table, int max_blocks, int num_blocks,
                                int block_size, int actual_history_len, float softmax_scale, int num_kv_groups,
                                int Hq, int Hkv, int Lq, int D, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return ATTN_ERR_WORKSPACE;
  return prefill_common(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, num_blocks, block_size,
                        actual_history_len, nullptr, nullptr, softmax_scale, num_kv_groups, Hq, Hkv, Lq, D, out, lse,
                        nullptr, 0, workspace, workspace_bytes, nullptr, stream);
}

size_t attn_prefill_paged_causal_workspace_size(int Hq, int Hkv, int Lq, int D) {
  if (Hq <= 0 || Hkv <= 0 || Lq <= 0 || D <= 0 || Hq % Hkv) return 0;
  return (size_t)prefill_handoff_o_bytes(Hq, Hkv, Lq, D) + (size_t)Hq * Lq * 4;
}

size_t attn_prefill_paged_causal_expanded_workspace_size(int Hq, int Hkv, int Lq, int actual_history_len, int D) {
  const size_t hand = attn_prefill_paged_causal_workspace_size(Hq, Hkv, Lq, D);
  if (hand == 0 || actual_history_len < 0) return 0;
  const size_t img = actual_history_len > 0 ? attn_prefill_paged_expanded_workspace_size(Hkv, actual_history_len, D) : 0;
  const size_t cur = attn_prefill_paged_expanded_workspace_size(Hkv, Lq, D);  // the current tokens' images
  if ((actual_history_len > 0 && img == 0) || cur == 0) return 0;
  return (hand + 255) / 256 * 256 + img + cur;
}

int attn_prefill_paged_causal_expanded(const void *q, const void *k_cache, const void *v_cache, float k_scale,
                                       float v_scale, const int32_t *block_table, int max_blocks, int num_blocks,
                                       int block_size, int actual_history_len, const void *k_cur,
                                       const void *v_cur, float softmax_scale, int num_kv_groups, int Hq, int Hkv,
                                       int Lq, int D, void *out, float *lse, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (!k_cur || !v_cur) return ATTN_ERR_INVALID_ARG;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  const size_t need = attn_prefill_paged_causal_expanded_workspace_size(Hq, Hkv, Lq, actual_history_len, D);
  if (need == 0) {  // invalid or unsupported arguments: let the shared validation name them
    return prefill_common(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, num_blocks, block_size,
                          actual_history_len, k_cur, v_cur, softmax_scale, num_kv_groups, Hq, Hkv, Lq, D, out,
                          lse, workspace, workspace_bytes, nullptr, 0, nullptr, stream);
  }
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  // hand-off state first, then the history's tile images, then the current
  // tokens' (each a multiple of 256 bytes)
  const size_t hand = (attn_prefill_paged_causal_workspace_size(Hq, Hkv, Lq, D) + 255) / 256 * 256;
  const size_t himg =
      actual_history_len > 0 ? attn_prefill_paged_expanded_workspace_size(Hkv, actual_history_len, D) : 0;
  char *const base = static_cast<char *>(workspace);
  return prefill_common(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, num_blocks, block_size,
                        actual_history_len, k_cur, v_cur, softmax_scale, num_kv_groups, Hq, Hkv, Lq, D, out, lse,
                        workspace, hand, himg ? base + hand : nullptr, himg, base + hand + himg, stream);
}

int attn_prefill_paged_causal(const void *q, const void *k_cache, const void *v_cache, float k_scale, float v_scale,
                              const int32_t *block_table, int max_blocks, int num_blocks, int block_size,
                              int actual_history_len, const void *k_cur, const void *v_cur, float softmax_scale,
                              int num_kv_groups, int Hq, int Hkv, int Lq, int D, void *out, float *lse,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!k_cur || !v_cur) return ATTN_ERR_INVALID_ARG;
  return prefill_common(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks, num_blocks, block_size,
                        actual_history_len, k_cur, v_cur, softmax_scale, num_kv_groups, Hq, Hkv, Lq, D, out, lse,
                        workspace, workspace_bytes, nullptr, 0, nullptr, stream);
}

int res_ln(const float *residual, const void *x, attn_dtype_t x_dtype, const float *gamma, const float *beta,
           float eps, int rows, int hidden, float *residual_out, void *y, attn_dtype_t y_dtype, float *mean,
           float *rstd, hipStream_t stream) {
  if (!residual || !y) return ATTN_ERR_INVALID_ARG;
  if (rows <= 0 || hidden <= 0 || hidden % 8) return ATTN_ERR_INVALID_ARG;
  if (hidden > res_ln_max_hidden()) return ATTN_ERR_UNSUPPORTED;
  if (x && x_dtype != ATTN_BF16 && x_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (y_dtype != ATTN_BF16 && y_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (!finite(eps) || !(eps >= 0.0f)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(residual) || !aligned16(y) || (x && !aligned16(x)) || (residual_out && !aligned16(residual_out)) ||
      (gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
    return ATTN_ERR_INVALID_ARG;
  ResLnLaunch R;
  memset(&R, 0, sizeof R);
  R.res = residual;
  R.x = x;
  R.x_bf16 = x_dtype == ATTN_BF16;
  R.gamma = gamma;
  R.beta = beta;
  R.eps = eps;
  R.rows = rows;
  R.hidden = hidden;
  R.res_out = residual_out;
  R.y = y;
  R.y_bf16 = y_dtype == ATTN_BF16;
  R.mean = mean;
  R.rstd = rstd;
  return hip_status(launch_res_ln(R, stream));
}

}  // extern "C"
