// Kernel launch records passed by value from the C-ABI layer to the kernels.
// Host-validated; the kernels trust these fields.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

struct EncoderLaunch {
  const void *q, *k, *v;
  int64_t qs[4], ks[4], vs[4];  // element strides {b,h,s,d}, d stride 1
  const float *mask;            // nullable, natural-log additive [B, S_kv] rows
  int64_t mask_sb;
  int B, H, Sq, Skv;
  float c;                      // |softmax_scale| * log2(e), > 0
  int q_neg;                    // 1: the scale was negative, q is negated on load
  void *out;                    // nullable
  int64_t os[4];
  int out_f32;
  float *lse;                   // nullable [B,H,Sq]
  const float *res;             // nullable [B,Sq,H*D]
  float *res_out;               // nullable (non-null iff res non-null)
  const float *rope_cos, *rope_sin;  // RoPE tables [rows, D/2] fp32 (rope != 0; q rows only, K comes rotated)
  int64_t rope_sb;              // table batch stride in floats (0: shared)
  int rope;                     // 0 none, 1 rotate-half pairing, 2 interleaved pairing
  const int *key_len;           // nullable [B]: batch row b attends keys 0 .. key_len[b]-1 (clamped)
};

// K rotation pass of the encoder's RoPE: k [B,H,S,D] strided -> out [B,H,S,D]
// contiguous, same dtype.
struct RopeLaunch {
  const void *k;
  int64_t ks[4];                 // element strides {b,h,s,d}, d stride 1
  void *out;
  int B, H, S, D, f32, rope;     // rope: 1 rotate-half, 2 interleaved
  const float *cos, *sin;        // [rows, D/2] per batch entry (+ b * sb)
  int64_t sb;
};

struct PrefillLaunch {
  const __bf16 *q;
  const uint8_t *kc, *vc;
  const int32_t *bt;
  int bs, L_act, Hkv, G, Lq;
  float c;        // |softmax_scale| * k_scale * log2(e), > 0
  int q_neg;      // 1: the scale was negative, q is negated on load
  float v_scale;
  const __bf16 *kcur, *vcur;  // nullable: current tokens' K/V [Hkv, Lq, D] (causal part)
  float c_cur;                // |softmax_scale| * log2(e), > 0
  float *ws_o, *ws_ml;        // history -> current-token handoff (causal part with a history)
  char *img;                  // nullable: bf16 tile images of the history [Hkv, n_tiles, image] (workspace)
  int n_tiles;                // tiles of prefill_key_tile() keys per KV head in img
  char *img_cur;              // nullable: tile images of the current tokens' K/V [Hkv, n_tiles_cur, image]
  int n_tiles_cur;
  __bf16 *out;
  float *lse;     // nullable
};

struct DecodeLaunch {
  const __bf16 *q, *k, *v;
  const float *mask;  // nullable [B, S_ctx]
  const int32_t *key_begin, *key_end;  // nullable [B]: per-sequence key range
  int max_keys;       // keys per sequence the grid covers (S_ctx without a range)
  int B, Hq, Hkv, G, S_ctx, D, n_chunks;
  float c;            // softmax_scale * log2(e)
  float *ws_o;        // [B*Hq*n_chunks, D]
  float *ws_ml;       // [B*Hq*n_chunks, 2]
  __bf16 *out;
};

struct ResLnLaunch {
  const float *res;
  const void *x;      // nullable
  int x_bf16;
  const float *gamma, *beta;
  float eps;
  int rows, hidden;
  float *res_out;     // nullable
  void *y;
  int y_bf16;
  float *mean, *rstd; // nullable
};

hipError_t launch_encoder(const EncoderLaunch &a, bool f32_in, hipStream_t stream);
int encoder_rows_per_block();
hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream);
int prefill_key_tile();
int prefill_rows_per_block();
int64_t prefill_tile_image_bytes();  // bytes of one tile's K and V images
hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream);
// Bytes of the decode's file-scope device scratch, and its address on the
// device of `stream` (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(hipStream_t stream, void **ptr);
int decode_chunk_keys();
int decode_max_groups();
hipError_t launch_res_ln(const ResLnLaunch &a, hipStream_t stream);
hipError_t launch_rope_k(const RopeLaunch &a, hipStream_t stream);
int res_ln_max_hidden();

}  // namespace mi355
