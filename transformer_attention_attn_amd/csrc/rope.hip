// Rotary position embedding of the encoder's keys, one pass over K.
//
// vit-encoder-neuron-kernels, "Kernels": pair k of token s turns by the angle
// whose cosine and sine the tables hold at [s, k]; pairing 1 ("half") pairs
// lane k with lane k + D/2, pairing 2 ("interleaved") lane 2k with 2k + 1.
// For a pair (a, b): a' = a cos - b sin, b' = b cos + a sin, in fp32.
//
// The attention kernel rotates its Q rows as it loads them, but every
// workgroup of a (batch, head) streams all of that head's keys: rotating K
// there would repeat the same rotation once per query tile, on the VALU the
// key loop is bound by.  Rotating K once here costs one read and one write of
// K over HBM.  The output keeps the input dtype (fp32 stays fp32 until the
// attention kernel rounds it to bf16, as it does for unrotated inputs).
//
// One thread per (key, group of 8 pairs): the half pairing reads 8 lanes at
// d = 8j and their partners at d = D/2 + 8j, the interleaved pairing the 16
// lanes at d = 16j; both read the tables at pairs 8j .. 8j+7.
#include "device_common.h"
#include "launch.h"

namespace mi355 {

constexpr int kRopeThreads = 256;

template <bool F32>
__device__ __forceinline__ void load_lanes8(const char *p, float (&f)[8]) {
  if constexpr (F32) {
    const f32x4_t x0 = ldg<f32x4_t>(p), x1 = ldg<f32x4_t>(p + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = x0[i];
      f[4 + i] = x1[i];
    }
  } else {
    const u32x4_t x = ldg<u32x4_t>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(x[i]);
      f[2 * i + 1] = bf16_hi(x[i]);
    }
  }
}

template <bool F32>
__device__ __forceinline__ void store_lanes8(char *p, const float (&f)[8]) {
  if constexpr (F32) {
    *reinterpret_cast<f32x4_t *>(p) = f32x4_t{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4_t *>(p + 16) = f32x4_t{f[4], f[5], f[6], f[7]};
  } else {
    *reinterpret_cast<u32x4_t *>(p) =
        u32x4_t{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
  }
}

__device__ __forceinline__ void turn(float &a, float &b, float c, float s) {
  const float a2 = __builtin_fmaf(-b, s, a * c);
  b = __builtin_fmaf(a, s, b * c);
  a = a2;
}

template <bool F32, int ROPE>
__global__ __launch_bounds__(kRopeThreads) void rope_k_kernel(RopeLaunch a) {
  constexpr int ES = F32 ? 4 : 2;
  const int groups = a.D / 16;  // groups of 8 pairs per key
  const int64_t item = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int64_t n_items = (int64_t)a.B * a.H * a.S * groups;
  if (item >= n_items) return;
  const int j = (int)(item % groups);
  const int64_t key = item / groups;  // (b, h, s) flattened
  const int s = (int)(key % a.S);
  const int64_t bh = key / a.S;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const char *src = reinterpret_cast<const char *>(a.k) + (b * a.ks[0] + h * a.ks[1] + s * a.ks[2]) * ES;
  char *dst = reinterpret_cast<char *>(a.out) + key * a.D * ES;
  const float *ct = a.cos + b * a.sb + (int64_t)s * (a.D / 2) + 8 * j;
  const float *st = a.sin + b * a.sb + (int64_t)s * (a.D / 2) + 8 * j;
  const f32x4_t c0 = ldg<f32x4_t>(ct), c1 = ldg<f32x4_t>(ct + 4);
  const f32x4_t s0 = ldg<f32x4_t>(st), s1 = ldg<f32x4_t>(st + 4);
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  float x[8], y[8];
  if constexpr (ROPE == 1) {
    // x: lanes 8j .. 8j+7 (the a of pairs 8j ..), y: their partners D/2 + 8j ..
    load_lanes8<F32>(src + 8 * j * ES, x);
    load_lanes8<F32>(src + (a.D / 2 + 8 * j) * ES, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) turn(x[e], y[e], c[e], sn[e]);
    store_lanes8<F32>(dst + 8 * j * ES, x);
    store_lanes8<F32>(dst + (a.D / 2 + 8 * j) * ES, y);
  } else {
    // lanes 16j .. 16j+15: pairs (16j + 2e, 16j + 2e + 1), e < 8
    load_lanes8<F32>(src + 16 * j * ES, x);
    load_lanes8<F32>(src + (16 * j + 8) * ES, y);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      turn(x[2 * e], x[2 * e + 1], c[e], sn[e]);
      turn(y[2 * e], y[2 * e + 1], c[4 + e], sn[4 + e]);
    }
    store_lanes8<F32>(dst + 16 * j * ES, x);
    store_lanes8<F32>(dst + (16 * j + 8) * ES, y);
  }
}

hipError_t launch_rope_k(const RopeLaunch &a, hipStream_t stream) {
  const int64_t n_items = (int64_t)a.B * a.H * a.S * (a.D / 16);
  const int64_t blocks = (n_items + kRopeThreads - 1) / kRopeThreads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kRopeThreads);
  if (a.f32 && a.rope == 1) hipLaunchKernelGGL((rope_k_kernel<true, 1>), grid, block, 0, stream, a);
  else if (a.f32) hipLaunchKernelGGL((rope_k_kernel<true, 2>), grid, block, 0, stream, a);
  else if (a.rope == 1) hipLaunchKernelGGL((rope_k_kernel<false, 1>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((rope_k_kernel<false, 2>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mi355
