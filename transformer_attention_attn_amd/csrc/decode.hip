// GQA single-token decode, head_dim 256, split-K ("flash-decode") + combine.
//
// head_dim>128 (256/512) GQA Flash-Decode NKI Kernel for AWS Trainium,
// "Input contract" fixes the operands (q [B,Hq,1,D], k/v [B,Hkv,S_ctx,D],
// additive 0/-inf mask [B,1,1,S_ctx], softmax_scale, num_kv_groups); its
// "Perf caveat" and "Future performance follow-on" note that one program
// re-streaming the whole cache is bandwidth-starved and that the KV stream
// should be sharded over many programs.  Here every (batch, KV head, chunk of
// 128 keys) is its own workgroup, the G query heads of a KV head share the
// one pass over its K/V, and a second kernel merges the chunk partials.
//
// Split kernel, per workgroup (4 waves, 32 keys each as 2 rounds of 16):
//   QK^T : v_mfma_f32_16x16x32_bf16 with the 16 keys on M and the G query
//          heads on N (padded to 16), K streamed straight from HBM into the
//          A operand (64 contiguous bytes per key per load);
//   mask : additive, in log2 units; a round whose 16 mask entries are all
//          -inf issues no K/V loads, a chunk with no live key exits at once;
//   PV   : on the VALU, each lane owning 4 of the 256 output columns, V read
//          with 512 contiguous bytes per key per wave;
//   merge: the 4 wave partials combine through LDS; the chunk partial
//          (m, l in log2 units, unnormalised o) goes to the workspace.
// Combine kernel, per (b, query head): M = max m_c, L = sum 2^(m_c-M) l_c,
//   o = sum 2^(m_c-M) o_c / L over the chunks in index order (deterministic).
#include "device_common.h"
#include "launch.h"

namespace mi355 {

constexpr int kDecD = 256;
constexpr int kDecChunk = 128;  // keys per workgroup
constexpr int kDecGmax = 8;     // query heads per KV head supported

template <int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeLaunch a) {
  constexpr int KW = kDecChunk / 4;  // keys per wave (two MFMA groups of 16)
  __shared__ __attribute__((aligned(16))) float sc[4][G][KW];
  __shared__ __attribute__((aligned(16))) float red_o[4][G][kDecD];
  __shared__ float red_ml[4][G][2];

  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *mrow = a.mask ? a.mask + (int64_t)b * a.S_ctx : nullptr;
  const int64_t part0 = ((int64_t)b * a.Hq + (int64_t)kvh * G) * a.n_chunks + chunk;  // head g adds g*n_chunks
  const int key0 = chunk * kDecChunk + wave * KW;

  // Liveness of this wave's 32 keys (one mask read per lane, then a vote).
  bool kl = false;
  if (lane < KW) {
    const int key = key0 + lane;
    kl = key < a.S_ctx && (mrow == nullptr || mrow[key] != -INFINITY);
  }
  const uint64_t live = __ballot(kl);

  float m[G], l[G];
  f32x4_t o[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    o[g] = f32x4_t{0, 0, 0, 0};
  }

  if (live != 0) {
    const int gq = lane & 15, quad = lane >> 4;
    const int64_t kv_off = ((int64_t)b * a.Hkv + kvh) * a.S_ctx * kDecD;
    const __bf16 *kbase = a.k + kv_off;
    const __bf16 *vbase = a.v + kv_off;
    // All K/V loads of the wave go out together; dead keys are not loaded.
    u32x4_t kf[2][kDecD / 32];
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const bool kin = (live >> (grp * 16 + gq)) & 1;
#pragma unroll
      for (int s = 0; s < kDecD / 32; ++s)
        kf[grp][s] = kin ? ldg<u32x4_t>(kbase + (int64_t)(key0 + grp * 16 + gq) * kDecD + 32 * s + 8 * quad)
                         : u32x4_t{0, 0, 0, 0};
    }
    u32x2_t vf[KW];
#pragma unroll
    for (int j = 0; j < KW; ++j)
      vf[j] = ((live >> j) & 1) ? ldg<u32x2_t>(vbase + (int64_t)(key0 + j) * kDecD + 4 * lane) : u32x2_t{0, 0};
    // q^T as the B operand: lane l holds q[g = l%16][32s + 8(l/16) .. +7], zero for g >= G.
    u32x4_t qf[kDecD / 32];
    const __bf16 *qrow = a.q + ((int64_t)b * a.Hq + (int64_t)kvh * G + gq) * kDecD;
#pragma unroll
    for (int s = 0; s < kDecD / 32; ++s)
      qf[s] = gq < G ? ldg<u32x4_t>(qrow + 32 * s + 8 * quad) : u32x4_t{0, 0, 0, 0};

#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      f32x4_t s4 = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < kDecD / 32; ++s) s4 = mfma16(as_bf16x8(kf[grp][s]), as_bf16x8(qf[s]), s4);
      // lane l holds S^T[key = grp*16 + 4*(l/16) + i][head g = l%16]
      if (gq < G) {
        f32x4_t x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kj = grp * 16 + 4 * quad + i;
          const float mk = ((live >> kj) & 1) ? (mrow ? mrow[key0 + kj] : 0.0f) : -INFINITY;
          x[i] = mk == -INFINITY ? -INFINITY : s4[i] * a.c + mk * kLog2e;
        }
        *reinterpret_cast<f32x4_t *>(&sc[wave][gq][grp * 16 + 4 * quad]) = x;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();

    // Softmax over the wave's 32 keys for each head, then PV on the VALU.
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float p[KW];
#pragma unroll
      for (int q4 = 0; q4 < KW / 4; ++q4) {
        const f32x4_t t = *reinterpret_cast<const f32x4_t *>(&sc[wave][g][4 * q4]);
        p[4 * q4 + 0] = t[0];
        p[4 * q4 + 1] = t[1];
        p[4 * q4 + 2] = t[2];
        p[4 * q4 + 3] = t[3];
      }
      float mr = p[0];
#pragma unroll
      for (int j = 1; j < KW; ++j) mr = fmaxf(mr, p[j]);
      m[g] = mr;
      const float m_use = mr == -INFINITY ? 0.0f : mr;
      float ls = 0.0f;
      f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const float pj = fast_exp2(p[j] - m_use);
        ls += pj;
        acc[0] += pj * bf16_lo(vf[j][0]);
        acc[1] += pj * bf16_hi(vf[j][0]);
        acc[2] += pj * bf16_lo(vf[j][1]);
        acc[3] += pj * bf16_hi(vf[j][1]);
      }
      l[g] = ls;
      o[g] = acc;
    }
  }

  // Merge the 4 waves' partials (fixed order) and write the chunk partial.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    *reinterpret_cast<f32x4_t *>(&red_o[wave][g][4 * lane]) = o[g];
    if (lane == 0) {
      red_ml[wave][g][0] = m[g];
      red_ml[wave][g][1] = l[g];
    }
  }
  __syncthreads();
  // thread tid handles column tid of every head
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[w][g][0]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sw = fast_exp2(red_ml[w][g][0] - Mu);
      L += red_ml[w][g][1] * sw;
      acc += red_o[w][g][tid] * sw;
    }
    const int64_t part = part0 + (int64_t)g * a.n_chunks;
    if (M != -INFINITY) a.ws_o[part * kDecD + tid] = acc;
    if (tid == 0) {
      a.ws_ml[part * 2 + 0] = M;
      a.ws_ml[part * 2 + 1] = L;
    }
  }
}

// One workgroup per (batch, query head); thread d owns output column d.  The
// chunk statistics are loaded first (independent loads), then every live
// chunk's partial column, weighted by 2^(m_c - M); dead chunks (m_c = -inf,
// whose partial was never written) are selected away, not branched around.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeLaunch a) {
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int64_t p0 = ((int64_t)b * a.Hq + hq) * a.n_chunks;
  float M = -INFINITY;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, a.ws_ml[(p0 + c) * 2]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float L = 0.0f, acc = 0.0f;
#pragma unroll 8
  for (int c = 0; c < a.n_chunks; ++c) {
    const float mc = a.ws_ml[(p0 + c) * 2];
    const float lc = a.ws_ml[(p0 + c) * 2 + 1];
    const float oc = a.ws_o[(p0 + c) * kDecD + d];
    const bool dead = mc == -INFINITY;
    const float w = dead ? 0.0f : fast_exp2(mc - Mu);
    L += dead ? 0.0f : lc * w;
    acc += dead ? 0.0f : oc * w;
  }
  const float r = L > 0.0f ? acc / L : 0.0f;
  a.out[((int64_t)b * a.Hq + hq) * kDecD + d] = (__bf16)r;
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream) {
  const dim3 grid(a.n_chunks, a.Hkv, a.B), block(256);
  switch (a.G) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(kDecD), 0, stream, a);
  return hipGetLastError();
}

int decode_chunk_keys() { return kDecChunk; }
int decode_max_groups() { return kDecGmax; }

}  // namespace mi355
