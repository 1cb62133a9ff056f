// (Residual +) LayerNorm over the last dimension, fp32 statistics.
//
// gte-encoder-neuron-kernels, "Repository layout": a (residual +) LayerNorm
// kernel; vit-encoder-neuron-kernels, "Supported shapes and limits": standard
// LayerNorm (not RMSNorm) on an fp32 residual stream.
//
// One wave per row; the row stays in registers (VPL float4 per lane) between
// the mean pass and the variance pass, so HBM sees one read of the residual
// (and x) and one write of each output.  Statistics: mean = sum/N, biased
// variance = sum((x-mean)^2)/N, rstd = 1/sqrt(var + eps), all fp32.
//
// Latency, not bandwidth, sets the time of a pass this short, so:
//   * every load of the row (residual, x, gamma, beta) is issued before the
//     first wait: raw buffer loads over the row's byte range, so chunks past
//     the row read as zeros without a branch, and x's presence and dtype are
//     template parameters (a runtime branch around each load made the
//     compiler wait for every load before issuing the next);
//   * the two row reductions use lane exchanges on the VALU (DPP mirrors and
//     quad permutes within 16 lanes, then the 16- and 32-lane swaps), which
//     leave the same sum, bit for bit, in every lane.
#include "device_common.h"
#include "launch.h"

namespace mi355 {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ln_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p), hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                   false));
}

// Sum over the wave; every lane receives the same bits.
__device__ __forceinline__ float ln_wave_sum(float x) {
  x = dpp_add<0x140>(x);  // row_mirror: lane i + lane 15-i of its 16-lane row
  x = dpp_add<0x141>(x);  // row_half_mirror: lane i + lane 7-i of its 8-lane half
  x = dpp_add<0x4e>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x = dpp_add<0xb1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  const auto r16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
  // (__uint_as_float on each element: hipcc folds a bit_cast of an
  // ext-vector element to element 0)
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);  // lane ^ 16
  const auto r32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);  // lane ^ 32
}

// XK: 0 = no x, 1 = bf16 x, 2 = fp32 x.
template <int VPL, int XK>
__global__ __launch_bounds__(256) void res_ln_kernel(ResLnLaunch a) {
  const int lane = threadIdx.x & 63;
  const int row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (row >= a.rows) return;
  const int N = a.hidden;  // a multiple of 8: every float4 chunk is wholly inside or past the row
  const int64_t base = (int64_t)row * N;
  constexpr bool PRE = VPL <= 8;  // gamma/beta loaded with the row (registers permitting)

  const auto rr = ln_rsrc(a.res + base, (uint32_t)N * 4);
  const auto rx = ln_rsrc(XK == 0 ? nullptr : static_cast<const char *>(a.x) + base * (XK == 1 ? 2 : 4),
                          XK == 0 ? 0u : (uint32_t)N * (XK == 1 ? 2 : 4));
  const auto rg = ln_rsrc(a.gamma, a.gamma ? (uint32_t)N * 4 : 0u);
  const auto rb = ln_rsrc(a.beta, a.beta ? (uint32_t)N * 4 : 0u);
  // x is held apart from the residual until both have arrived, except for
  // the widest rows (registers)
  constexpr bool XSEP = VPL <= 16;
  f32x4_t x[VPL], g[PRE ? VPL : 1], bt[PRE ? VPL : 1];
  u32x2_t xb[XK == 1 && XSEP ? VPL : 1];
  f32x4_t xf[XK == 2 && XSEP ? VPL : 1];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t c = (uint32_t)(j * 64 + lane) * 4;  // first column of the lane's chunk j
    x[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rr, c * 4, 0, 0));
    if constexpr (XK == 1) {
      const u32x2_t w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rx, c * 2, 0, 0));
      if constexpr (XSEP) xb[j] = w;
      else x[j] += f32x4_t{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
    }
    if constexpr (XK == 2) {
      const f32x4_t w = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, c * 4, 0, 0));
      if constexpr (XSEP) xf[j] = w;
      else x[j] += w;
    }
    if constexpr (PRE) {
      g[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rg, c * 4, 0, 0));
      bt[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, c * 4, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load above the first wait
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    if constexpr (XK == 1 && XSEP)
      x[j] += f32x4_t{bf16_lo(xb[j][0]), bf16_hi(xb[j][0]), bf16_lo(xb[j][1]), bf16_hi(xb[j][1])};
    if constexpr (XK == 2 && XSEP) x[j] += xf[j];
    s += (x[j][0] + x[j][1]) + (x[j][2] + x[j][3]);  // chunks past the row are zeros
  }
  const float mean = ln_wave_sum(s) / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const f32x4_t d = x[j] - mean;
    const float qj = (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    q += (j * 64 + lane) * 4 < N ? qj : 0.0f;
  }
  const float var = ln_wave_sum(q) / (float)N;
  const float rstd = 1.0f / __builtin_sqrtf(var + a.eps);
  if (lane == 0) {
    if (a.mean) a.mean[row] = mean;
    if (a.rstd) a.rstd[row] = rstd;
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c >= N) continue;
    if (a.res_out) *reinterpret_cast<f32x4_t *>(a.res_out + base + c) = x[j];
    f32x4_t gj, bj;  // absent gamma/beta read as zeros through their empty ranges
    if constexpr (PRE) {
      gj = g[j];
      bj = bt[j];
    } else {
      gj = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)c * 4, 0, 0));
      bj = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)c * 4, 0, 0));
    }
    if (!a.gamma) gj = f32x4_t{1, 1, 1, 1};
    f32x4_t y = (x[j] - mean) * rstd * gj + bj;
    if (a.y_bf16)
      *reinterpret_cast<u32x2_t *>(reinterpret_cast<__bf16 *>(a.y) + base + c) =
          u32x2_t{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
    else
      *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(a.y) + base + c) = y;
  }
}

template <int VPL>
static void launch_vpl(const ResLnLaunch &a, dim3 grid, hipStream_t stream) {
  if (!a.x)
    hipLaunchKernelGGL((res_ln_kernel<VPL, 0>), grid, dim3(256), 0, stream, a);
  else if (a.x_bf16)
    hipLaunchKernelGGL((res_ln_kernel<VPL, 1>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((res_ln_kernel<VPL, 2>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_res_ln(const ResLnLaunch &a, hipStream_t stream) {
  const dim3 grid((a.rows + 3) / 4);
  const int need = (a.hidden + 255) / 256;
  if (need <= 1)
    launch_vpl<1>(a, grid, stream);
  else if (need <= 2)
    launch_vpl<2>(a, grid, stream);
  else if (need <= 4)
    launch_vpl<4>(a, grid, stream);
  else if (need <= 8)
    launch_vpl<8>(a, grid, stream);
  else if (need <= 16)
    launch_vpl<16>(a, grid, stream);
  else
    launch_vpl<32>(a, grid, stream);
  return hipGetLastError();
}

int res_ln_max_hidden() { return 32 * 256; }

}  // namespace mi355
