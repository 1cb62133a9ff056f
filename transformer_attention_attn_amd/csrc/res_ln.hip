// (Residual +) LayerNorm over the last dimension, fp32 statistics.
//
// gte-encoder-neuron-kernels, "Repository layout": a (residual +) LayerNorm
// kernel; vit-encoder-neuron-kernels, "Supported shapes and limits": standard
// LayerNorm (not RMSNorm) on an fp32 residual stream.
//
// One wave per row; the row stays in registers (VPL float4 per lane) between
// the mean pass and the variance pass, so HBM sees one read of the residual
// (and x) and one write of each output.  Statistics: mean = sum/N, biased
// variance = sum((x-mean)^2)/N, rstd = 1/sqrt(var + eps), all fp32 with wave
// tree reductions.
#include "device_common.h"
#include "launch.h"

namespace mi355 {

template <int VPL>
__global__ __launch_bounds__(256) void res_ln_kernel(ResLnLaunch a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int N = a.hidden;
  const int64_t base = (int64_t)row * N;

  f32x4_t x[VPL];
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c < N) {
      f32x4_t r = ldg<f32x4_t>(a.res + base + c);
      if (a.x) {
        if (a.x_bf16) {
          const u32x2_t w = ldg<u32x2_t>(reinterpret_cast<const __bf16 *>(a.x) + base + c);
          r += f32x4_t{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
        } else {
          r += ldg<f32x4_t>(reinterpret_cast<const float *>(a.x) + base + c);
        }
      }
      x[j] = r;
      s += (r[0] + r[1]) + (r[2] + r[3]);
    } else {
      x[j] = f32x4_t{0, 0, 0, 0};
    }
  }
  const float mean = wave_sum(s) / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c < N) {
      const f32x4_t d = x[j] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float var = wave_sum(q) / (float)N;
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
    f32x4_t y = (x[j] - mean) * rstd;
    if (a.gamma) y *= ldg<f32x4_t>(a.gamma + c);
    if (a.beta) y += ldg<f32x4_t>(a.beta + c);
    if (a.y_bf16)
      *reinterpret_cast<u32x2_t *>(reinterpret_cast<__bf16 *>(a.y) + base + c) =
          u32x2_t{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
    else
      *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(a.y) + base + c) = y;
  }
}

hipError_t launch_res_ln(const ResLnLaunch &a, hipStream_t stream) {
  const dim3 grid((a.rows + 3) / 4), block(256);
  const int need = (a.hidden + 255) / 256;
  if (need <= 1)
    hipLaunchKernelGGL(res_ln_kernel<1>, grid, block, 0, stream, a);
  else if (need <= 2)
    hipLaunchKernelGGL(res_ln_kernel<2>, grid, block, 0, stream, a);
  else if (need <= 4)
    hipLaunchKernelGGL(res_ln_kernel<4>, grid, block, 0, stream, a);
  else if (need <= 8)
    hipLaunchKernelGGL(res_ln_kernel<8>, grid, block, 0, stream, a);
  else if (need <= 16)
    hipLaunchKernelGGL(res_ln_kernel<16>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(res_ln_kernel<32>, grid, block, 0, stream, a);
  return hipGetLastError();
}

int res_ln_max_hidden() { return 32 * 256; }

}  // namespace mi355
