// norm.hip -- the HGRN2 layer's readout normalisation and output gate for gfx950.
//
// frankenstein-transformer documentation, "HGRN2 Attention": a layer normalisation is applied to
// the recurrent readout before the silu-gated output.  Per row of `width` features
//   y = ((o - mean) / sqrt(var + eps) * weight + bias) * silu(gate),
// with the mean and the biased variance over the row (torch.nn.LayerNorm's definition).
//
// One workgroup of 256 threads per row; the row stays in registers (VPT values per thread, element
// c = tid + 256 k, so loads and stores are coalesced).  The mean and the variance (of the centred
// values, not E[x^2] - mean^2) are each reduced within the waves and then over the four waves in a
// fixed order, so results are deterministic.  The kernel is HBM-bound: o is read once, y written
// once.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

__device__ __forceinline__ float block_sum(float v, float* red, int tid) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();  // red is reused by the next sum
  return t;
}

template <typename Tg, typename Tout, int VPT>
__global__ __launch_bounds__(256) void readout_norm_kernel(ReadoutNormArgs a) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int width = (int)a.width;
  const float* x = a.o + row * a.width;
  float v[VPT];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = tid + 256 * k;
    v[k] = c < width ? x[c] : 0.0f;
    s += v[k];
  }
  const float mean = block_sum(s, red, tid) / (float)width;
  float q = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = tid + 256 * k;
    const float dv = v[k] - mean;
    q = c < width ? fmaf(dv, dv, q) : q;
  }
  const float var = block_sum(q, red, tid) / (float)width;
  const float inv = 1.0f / sqrtf(var + a.eps);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = tid + 256 * k;
    if (c < width) {
      float y = (v[k] - mean) * inv;
      if (a.weight) y *= a.weight[c];
      if (a.bias) y += a.bias[c];
      if (a.gate) y *= silu_f(io<Tg>::load(a.gate, row * a.width + c));
      io<Tout>::store(a.y, row * a.width + c, y);
    }
  }
}

template <typename Tg, typename Tout>
hipError_t launch_t(const ReadoutNormArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.rows);
  const int vpt = (int)((a.width + 255) / 256);
  if (vpt <= 1)
    hipLaunchKernelGGL((readout_norm_kernel<Tg, Tout, 1>), grid, dim3(256), 0, s, a);
  else if (vpt <= 2)
    hipLaunchKernelGGL((readout_norm_kernel<Tg, Tout, 2>), grid, dim3(256), 0, s, a);
  else if (vpt <= 4)
    hipLaunchKernelGGL((readout_norm_kernel<Tg, Tout, 4>), grid, dim3(256), 0, s, a);
  else if (vpt <= 8)
    hipLaunchKernelGGL((readout_norm_kernel<Tg, Tout, 8>), grid, dim3(256), 0, s, a);
  else if (vpt <= 16)
    hipLaunchKernelGGL((readout_norm_kernel<Tg, Tout, 16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((readout_norm_kernel<Tg, Tout, 32>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_readout_norm(const ReadoutNormArgs& a, hipStream_t s) {
  if (!a.in_bf16) return launch_t<float, float>(a, s);
  return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, s) : launch_t<bf16_t, float>(a, s);
}

}  // namespace ssd
