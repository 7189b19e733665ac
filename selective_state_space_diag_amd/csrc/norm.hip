// norm.hip -- the HGRN2 layer's readout normalisation and output gate for gfx950.
//
// frankenstein-transformer documentation, "HGRN2 Attention": a layer normalisation is applied to
// the recurrent readout before the silu-gated output.  Per row of `width` features
//   y = ((o - mean) / sqrt(var + eps) * weight + bias) * silu(gate),
// with the mean and the biased variance over the row (torch.nn.LayerNorm's definition).
//
// Widths that are a multiple of 4 (the layer's H d): one wave per row, the row in registers as
// 16-byte chunks, all sums inside the wave.  Other widths: one workgroup of 256 threads per row;
// the row stays in registers (VPT values per thread, element c = tid + 256 k, so loads and stores
// are coalesced).  The mean and the variance (of the centred
// values, not E[x^2] - mean^2) are each reduced within the waves and then over the four waves in a
// fixed order, so results are deterministic.  The kernel is HBM-bound: o is read once, y written
// once.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Rows whose width is a multiple of 4: one wave per row, 16-byte chunks c = 4 lane + 256 k
// (k < NC), reductions inside the wave only (no barriers).  Every access goes through a window over
// the row, so chunks past the row read as 0 and are not stored; they are masked out of the
// variance.
template <typename Tg, typename Tout, int NC>
__global__ __launch_bounds__(256) void readout_norm_wave_kernel(ReadoutNormArgs a) {
  const int lane = threadIdx.x & 63;
  // the wave's row, in scalar registers: the windows over it stay wave-uniform
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.rows) return;  // whole wave
  const uint32_t width = (uint32_t)a.width;
  const auto wo = make_window(a.o + row * a.width, width * 4);
  const auto wg = make_window(a.gate ? static_cast<const char*>(a.gate) + row * a.width * sizeof(Tg) : nullptr,
                              a.gate ? width * (uint32_t)sizeof(Tg) : 0u);
  const auto ww = make_window(a.weight, a.weight ? width * 4 : 0u);
  const auto wb = make_window(a.bias, a.bias ? width * 4 : 0u);
  const auto wy = make_window(static_cast<char*>(a.y) + row * a.width * sizeof(Tout), width * (uint32_t)sizeof(Tout));
  float x[NC][4];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const uint32_t c = 4u * lane + 256u * k;
    const v4i_t d = __builtin_amdgcn_raw_buffer_load_b128(wo, (int)(c * 4), 0, 0);
    x[k][0] = __int_as_float(d.x); x[k][1] = __int_as_float(d.y);
    x[k][2] = __int_as_float(d.z); x[k][3] = __int_as_float(d.w);
    s += (x[k][0] + x[k][1]) + (x[k][2] + x[k][3]);
  }
  const float mean = wave_sum(s) / (float)width;
  float q = 0.0f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const bool in = 4u * lane + 256u * k < width;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dv = x[k][e] - mean;
      q = in ? fmaf(dv, dv, q) : q;
    }
  }
  const float inv = 1.0f / sqrtf(wave_sum(q) / (float)width + a.eps);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const uint32_t c = 4u * lane + 256u * k;
    float w[4] = {1.0f, 1.0f, 1.0f, 1.0f}, b[4] = {0.0f, 0.0f, 0.0f, 0.0f}, g[4];
    if (a.weight) {
      const v4i_t d = __builtin_amdgcn_raw_buffer_load_b128(ww, (int)(c * 4), 0, 0);
      w[0] = __int_as_float(d.x); w[1] = __int_as_float(d.y); w[2] = __int_as_float(d.z); w[3] = __int_as_float(d.w);
    }
    if (a.bias) {
      const v4i_t d = __builtin_amdgcn_raw_buffer_load_b128(wb, (int)(c * 4), 0, 0);
      b[0] = __int_as_float(d.x); b[1] = __int_as_float(d.y); b[2] = __int_as_float(d.z); b[3] = __int_as_float(d.w);
    }
    if (a.gate) {
      if constexpr (sizeof(Tg) == 2) {
        const u32x2_t d = __builtin_amdgcn_raw_buffer_load_b64(wg, (int)(c * 2), 0, 0);
        g[0] = bf16_lo(d.x); g[1] = bf16_hi(d.x); g[2] = bf16_lo(d.y); g[3] = bf16_hi(d.y);
      } else {
        const v4i_t d = __builtin_amdgcn_raw_buffer_load_b128(wg, (int)(c * 4), 0, 0);
        g[0] = __int_as_float(d.x); g[1] = __int_as_float(d.y); g[2] = __int_as_float(d.z); g[3] = __int_as_float(d.w);
      }
    }
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = fmaf((x[k][e] - mean) * inv, w[e], b[e]);
      if (a.gate) y[e] *= silu_f(g[e]);
    }
    if constexpr (sizeof(Tout) == 4) {
      const v4i_t d = {(int)__float_as_uint(y[0]), (int)__float_as_uint(y[1]), (int)__float_as_uint(y[2]),
                       (int)__float_as_uint(y[3])};
      __builtin_amdgcn_raw_buffer_store_b128(d, wy, (int)(c * 4), 0, 0);
    } else {
      u32x2_t d;
      d.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
      d.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
      __builtin_amdgcn_raw_buffer_store_b64(d, wy, (int)(c * 2), 0, 0);
    }
  }
}

template <typename Tg, typename Tout>
hipError_t launch_t(const ReadoutNormArgs& a, hipStream_t s) {
  if (a.width % 4 == 0) {
    const dim3 grid((unsigned)((a.rows + 3) / 4));
    const int nc = (int)((a.width + 255) / 256);
    if (nc <= 1)
      hipLaunchKernelGGL((readout_norm_wave_kernel<Tg, Tout, 1>), grid, dim3(256), 0, s, a);
    else if (nc <= 2)
      hipLaunchKernelGGL((readout_norm_wave_kernel<Tg, Tout, 2>), grid, dim3(256), 0, s, a);
    else if (nc <= 4)
      hipLaunchKernelGGL((readout_norm_wave_kernel<Tg, Tout, 4>), grid, dim3(256), 0, s, a);
    else if (nc <= 8)
      hipLaunchKernelGGL((readout_norm_wave_kernel<Tg, Tout, 8>), grid, dim3(256), 0, s, a);
    else if (nc <= 16)
      hipLaunchKernelGGL((readout_norm_wave_kernel<Tg, Tout, 16>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((readout_norm_wave_kernel<Tg, Tout, 32>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
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
