// hgrn2.hip -- HGRN2 matrix-state scan and decode update for gfx950.
//
// Recurrence (frankenstein-transformer documentation, "HGRN2 Attention", state update):
//   g_i = lb + (1 - lb) sigmoid(g_logit_i),  S[i][j] = g_i S[i][j] + v_i k_j,  o_i = sum_j S[i][j] q_j.
// The gate scales row i of S (the value index); rows evolve independently of each other.
//
// Recurrent scan: one workgroup per (batch, head), one lane per value row i holding S[i][:] in
// registers; k_t and q_t of each step are staged in LDS (double-buffered) and read as broadcasts.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

struct H2Params {
  int64_t B, L, H, d;
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  float lb;
  const float* S0;
  void* o;
  float* S_last;
};

template <typename Tin, typename Tout, int DH>
__global__ __launch_bounds__(DH < 64 ? 64 : DH) void hgrn2_recurrent_kernel(H2Params p) {
  __shared__ float sk[2][DH];
  __shared__ float sq[2][DH];
  const int i = threadIdx.x;
  const bool row_ok = i < DH;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.H;
  const int64_t hh = bh - b * p.H;
  float S[DH];
  const int64_t sbase = (bh * DH + (row_ok ? i : 0)) * DH;
#pragma unroll
  for (int j = 0; j < DH; ++j) S[j] = (p.S0 && row_ok) ? p.S0[sbase + j] : 0.0f;
  const float one_m_lb = 1.0f - p.lb;
  for (int64_t t = 0; t < p.L; ++t) {
    const int buf = (int)(t & 1);
    const int64_t base = ((b * p.L + t) * p.H + hh) * DH;
    float vi = 0.0f, gl = 0.0f;
    if (row_ok) {
      sk[buf][i] = io<Tin>::load(p.k, base + i);
      sq[buf][i] = io<Tin>::load(p.q, base + i);
      vi = io<Tin>::load(p.v, base + i);
      gl = io<Tin>::load(p.g, base + i);
    }
    __syncthreads();
    const float g = fmaf(one_m_lb, sigmoid_f(gl), p.lb);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < DH; ++j) {
      S[j] = fmaf(g, S[j], vi * sk[buf][j]);
      acc = fmaf(S[j], sq[buf][j], acc);
    }
    if (row_ok) io<Tout>::store(p.o, base + i, acc);
  }
  if (p.S_last && row_ok) {
#pragma unroll
    for (int j = 0; j < DH; ++j) p.S_last[sbase + j] = S[j];
  }
}

// Decode step: one wave per value row; o_i reduced across the wave.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void hgrn2_update_kernel(int64_t rows, int64_t d, const void* q, const void* k,
                                                           const void* v, const void* g, float lb, float* S,
                                                           void* o) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int64_t bh = r / d;
  const int64_t i = r - bh * d;
  const float gi = fmaf(1.0f - lb, sigmoid_f(io<Tin>::load(g, bh * d + i)), lb);
  const float vi = io<Tin>::load(v, bh * d + i);
  float acc = 0.0f;
  for (int64_t j = lane; j < d; j += 64) {
    const int64_t e = r * d + j;
    const float s = fmaf(gi, S[e], vi * io<Tin>::load(k, bh * d + j));
    S[e] = s;
    acc = fmaf(s, io<Tin>::load(q, bh * d + j), acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) io<Tout>::store(o, bh * d + i, acc);
}

template <typename Tin, typename Tout>
hipError_t launch_recurrent_t(const H2Params& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.H));
  switch (p.d) {
    case 16: hipLaunchKernelGGL((hgrn2_recurrent_kernel<Tin, Tout, 16>), grid, dim3(64), 0, s, p); break;
    case 32: hipLaunchKernelGGL((hgrn2_recurrent_kernel<Tin, Tout, 32>), grid, dim3(64), 0, s, p); break;
    case 64: hipLaunchKernelGGL((hgrn2_recurrent_kernel<Tin, Tout, 64>), grid, dim3(64), 0, s, p); break;
    default: hipLaunchKernelGGL((hgrn2_recurrent_kernel<Tin, Tout, 128>), grid, dim3(128), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hgrn2_scan(const Hgrn2ScanArgs& a, hipStream_t s) {
  H2Params p;
  p.B = a.B; p.L = a.L; p.H = a.H; p.d = a.d;
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g_logit; p.lb = a.lower_bound;
  p.S0 = a.S0; p.o = a.o; p.S_last = a.S_last;
  if (!a.in_bf16) return launch_recurrent_t<float, float>(p, s);
  return a.out_bf16 ? launch_recurrent_t<bf16_t, bf16_t>(p, s) : launch_recurrent_t<bf16_t, float>(p, s);
}

hipError_t launch_hgrn2_update(const Hgrn2UpdateArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.H * a.d;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (!a.in_bf16)
    hipLaunchKernelGGL((hgrn2_update_kernel<float, float>), grid, dim3(256), 0, s, rows, a.d, a.q, a.k, a.v,
                       a.g_logit, a.lower_bound, a.S, a.o);
  else if (a.out_bf16)
    hipLaunchKernelGGL((hgrn2_update_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, rows, a.d, a.q, a.k, a.v,
                       a.g_logit, a.lower_bound, a.S, a.o);
  else
    hipLaunchKernelGGL((hgrn2_update_kernel<bf16_t, float>), grid, dim3(256), 0, s, rows, a.d, a.q, a.k, a.v,
                       a.g_logit, a.lower_bound, a.S, a.o);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}
}  // namespace

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0 || !dst) return hipSuccess;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace ssd
