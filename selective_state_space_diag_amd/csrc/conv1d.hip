// conv1d.hip -- causal depthwise convolution of the RG-LRU block and its decode step, for gfx950.
//
// Definition (lrnnx documentation, "lrnnx.models.ltv.rglru": the block's nn.Conv1d with groups =
// channels, kernel W = d_conv, padding W - 1, of which the first L outputs are kept; and step(),
// whose conv_state window shifts left by one, takes the new input last and is summed against the
// weights plus the bias):
//   y[b, t, d] = bias[d] + sum_{k < W} weight[d][k] x[b, t - (W-1) + k, d]
// Inputs before the sequence come from a carried window state[b][d][0..W-1] (entry W + tau holds
// time tau < 0) or are zero.
//
// Scan form: streaming, every input read once.  A workgroup covers 64 rows x 64 V channels of one
// batch row; each of its 4 waves owns 16 consecutive rows, each lane V adjacent channels.  A lane
// keeps the previous W - 1 inputs of its channels in registers (loaded once as a halo: 3 extra rows
// per 16, served from L2 since the neighbouring wave reads them too), loads its 16 rows up front
// and slides the window down them.  The lane whose rows end the sequence also writes the final
// window (the last W inputs) to state_out.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 16;              // rows per wave
constexpr int kTile = kWaves * kRows;  // rows per workgroup

struct ConvParams {
  int64_t B, L, D;
  int64_t n_tiles, n_rowblk;
  const void* x;
  const float* weight;  // [D][W]
  const float* bias;    // [D] or NULL
  const float* state_in;  // [B][D][W] or NULL
  void* y;
  float* state_out;       // [B][D][W] or NULL
};

template <typename Tin, typename Tout, int V, int W>
__global__ __launch_bounds__(kWaves * 64) void conv1d_kernel(ConvParams p) {
  using LD = win<Tin, V>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // blockIdx.x = (b * n_rowblk + row block) * n_tiles + channel tile
  const int64_t tile = blockIdx.x % p.n_tiles;
  const int64_t rest = blockIdx.x / p.n_tiles;
  const int64_t rb = rest % p.n_rowblk;
  const int64_t b = rest / p.n_rowblk;
  const int64_t ch0 = tile * 64 * V + (int64_t)lane * V;
  const bool ch_ok = ch0 < p.D;  // V = 2 only when D is even
  const int64_t chl = ch_ok ? ch0 : p.D - V;
  const int64_t t0 = rb * kTile + (int64_t)wave * kRows;  // first row of this wave
  if (t0 >= p.L) return;
  const int nrows = (int)min<int64_t>(kRows, p.L - t0);

  // rows [t0 - (W-1), t0 + nrows) of this batch row that lie in [0, L): window for loads
  const int64_t lo_row = max<int64_t>(0, t0 - (W - 1));
  const int64_t hi_row = t0 + nrows;
  const auto wx = make_window(static_cast<const char*>(p.x) + ((b * p.L + lo_row) * p.D) * (int64_t)sizeof(Tin),
                              (uint32_t)((hi_row - lo_row) * p.D * (int64_t)sizeof(Tin)));
  const uint32_t row_bytes = (uint32_t)(p.D * (int64_t)sizeof(Tin));
  const uint32_t lane_off = (uint32_t)(chl * (int64_t)sizeof(Tin));

  typename LD::raw raw[kRows];
#pragma unroll
  for (int s = 0; s < kRows; ++s) {
    const int r = min(s, nrows - 1);
    raw[s] = LD::load(wx, lane_off, (uint32_t)(t0 + r - lo_row) * row_bytes);
  }
  // window[k] = input at time t0 - (W-1) + k, k < W - 1 (the halo)
  float win_v[W][V];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t tau = t0 - (W - 1) + k;
    if (tau >= 0) {
      const auto r = LD::load(wx, lane_off, (uint32_t)(tau - lo_row) * row_bytes);
#pragma unroll
      for (int v = 0; v < V; ++v) win_v[k][v] = LD::get(r, v);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v)
        win_v[k][v] = p.state_in ? p.state_in[(b * p.D + chl + v) * W + (W + tau)] : 0.0f;
    }
  }
  float w[V][W], bs[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < W; ++k) w[v][k] = p.weight[(chl + v) * W + k];
    bs[v] = p.bias ? p.bias[chl + v] : 0.0f;
  }

  const auto wy = make_window(static_cast<char*>(p.y) + ((b * p.L + t0) * p.D) * (int64_t)sizeof(Tout),
                              (uint32_t)(nrows * p.D * (int64_t)sizeof(Tout)));
  const uint32_t out_row = (uint32_t)(p.D * (int64_t)sizeof(Tout));
  const uint32_t out_lane = (uint32_t)(chl * (int64_t)sizeof(Tout));
#pragma unroll
  for (int s = 0; s < kRows; ++s) {
    float out[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      win_v[W - 1][v] = LD::get(raw[s], v);
      float acc = bs[v];
#pragma unroll
      for (int k = 0; k < W; ++k) acc = fmaf(w[v][k], win_v[k][v], acc);
      out[v] = acc;
    }
    if (s < nrows) {
      if (ch_ok) win<Tout, V, kStreaming>::store(wy, out_lane, (uint32_t)s * out_row, out);
      if (p.state_out && ch_ok && t0 + s == p.L - 1) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < W; ++k) p.state_out[(b * p.D + ch0 + v) * W + k] = win_v[k][v];
      }
    }
#pragma unroll
    for (int k = 0; k + 1 < W; ++k)
#pragma unroll
      for (int v = 0; v < V; ++v) win_v[k][v] = win_v[k + 1][v];
  }
}

// Decode step: one thread per (b, d); the window shifts left, x enters last.
template <typename Tin, typename Tout, int W>
__global__ __launch_bounds__(256) void conv1d_update_kernel(int64_t B, int64_t D, const void* x, const float* weight,
                                                            const float* bias, float* state, void* y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * D) return;
  const int64_t d = idx % D;
  float* st = state + idx * W;
  float win_v[W];
#pragma unroll
  for (int k = 0; k + 1 < W; ++k) win_v[k] = st[k + 1];
  win_v[W - 1] = io<Tin>::load(x, idx);
  float acc = bias ? bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    acc = fmaf(weight[d * W + k], win_v[k], acc);
    st[k] = win_v[k];
  }
  io<Tout>::store(y, idx, acc);
}

template <typename Tin, typename Tout, int V>
hipError_t launch_conv_v(const ConvParams& p, int W, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.n_rowblk * p.n_tiles)), blk(kWaves * 64);
  switch (W) {
    case 1: hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, V, 1>), grid, blk, 0, s, p); break;
    case 2: hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, V, 2>), grid, blk, 0, s, p); break;
    case 3: hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, V, 3>), grid, blk, 0, s, p); break;
    default: hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, V, 4>), grid, blk, 0, s, p); break;
  }
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_conv_t(const ConvParams& p, int W, hipStream_t s) {
  return p.D % 2 == 0 ? launch_conv_v<Tin, Tout, 2>(p, W, s) : launch_conv_v<Tin, Tout, 1>(p, W, s);
}

template <typename Tin, typename Tout>
hipError_t launch_conv_update_t(const Conv1dUpdateArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.B * a.D + 255) / 256)), blk(256);
  switch (a.W) {
    case 1: hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, 1>), grid, blk, 0, s, a.B, a.D, a.x, a.weight, a.bias, a.state, a.y); break;
    case 2: hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, 2>), grid, blk, 0, s, a.B, a.D, a.x, a.weight, a.bias, a.state, a.y); break;
    case 3: hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, 3>), grid, blk, 0, s, a.B, a.D, a.x, a.weight, a.bias, a.state, a.y); break;
    default: hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, 4>), grid, blk, 0, s, a.B, a.D, a.x, a.weight, a.bias, a.state, a.y); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_conv1d(const Conv1dArgs& a, hipStream_t s) {
  ConvParams p{};
  p.B = a.B; p.L = a.L; p.D = a.D;
  const int V = a.D % 2 == 0 ? 2 : 1;
  p.n_tiles = (a.D + 64 * V - 1) / (64 * V);
  p.n_rowblk = (a.L + kTile - 1) / kTile;
  p.x = a.x; p.weight = a.weight; p.bias = a.bias; p.state_in = a.state_in; p.y = a.y; p.state_out = a.state_out;
  if (!a.in_bf16) return launch_conv_t<float, float>(p, (int)a.W, s);
  return a.out_bf16 ? launch_conv_t<bf16_t, bf16_t>(p, (int)a.W, s) : launch_conv_t<bf16_t, float>(p, (int)a.W, s);
}

hipError_t launch_causal_conv1d_update(const Conv1dUpdateArgs& a, hipStream_t s) {
  if (!a.in_bf16) return launch_conv_update_t<float, float>(a, s);
  return a.out_bf16 ? launch_conv_update_t<bf16_t, bf16_t>(a, s) : launch_conv_update_t<bf16_t, float>(a, s);
}

}  // namespace ssd
