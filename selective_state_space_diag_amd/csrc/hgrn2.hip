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

// ----------------------------------------------------------------------------- chunked MFMA form
// For chunks of 64 tokens with Gamma[t][i] = prod_{u<=t} g[u][i] (within the chunk) the row-gated
// recurrence unrolls to
//   O      = Gamma (.) ( (Q K^T (.) M) (V (/) Gamma)  +  Q S0^T )          (M: causal, diagonal included)
//   S_next = diag(Gamma_C) S0  +  ((Gamma_C (/) Gamma) (.) V)^T K
// (rows of S and columns of O index the value dimension).  All products run on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Q, K are bf16 inputs and enter exactly; every
// derived operand (Q K^T, V / Gamma, the W factor, the state copy) is split into a bf16 pair
// hi + lo, so its products carry about 16 significant bits instead of 8; the state S itself stays in
// fp32 accumulators for the whole sequence.
// V (/) Gamma needs Gamma >= lower_bound^64 to stay far from underflow: the launcher uses this form
// only for lower_bound >= 2^-1.5 (Gamma >= 2^-96); smaller bounds take the recurrent kernel.
//
// Workgroup = (batch, head, half of the 128 value rows); 4 waves, wave w owns value rows
// [16w, 16w+16) of the half: 16 x 128 state entries = 8 accumulator tiles.  LDS rows are padded by
// 16 bytes so the 16-row operand reads of an MFMA spread over all banks.  The next chunk's global
// data is loaded into registers while the current chunk computes.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;

constexpr int kCh = 64;    // chunk length (tokens)
constexpr int kDh = 128;   // head dim
constexpr int kRows = 64;  // value rows per workgroup
constexpr int kPadD = kDh + 8;
constexpr int kPadC = kCh + 8;

__device__ __forceinline__ floatx4_t mfma(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                  0, 0, 0);
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

struct H2Lds {
  uint16_t q[kCh][kPadD];          // Q chunk [t][j]
  uint16_t k[kCh][kPadD];          // K chunk [s][j]
  uint16_t kt[kDh][kPadC];         // K transposed [j][t]
  union {
    struct {
      uint16_t vraw[kCh][kRows];   // V chunk [t][i]          (read by the gate step)
      uint16_t graw[kCh][kRows];   // gate logits [t][i]      (read by the gate step)
    } in;
    struct {
      uint16_t a[kCh][kPadC];      // masked Q K^T [t][s], hi (written after the gate step)
      uint16_t a_lo[kCh][kPadC];
    } qk;
  } u;
  uint16_t vs[kRows][kPadC];       // V / Gamma, [i][t], hi and lo
  uint16_t vs_lo[kRows][kPadC];
  uint16_t w[kRows][kPadC];        // V * Gamma_C / Gamma, [i][t], hi and lo
  uint16_t w_lo[kRows][kPadC];
  uint16_t sb[kRows][kPadD];       // state S [i][j] entering the chunk, hi and lo
  uint16_t sb_lo[kRows][kPadD];
  float gam[kRows][kCh + 4];       // Gamma [i][t]
  float gtot[4][kRows];            // per-quarter gate products
};

struct H2Prefetch {
  uint4 q[4], k[4], v[2], g[2];
};

__device__ __forceinline__ void h2_fetch(const H2Params& p, int64_t b, int64_t hh, int64_t i0, int64_t t0, int tid,
                                         H2Prefetch& f) {
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const uint16_t* K = static_cast<const uint16_t*>(p.k);
  const uint16_t* V = static_cast<const uint16_t*>(p.v);
  const uint16_t* G = static_cast<const uint16_t*>(p.g);
  const int valid = (int)min((int64_t)kCh, p.L - t0);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = it * 256 + tid;  // 1024 segments of 8 elements: row t, segment seg
    const int t = idx >> 4, seg = idx & 15;
    f.q[it] = f.k[it] = make_uint4(0, 0, 0, 0);
    if (t < valid) {
      const int64_t off = ((b * p.L + t0 + t) * p.H + hh) * kDh + seg * 8;
      f.q[it] = *reinterpret_cast<const uint4*>(Q + off);
      f.k[it] = *reinterpret_cast<const uint4*>(K + off);
    }
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = it * 256 + tid;  // 512 segments of 8 elements
    const int t = idx >> 3, seg = idx & 7;
    f.v[it] = f.g[it] = make_uint4(0, 0, 0, 0);
    if (t < valid) {
      const int64_t off = ((b * p.L + t0 + t) * p.H + hh) * kDh + i0 + seg * 8;
      f.v[it] = *reinterpret_cast<const uint4*>(V + off);
      f.g[it] = *reinterpret_cast<const uint4*>(G + off);
    }
  }
}

__device__ __forceinline__ void h2_stage(H2Lds& sm, int tid, const H2Prefetch& f) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = it * 256 + tid;
    const int t = idx >> 4, seg = idx & 15;
    *reinterpret_cast<uint4*>(&sm.q[t][seg * 8]) = f.q[it];
    *reinterpret_cast<uint4*>(&sm.k[t][seg * 8]) = f.k[it];
    const uint16_t* ke = reinterpret_cast<const uint16_t*>(&f.k[it]);
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.kt[seg * 8 + e][t] = ke[e];
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = it * 256 + tid;
    const int t = idx >> 3, seg = idx & 7;
    *reinterpret_cast<uint4*>(&sm.u.in.vraw[t][seg * 8]) = f.v[it];
    *reinterpret_cast<uint4*>(&sm.u.in.graw[t][seg * 8]) = f.g[it];
  }
}

template <typename Tout>
__global__ __launch_bounds__(256) void hgrn2_chunk_kernel(H2Params p) {
  __shared__ H2Lds sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;  // 0..3
  // both halves of a head on the same XCD (blockIdx % 8) so their Q / K reads share an L2
  int64_t bh, half;
  if ((p.B * p.H) % 8 == 0) {
    const int64_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    half = slot % 2;
    bh = (slot / 2) * 8 + xcd;
  } else {
    bh = blockIdx.x / 2;
    half = blockIdx.x % 2;
  }
  const int64_t b = bh / p.H, hh = bh - b * p.H;
  const int64_t i0 = half * kRows;  // first value row of this workgroup
  const float lb = p.lb, one_m_lb = 1.0f - p.lb;

  // ---- state accumulators: rows r0 + 4*lg + e (e = 0..3) of the half, columns 16*nt + l16
  const int r0 = wave * 16;
  floatx4_t S[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[nt][e] = p.S0 ? p.S0[(bh * kDh + i0 + r0 + 4 * lg + e) * kDh + 16 * nt + l16] : 0.0f;

  const int64_t nchunks = (p.L + kCh - 1) / kCh;
  H2Prefetch f;
  h2_fetch(p, b, hh, i0, 0, tid, f);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * kCh;
    const int valid = (int)min((int64_t)kCh, p.L - t0);
    h2_stage(sm, tid, f);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t hi, lo;
        split_bf16(S[nt][e], hi, lo);
        sm.sb[r0 + 4 * lg + e][16 * nt + l16] = hi;
        sm.sb_lo[r0 + 4 * lg + e][16 * nt + l16] = lo;
      }
    __syncthreads();
    if (c + 1 < nchunks) h2_fetch(p, b, hh, i0, t0 + kCh, tid, f);  // in flight during this chunk

    // ---- gates and their cumulative products: thread (row i, quarter q of the chunk)
    {
      const int i = tid & 63, q = tid >> 6;
      float gl[16], vv[16];
      float run = 1.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int t = q * 16 + u;
        const float g = (t < valid) ? fmaf(one_m_lb, sigmoid_f(bf16_to_f32(sm.u.in.graw[t][i])), lb) : 1.0f;
        run *= g;
        gl[u] = run;
        vv[u] = bf16_to_f32(sm.u.in.vraw[t][i]);
      }
      sm.gtot[q][i] = run;
      __syncthreads();  // quarter products visible; vraw / graw fully read
      float pre = 1.0f, all = 1.0f;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (qq < q) pre *= sm.gtot[qq][i];
        all *= sm.gtot[qq][i];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int t = q * 16 + u;
        const float gam = pre * gl[u];
        const float inv = hw_rcp(gam);
        sm.gam[i][t] = gam;
        split_bf16(vv[u] * inv, sm.vs[i][t], sm.vs_lo[i][t]);
        split_bf16(vv[u] * (all * inv), sm.w[i][t], sm.w_lo[i][t]);
      }
    }

    // ---- A = Q K^T (rows t in [16*wave, +16)), causal mask, bf16 hi / lo into LDS
    {
      floatx4_t acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sm.q[16 * wave + l16][32 * ks + 8 * lg]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const uint4 bb = *reinterpret_cast<const uint4*>(&sm.k[16 * nt + l16][32 * ks + 8 * lg]);
          acc[nt] = mfma(a, bb, acc[nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * wave + 4 * lg + e, sidx = 16 * nt + l16;
          split_bf16(sidx <= t ? acc[nt][e] : 0.0f, sm.u.qk.a[t][sidx], sm.u.qk.a_lo[t][sidx]);
        }
    }
    __syncthreads();

    // ---- O for this wave's 16 value rows, all 64 tokens: Gamma (.) (A Vs + Q S^T)
    {
      float gc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r0 + 4 * lg + e;
        gc[e] = sm.gtot[0][row] * sm.gtot[1][row] * sm.gtot[2][row] * sm.gtot[3][row];
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (32 * ks <= 16 * mt + 15) {  // key blocks past the query block are fully masked
            const uint4 ah = *reinterpret_cast<const uint4*>(&sm.u.qk.a[16 * mt + l16][32 * ks + 8 * lg]);
            const uint4 al = *reinterpret_cast<const uint4*>(&sm.u.qk.a_lo[16 * mt + l16][32 * ks + 8 * lg]);
            const uint4 vh = *reinterpret_cast<const uint4*>(&sm.vs[r0 + l16][32 * ks + 8 * lg]);
            const uint4 vl = *reinterpret_cast<const uint4*>(&sm.vs_lo[r0 + l16][32 * ks + 8 * lg]);
            acc = mfma(ah, vh, acc);
            acc = mfma(al, vh, acc);
            acc = mfma(ah, vl, acc);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint4 a = *reinterpret_cast<const uint4*>(&sm.q[16 * mt + l16][32 * ks + 8 * lg]);
          const uint4 sh = *reinterpret_cast<const uint4*>(&sm.sb[r0 + l16][32 * ks + 8 * lg]);
          const uint4 sl = *reinterpret_cast<const uint4*>(&sm.sb_lo[r0 + l16][32 * ks + 8 * lg]);
          acc = mfma(a, sh, acc);
          acc = mfma(a, sl, acc);
        }
        // acc[e] = O[t = 16 mt + 4 lg + e][i = r0 + l16]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * mt + 4 * lg + e;
          if (t < valid) {
            const float o = acc[e] * sm.gam[r0 + l16][t];
            io<Tout>::store(p.o, ((b * p.L + t0 + t) * p.H + hh) * kDh + i0 + r0 + l16, o);
          }
        }
      }
      // ---- state update: S = diag(Gamma_C) S + W^T K  (rows r0 + 4 lg + e, columns 16 nt + l16)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[nt][e] *= gc[e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 wh = *reinterpret_cast<const uint4*>(&sm.w[r0 + l16][32 * ks + 8 * lg]);
        const uint4 wl = *reinterpret_cast<const uint4*>(&sm.w_lo[r0 + l16][32 * ks + 8 * lg]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const uint4 bb = *reinterpret_cast<const uint4*>(&sm.kt[16 * nt + l16][32 * ks + 8 * lg]);
          S[nt] = mfma(wh, bb, S[nt]);
          S[nt] = mfma(wl, bb, S[nt]);
        }
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  if (p.S_last) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.S_last[(bh * kDh + i0 + r0 + 4 * lg + e) * kDh + 16 * nt + l16] = S[nt][e];
  }
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
  // chunked MFMA form: bf16 inputs, d = 128, lower_bound >= 2^-1.5 (see hgrn2_chunk_kernel)
  if (a.in_bf16 && a.d == kDh && a.lower_bound >= 0.35355339f) {
    const dim3 grid((unsigned)(a.B * a.H * 2));
    if (a.out_bf16)
      hipLaunchKernelGGL((hgrn2_chunk_kernel<bf16_t>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((hgrn2_chunk_kernel<float>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
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
