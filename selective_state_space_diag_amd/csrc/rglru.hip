// rglru.hip -- RG-LRU scan and decode update for gfx950.
//
// Recurrence (lrnnx documentation, "lrnnx.models.ltv.rglru": RGLRU.forward gates and the
// RGLRU.step update): r = sigmoid(r_logit), i = sigmoid(i_logit), log a_t = c * r * a_log,
// h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i x).
//
// Scan design (single pass, every input read once from HBM):
//   * A work unit is (batch b, channel tile k of 64*V channels, chunk c of 64 steps).  Lanes run
//     along channels (coalesced rows of the [B, L, D] layout); the 4 waves of a workgroup each own
//     16 consecutive steps of the chunk.
//   * Each lane turns its 16 steps into affine pairs (a_t, b_t) kept in registers and folds them
//     into the wave's aggregate (P = prod a, H = state reached from 0).
//   * Aggregates of the 4 waves meet in LDS; the chunk's carry-in comes from a lookback over
//     earlier chunks of the same (b, k), which publish aggregates and block-end inclusive states
//     as self-validating 64-bit words (value, launch epoch).  Tickets are handed out chunk-major,
//     so a unit only ever waits for lower tickets, which are running or done: the lookback always
//     terminates, and its fixed combine order makes the result bitwise reproducible.
//   * With the carry known, each wave re-runs h = a h + b over its registers and stores y.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kWaves = 4;
constexpr int kSteps = 16;                 // steps per wave
constexpr int kChunk = kWaves * kSteps;    // steps per work unit
constexpr int kBlock = 2;                  // chunks per lookback block

struct RgParams {
  int64_t B, L, D;
  int64_t n_tiles, n_chunks;
  const void* x;
  const void* r;
  const void* i;
  const float* a_log;
  float c;
  const float* h0;
  void* y;
  float* h_last;
  LookbackCtl* ctl;
  unsigned long long* words;  // [unit][3][tile width]: aggregate P, aggregate H, inclusive h
  int one_unit_each;          // grid == number of units: every workgroup takes exactly one ticket
};

// 1 - a^2 for a = 2^l2 (l2 <= 0), accurate near a = 1: series of -expm1(2 l2 ln2) for small
// arguments, else fma(-a, a, 1).
__device__ __forceinline__ float one_minus_a2(float l2, float a) {
  float u = 2.0f * l2 * kLn2;
  float p = fmaf(u, 1.0f / 720.0f, 1.0f / 120.0f);
  p = fmaf(u, p, 1.0f / 24.0f);
  p = fmaf(u, p, 1.0f / 6.0f);
  p = fmaf(u, p, 0.5f);
  p = fmaf(u, p, 1.0f);
  float small = -u * p;
  float big = fmaf(-a, a, 1.0f);
  return fabsf(u) < 0.25f ? small : big;
}

// One RG-LRU element: returns (a_t, b_t) of the affine step from raw inputs.
// kc = c * a_log * log2(e) so that log2 a_t = kc * r.
__device__ __forceinline__ void rglru_ab(float xx, float rl, float il, float kc, float& a, float& b) {
  float r = sigmoid_f(rl);
  float i = sigmoid_f(il);
  float l2 = kc * r;
  a = hw_exp2(l2);
  float beta = hw_sqrt(one_minus_a2(l2, a));
  b = beta * (i * xx);
}

// Raw inputs of one wave's kSteps steps (the loads of a unit, kept in flight until needed).
template <typename Tin, int V>
struct RgRaw {
  typename win<Tin, V, kStreaming>::raw x[kSteps], r[kSteps], i[kSteps];
};

struct RgUnit {
  int64_t c, b, k;
  int rows;  // valid steps in the chunk (kChunk except for a ragged last chunk)
};

__device__ __forceinline__ RgUnit rg_unit(const RgParams& p, int64_t ticket) {
  const int64_t per_round = p.B * p.n_tiles;
  RgUnit u;
  u.c = ticket / per_round;  // chunk-major ticket order
  const int64_t rr = ticket - u.c * per_round;
  u.b = rr / p.n_tiles;
  u.k = rr - u.b * p.n_tiles;
  u.rows = (int)min<int64_t>(kChunk, p.L - u.c * kChunk);
  return u;
}

// Window over the unit's rows of a [B, L, D] array with elements of `es` bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rg_window(const RgParams& p, const RgUnit& u, const void* a,
                                                            int es) {
  const char* base = static_cast<const char*>(a) + ((u.b * p.L + u.c * kChunk) * p.D) * es;
  return make_window(base, (uint32_t)(u.rows * p.D * es));
}

// Issue the loads of unit u for this wave.  Lanes past D read channel D - V and steps past the
// chunk's valid rows read its last row: every offset stays inside the window (results unused).
template <typename Tin, int V>
__device__ __forceinline__ void rg_fetch(const RgParams& p, const RgUnit& u, uint32_t lane_off, int wave,
                                         RgRaw<Tin, V>& raw) {
  constexpr int es = sizeof(Tin);
  const auto wx = rg_window(p, u, p.x, es), wr = rg_window(p, u, p.r, es), wi = rg_window(p, u, p.i, es);
  const uint32_t row_bytes = (uint32_t)(p.D * es);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const uint32_t ro = (uint32_t)min(wave * kSteps + s, u.rows - 1) * row_bytes;
    raw.x[s] = win<Tin, V, kStreaming>::load(wx, lane_off, ro);
    raw.r[s] = win<Tin, V, kStreaming>::load(wr, lane_off, ro);
    raw.i[s] = win<Tin, V, kStreaming>::load(wi, lane_off, ro);
  }
}

// Persistent workgroups: each takes tickets (work units) until none are left.  For unit t it
//   1. folds the raw inputs of t (loaded earlier) into affine pairs and wave aggregates,
//   2. issues the loads of its next unit, so they are in flight during the lookback of t,
//   3. resolves the carry of t (wave 0), then re-runs the recurrence and stores y.
// The next ticket is requested one unit ahead, so its latency is hidden too.
// Occupancy hint: with bf16 inputs the kernel fits 3 workgroups per SIMD group without spills.
template <typename Tin> constexpr int rg_waves_per_eu() { return sizeof(Tin) == 2 ? 3 : 1; }

template <typename Tin, typename Tout, int V>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(rg_waves_per_eu<Tin>())))
void rglru_scan_kernel(RgParams p) {
  constexpr int TW = 64 * V;  // channels per tile
  __shared__ unsigned long long s_tick[2];
  __shared__ float s_aggP[kWaves][TW];
  __shared__ float s_aggH[kWaves][TW];
  __shared__ float s_carry[TW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t total = p.B * p.n_tiles * p.n_chunks;
  using LD = win<Tin, V, kStreaming>;

  if (threadIdx.x == 0) s_tick[0] = atomicAdd(&p.ctl->tick, 1ull);
  __syncthreads();
  const uint32_t E = (uint32_t)(s_tick[0] >> 32) + 1u;  // epoch carried by this launch's words
  int64_t ticket = (int64_t)(s_tick[0] & 0xffffffffull);
  RgRaw<Tin, V> raw;
  // The lane's channels within a tile are the same for every unit; the tile base moves.
  auto lane_off_of = [&](const RgUnit& u) -> uint32_t {
    const int64_t ch0 = u.k * TW + (int64_t)lane * V;
    return (uint32_t)(min<int64_t>(ch0, p.D - V) * (int64_t)sizeof(Tin));
  };
  if (ticket < total) {
    const RgUnit u0 = rg_unit(p, ticket);
    rg_fetch<Tin, V>(p, u0, lane_off_of(u0), wave, raw);
  }
  int parity = 0;

  while (ticket < total) {
    const RgUnit u = rg_unit(p, ticket);
    if (threadIdx.x == 0)  // next ticket, one unit ahead (none needed when the grid covers every unit)
      s_tick[parity ^ 1] = p.one_unit_each ? ~0ull : atomicAdd(&p.ctl->tick, 1ull);
    const int64_t ch0 = u.k * TW + (int64_t)lane * V;
    const bool ch_ok = ch0 < p.D;  // V = 2 only when D is even
    const int64_t chl = ch_ok ? ch0 : p.D - V;
    const int64_t t0 = u.c * kChunk + (int64_t)wave * kSteps;  // first step of this wave

    // ---- affine pairs and the wave's aggregate
    float kc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) kc[v] = p.c * p.a_log[chl + v] * kLog2e;
    float av[kSteps][V], bv[kSteps][V];
    float P[V], Hs[V];
#pragma unroll
    for (int v = 0; v < V; ++v) { P[v] = 1.0f; Hs[v] = 0.0f; }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bool ok = ch_ok && (t0 + s < p.L);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float a, bb;
        rglru_ab(LD::get(raw.x[s], v), LD::get(raw.r[s], v), LD::get(raw.i[s], v), kc[v], a, bb);
        a = ok ? a : 1.0f;  // steps past L and idle lanes are the identity map
        bb = ok ? bb : 0.0f;
        av[s][v] = a;
        bv[s][v] = bb;
        Hs[v] = fmaf(a, Hs[v], bb);
        P[v] *= a;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      s_aggP[wave][lane * V + v] = P[v];
      s_aggH[wave][lane * V + v] = Hs[v];
    }
    __syncthreads();  // aggregates in LDS; the next ticket is visible
    const int64_t next = p.one_unit_each ? total : (int64_t)(s_tick[parity ^ 1] & 0xffffffffull);
    if (next < total) {  // in flight during the lookback
      const RgUnit un = rg_unit(p, next);
      rg_fetch<Tin, V>(p, un, lane_off_of(un), wave, raw);
    }

    // ---- wave 0: chunk aggregate, publish, carry-in, inclusive
    // Chunks form blocks of kBlock.  The carry into chunk c is the inclusive state published by the
    // last chunk of the previous block (h0 for the first block), followed by the aggregates of the
    // earlier chunks of c's own block, applied in chunk order.  Every carry is therefore one fixed
    // function of the inputs (bitwise reproducible), and the serial chain has n_chunks / kBlock
    // links.  All the words a unit needs are requested at once; only missing ones are polled again.
    // Waves 0 .. V-1 each resolve 64 of the tile's channels, one per lane.
    if (wave < V) {
      const int64_t seq_unit = (u.b * p.n_tiles + u.k) * p.n_chunks;
      unsigned long long* W = p.words + (seq_unit + u.c) * 3 * TW;
      const int64_t base = (u.c / kBlock) * kBlock;
      const int nprev = (int)(u.c - base);  // aggregates of block-mates before c
      {
        const int j = wave * 64 + lane;
        const int64_t ch = u.k * TW + j;
        const bool j_ok = ch < p.D;
        float Pc = 1.0f, Hc = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          Hc = fmaf(s_aggP[w][j], Hc, s_aggH[w][j]);
          Pc *= s_aggP[w][j];
        }
        if (u.c + 1 < base + kBlock && u.c + 1 < p.n_chunks) {  // block-mates after c read the aggregate
          word_store(&W[0 * TW + j], E, Pc);
          word_store(&W[1 * TW + j], E, Hc);
        }
        // words: [0] inclusive of chunk base-1 (if base > 0), then (P, H) of chunks base .. c-1
        unsigned long long wd[1 + 2 * (kBlock - 1)];
        const unsigned long long* Wb = p.words + (seq_unit + base - 1) * 3 * TW;
        wd[0] = base > 0 ? word_load(&Wb[2 * TW + j]) : ((unsigned long long)E << 32);
#pragma unroll
        for (int q = 0; q < kBlock - 1; ++q) {
          const unsigned long long* Wq = p.words + (seq_unit + base + q) * 3 * TW;
          if (q < nprev) {
            wd[1 + 2 * q] = word_load(&Wq[0 * TW + j]);
            wd[2 + 2 * q] = word_load(&Wq[1 * TW + j]);
          } else {
            wd[1 + 2 * q] = wd[2 + 2 * q] = (unsigned long long)E << 32;
          }
        }
        unsigned int spins = 0;
        while (true) {
          bool all = word_ready(wd[0], E);
#pragma unroll
          for (int q = 0; q < 2 * (kBlock - 1); ++q) all = all && word_ready(wd[1 + q], E);
          if (all || spins >= kSpinLimit) break;
          ++spins;
          __builtin_amdgcn_s_sleep(1);
          if (!word_ready(wd[0], E)) wd[0] = word_load(&Wb[2 * TW + j]);
#pragma unroll
          for (int q = 0; q < kBlock - 1; ++q) {
            const unsigned long long* Wq = p.words + (seq_unit + base + q) * 3 * TW;
            if (!word_ready(wd[1 + 2 * q], E)) wd[1 + 2 * q] = word_load(&Wq[0 * TW + j]);
            if (!word_ready(wd[2 + 2 * q], E)) wd[2 + 2 * q] = word_load(&Wq[1 * TW + j]);
          }
        }
        if (spins >= kSpinLimit) atomicOr(&p.ctl->error, 1u);
        float hin = (base > 0) ? word_value(wd[0]) : (p.h0 ? p.h0[u.b * p.D + (j_ok ? ch : p.D - 1)] : 0.0f);
#pragma unroll
        for (int q = 0; q < kBlock - 1; ++q)
          if (q < nprev) hin = fmaf(word_value(wd[1 + 2 * q]), hin, word_value(wd[2 + 2 * q]));
        const float incl = fmaf(Pc, hin, Hc);
        if (u.c == base + kBlock - 1 && u.c + 1 < p.n_chunks) word_store(&W[2 * TW + j], E, incl);
        if (p.h_last && j_ok && u.c == p.n_chunks - 1) p.h_last[u.b * p.D + ch] = incl;
        s_carry[j] = hin;
      }
    }
    __syncthreads();

    // ---- carry into this wave, re-run the recurrence, store
    float h[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int j = lane * V + v;
      float hv = s_carry[j];
      for (int w = 0; w < wave; ++w) hv = fmaf(s_aggP[w][j], hv, s_aggH[w][j]);
      h[v] = hv;
    }
    {
      const auto wy = rg_window(p, u, p.y, (int)sizeof(Tout));
      const uint32_t row_bytes = (uint32_t)(p.D * (int64_t)sizeof(Tout));
      const uint32_t lo = (uint32_t)(chl * (int64_t)sizeof(Tout));
      const int nvalid = u.rows - wave * kSteps;  // rows of this wave inside the chunk
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        float out[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          h[v] = fmaf(av[s][v], h[v], bv[s][v]);
          out[v] = h[v];
        }
        if (ch_ok && s < nvalid) win<Tout, V, kStreaming>::store(wy, lo, (uint32_t)(wave * kSteps + s) * row_bytes, out);
      }
    }
    __syncthreads();  // LDS (aggregates, carry, ticket slot) is reused by the next unit
    ticket = next;
    parity ^= 1;
  }

  // ---- last workgroup to finish resets the ticket and advances the epoch
  if (threadIdx.x == 0) {
    const unsigned int old = atomicAdd(&p.ctl->done, 1u);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(&p.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.ctl->tick, (unsigned long long)E << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void rglru_update_kernel(int64_t B, int64_t D, const void* x, const void* r,
                                                           const void* i, const float* a_log, float c,
                                                           float* state, void* y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * D) return;
  const int64_t d = idx % D;
  float a, bb;
  rglru_ab(io<Tin>::load(x, idx), io<Tin>::load(r, idx), io<Tin>::load(i, idx), c * a_log[d] * kLog2e, a, bb);
  const float h = fmaf(a, state[idx], bb);
  state[idx] = h;
  io<Tout>::store(y, idx, h);
}

// Persistent grid: as many workgroups as stay resident together (by the kernel's own occupancy),
// never more than there are work units.
template <typename Tin, typename Tout, int V>
hipError_t launch_scan_t(const RgParams& p, hipStream_t s) {
  const int64_t total = p.B * p.n_tiles * p.n_chunks;
  static int per_cu = 0, cus = 0;
  if (per_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rglru_scan_kernel<Tin, Tout, V>, kWaves * 64, 0) !=
            hipSuccess || per_cu <= 0)
      per_cu = 1;
  }
  const int64_t grid = std::min<int64_t>(total, (int64_t)per_cu * cus);
  RgParams q = p;
  q.one_unit_each = grid == total;
  hipLaunchKernelGGL((rglru_scan_kernel<Tin, Tout, V>), dim3((unsigned)grid), dim3(kWaves * 64), 0, s, q);
  return hipGetLastError();
}

int vec_width(int64_t D) { return (D % 2 == 0) ? 2 : 1; }

}  // namespace

size_t rglru_scan_scratch_bytes(int64_t B, int64_t L, int64_t D) {
  const int V = vec_width(D);
  const int64_t TW = 64 * V;
  const int64_t n_tiles = (D + TW - 1) / TW;
  const int64_t n_chunks = (L + kChunk - 1) / kChunk;
  return 256 + (size_t)(B * n_tiles * n_chunks) * 3 * TW * sizeof(unsigned long long);
}

hipError_t launch_rglru_scan(const RglruScanArgs& a, hipStream_t s) {
  const int V = vec_width(a.D);
  const int64_t TW = 64 * V;
  RgParams p;
  p.B = a.B; p.L = a.L; p.D = a.D;
  p.n_tiles = (a.D + TW - 1) / TW;
  p.n_chunks = (a.L + kChunk - 1) / kChunk;
  p.x = a.x; p.r = a.r_logit; p.i = a.i_logit;
  p.a_log = a.a_log; p.c = a.c; p.h0 = a.h0; p.y = a.y; p.h_last = a.h_last;
  p.ctl = static_cast<LookbackCtl*>(a.scratch);
  p.words = reinterpret_cast<unsigned long long*>(static_cast<char*>(a.scratch) + 256);
  if (V == 2) {
    if (!a.in_bf16) return launch_scan_t<float, float, 2>(p, s);
    return a.out_bf16 ? launch_scan_t<bf16_t, bf16_t, 2>(p, s) : launch_scan_t<bf16_t, float, 2>(p, s);
  }
  if (!a.in_bf16) return launch_scan_t<float, float, 1>(p, s);
  return a.out_bf16 ? launch_scan_t<bf16_t, bf16_t, 1>(p, s) : launch_scan_t<bf16_t, float, 1>(p, s);
}

hipError_t launch_rglru_update(const RglruUpdateArgs& a, hipStream_t s) {
  const int64_t n = a.B * a.D;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (!a.in_bf16)
    hipLaunchKernelGGL((rglru_update_kernel<float, float>), grid, dim3(256), 0, s, a.B, a.D, a.x, a.r_logit,
                       a.i_logit, a.a_log, a.c, a.state, a.y);
  else if (a.out_bf16)
    hipLaunchKernelGGL((rglru_update_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, a.B, a.D, a.x, a.r_logit,
                       a.i_logit, a.a_log, a.c, a.state, a.y);
  else
    hipLaunchKernelGGL((rglru_update_kernel<bf16_t, float>), grid, dim3(256), 0, s, a.B, a.D, a.x, a.r_logit,
                       a.i_logit, a.a_log, a.c, a.state, a.y);
  return hipGetLastError();
}

}  // namespace ssd
