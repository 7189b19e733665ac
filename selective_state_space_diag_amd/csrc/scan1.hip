// scan1.hip -- diagonal scans with one state per channel for gfx950: the RG-LRU recurrence and the
// MinMax recurrence, each with its decode step.
//
// RG-LRU (lrnnx documentation, "lrnnx.models.ltv.rglru": RGLRU.forward gates and the RGLRU.step
// update): r = sigmoid(r_logit), i = sigmoid(i_logit), log a_t = c * r * a_log,
// h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i x).  The block around it multiplies the result by
// gelu(gate) before its output projection; that multiply is optional here.
// MinMax (minmaxrnc package, minmax_neuron.py and minmax_operator.py): x_t = max(min(r_t, x_{t-1}),
// s_t) from the initial state; the neuron's output gate multiplies x_t by g_t (optional here).
//
// Both steps are maps h -> f(a, b; h) of a family closed under composition:
//   affine  f = a h + b,             (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2)
//   minmax  f = max(min(a, h), b),   (a2, b2) o (a1, b1) = (min(a2, a1), max(min(a2, b1), b2))
// (the MinMax rule is the composition the minmax_operator page states), so one chunked scan serves
// both.  MinMax's min and max order -0 below +0 and turn any NaN operand into NaN: each is then a
// well-defined function of its operands' values, commutative and associative bit for bit, and the
// chunked evaluation equals the sequential loop exactly.
//
// Scan design (single pass, every input read once from HBM):
//   * A work unit is (batch b, channel tile k of 64*V channels, chunk c of 64 steps).  Lanes run
//     along channels (coalesced rows of the [B, L, D] layout); the 4 waves of a workgroup each own
//     16 consecutive steps of the chunk.
//   * Each lane turns its 16 steps into pairs (a_t, b_t) kept in registers and folds them into the
//     wave's aggregate (the composed map of its 16 steps).
//   * Aggregates of the 4 waves meet in LDS; the chunk's carry-in comes from a lookback over
//     earlier chunks of the same (b, k), which publish aggregates and block-end inclusive states
//     as self-validating 64-bit words (value, launch epoch).  Tickets are handed out chunk-major,
//     so a unit only ever waits for lower tickets, which are running or done: the lookback always
//     terminates, and its fixed combine order makes the result bitwise reproducible.
//   * With the carry known, each wave re-runs h = f(a_t, b_t; h) over its registers and stores y.
#include <algorithm>

#include <mutex>
#include <unordered_map>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kWaves = 4;
constexpr int kSteps = 16;                 // steps per wave
constexpr int kChunk = kWaves * kSteps;    // steps per work unit
constexpr int kBlock = 2;                  // chunks per lookback block

struct Scan1Params {
  int64_t B, L, D;
  int64_t n_tiles, n_chunks;
  const void* in[3];   // step inputs: RG-LRU (x, r_logit, i_logit), MinMax (r, s)
  const void* gate;    // output gate or NULL
  const float* a_log;  // RG-LRU only
  float c;
  const float* h0;
  void* y;
  float* h_last;
  float* carry_out;    // [B][n_chunks][D]: state entering each chunk (record passes)
  LookbackCtl* ctl;
  unsigned long long* words;  // [unit][3][tile width]: aggregate a, aggregate b, inclusive h
  WaitCfg wait;
};

// ------------------------------------------------------------------ RG-LRU step
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

// gelu(v) = v * Phi(v) = v/2 (1 + erf(v / sqrt 2)), the exact form (torch's default).  erf by
// Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26 (absolute error below
// 1.5e-7): for x >= 0, 1 - erf(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-x^2) with
// t = 1 / (1 + p x).  With q = 1 - erf(|v| / sqrt 2), 1 + erf(v / sqrt 2) is 2 - q for v >= 0 and q
// itself for v < 0, so the negative tail is formed without cancellation.
__device__ __forceinline__ float gelu_f(float v) {
  const float x = fabsf(v) * 0.70710678118654752f;
  const float t = hw_rcp(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  const float q = poly * t * hw_exp2(-(x * x) * kLog2e);
  return 0.5f * v * (v >= 0.0f ? 2.0f - q : q);
}

struct AffineOp {
  static constexpr int kIn = 3;
  struct Chan {
    float kc;  // c * a_log * log2(e), so that log2 a_t = kc * r
  };
  // The channel parameter is loaded with a unit's inputs (param) and turned into Chan when used.
  static __device__ __forceinline__ float param(const Scan1Params& p, int64_t ch) { return p.a_log[ch]; }
  static __device__ __forceinline__ Chan chan(const Scan1Params& p, float a_log) { return Chan{p.c * a_log * kLog2e}; }
  static __device__ __forceinline__ void step(const float (&v)[3], const Chan& ch, float& a, float& b) {
    const float r = sigmoid_f(v[1]);
    const float i = sigmoid_f(v[2]);
    const float l2 = ch.kc * r;
    a = hw_exp2(l2);
    b = hw_sqrt(one_minus_a2(l2, a)) * (i * v[0]);
  }
  static __device__ __forceinline__ float id_a() { return 1.0f; }
  static __device__ __forceinline__ float id_b() { return 0.0f; }
  static __device__ __forceinline__ float apply(float a, float b, float h) { return fmaf(a, h, b); }
  static __device__ __forceinline__ float fold_a(float a2, float a1) { return a2 * a1; }
  static __device__ __forceinline__ float gated(float h, float g) { return gelu_f(g) * h; }
};

// ------------------------------------------------------------------ MinMax step
// min / max on the reals with -0 below +0, NaN when either operand is NaN: IEEE 754-2019 minimum
// and maximum, one gfx950 instruction each (v_minimum3_f32 / v_maximum3_f32).
__device__ __forceinline__ float mm_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float mm_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

struct MinMaxOp {
  static constexpr int kIn = 2;
  struct Chan {};
  static __device__ __forceinline__ float param(const Scan1Params&, int64_t) { return 0.0f; }
  static __device__ __forceinline__ Chan chan(const Scan1Params&, float) { return Chan{}; }
  static __device__ __forceinline__ void step(const float (&v)[3], const Chan&, float& a, float& b) {
    a = v[0];
    b = v[1];
  }
  static __device__ __forceinline__ float id_a() { return __int_as_float(0x7f800000); }   // +inf
  static __device__ __forceinline__ float id_b() { return __int_as_float((int)0xff800000u); }  // -inf
  static __device__ __forceinline__ float apply(float a, float b, float h) { return mm_max(mm_min(a, h), b); }
  static __device__ __forceinline__ float fold_a(float a2, float a1) { return mm_min(a2, a1); }
  static __device__ __forceinline__ float gated(float h, float g) { return h * g; }
};

// ------------------------------------------------------------------ work tickets
// Sequences (batch row x channel tile) of ticket class x: x, x + K, x + 2K, ... below n_seq.  Every
// count here is below 2^31 (the entry points bound the number of units).
__device__ __forceinline__ uint32_t class_seqs(uint32_t n_seq, uint32_t x) {
  return x < n_seq ? (n_seq - 1 - x) / kTicketClasses + 1 : 0u;
}

constexpr unsigned long long kNoUnit = ~0ull;

// Taking a unit is split in two so that the atomic's round trip overlaps the caller's work (waiting
// on it at once would also wait for every load issued before it).  Thread 0 only.  xc is the class
// being drawn from (initially the home class, blockIdx mod kTicketClasses; it only moves forward)
// and left counts the classes not yet found empty.
__device__ __forceinline__ uint32_t take_begin(LookbackCtl* ctl, int xc, int left) {
  return left > 0 ? atomicAdd(&ctl->cls[xc].next, 1u) : ~0u;
}
// The unit as (class << 32) | local ticket, or kNoUnit once every class is exhausted.  When the
// ticket drawn by take_begin is past its class's end, the following classes are tried in turn; an
// exhausted class is recognised there by a plain load before an atomic is spent on it.
__device__ __forceinline__ unsigned long long take_next_class(LookbackCtl* ctl, uint32_t n_seq, uint32_t n_chunks,
                                                              int* xc, int* left) {
  while (--*left > 0) {
    *xc = *xc + 1 == kTicketClasses ? 0 : *xc + 1;
    const uint32_t lim = class_seqs(n_seq, (uint32_t)*xc) * n_chunks;
    unsigned int* ctr = &ctl->cls[*xc].next;
    if (lim > 0 && __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < lim) {
      const uint32_t m = atomicAdd(ctr, 1u);
      if (m < lim) return ((unsigned long long)*xc << 32) | m;
    }
  }
  return kNoUnit;
}
__device__ __forceinline__ unsigned long long take_end(LookbackCtl* ctl, uint32_t n_seq, uint32_t n_chunks, int& xc,
                                                       int& left, uint32_t m) {
  if (left <= 0) return kNoUnit;
  if (m < class_seqs(n_seq, (uint32_t)xc) * n_chunks) return ((unsigned long long)xc << 32) | m;
  return take_next_class(ctl, n_seq, n_chunks, &xc, &left);
}
__device__ __forceinline__ unsigned long long take_unit(LookbackCtl* ctl, uint32_t n_seq, uint32_t n_chunks, int& xc,
                                                       int& left) {
  return take_end(ctl, n_seq, n_chunks, xc, left, take_begin(ctl, xc, left));
}

// A ticket read from LDS is the same in every lane: keep it (and all index arithmetic on it) scalar.
__device__ __forceinline__ unsigned long long uniform_ticket(unsigned long long t) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)t), hi = __builtin_amdgcn_readfirstlane((uint32_t)(t >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Sequence and chunk of a unit: a class hands its sequences' units out chunk by chunk.
struct SeqChunk {
  int64_t seq, chunk;
};
__device__ __forceinline__ SeqChunk unit_seq_chunk(unsigned long long t, uint32_t n_seq) {
  const uint32_t x = (uint32_t)(t >> 32), m = (uint32_t)t;
  const uint32_t n = class_seqs(n_seq, x);
  const uint32_t c = m / n;
  return SeqChunk{(int64_t)x + (int64_t)kTicketClasses * (m - c * n), (int64_t)c};
}

__device__ __forceinline__ uint32_t launch_epoch(LookbackCtl* ctl) {
  return (uint32_t)(__hip_atomic_load(&ctl->tick, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) + 1u;
}

// Thread 0 of every workgroup, once, after its last unit.  The last workgroup of each home class
// reports to done_all; the last of those resets every counter and publishes the launch count E (all
// workgroups have then taken their last ticket).
__device__ void finish_launch(LookbackCtl* ctl, uint32_t E) {
  const int h = (int)(blockIdx.x % kTicketClasses);
  const unsigned int n_home = (gridDim.x - 1 - h) / kTicketClasses + 1;
  if (atomicAdd(&ctl->cls[h].done, 1u) != n_home - 1) return;
  __hip_atomic_store(&ctl->cls[h].done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned int homes = gridDim.x < (unsigned)kTicketClasses ? gridDim.x : (unsigned)kTicketClasses;
  if (atomicAdd(&ctl->done_all, 1u) != homes - 1) return;
  for (int x = 0; x < kTicketClasses; ++x)
    __hip_atomic_store(&ctl->cls[x].next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&ctl->done_all, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&ctl->tick, (unsigned long long)E << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ work units and loads
// Raw inputs of one wave's kSteps steps (the loads of a unit, kept in flight until needed).
template <class Op, typename Tin, int V>
struct Raw {
  typename win<Tin, V, kStreaming>::raw v[Op::kIn][kSteps];
  float prm[V];  // the channels' parameters (Op::param)
};

struct Unit {
  int64_t c, b, k;
  int rows;  // valid steps in the chunk (kChunk except for a ragged last chunk)
};

// CLASSES: the ticket is (class << 32) | local ticket; otherwise units go chunk by chunk, all
// (batch row, tile) sequences of a chunk in turn.
template <bool CLASSES>
__device__ __forceinline__ Unit unit_of(const Scan1Params& p, unsigned long long ticket) {
  Unit u;
  if constexpr (CLASSES) {
    const SeqChunk sc = unit_seq_chunk(ticket, (uint32_t)(p.B * p.n_tiles));
    u.c = sc.chunk;
    u.b = sc.seq / p.n_tiles;
    u.k = sc.seq - u.b * p.n_tiles;
  } else {
    const int64_t per_round = p.B * p.n_tiles;
    u.c = (int64_t)ticket / per_round;
    const int64_t rr = (int64_t)ticket - u.c * per_round;
    u.b = rr / p.n_tiles;
    u.k = rr - u.b * p.n_tiles;
  }
  u.rows = (int)min<int64_t>(kChunk, p.L - u.c * kChunk);
  return u;
}

// Window over the unit's rows of a [B, L, D] array with elements of `es` bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_window(const Scan1Params& p, const Unit& u, const void* a,
                                                              int es) {
  const char* base = static_cast<const char*>(a) + ((u.b * p.L + u.c * kChunk) * p.D) * es;
  return make_window(base, (uint32_t)(u.rows * p.D * es));
}

// Issue the loads of unit u for this wave.  Lanes past D read channel D - V and steps past the
// chunk's valid rows read its last row: every offset stays inside the window (results unused).
template <class Op, typename Tin, int V>
__device__ __forceinline__ void fetch(const Scan1Params& p, const Unit& u, uint32_t lane_off, int wave,
                                      Raw<Op, Tin, V>& raw) {
  using LD = win<Tin, V, kStreaming>;
  constexpr int es = sizeof(Tin);
  __amdgpu_buffer_rsrc_t w[Op::kIn];
#pragma unroll
  for (int q = 0; q < Op::kIn; ++q) w[q] = unit_window(p, u, p.in[q], es);
  const uint32_t row_bytes = (uint32_t)(p.D * es);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const uint32_t ro = (uint32_t)min(wave * kSteps + s, u.rows - 1) * row_bytes;
#pragma unroll
    for (int q = 0; q < Op::kIn; ++q) raw.v[q][s] = LD::load(w[q], lane_off, ro);
  }
  const int64_t chl = lane_off / es;
#pragma unroll
  for (int v = 0; v < V; ++v) raw.prm[v] = Op::param(p, chl + v);
}

// The output gate of unit u for this wave (same clamping), loaded when the unit's carry is being
// resolved and consumed by its stores.
template <typename Tin, int V>
__device__ __forceinline__ void fetch_gate(const Scan1Params& p, const Unit& u, uint32_t lane_off, int wave,
                                           typename win<Tin, V, kStreaming>::raw (&g)[kSteps]) {
  constexpr int es = sizeof(Tin);
  const auto wg = unit_window(p, u, p.gate, es);
  const uint32_t row_bytes = (uint32_t)(p.D * es);
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    g[s] = win<Tin, V, kStreaming>::load(wg, lane_off, (uint32_t)min(wave * kSteps + s, u.rows - 1) * row_bytes);
}

// ------------------------------------------------------------------ chunk lookback
// Carry into chunk `cix` of one sequence of units (chunks of 64 steps, one channel per lane).
// Chunks form blocks of kBlock.  The carry into chunk cix is the inclusive state published by the
// last chunk of the previous block (`init` for the first block), followed by the aggregates of the
// earlier chunks of its own block, applied in chunk order: every carry is one fixed function of the
// inputs (bitwise reproducible), and the serial chain has n_chunks / kBlock links.  This chunk's
// aggregate (Ac, Bc) is published for its later block-mates and, at a block end, its inclusive
// state for the next block.  Words are (value, epoch) pairs; every wait is bounded, and a unit only
// waits on units with lower tickets, which are running or done.  Returns the carry; *incl receives
// the inclusive state.
template <class Op, int TW>
__device__ __forceinline__ float lookback_carry(LookbackCtl* ctl, unsigned long long* words, int64_t seq_unit,
                                                int64_t cix, int64_t n_chunks, int j, uint32_t E, const WaitCfg& wc,
                                                float Ac, float Bc, float init, float* incl) {
  unsigned long long* W = words + (seq_unit + cix) * 3 * TW;
  const int64_t base = (cix / kBlock) * kBlock;
  const int nprev = (int)(cix - base);  // aggregates of block-mates before cix
  const uint32_t Ew = E + wc.skew;      // the epoch accepted while waiting (E unless testing timeouts)
  if (cix + 1 < base + kBlock && cix + 1 < n_chunks) {
    word_store(&W[0 * TW + j], E, Ac);
    word_store(&W[1 * TW + j], E, Bc);
  }
  // words: [0] inclusive of chunk base-1 (if base > 0), then (a, b) of chunks base .. cix-1
  unsigned long long wd[1 + 2 * (kBlock - 1)];
  const unsigned long long* Wb = words + (seq_unit + base - 1) * 3 * TW;
  wd[0] = base > 0 ? word_load(&Wb[2 * TW + j]) : ((unsigned long long)Ew << 32);
#pragma unroll
  for (int q = 0; q < kBlock - 1; ++q) {
    const unsigned long long* Wq = words + (seq_unit + base + q) * 3 * TW;
    if (q < nprev) {
      wd[1 + 2 * q] = word_load(&Wq[0 * TW + j]);
      wd[2 + 2 * q] = word_load(&Wq[1 * TW + j]);
    } else {
      wd[1 + 2 * q] = wd[2 + 2 * q] = (unsigned long long)Ew << 32;
    }
  }
  unsigned int spins = 0;
  bool all;
  while (true) {
    all = word_ready(wd[0], Ew);
#pragma unroll
    for (int q = 0; q < 2 * (kBlock - 1); ++q) all = all && word_ready(wd[1 + q], Ew);
    if (all || spins >= wc.spin_limit) break;
    ++spins;
    __builtin_amdgcn_s_sleep(1);
    if (!word_ready(wd[0], Ew)) wd[0] = word_load(&Wb[2 * TW + j]);
#pragma unroll
    for (int q = 0; q < kBlock - 1; ++q) {
      const unsigned long long* Wq = words + (seq_unit + base + q) * 3 * TW;
      if (!word_ready(wd[1 + 2 * q], Ew)) wd[1 + 2 * q] = word_load(&Wq[0 * TW + j]);
      if (!word_ready(wd[2 + 2 * q], Ew)) wd[2 + 2 * q] = word_load(&Wq[1 * TW + j]);
    }
  }
  float hin = base > 0 ? word_value(wd[0]) : init;
#pragma unroll
  for (int q = 0; q < kBlock - 1; ++q)
    if (q < nprev) hin = Op::apply(word_value(wd[1 + 2 * q]), word_value(wd[2 + 2 * q]), hin);
  if (!all) {  // the wait gave up: record it, and hand on NaN rather than a carry built from stale words
    atomicOr(&ctl->error, 1u);
    hin = __builtin_nanf("");
  }
  *incl = Op::apply(Ac, Bc, hin);
  if (cix == base + kBlock - 1 && cix + 1 < n_chunks) word_store(&W[2 * TW + j], E, *incl);
  return hin;
}

// ------------------------------------------------------------------ the scan kernel
// Persistent workgroups: each takes tickets (work units) until none are left.  For unit t it
//   1. folds the raw inputs of t (loaded earlier) into step pairs and wave aggregates,
//   2. issues the loads of its next unit, so they are in flight during the lookback of t,
//   3. resolves the carry of t (waves 0 .. V-1), then re-runs the recurrence and stores y.
// The next ticket is requested one unit ahead, so its latency is hidden too.
// Occupancy hint: with bf16 inputs the kernel fits 3 workgroups per SIMD group without spills.
template <typename Tin> constexpr int waves_per_eu() { return sizeof(Tin) == 2 ? 3 : 1; }

// RECORD: a pass that stores no outputs and records the state entering every chunk (carry_out).
template <class Op, typename Tin, typename Tout, int V, bool GATE, bool RECORD>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(waves_per_eu<Tin>())))
void scan1_kernel(Scan1Params p) {
  constexpr int TW = 64 * V;  // channels per tile
  __shared__ unsigned long long s_tick[2];
  __shared__ uint32_t s_epoch;
  __shared__ float s_aggA[kWaves][TW];
  __shared__ float s_aggB[kWaves][TW];
  __shared__ float s_carry[TW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  using LD = win<Tin, V, kStreaming>;

  // Tickets: the output pass, whose units are long, draws them from the single counter; the record
  // pass, with short units, from the ticket classes.
  constexpr bool CLS = RECORD;
  const int64_t total = p.B * p.n_tiles * p.n_chunks;
  const uint32_t n_seq = (uint32_t)(p.B * p.n_tiles);
  auto unit_ticket = [&](unsigned long long t) -> unsigned long long {
    if constexpr (CLS) return uniform_ticket(t);
    const int64_t q = (int64_t)(t & 0xffffffffull);
    return q < total ? (unsigned long long)q : kNoUnit;
  };
  int xc = (int)(blockIdx.x % kTicketClasses), left = kTicketClasses;  // class cursor (thread 0)
  if (threadIdx.x == 0) {
    if constexpr (CLS) {
      s_epoch = launch_epoch(p.ctl);
      s_tick[0] = take_unit(p.ctl, n_seq, (uint32_t)p.n_chunks, xc, left);
    } else {
      s_tick[0] = atomicAdd(&p.ctl->tick, 1ull);
    }
  }
  __syncthreads();
  // epoch carried by this launch's words
  const uint32_t E = CLS ? __builtin_amdgcn_readfirstlane(s_epoch) : (uint32_t)(s_tick[0] >> 32) + 1u;
  unsigned long long ticket = unit_ticket(s_tick[0]);
  Raw<Op, Tin, V> raw;
  // The lane's channels within a tile are the same for every unit; the tile base moves.
  auto lane_off_of = [&](const Unit& u) -> uint32_t {
    const int64_t ch0 = u.k * TW + (int64_t)lane * V;
    return (uint32_t)(min<int64_t>(ch0, p.D - V) * (int64_t)sizeof(Tin));
  };
  if (ticket != kNoUnit) {
    const Unit u0 = unit_of<CLS>(p, ticket);
    fetch<Op, Tin, V>(p, u0, lane_off_of(u0), wave, raw);
  }
  int parity = 0;

  while (ticket != kNoUnit) {
    const Unit u = unit_of<CLS>(p, ticket);
    uint32_t m_next = 0;  // next ticket, one unit ahead (thread 0)
    if (threadIdx.x == 0) {
      if constexpr (CLS) m_next = take_begin(p.ctl, xc, left);
      else s_tick[parity ^ 1] = atomicAdd(&p.ctl->tick, 1ull);
    }
    const int64_t ch0 = u.k * TW + (int64_t)lane * V;
    const bool ch_ok = ch0 < p.D;  // V = 2 only when D is even
    const int64_t chl = ch_ok ? ch0 : p.D - V;
    const int64_t t0 = u.c * kChunk + (int64_t)wave * kSteps;  // first step of this wave

    // ---- step pairs and the wave's aggregate
    typename Op::Chan cc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) cc[v] = Op::chan(p, raw.prm[v]);
    float av[kSteps][V], bv[kSteps][V];
    float Ag[V], Bg[V];
#pragma unroll
    for (int v = 0; v < V; ++v) { Ag[v] = Op::id_a(); Bg[v] = Op::id_b(); }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bool ok = ch_ok && (t0 + s < p.L);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float in[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < Op::kIn; ++q) in[q] = LD::get(raw.v[q][s], v);
        float a, bb;
        Op::step(in, cc[v], a, bb);
        a = ok ? a : Op::id_a();  // steps past L and idle lanes are the identity map
        bb = ok ? bb : Op::id_b();
        av[s][v] = a;
        bv[s][v] = bb;
        Bg[v] = Op::apply(a, bb, Bg[v]);
        Ag[v] = Op::fold_a(a, Ag[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      s_aggA[wave][lane * V + v] = Ag[v];
      s_aggB[wave][lane * V + v] = Bg[v];
    }
    if constexpr (CLS)
      if (threadIdx.x == 0) s_tick[parity ^ 1] = take_end(p.ctl, n_seq, (uint32_t)p.n_chunks, xc, left, m_next);
    __syncthreads();  // aggregates in LDS; the next ticket is visible
    const unsigned long long next = unit_ticket(s_tick[parity ^ 1]);
    if (next != kNoUnit) {  // in flight during the lookback
      const Unit un = unit_of<CLS>(p, next);
      fetch<Op, Tin, V>(p, un, lane_off_of(un), wave, raw);
    }
    typename LD::raw graw[GATE ? kSteps : 1];
    if constexpr (GATE) fetch_gate<Tin, V>(p, u, lane_off_of(u), wave, graw);

    // ---- waves 0 .. V-1: chunk aggregate, publish, carry-in, inclusive (64 of the tile's
    //      channels per wave, one per lane)
    if (wave < V) {
      const int64_t seq_unit = (u.b * p.n_tiles + u.k) * p.n_chunks;
      const int j = wave * 64 + lane;
      const int64_t ch = u.k * TW + j;
      const bool j_ok = ch < p.D;
      float Ac = Op::id_a(), Bc = Op::id_b();
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        Bc = Op::apply(s_aggA[w][j], s_aggB[w][j], Bc);
        Ac = Op::fold_a(s_aggA[w][j], Ac);
      }
      const float init = p.h0 ? p.h0[u.b * p.D + (j_ok ? ch : p.D - 1)] : 0.0f;
      float incl;
      const float hin = lookback_carry<Op, TW>(p.ctl, p.words, seq_unit, u.c, p.n_chunks, j, E, p.wait, Ac, Bc, init, &incl);
      if (p.h_last && j_ok && u.c == p.n_chunks - 1) p.h_last[u.b * p.D + ch] = incl;
      if ((RECORD || p.carry_out) && j_ok) p.carry_out[(u.b * p.n_chunks + u.c) * p.D + ch] = hin;
      s_carry[j] = hin;
    }
    __syncthreads();

    // ---- carry into this wave, re-run the recurrence, store
    float h[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int j = lane * V + v;
      float hv = s_carry[j];
      for (int w = 0; w < wave; ++w) hv = Op::apply(s_aggA[w][j], s_aggB[w][j], hv);
      h[v] = hv;
    }
    if (!RECORD) {
      const auto wy = unit_window(p, u, p.y, (int)sizeof(Tout));
      const uint32_t row_bytes = (uint32_t)(p.D * (int64_t)sizeof(Tout));
      const uint32_t lo = (uint32_t)(chl * (int64_t)sizeof(Tout));
      const int nvalid = u.rows - wave * kSteps;  // rows of this wave inside the chunk
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        float out[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          h[v] = Op::apply(av[s][v], bv[s][v], h[v]);
          out[v] = GATE ? Op::gated(h[v], LD::get(graw[GATE ? s : 0], v)) : h[v];
        }
        if (ch_ok && s < nvalid)
          win<Tout, V, kStreaming>::store(wy, lo, (uint32_t)(wave * kSteps + s) * row_bytes, out);
      }
    }
    __syncthreads();  // LDS (aggregates, carry, ticket slot) is reused by the next unit
    ticket = next;
    parity ^= 1;
  }

  // ---- the last workgroup to finish resets the counters and advances the launch count
  if (CLS && threadIdx.x == 0) finish_launch(p.ctl, E);
  if (!CLS && threadIdx.x == 0) {
    const unsigned int old = atomicAdd(&p.ctl->done, 1u);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(&p.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.ctl->tick, (unsigned long long)E << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ short sequences
// L <= NW * SPW: one workgroup of NW waves per (batch row, tile of 64 channels, one per lane) covers
// every step at once (wave w owns steps [SPW w, SPW w + SPW)); the wave aggregates meet in LDS and
// each wave starts from h0 folded through the aggregates of the waves before it.  No tickets, no
// lookback, no workspace traffic: the whole scan is one round of loads, the combine and the stores,
// with few steps per lane so that the dependent chain of each lane stays short.
constexpr int kShortSpw = 8;  // steps per wave
template <class Op, typename Tin, typename Tout, bool GATE, int NW>
__global__ __launch_bounds__(NW * 64) void scan1_short_kernel(Scan1Params p) {
  constexpr int SPW = kShortSpw;
  __shared__ float s_aggA[NW][64];
  __shared__ float s_aggB[NW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  using LD = win<Tin, 1, kStreaming>;
  const int64_t n_tiles = (p.D + 63) / 64;
  const int64_t b = blockIdx.x / n_tiles;
  const int64_t ch0 = (blockIdx.x - b * n_tiles) * 64 + lane;
  const bool ch_ok = ch0 < p.D;
  const int64_t chl = ch_ok ? ch0 : p.D - 1;
  const uint32_t lo_in = (uint32_t)(chl * (int64_t)sizeof(Tin));
  const uint32_t rows_in = (uint32_t)(p.D * (int64_t)sizeof(Tin));
  const int t0 = wave * SPW;
  const int last = (int)p.L - 1;
  typename LD::raw raw[Op::kIn][SPW];
  typename LD::raw graw[GATE ? SPW : 1];
  {
    __amdgpu_buffer_rsrc_t w[Op::kIn];
#pragma unroll
    for (int q = 0; q < Op::kIn; ++q)
      w[q] = make_window(static_cast<const char*>(p.in[q]) + b * p.L * p.D * (int64_t)sizeof(Tin), (uint32_t)(p.L * rows_in));
    const auto wg = make_window(static_cast<const char*>(GATE ? p.gate : p.in[0]) + b * p.L * p.D * (int64_t)sizeof(Tin),
                                (uint32_t)(p.L * rows_in));
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      const uint32_t ro = (uint32_t)min(t0 + st, last) * rows_in;  // steps past L read the last row
#pragma unroll
      for (int q = 0; q < Op::kIn; ++q) raw[q][st] = LD::load(w[q], lo_in, ro);
      if (GATE) graw[st] = LD::load(wg, lo_in, ro);
    }
  }
  const typename Op::Chan cc = Op::chan(p, Op::param(p, chl));
  float av[SPW], bv[SPW], Ag = Op::id_a(), Bg = Op::id_b();
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    const bool ok = t0 + st < p.L;
    float in[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < Op::kIn; ++q) in[q] = LD::get(raw[q][st], 0);
    float a, bb;
    Op::step(in, cc, a, bb);
    av[st] = ok ? a : Op::id_a();  // steps past L are the identity map
    bv[st] = ok ? bb : Op::id_b();
    Bg = Op::apply(av[st], bv[st], Bg);
    Ag = Op::fold_a(av[st], Ag);
  }
  s_aggA[wave][lane] = Ag;
  s_aggB[wave][lane] = Bg;
  __syncthreads();
  float h = p.h0 ? p.h0[b * p.D + chl] : 0.0f;
  for (int w = 0; w < wave; ++w) h = Op::apply(s_aggA[w][lane], s_aggB[w][lane], h);
  // the state entering each 64-step chunk is the carry of the wave that starts it
  if (p.carry_out && ch_ok && (t0 % kChunk) == 0 && t0 < p.L) p.carry_out[(b * p.n_chunks + t0 / kChunk) * p.D + ch0] = h;
  const auto wy = make_window(static_cast<char*>(p.y) + b * p.L * p.D * (int64_t)sizeof(Tout),
                              (uint32_t)(p.L * p.D * (int64_t)sizeof(Tout)));
  const uint32_t lo_out = (uint32_t)(chl * (int64_t)sizeof(Tout)), rows_out = (uint32_t)(p.D * (int64_t)sizeof(Tout));
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    h = Op::apply(av[st], bv[st], h);
    const float out = GATE ? Op::gated(h, LD::get(graw[GATE ? st : 0], 0)) : h;
    if (ch_ok && t0 + st < p.L) win<Tout, 1, kStreaming>::store(wy, lo_out, (uint32_t)(t0 + st) * rows_out, &out);
  }
  // steps past L are identities, so the last wave ends holding h_L
  if (p.h_last && ch_ok && wave == NW - 1) p.h_last[b * p.D + ch0] = h;
}

// ------------------------------------------------------------------ decode steps
struct Upd1Params {
  int64_t B, D;
  const void* in[3];
  const void* gate;
  const float* a_log;
  float c;
  float* state;
  void* y;
};

template <class Op, typename Tin, typename Tout, bool GATE>
__global__ __launch_bounds__(256) void update1_kernel(Upd1Params p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.B * p.D) return;
  const int64_t d = idx % p.D;
  Scan1Params q{};
  q.a_log = p.a_log;
  q.c = p.c;
  float in[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < Op::kIn; ++k) in[k] = io<Tin>::load(p.in[k], idx);
  float a, b;
  Op::step(in, Op::chan(q, Op::param(q, d)), a, b);
  const float h = Op::apply(a, b, p.state[idx]);
  p.state[idx] = h;
  io<Tout>::store(p.y, idx, GATE ? Op::gated(h, io<Tin>::load(p.gate, idx)) : h);
}

// Decode step with V consecutive channels per vector and U vectors per lane (D a multiple of V,
// every operand under 2^31 bytes): x / r / i / gate, the state and y go through buffer windows with
// 32-bit offsets, one 2V- or 4V-byte access per operand and vector; the channel parameters come in
// one access as well.  All loads of a lane are issued before any arithmetic: a decode step is one
// round trip to memory.
constexpr unsigned kUpdThreads = 128;  // workgroup size of the vector decode step (see launch_update_v)
template <class Op, typename Tin, typename Tout, bool GATE, int V, int U>
__global__ __launch_bounds__(kUpdThreads) void update1v_kernel(Upd1Params p) {
  const uint32_t n = (uint32_t)(p.B * p.D / V);  // vectors of V channels
  const uint32_t per_row = (uint32_t)(p.D / V);
  const uint32_t elems = (uint32_t)(p.B * p.D);
  Scan1Params q{};
  q.a_log = p.a_log;
  q.c = p.c;
  using Wi = win<Tin, V, kStreaming>;  // this step's inputs and output are touched once
  using Wf = win<float, V>;            // the state is read again by the next step
  __amdgpu_buffer_rsrc_t win_in[3];
#pragma unroll
  for (int k = 0; k < Op::kIn; ++k) win_in[k] = make_window(p.in[k], elems * sizeof(Tin));
  const auto wgt = make_window(GATE ? p.gate : p.in[0], elems * sizeof(Tin));
  const auto ws = make_window(p.state, elems * sizeof(float));
  const auto wa = make_window(p.a_log ? p.a_log : p.state, (uint32_t)(p.D * sizeof(float)));
  uint32_t g[U];
  typename Wi::raw rin[U][3], rg[U];
  typename Wf::raw rs[U], ra[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    g[u] = blockIdx.x * (kUpdThreads * U) + u * kUpdThreads + threadIdx.x;
    const uint32_t gc = g[u] < n ? g[u] : n - 1;  // lanes past the end reread the last vector
    const uint32_t d0 = (gc % per_row) * V;
#pragma unroll
    for (int k = 0; k < Op::kIn; ++k) rin[u][k] = Wi::load(win_in[k], gc * V * sizeof(Tin), 0);
    if (GATE) rg[u] = Wi::load(wgt, gc * V * sizeof(Tin), 0);
    rs[u] = Wf::load(ws, gc * V * sizeof(float), 0);
    if (p.a_log) ra[u] = Wf::load(wa, d0 * sizeof(float), 0);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float h[V], y[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float in[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < Op::kIn; ++k) in[k] = Wi::get(rin[u][k], v);
      float a, b;
      Op::step(in, Op::chan(q, p.a_log ? Wf::get(ra[u], v) : 0.0f), a, b);
      h[v] = Op::apply(a, b, Wf::get(rs[u], v));
      y[v] = GATE ? Op::gated(h[v], Wi::get(rg[u], v)) : h[v];
    }
    if (g[u] < n) {
      Wf::store(ws, g[u] * V * sizeof(float), 0, h);
      win<Tout, V, kStreaming>::store(make_window(p.y, elems * sizeof(Tout)), g[u] * V * sizeof(Tout), 0, y);
    }
  }
}

// ------------------------------------------------------------------ RG-LRU backward
// Reverse-time adjoint of the affine recurrence (the gradient of  sum dy y + sum dh_last h_last).
// With e_t = dy_t G_t (G_t = gelu(gate_t), or 1) and q_t the gradient leaving step t towards
// h_{t-1}:  g_t = dL/dh_t = e_t + q_{t+1},  q_t = a_t g_t,  q_L = dh_last.  So q runs backwards
// through the affine maps q -> a_t q + a_t e_t: the chunked lookback applies unchanged with the
// chunks taken in reverse order.  Per step, with h_{t-1} recomputed forward inside the chunk from
// the chunk's carry-in (recorded by a forward pass), l = log a = c r a_log and b = beta i x:
//   dx = g beta i,  d i_logit = g beta x i (1 - i),  dl = g h_{t-1} a - g (i x) a^2 / beta,
//   d r_logit = dl c a_log r (1 - r),  d a_log += dl c r,  d gate = dy h_t gelu'(gate),
//   and dh0 = q_0.
// Work units are (batch row, tile of 64 V channels, chunk), one channel pair per lane, 8 waves x 8
// steps; a resident grid takes them from the ticket classes, chunks in reverse order.
struct Bwd1Params {
  int64_t B, L, D;
  int64_t n_tiles, n_chunks;
  const void* x;
  const void* r;
  const void* i;
  const void* gate;   // or NULL
  const void* dy;
  const float* a_log;
  float c;
  const float* carry;    // [B][n_chunks][D] forward state entering each chunk
  const float* dh_last;  // [B][D] or NULL
  void* dx;
  void* dr;
  void* di;
  void* dgate;           // or NULL
  float* dalog_part;     // [B][n_chunks][D]: per-unit partial sums of d a_log
  float* dh0;            // [B][D] or NULL
  LookbackCtl* ctl;
  unsigned long long* words;
  WaitCfg wait;
};

// gelu'(v) = Phi(v) + v phi(v), with Phi through the same erf as gelu_f.
__device__ __forceinline__ float gelu_grad_f(float v) {
  const float x = fabsf(v) * 0.70710678118654752f;
  const float t = hw_rcp(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  const float ex = hw_exp2(-(x * x) * kLog2e);  // e^(-v^2/2)
  const float q = poly * t * ex;                // 1 - erf(|v| / sqrt 2)
  const float Phi = 0.5f * (v >= 0.0f ? 2.0f - q : q);
  return Phi + v * (0.3989422804014327f * ex);  // phi(v) = e^(-v^2/2) / sqrt(2 pi)
}

constexpr int kBWaves = 8;                 // waves of a backward workgroup
constexpr int kBSteps = kChunk / kBWaves;  // steps per wave

template <typename Tin, typename Tout, int V, bool GATE>
__global__ __launch_bounds__(kBWaves * 64) void rglru_bwd_kernel(Bwd1Params p) {
  constexpr int TW = 64 * V;  // channels per tile
  __shared__ unsigned long long s_tick[2];
  __shared__ uint32_t s_epoch;
  __shared__ float s_fA[kBWaves][TW], s_fB[kBWaves][TW];  // forward wave aggregates
  __shared__ float s_rA[kBWaves][TW], s_rB[kBWaves][TW];  // reverse wave aggregates
  __shared__ float s_qin[TW];
  __shared__ float s_dal[kBWaves][TW];
  using LD = win<Tin, V, kStreaming>;
  using ST = win<Tout, V, kStreaming>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int xc = (int)(blockIdx.x % kTicketClasses), left = kTicketClasses;  // ticket cursor (thread 0)
  const uint32_t n_seq = (uint32_t)(p.B * p.n_tiles);
  if (threadIdx.x == 0) {
    s_epoch = launch_epoch(p.ctl);
    s_tick[0] = take_unit(p.ctl, n_seq, (uint32_t)p.n_chunks, xc, left);
  }
  __syncthreads();
  const uint32_t E = __builtin_amdgcn_readfirstlane(s_epoch);
  constexpr int es = sizeof(Tin);
  const uint32_t row_in = (uint32_t)(p.D * es);
  // Geometry of a unit (its reverse and forward chunk index, batch row, tile and rows) and the
  // window over its rows of one [B, L, D] array with e-byte elements.
  struct G {
    int64_t cr, c, b, k;
    int rows;
  };
  auto geom = [&](unsigned long long t) {
    const SeqChunk sc = unit_seq_chunk(t, n_seq);
    G g;
    g.cr = sc.chunk;
    g.c = p.n_chunks - 1 - g.cr;
    g.b = sc.seq / p.n_tiles;
    g.k = sc.seq - g.b * p.n_tiles;
    g.rows = (int)min<int64_t>(kChunk, p.L - g.c * kChunk);
    return g;
  };
  auto window_of = [&](const G& g, const void* a, int e) {
    return make_window(static_cast<const char*>(a) + ((g.b * p.L + g.c * kChunk) * p.D) * e, (uint32_t)(g.rows * p.D * e));
  };
  // Loads of a unit's x, r, i and dy rows (rows past the chunk read its last row; results unused).
  // Without an output gate the next unit's rows are loaded while this unit resolves its carry and
  // writes its gradients (PREFETCH); with one, the registers are not there and each unit loads its
  // own rows first.
  constexpr bool PREFETCH = !GATE;
  typedef typename LD::raw Raw4[4][kBSteps];
  auto fetch4 = [&](unsigned long long t, Raw4& r4) {
    const G g = geom(t);
    const int64_t c0 = g.k * TW + (int64_t)lane * V;
    const uint32_t li = (uint32_t)((c0 < p.D ? c0 : p.D - V) * es);
    const auto w0 = window_of(g, p.x, es), w1 = window_of(g, p.r, es), w2 = window_of(g, p.i, es),
               w3 = window_of(g, p.dy, es);
  #pragma unroll
    for (int s = 0; s < kBSteps; ++s) {
      const uint32_t ro = (uint32_t)min(wave * kBSteps + s, g.rows - 1) * row_in;
      r4[0][s] = LD::load(w0, li, ro);
      r4[1][s] = LD::load(w1, li, ro);
      r4[2][s] = LD::load(w2, li, ro);
      r4[3][s] = LD::load(w3, li, ro);
    }
  };
  Raw4 cur, nxt;
  unsigned long long ticket = uniform_ticket(s_tick[0]);
  if (ticket != kNoUnit) fetch4(ticket, cur);
  for (int parity = 0; ticket != kNoUnit; parity ^= 1) {
    const G gu = geom(ticket);
    const int64_t cr = gu.cr, c = gu.c, b = gu.b, k = gu.k;
    const int rows = gu.rows;
    const int64_t ch0 = k * TW + (int64_t)lane * V;
    const bool ch_ok = ch0 < p.D;  // V = 2 only when D is even
    const int64_t chl = ch_ok ? ch0 : p.D - V;
    const int64_t t0 = c * kChunk + (int64_t)wave * kBSteps;
    const int nvalid = rows - wave * kBSteps;
    auto window = [&](const void* a, int e) { return window_of(gu, a, e); };
    const uint32_t lane_in = (uint32_t)(chl * es);
    typename LD::raw(&rx)[kBSteps] = cur[0];
    typename LD::raw(&rrl)[kBSteps] = cur[1];
    typename LD::raw(&ril)[kBSteps] = cur[2];
    typename LD::raw(&rdy)[kBSteps] = cur[3];
    typename LD::raw rg[GATE ? kBSteps : 1];
    if (GATE) {
      const auto wg = window(p.gate, es);
  #pragma unroll
      for (int s = 0; s < kBSteps; ++s)
        rg[GATE ? s : 0] = LD::load(wg, lane_in, (uint32_t)min(wave * kBSteps + s, rows - 1) * row_in);
    }
    uint32_t m_next = 0;  // next unit, one ahead (thread 0; resolved before the first barrier)
    if (threadIdx.x == 0) m_next = take_begin(p.ctl, xc, left);
    float kc[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) kc[v] = p.c * p.a_log[chl + v] * kLog2e;

    // ---- forward pairs (keeping the gates r, i and beta for the gradients), reverse pairs, and
    //      both wave aggregates
    float av[kBSteps][V], bv[kBSteps][V], ev[kBSteps][V], rv[kBSteps][V], iv[kBSteps][V], btv[kBSteps][V];
    float fA[V], fB[V], rA[V], rB[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) { fA[v] = 1.0f; fB[v] = 0.0f; rA[v] = 1.0f; rB[v] = 0.0f; }
  #pragma unroll
    for (int s = 0; s < kBSteps; ++s) {
      const bool ok = ch_ok && (t0 + s < p.L);
  #pragma unroll
      for (int v = 0; v < V; ++v) {
        // AffineOp::step, with its intermediates kept
        const float r = sigmoid_f(LD::get(rrl[s], v));
        const float i = sigmoid_f(LD::get(ril[s], v));
        const float l2 = kc[v] * r;
        const float a = hw_exp2(l2);
        const float beta = hw_sqrt(one_minus_a2(l2, a));
        const float bb = beta * (i * LD::get(rx[s], v));
        rv[s][v] = r;
        iv[s][v] = i;
        btv[s][v] = beta;
        const float G = GATE ? gelu_f(LD::get(rg[GATE ? s : 0], v)) : 1.0f;
        av[s][v] = ok ? a : 1.0f;
        bv[s][v] = ok ? bb : 0.0f;
        ev[s][v] = ok ? LD::get(rdy[s], v) * G : 0.0f;
        fB[v] = fmaf(av[s][v], fB[v], bv[s][v]);
        fA[v] *= av[s][v];
      }
    }
  #pragma unroll
    for (int s = kBSteps - 1; s >= 0; --s)
  #pragma unroll
      for (int v = 0; v < V; ++v) {
        rB[v] = fmaf(av[s][v], rB[v], av[s][v] * ev[s][v]);
        rA[v] *= av[s][v];
      }
  #pragma unroll
    for (int v = 0; v < V; ++v) {
      s_fA[wave][lane * V + v] = fA[v];
      s_fB[wave][lane * V + v] = fB[v];
      s_rA[wave][lane * V + v] = rA[v];
      s_rB[wave][lane * V + v] = rB[v];
    }
    if (threadIdx.x == 0) s_tick[parity ^ 1] = take_end(p.ctl, n_seq, (uint32_t)p.n_chunks, xc, left, m_next);
    __syncthreads();  // wave aggregates in LDS; the next ticket is visible
    const unsigned long long next = uniform_ticket(s_tick[parity ^ 1]);
    if (PREFETCH && next != kNoUnit) fetch4(next, nxt);  // in flight during this unit's lookback and stores

    // ---- waves 0 .. V-1: chunk reverse aggregate, publish, reverse carry (lookback over later
    //      chunks), one channel of the tile per lane
    if (wave < V) {
      const int j = wave * 64 + lane;
      const int64_t seq_unit = (b * p.n_tiles + k) * p.n_chunks;
      float Ac = 1.0f, Bc = 0.0f;
  #pragma unroll
      for (int w = kBWaves - 1; w >= 0; --w) {
        Bc = fmaf(s_rA[w][j], Bc, s_rB[w][j]);
        Ac *= s_rA[w][j];
      }
      const int64_t chj = k * TW + j;
      const float init = p.dh_last ? p.dh_last[b * p.D + (chj < p.D ? chj : p.D - 1)] : 0.0f;
      float incl;
      s_qin[j] = lookback_carry<AffineOp, TW>(p.ctl, p.words, seq_unit, cr, p.n_chunks, j, E, p.wait, Ac, Bc, init, &incl);
    }
    __syncthreads();

    // ---- forward states entering each step of this wave, and the reverse carry into it
    float hp[kBSteps][V], q[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) {
      const int j = lane * V + v;
      float h = p.carry[(b * p.n_chunks + c) * p.D + chl + v];
      for (int w = 0; w < wave; ++w) h = fmaf(s_fA[w][j], h, s_fB[w][j]);
  #pragma unroll
      for (int s = 0; s < kBSteps; ++s) {
        hp[s][v] = h;
        h = fmaf(av[s][v], h, bv[s][v]);
      }
      float qq = s_qin[j];
      for (int w = kBWaves - 1; w > wave; --w) qq = fmaf(s_rA[w][j], qq, s_rB[w][j]);
      q[v] = qq;
    }
    // ---- per-step gradients, last step first
    const auto wdx = window(p.dx, (int)sizeof(Tout)), wdr = window(p.dr, (int)sizeof(Tout));
    const auto wdi = window(p.di, (int)sizeof(Tout)), wdg = window(GATE && p.dgate ? p.dgate : p.dx, (int)sizeof(Tout));
    const uint32_t row_out = (uint32_t)(p.D * (int64_t)sizeof(Tout)), lane_out = (uint32_t)(chl * (int64_t)sizeof(Tout));
    float ca[V], dal[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) { ca[v] = p.c * p.a_log[chl + v]; dal[v] = 0.0f; }
  #pragma unroll
    for (int s = kBSteps - 1; s >= 0; --s) {
      float o_dx[V], o_dr[V], o_di[V], o_dg[V];
  #pragma unroll
      for (int v = 0; v < V; ++v) {
        const float g = ev[s][v] + q[v];
        q[v] = av[s][v] * g;
        const float xx = LD::get(rx[s], v);
        const float r = rv[s][v], i = iv[s][v], beta = btv[s][v];
        const float a = av[s][v];
        const float gb = g * beta;
        const float dl = g * a * (hp[s][v] - (i * xx) * a * hw_rcp(beta));
        o_dx[v] = gb * i;
        o_di[v] = gb * xx * i * (1.0f - i);
        o_dr[v] = dl * ca[v] * r * (1.0f - r);
        if (s < nvalid) dal[v] = fmaf(dl * p.c, r, dal[v]);
        if (GATE) o_dg[v] = LD::get(rdy[s], v) * fmaf(a, hp[s][v], bv[s][v]) * gelu_grad_f(LD::get(rg[GATE ? s : 0], v));
      }
      if (ch_ok && s < nvalid) {
        const uint32_t ro = (uint32_t)(wave * kBSteps + s) * row_out;
        ST::store(wdx, lane_out, ro, o_dx);
        ST::store(wdr, lane_out, ro, o_dr);
        ST::store(wdi, lane_out, ro, o_di);
        if (GATE && p.dgate) ST::store(wdg, lane_out, ro, o_dg);
      }
    }
    if (p.dh0 && ch_ok && c == 0 && wave == 0)
  #pragma unroll
      for (int v = 0; v < V; ++v) p.dh0[b * p.D + ch0 + v] = q[v];
  #pragma unroll
    for (int v = 0; v < V; ++v) s_dal[wave][lane * V + v] = ch_ok ? dal[v] : 0.0f;
    __syncthreads();
    if (wave < V) {
      const int j = wave * 64 + lane;
      const int64_t chj = k * TW + j;
      if (chj < p.D) {
        float acc = 0.0f;
  #pragma unroll
        for (int w = 0; w < kBWaves; ++w) acc += s_dal[w][j];
        p.dalog_part[(b * p.n_chunks + c) * p.D + chj] = acc;
      }
    }
    __syncthreads();  // this unit's LDS is free
    if (next != kNoUnit) {
      if (PREFETCH) {
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
  #pragma unroll
          for (int s = 0; s < kBSteps; ++s) cur[q4][s] = nxt[q4][s];
      } else {
        fetch4(next, cur);
      }
    }
    ticket = next;
  }
  if (threadIdx.x == 0) finish_launch(p.ctl, E);
}

// ------------------------------------------------------------------ MinMax backward
// Reverse-time adjoint of x_t = max(min(r_t, x_{t-1}), s_t), y_t = x_t (or x_t gate_t), for the loss
// sum dy y + sum dx_last x_last, with the derivative convention of torch.minimum / torch.maximum
// (the training framework of the minmaxrnc package): each operand receives the gradient when it is
// the selected one, half of it when the two are equal, and -- as those comparisons give -- all of
// it when either operand is NaN.  With m_t = min(r_t, x_{t-1}):
//   wR = [r < x] + [r == x]/2 (to r),  wX = [r > x] + [r == x]/2 (to x_{t-1}), and the same pair
//   wM (to m), wS (to s_t) for max(m, s_t), the NaN case giving 1 to both.
// g_t = e_t + q_{t+1} (e_t = dy_t gate_t, or dy_t), q_t = wM wX g_t, q_L = dx_last:
//   dr_t = g_t wM wR,  ds_t = g_t wS,  dgate_t = dy_t x_t,  dx0 = q_0.
// q runs backwards through affine maps q -> a'_t q + a'_t e_t whose coefficients a'_t = wM wX are
// in {0, 1/4, 1/2, 1} and depend on the forward state, so a unit first rebuilds the forward states
// of its chunk (from the carry recorded by a forward pass and the MinMax wave aggregates), then
// resolves the reverse carry with the affine lookback over chunks taken in reverse order.
struct MmBwdParams {
  int64_t B, L, D;
  int64_t n_tiles, n_chunks;
  const void* r;
  const void* s;
  const void* gate;      // or NULL
  const void* dy;
  const float* carry;    // [B][n_chunks][D] forward state entering each chunk
  const float* dx_last;  // [B][D] or NULL
  void* dr;
  void* ds;
  void* dgate;           // or NULL
  float* dx0;            // [B][D] or NULL
  LookbackCtl* ctl;
  unsigned long long* words;
  WaitCfg wait;
};

// d min(u, w) / du and d max(u, w) / du under the convention above.
__device__ __forceinline__ float sel_lo(float u, float w) { return u == w ? 0.5f : (u > w ? 0.0f : 1.0f); }
__device__ __forceinline__ float sel_hi(float u, float w) { return u == w ? 0.5f : (u < w ? 0.0f : 1.0f); }

// The step weights are products of {0, 1/2, 1}, i.e. {0, 1/4, 1/2, 1}: four times a weight is a
// byte, packed four to a register (one v_cvt_pk_u8_f32 to store, one v_cvt_f32_ubyte to read back).
template <int N>
struct Bytes4 {
  uint32_t u[(N + 3) / 4] = {};
  __device__ __forceinline__ void set(int i, float x4) { u[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(x4, i & 3, u[i >> 2]); }
  __device__ __forceinline__ float get(int i) const { return (float)((u[i >> 2] >> (8 * (i & 3))) & 0xffu); }
};

template <typename Tin, typename Tout, int V, bool GATE>
__global__ __launch_bounds__(kBWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void minmax_bwd_kernel(MmBwdParams p) {
  constexpr int TW = 64 * V;  // channels per tile
  __shared__ unsigned long long s_tick[2];
  __shared__ uint32_t s_epoch;
  __shared__ float s_fA[kBWaves][TW], s_fB[kBWaves][TW];  // forward wave aggregates
  __shared__ float s_rA[kBWaves][TW], s_rB[kBWaves][TW];  // reverse wave aggregates
  __shared__ float s_qin[TW];
  using LD = win<Tin, V, kStreaming>;
  using ST = win<Tout, V, kStreaming>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int xc = (int)(blockIdx.x % kTicketClasses), left = kTicketClasses;  // ticket cursor (thread 0)
  const uint32_t n_seq = (uint32_t)(p.B * p.n_tiles);
  if (threadIdx.x == 0) {
    s_epoch = launch_epoch(p.ctl);
    s_tick[0] = take_unit(p.ctl, n_seq, (uint32_t)p.n_chunks, xc, left);
  }
  __syncthreads();
  const uint32_t E = __builtin_amdgcn_readfirstlane(s_epoch);
  for (int parity = 0;; parity ^= 1) {
    const unsigned long long ticket = uniform_ticket(s_tick[parity]);
    if (ticket == kNoUnit) break;
    const SeqChunk sc = unit_seq_chunk(ticket, n_seq);
    const int64_t cr = sc.chunk;  // reverse chunk index
    const int64_t c = p.n_chunks - 1 - cr;
    const int64_t b = sc.seq / p.n_tiles, k = sc.seq - b * p.n_tiles;
    const int rows = (int)min<int64_t>(kChunk, p.L - c * kChunk);
    const int64_t ch0 = k * TW + (int64_t)lane * V;
    const bool ch_ok = ch0 < p.D;  // V = 2 only when D is even
    const int64_t chl = ch_ok ? ch0 : p.D - V;
    const int64_t t0 = c * kChunk + (int64_t)wave * kBSteps;
    const int nvalid = rows - wave * kBSteps;

    // ---- loads of the unit's rows (rows past the chunk read its last row; results unused)
    constexpr int es = sizeof(Tin);
    auto window = [&](const void* a, int e) {
      return make_window(static_cast<const char*>(a) + ((b * p.L + c * kChunk) * p.D) * e, (uint32_t)(rows * p.D * e));
    };
    const auto wr = window(p.r, es), ws = window(p.s, es), wd = window(p.dy, es);
    const auto wg = window(GATE ? p.gate : p.r, es);
    const uint32_t row_in = (uint32_t)(p.D * es), lane_in = (uint32_t)(chl * es);
    typename LD::raw raw_r[kBSteps], raw_s[kBSteps], rdy[kBSteps], rg[GATE ? kBSteps : 1];
  #pragma unroll
    for (int s = 0; s < kBSteps; ++s) {
      const uint32_t ro = (uint32_t)min(wave * kBSteps + s, rows - 1) * row_in;
      raw_r[s] = LD::load(wr, lane_in, ro);
      raw_s[s] = LD::load(ws, lane_in, ro);
      rdy[s] = LD::load(wd, lane_in, ro);
    }
    uint32_t m_next = 0;  // next unit, one ahead (thread 0; resolved at the end of this unit)
    if (threadIdx.x == 0) m_next = take_begin(p.ctl, xc, left);
    float hc[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) hc[v] = p.carry[(b * p.n_chunks + c) * p.D + chl + v];

    // ---- forward maps (identity past L and on idle lanes) and the wave's forward aggregate
    float av[kBSteps][V], bv[kBSteps][V];
    float fA[V], fB[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) { fA[v] = MinMaxOp::id_a(); fB[v] = MinMaxOp::id_b(); }
  #pragma unroll
    for (int s = 0; s < kBSteps; ++s) {
      const bool ok = ch_ok && (t0 + s < p.L);
  #pragma unroll
      for (int v = 0; v < V; ++v) {
        av[s][v] = ok ? LD::get(raw_r[s], v) : MinMaxOp::id_a();
        bv[s][v] = ok ? LD::get(raw_s[s], v) : MinMaxOp::id_b();
        fB[v] = MinMaxOp::apply(av[s][v], bv[s][v], fB[v]);
        fA[v] = MinMaxOp::fold_a(av[s][v], fA[v]);
      }
    }
  #pragma unroll
    for (int v = 0; v < V; ++v) {
      s_fA[wave][lane * V + v] = fA[v];
      s_fB[wave][lane * V + v] = fB[v];
    }
    // the gate is first needed after the barrier: its loads are issued here, once r and s are spent
    if (GATE)
  #pragma unroll
      for (int s = 0; s < kBSteps; ++s)
        rg[GATE ? s : 0] = LD::load(wg, lane_in, (uint32_t)min(wave * kBSteps + s, rows - 1) * row_in);
    __syncthreads();

    // ---- forward states of this wave's steps: the output-gate gradient (stored now, in step order),
    //      the step weights, and the wave's reverse aggregate
    const uint32_t row_out = (uint32_t)(p.D * (int64_t)sizeof(Tout)), lane_out = (uint32_t)(chl * (int64_t)sizeof(Tout));
    const auto wdg = window(GATE && p.dgate ? p.dgate : p.dr, (int)sizeof(Tout));
    // 4 a'_t = 4 wM wX, 4 wM wR and 4 wS of step s, channel v at bytes (k kBSteps + s) V + v, k = 0, 1, 2
    Bytes4<3 * kBSteps * V> wt;
    auto wi = [](int k, int s, int v) { return (k * kBSteps + s) * V + v; };
    float ev[kBSteps][V];
    {
      float h[V];
  #pragma unroll
      for (int v = 0; v < V; ++v) {
        const int j = lane * V + v;
        h[v] = hc[v];
        for (int w = 0; w < wave; ++w) h[v] = MinMaxOp::apply(s_fA[w][j], s_fB[w][j], h[v]);
      }
  #pragma unroll
      for (int s = 0; s < kBSteps; ++s) {
        const bool ok = ch_ok && (t0 + s < p.L);
        float o_dg[V];
  #pragma unroll
        for (int v = 0; v < V; ++v) {
          const float r = av[s][v], sv = bv[s][v];
          const float m = mm_min(r, h[v]);
          const float wm2 = 2.0f * sel_hi(m, sv);
          wt.set(wi(0, s, v), ok ? wm2 * (2.0f * sel_lo(h[v], r)) : 4.0f);
          wt.set(wi(1, s, v), wm2 * (2.0f * sel_lo(r, h[v])));
          wt.set(wi(2, s, v), 4.0f * sel_hi(sv, m));
          const float dy = LD::get(rdy[s], v);
          ev[s][v] = ok ? (GATE ? dy * LD::get(rg[GATE ? s : 0], v) : dy) : 0.0f;
          h[v] = mm_max(m, sv);
          o_dg[v] = dy * h[v];
        }
        if (GATE && p.dgate && ch_ok && s < nvalid) ST::store(wdg, lane_out, (uint32_t)(wave * kBSteps + s) * row_out, o_dg);
      }
    }
    // the packed weights are final here: keep them packed (rather than their inputs) from now on
  #pragma unroll
    for (int i = 0; i < (3 * kBSteps * V + 3) / 4; ++i) asm volatile("" : "+v"(wt.u[i]));
  #pragma unroll
    for (int v = 0; v < V; ++v) {
      float rA = 1.0f, rB = 0.0f;
  #pragma unroll
      for (int s = kBSteps - 1; s >= 0; --s) {
        const float a = 0.25f * wt.get(wi(0, s, v));
        rB = fmaf(a, rB, a * ev[s][v]);
        rA *= a;
      }
      s_rA[wave][lane * V + v] = rA;
      s_rB[wave][lane * V + v] = rB;
    }
    __syncthreads();

    // ---- waves 0 .. V-1: chunk reverse aggregate, publish, reverse carry over later chunks
    if (wave < V) {
      const int j = wave * 64 + lane;
      const int64_t seq_unit = (b * p.n_tiles + k) * p.n_chunks;
      float Ac = 1.0f, Bc = 0.0f;
  #pragma unroll
      for (int w = kBWaves - 1; w >= 0; --w) {
        Bc = fmaf(s_rA[w][j], Bc, s_rB[w][j]);
        Ac *= s_rA[w][j];
      }
      const int64_t chj = k * TW + j;
      const float init = p.dx_last ? p.dx_last[b * p.D + (chj < p.D ? chj : p.D - 1)] : 0.0f;
      float incl;
      s_qin[j] = lookback_carry<AffineOp, TW>(p.ctl, p.words, seq_unit, cr, p.n_chunks, j, E, p.wait, Ac, Bc, init, &incl);
    }
    __syncthreads();

    // ---- per-step gradients, last step first (the packed weights are decoded again here rather than
    //      kept unpacked through the lookback: the empty asm hides the earlier decode)
  #pragma unroll
    for (int i = 0; i < (3 * kBSteps * V + 3) / 4; ++i) asm volatile("" : "+v"(wt.u[i]));
    float q[V];
  #pragma unroll
    for (int v = 0; v < V; ++v) {
      const int j = lane * V + v;
      float qq = s_qin[j];
      for (int w = kBWaves - 1; w > wave; --w) qq = fmaf(s_rA[w][j], qq, s_rB[w][j]);
      q[v] = qq;
    }
    const auto wdr = window(p.dr, (int)sizeof(Tout)), wds = window(p.ds, (int)sizeof(Tout));
  #pragma unroll
    for (int s = kBSteps - 1; s >= 0; --s) {
      float o_dr[V], o_ds[V];
  #pragma unroll
      for (int v = 0; v < V; ++v) {
        const float g4 = 0.25f * (ev[s][v] + q[v]);
        q[v] = wt.get(wi(0, s, v)) * g4;
        o_dr[v] = wt.get(wi(1, s, v)) * g4;
        o_ds[v] = wt.get(wi(2, s, v)) * g4;
      }
      if (ch_ok && s < nvalid) {
        const uint32_t ro = (uint32_t)(wave * kBSteps + s) * row_out;
        ST::store(wdr, lane_out, ro, o_dr);
        ST::store(wds, lane_out, ro, o_ds);
      }
    }
    if (p.dx0 && ch_ok && c == 0 && wave == 0)
  #pragma unroll
      for (int v = 0; v < V; ++v) p.dx0[b * p.D + ch0 + v] = q[v];
    if (threadIdx.x == 0) s_tick[parity ^ 1] = take_end(p.ctl, n_seq, (uint32_t)p.n_chunks, xc, left, m_next);
    __syncthreads();  // this unit's LDS is free; the next ticket is visible
  }
  if (threadIdx.x == 0) finish_launch(p.ctl, E);
}

// d a_log[d] = sum over (batch, chunk) of the unit partials, in a fixed order: slice s of
// kDalSlices sums units [s n / S, (s + 1) n / S), then the slices are added in order.
constexpr int kDalSlices = 32;
__global__ __launch_bounds__(256) void dalog_slice_kernel(const float* part, int64_t n, int64_t D, float* slices) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  const int64_t s = blockIdx.y, u0 = s * n / kDalSlices, u1 = (s + 1) * n / kDalSlices;
  float acc = 0.0f;
  for (int64_t u = u0; u < u1; ++u) acc += part[u * D + d];
  slices[s * D + d] = acc;
}
__global__ __launch_bounds__(256) void dalog_final_kernel(const float* slices, int64_t D, float* out) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  float acc = 0.0f;
  for (int s = 0; s < kDalSlices; ++s) acc += slices[s * D + d];
  out[d] = acc;
}

// ------------------------------------------------------------------ launchers
// Persistent grids: as many workgroups as stay resident together (by the kernel's own occupancy,
// cached per kernel), never more than there are work units.
int64_t resident_blocks(const void* kern, int threads) {
  static std::mutex mu;
  static std::unordered_map<const void*, int64_t> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(kern);
  if (it != cache.end()) return it->second;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess || per_cu <= 0) per_cu = 1;
  return cache[kern] = (int64_t)per_cu * cus;
}
template <class Op, typename Tin, typename Tout, int V, bool GATE, bool RECORD>
hipError_t launch_scan_t(const Scan1Params& p, hipStream_t s) {
  const auto kern = scan1_kernel<Op, Tin, Tout, V, GATE, RECORD>;
  const int64_t total = p.B * p.n_tiles * p.n_chunks;
  const int64_t grid = std::min<int64_t>(total, resident_blocks(reinterpret_cast<const void*>(kern), kWaves * 64));
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

template <class Op, int V, bool GATE>
hipError_t launch_scan_dt(const Scan1Params& p, int in_bf16, int out_bf16, hipStream_t s) {
  if (!in_bf16) return launch_scan_t<Op, float, float, V, GATE, false>(p, s);
  return out_bf16 ? launch_scan_t<Op, bf16_t, bf16_t, V, GATE, false>(p, s)
                  : launch_scan_t<Op, bf16_t, float, V, GATE, false>(p, s);
}

int vec_width(int64_t D) { return (D % 2 == 0) ? 2 : 1; }

template <class Op>
void scan_geometry(Scan1Params& p, void* scratch) {
  const int V = vec_width(p.D);
  const int64_t TW = 64 * V;
  p.n_tiles = (p.D + TW - 1) / TW;
  p.n_chunks = (p.L + kChunk - 1) / kChunk;
  p.ctl = static_cast<LookbackCtl*>(scratch);
  p.words = reinterpret_cast<unsigned long long*>(static_cast<char*>(scratch) + kCtlBytes);
}

// The record pass of the backward: no outputs, the state entering each chunk to p.carry_out.
template <class Op>
hipError_t launch_record_op(Scan1Params& p, int in_bf16, void* scratch, hipStream_t s) {
  scan_geometry<Op>(p, scratch);
  if (vec_width(p.D) == 2)
    return in_bf16 ? launch_scan_t<Op, bf16_t, float, 2, false, true>(p, s) : launch_scan_t<Op, float, float, 2, false, true>(p, s);
  return in_bf16 ? launch_scan_t<Op, bf16_t, float, 1, false, true>(p, s) : launch_scan_t<Op, float, float, 1, false, true>(p, s);
}

template <class Op, bool GATE, int NW>
hipError_t launch_short_dt(const Scan1Params& p, int in_bf16, int out_bf16, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * ((p.D + 63) / 64))), block(NW * 64);
  if (!in_bf16)
    hipLaunchKernelGGL((scan1_short_kernel<Op, float, float, GATE, NW>), grid, block, 0, s, p);
  else if (out_bf16)
    hipLaunchKernelGGL((scan1_short_kernel<Op, bf16_t, bf16_t, GATE, NW>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((scan1_short_kernel<Op, bf16_t, float, GATE, NW>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <class Op, bool GATE>
hipError_t launch_short_g(const Scan1Params& p, int in_bf16, int out_bf16, hipStream_t s) {
  if (p.L <= 4 * kShortSpw) return launch_short_dt<Op, GATE, 4>(p, in_bf16, out_bf16, s);
  if (p.L <= 8 * kShortSpw) return launch_short_dt<Op, GATE, 8>(p, in_bf16, out_bf16, s);
  return launch_short_dt<Op, GATE, 16>(p, in_bf16, out_bf16, s);
}

// Sequences of at most this many steps take the one-pass short kernel.
constexpr int64_t kShortSteps = 16 * kShortSpw;

template <class Op>
hipError_t launch_scan_op(Scan1Params& p, int in_bf16, int out_bf16, void* scratch, hipStream_t s) {
  const int V = vec_width(p.D);
  scan_geometry<Op>(p, scratch);
  const bool gate = p.gate != nullptr;
  if (p.L <= kShortSteps && p.B * ((p.D + 63) / 64) < ((int64_t)1 << 31) && p.L * p.D * 4 < ((int64_t)1 << 31))
    return gate ? launch_short_g<Op, true>(p, in_bf16, out_bf16, s) : launch_short_g<Op, false>(p, in_bf16, out_bf16, s);
  if (V == 2)
    return gate ? launch_scan_dt<Op, 2, true>(p, in_bf16, out_bf16, s) : launch_scan_dt<Op, 2, false>(p, in_bf16, out_bf16, s);
  return gate ? launch_scan_dt<Op, 1, true>(p, in_bf16, out_bf16, s) : launch_scan_dt<Op, 1, false>(p, in_bf16, out_bf16, s);
}

// Vectors per lane in the decode step, and channels per vector (below): a step is one round trip to
// memory followed by a short chain of arithmetic per lane, so many short lanes finish first.  Measured
// at B = 256, D = 2560 bf16 from a HIP graph, with the step's inputs and y non-temporal, 256-thread
// workgroups: 2 channels x 1 vector 3.26 us per step, 4 x 1 3.51 us, 2 x 2 3.74 us (a plain device
// copy of the same bytes: 2.6 us); with every access cached, 2 x 1 took 3.9 us.  Workgroups of 128
// threads: 3.15-3.19 us (64: 3.68-3.71, 512: 3.37, 1024: 3.66).
constexpr int kUpdVectors = 1;
template <class Op, bool GATE, int V>
hipError_t launch_update_v(const Upd1Params& p, int in_bf16, int out_bf16, hipStream_t s) {
  constexpr int U = kUpdVectors;
  constexpr int64_t per_wg = (int64_t)kUpdThreads * U;
  const dim3 grid((unsigned)((p.B * p.D / V + per_wg - 1) / per_wg)), block(kUpdThreads);
  if (!in_bf16)
    hipLaunchKernelGGL((update1v_kernel<Op, float, float, GATE, V, U>), grid, block, 0, s, p);
  else if (out_bf16)
    hipLaunchKernelGGL((update1v_kernel<Op, bf16_t, bf16_t, GATE, V, U>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((update1v_kernel<Op, bf16_t, float, GATE, V, U>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <class Op, bool GATE>
hipError_t launch_update_g(const Upd1Params& p, int in_bf16, int out_bf16, hipStream_t s) {
  const int64_t n = p.B * p.D;
  // vector path: every operand (the fp32 state is the largest) under 2^31 bytes
  if (n * (int64_t)sizeof(float) < ((int64_t)1 << 31)) {
    if (p.D % 2 == 0) return launch_update_v<Op, GATE, 2>(p, in_bf16, out_bf16, s);
  }
  const dim3 grid((unsigned)((n + 255) / 256));
  if (!in_bf16)
    hipLaunchKernelGGL((update1_kernel<Op, float, float, GATE>), grid, dim3(256), 0, s, p);
  else if (out_bf16)
    hipLaunchKernelGGL((update1_kernel<Op, bf16_t, bf16_t, GATE>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((update1_kernel<Op, bf16_t, float, GATE>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_update_op(const Upd1Params& p, int in_bf16, int out_bf16, hipStream_t s) {
  return p.gate ? launch_update_g<Op, true>(p, in_bf16, out_bf16, s) : launch_update_g<Op, false>(p, in_bf16, out_bf16, s);
}

}  // namespace

size_t workspace_head_bytes() { return (size_t)kCtlBytes; }
size_t workspace_error_offset() { return offsetof(LookbackCtl, error); }

size_t scan1_scratch_bytes(int64_t B, int64_t L, int64_t D) {
  const int V = vec_width(D);
  const int64_t TW = 64 * V;
  const int64_t n_tiles = (D + TW - 1) / TW;
  const int64_t n_chunks = (L + kChunk - 1) / kChunk;
  return (size_t)kCtlBytes + (size_t)(B * n_tiles * n_chunks) * 3 * TW * sizeof(unsigned long long);
}

// ------------------------------------------------------------------ fixed device scratch
// The lookback scratch of ssd_rglru_scan_noalloc, for callers that cannot allocate: one array per
// GPU, zero at module load and left ready for the next launch by every launch (the launch counter
// and ticket resets of the lookback protocol), so it is never cleared again.  Every call on a GPU
// shares it: calls whose work overlaps on one GPU race.  Host code uses only the per-device address
// from hipGetSymbolAddress, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    g_noalloc_ptr[dev] = ptr;
  }
  *out = g_noalloc_ptr[dev];
  return hipSuccess;
}

hipError_t launch_rglru_scan(const RglruScanArgs& a, hipStream_t s) {
  Scan1Params p{};
  p.B = a.B; p.L = a.L; p.D = a.D;
  p.in[0] = a.x; p.in[1] = a.r_logit; p.in[2] = a.i_logit;
  p.gate = a.gate;
  p.a_log = a.a_log; p.c = a.c; p.h0 = a.h0; p.y = a.y; p.h_last = a.h_last; p.carry_out = a.chunk_states;
  p.wait = a.wait;
  return launch_scan_op<AffineOp>(p, a.in_bf16, a.out_bf16, a.scratch, s);
}

hipError_t launch_minmax_scan(const MinmaxScanArgs& a, hipStream_t s) {
  Scan1Params p{};
  p.B = a.B; p.L = a.L; p.D = a.D;
  p.in[0] = a.r; p.in[1] = a.s;
  p.gate = a.gate;
  p.h0 = a.x0; p.y = a.y; p.h_last = a.x_last; p.carry_out = a.chunk_states;
  p.wait = a.wait;
  return launch_scan_op<MinMaxOp>(p, a.in_bf16, a.out_bf16, a.scratch, s);
}

template <typename Tin, typename Tout, int V, bool G>
hipError_t launch_bwd_k(const Bwd1Params& q, int64_t units, hipStream_t s) {
  const auto kern = rglru_bwd_kernel<Tin, Tout, V, G>;
  const int64_t grid = std::min<int64_t>(units, resident_blocks(reinterpret_cast<const void*>(kern), kBWaves * 64));
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBWaves * 64), 0, s, q);
  return hipGetLastError();
}
template <int V, bool G>
hipError_t launch_bwd_g(const Bwd1Params& q, int in_bf16, int out_bf16, int64_t units, hipStream_t s) {
  if (!in_bf16) return launch_bwd_k<float, float, V, G>(q, units, s);
  return out_bf16 ? launch_bwd_k<bf16_t, bf16_t, V, G>(q, units, s) : launch_bwd_k<bf16_t, float, V, G>(q, units, s);
}
template <int V>
hipError_t launch_bwd_dt(const Bwd1Params& q, bool gate, int in_bf16, int out_bf16, int64_t units, hipStream_t s) {
  return gate ? launch_bwd_g<V, true>(q, in_bf16, out_bf16, units, s) : launch_bwd_g<V, false>(q, in_bf16, out_bf16, units, s);
}

// Scratch of the backward call: lookback control block and words (sized for the larger of the
// forward and reverse tilings), then the chunk carries and the d a_log partials.
namespace {
// The reverse pass uses the same tiling as the forward (64 V channels per tile, V = 2 for even D),
// so one word layout serves both.
int64_t bwd_words_bytes(int64_t B, int64_t L, int64_t D) {
  return ((int64_t)scan1_scratch_bytes(B, L, D) - kCtlBytes + 255) / 256 * 256;
}
}  // namespace

size_t rglru_bwd_scratch_bytes(int64_t B, int64_t L, int64_t D) {
  const int64_t n_chunks = (L + kChunk - 1) / kChunk;
  const int64_t per = (B * n_chunks * D * 4 + 255) / 256 * 256;
  return (size_t)(kCtlBytes + bwd_words_bytes(B, L, D) + 2 * per + (int64_t)kDalSlices * D * 4);
}

hipError_t launch_rglru_scan_backward(const RglruBwdArgs& a, hipStream_t s) {
  const int64_t n_chunks = (a.L + kChunk - 1) / kChunk;
  const int64_t per = (a.B * n_chunks * a.D * 4 + 255) / 256 * 256;
  char* base = static_cast<char*>(a.scratch);
  float* rec = reinterpret_cast<float*>(base + kCtlBytes + bwd_words_bytes(a.B, a.L, a.D));
  float* dal = reinterpret_cast<float*>(reinterpret_cast<char*>(rec) + per);
  // 1. the state entering every chunk: the forward's, or a forward pass that records it (no outputs)
  const float* carry = a.chunk_states;
  hipError_t e = hipSuccess;
  if (!carry) {
    Scan1Params f{};
    f.B = a.B; f.L = a.L; f.D = a.D;
    f.in[0] = a.x; f.in[1] = a.r_logit; f.in[2] = a.i_logit;
    f.a_log = a.a_log; f.c = a.c; f.h0 = a.h0; f.y = nullptr; f.h_last = nullptr; f.carry_out = rec;
    f.wait = a.wait;
    e = launch_record_op<AffineOp>(f, a.in_bf16, a.scratch, s);
    if (e != hipSuccess) return e;
    carry = rec;
  }
  // 2. reverse pass, one workgroup per (batch, 64-channel tile, chunk)
  const int V = vec_width(a.D);
  Bwd1Params q{};
  q.B = a.B; q.L = a.L; q.D = a.D;
  q.n_tiles = (a.D + 64 * V - 1) / (64 * V); q.n_chunks = n_chunks;
  q.x = a.x; q.r = a.r_logit; q.i = a.i_logit; q.gate = a.gate; q.dy = a.dy;
  q.a_log = a.a_log; q.c = a.c; q.carry = carry; q.dh_last = a.dh_last;
  q.dx = a.dx; q.dr = a.dr_logit; q.di = a.di_logit; q.dgate = a.dgate; q.dalog_part = dal; q.dh0 = a.dh0;
  q.ctl = static_cast<LookbackCtl*>(a.scratch);
  q.words = reinterpret_cast<unsigned long long*>(base + kCtlBytes);
  q.wait = a.wait;
  const int64_t units = a.B * q.n_tiles * n_chunks;
  if (V == 2) e = launch_bwd_dt<2>(q, a.gate != nullptr, a.in_bf16, a.out_bf16, units, s);
  else e = launch_bwd_dt<1>(q, a.gate != nullptr, a.in_bf16, a.out_bf16, units, s);
  if (e != hipSuccess) return e;
  // 3. d a_log
  float* slices = reinterpret_cast<float*>(reinterpret_cast<char*>(dal) + per);
  const unsigned nb = (unsigned)((a.D + 255) / 256);
  hipLaunchKernelGGL(dalog_slice_kernel, dim3(nb, kDalSlices), dim3(256), 0, s, dal, a.B * n_chunks, a.D, slices);
  hipLaunchKernelGGL(dalog_final_kernel, dim3(nb), dim3(256), 0, s, slices, a.D, a.da_log);
  return hipGetLastError();
}

namespace {
template <typename Tin, typename Tout, int V, bool G>
hipError_t launch_mm_bwd_k(const MmBwdParams& q, int64_t units, hipStream_t s) {
  const auto kern = minmax_bwd_kernel<Tin, Tout, V, G>;
  const int64_t grid = std::min<int64_t>(units, resident_blocks(reinterpret_cast<const void*>(kern), kBWaves * 64));
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBWaves * 64), 0, s, q);
  return hipGetLastError();
}
template <int V, bool G>
hipError_t launch_mm_bwd_g(const MmBwdParams& q, int in_bf16, int out_bf16, int64_t units, hipStream_t s) {
  if (!in_bf16) return launch_mm_bwd_k<float, float, V, G>(q, units, s);
  return out_bf16 ? launch_mm_bwd_k<bf16_t, bf16_t, V, G>(q, units, s) : launch_mm_bwd_k<bf16_t, float, V, G>(q, units, s);
}
template <int V>
hipError_t launch_mm_bwd_dt(const MmBwdParams& q, bool gate, int in_bf16, int out_bf16, int64_t units, hipStream_t s) {
  return gate ? launch_mm_bwd_g<V, true>(q, in_bf16, out_bf16, units, s) : launch_mm_bwd_g<V, false>(q, in_bf16, out_bf16, units, s);
}
}  // namespace

size_t minmax_bwd_scratch_bytes(int64_t B, int64_t L, int64_t D) {
  const int64_t n_chunks = (L + kChunk - 1) / kChunk;
  return (size_t)(kCtlBytes + bwd_words_bytes(B, L, D) + B * n_chunks * D * 4);
}

hipError_t launch_minmax_scan_backward(const MinmaxBwdArgs& a, hipStream_t s) {
  const int64_t n_chunks = (a.L + kChunk - 1) / kChunk;
  char* base = static_cast<char*>(a.scratch);
  float* rec = reinterpret_cast<float*>(base + kCtlBytes + bwd_words_bytes(a.B, a.L, a.D));
  // 1. the state entering every chunk: the forward's, or a forward pass that records it (no outputs)
  const float* carry = a.chunk_states;
  if (!carry) {
    Scan1Params f{};
    f.B = a.B; f.L = a.L; f.D = a.D;
    f.in[0] = a.r; f.in[1] = a.s;
    f.h0 = a.x0; f.y = nullptr; f.h_last = nullptr; f.carry_out = rec;
    f.wait = a.wait;
    const hipError_t e = launch_record_op<MinMaxOp>(f, a.in_bf16, a.scratch, s);
    if (e != hipSuccess) return e;
    carry = rec;
  }
  // 2. reverse pass, one workgroup per (batch, 64-channel tile, chunk)
  const int V = vec_width(a.D);
  MmBwdParams q{};
  q.B = a.B; q.L = a.L; q.D = a.D;
  q.n_tiles = (a.D + 64 * V - 1) / (64 * V); q.n_chunks = n_chunks;
  q.r = a.r; q.s = a.s; q.gate = a.gate; q.dy = a.dy; q.carry = carry; q.dx_last = a.dx_last;
  q.dr = a.dr; q.ds = a.ds; q.dgate = a.dgate; q.dx0 = a.dx0;
  q.ctl = static_cast<LookbackCtl*>(a.scratch);
  q.words = reinterpret_cast<unsigned long long*>(base + kCtlBytes);
  q.wait = a.wait;
  const int64_t units = a.B * q.n_tiles * n_chunks;
  return V == 2 ? launch_mm_bwd_dt<2>(q, a.gate != nullptr, a.in_bf16, a.out_bf16, units, s)
                : launch_mm_bwd_dt<1>(q, a.gate != nullptr, a.in_bf16, a.out_bf16, units, s);
}

hipError_t launch_rglru_update(const RglruUpdateArgs& a, hipStream_t s) {
  Upd1Params p{};
  p.B = a.B; p.D = a.D;
  p.in[0] = a.x; p.in[1] = a.r_logit; p.in[2] = a.i_logit;
  p.gate = a.gate; p.a_log = a.a_log; p.c = a.c; p.state = a.state; p.y = a.y;
  return launch_update_op<AffineOp>(p, a.in_bf16, a.out_bf16, s);
}

hipError_t launch_minmax_update(const MinmaxUpdateArgs& a, hipStream_t s) {
  Upd1Params p{};
  p.B = a.B; p.D = a.D;
  p.in[0] = a.r; p.in[1] = a.s;
  p.gate = a.gate; p.state = a.state; p.y = a.y;
  return launch_update_op<MinMaxOp>(p, a.in_bf16, a.out_bf16, s);
}

}  // namespace ssd
