// selective.hip -- multi-scale selective scan (batched and packed varlen) and its decode update.
//
// Recurrence (cortexnet 3.2.1, cortexnet/ssm.py, MultiScaleSSM.forward / _selective_scan):
//   delta = softplus(dt + dt_bias) (or dt + dt_bias), abar_n = exp(min(delta A_n, 20)),
//   h_n = abar_n h_n + (delta B_n) x,  y = (sum_n C_n h_n + Dskip x) * silu(z).
//
// Layout: one lane per channel d (rows of [rows, D] are coalesced along d), the N states of the
// channel in registers, B_n / C_n of the current row uniform across the wave (scalar loads).
//
// Time parallelism: each sequence is cut into segments of T rows.  Pass 1 runs every segment
// except a sequence's last from a zero state and stores its aggregate per state (P = prod abar,
// H = end state).  A carry pass folds the aggregates of the earlier segments of the same sequence
// onto h0, and pass 2 runs the full recurrence from that carry-in with the readout, skip and gate,
// writing y (and the final state for a sequence's last segment).  No workgroup waits for another:
// the only dependency is the kernel boundary between the passes.
//
// Packed sequences with bf16 inputs take a second plan: a sequence is scanned from its start to its
// end by one workgroup per channel block unless it is longer than X rows (a fraction of the rows
// each compute unit scans on average); a longer one is cut into as few equal pieces as keep them
// within X.  Only the rows before a sequence's last piece pass through the aggregate kernel (in
// blocks of 256 rows), a small kernel folds each piece's blocks into the piece's aggregate, a later
// piece folds h0 through the earlier pieces' aggregates, and the scan units run longest first so
// that the long ones end with the rest.  For the 32-sequence benchmark shape
// half the rows are aggregated instead of nearly all.
//
// When dt goes through softplus (delta >= 0) and every A of the wave is <= 0, delta*A <= 0 and
// the clamp at 20 cannot act; that wave-uniform case skips it and forms P as 2^(A sum delta).
// Otherwise the clamp is applied and P = 2^(sum of the clamped exponents), both exact readings of
// prod abar.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr float kClampLog2 = 20.0f * kLog2e;  // clamp(delta*A, max=20) in the base-2 exponent

struct SelParams {
  int64_t L;        // rows per sequence (batched)
  int64_t D;
  int64_t N;
  int64_t nseq;
  int64_t T;        // segment length
  int64_t nseg;     // segments per sequence (batched)
  const int32_t* cu;      // varlen boundaries or NULL
  const int2* units;      // varlen (seq, seg) table or NULL
  const int* n_units;     // varlen unit count (device)
  const void* x;
  const void* dt;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const float* dt_bias;
  const float* h0;
  void* y;
  float* h_last;
  float* aggP;   // [unit][N][D]  product of abar over the segment (clamp variant only, see sdelta)
  float* aggH;   // [unit][N][D]  state reached from zero at the segment end
  float* sdelta;  // [unit][D]   delta summed over the segment: where the clamp cannot act (softplus
                  //  steps, A_n <= 0) the product of abar is 2^(A_n log2(e) sdelta), as pass 1 forms it
  int softplus;
  float* carry;  // [unit][N][D]  state entering the segment
  const int2* seq_units;  // varlen: (first unit, unit count) per sequence
  // Packed varlen forward plan (NULL for the other launches): scan units of whole sequences or of
  // long sequences cut into a few pieces, in two phases (first pieces, then the later ones), longest
  // first within a phase; aggregates only for the rows of a sequence's middle pieces.
  const int* vcount;      // [0] scan units, [1] aggregate units, [2] piece slots, [3] scan units of phase 1
  const int4* vscan;      // (sequence, first row in the sequence, rows, carry slot or -1)
  const int4* vagg;       // (sequence, first row in the sequence, rows, piece slot)
  const int4* vseq;       // per sequence: (first aggregate unit, aggregate units, aggregate units per
                          //  scan piece, first piece slot)
  const int2* vpiece;     // per piece slot: (first aggregate unit, aggregate units; 0 for a first piece)
  float* pieceP;          // [piece slot][N][D]: prod abar over a middle piece
  float* pieceH;          // [piece slot][N][D]: the state a middle piece reaches from zero; a first
                          //  piece's end state
  int64_t nblk;           // channel blocks (the packed plan's scan grid is units x channel blocks)
};

struct Unit {
  int64_t seq, seg, row0, row1, carry;
  bool last, valid;
};

__device__ __forceinline__ Unit unit_of(const SelParams& p, int64_t u) {
  Unit r;
  r.carry = -1;
  if (p.vscan != nullptr) {
    r.valid = u < (int64_t)p.vcount[0];
    if (!r.valid) return r;
    const int4 e = p.vscan[u];
    r.seq = e.x;
    r.row0 = (int64_t)p.cu[r.seq] + e.y;
    r.row1 = r.row0 + e.z;
    r.carry = e.w;
    r.seg = e.w < 0 ? 0 : 1;
    r.last = (r.row1 == (int64_t)p.cu[r.seq + 1]);
    return r;
  }
  if (p.cu == nullptr) {
    r.seq = u / p.nseg;
    r.seg = u - r.seq * p.nseg;
    r.row0 = r.seq * p.L + r.seg * p.T;
    const int64_t end = (r.seq + 1) * p.L;
    r.row1 = min(r.row0 + p.T, end);
    r.last = (r.row1 == end);
    r.valid = true;
  } else {
    r.valid = u < (int64_t)(*p.n_units);
    if (!r.valid) return r;
    const int2 e = p.units[u];
    r.seq = e.x;
    r.seg = e.y;
    const int64_t start = p.cu[r.seq];
    const int64_t end = p.cu[r.seq + 1];
    r.row0 = start + r.seg * p.T;
    r.row1 = min(r.row0 + p.T, end);
    r.last = (r.row1 == end);
  }
  return r;
}

// ----------------------------------------------------------------------------- row inputs
// x / dt / z / y of a unit are addressed through buffer windows over the unit's rows: a per-lane
// channel offset plus a wave-uniform row offset, no per-lane 64-bit address arithmetic.  The plan
// keeps every unit's window under 2^31 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_window(const void* a, int64_t row0, int64_t nrows, int64_t D,
                                                              int es) {
  return make_window(static_cast<const char*>(a) + row0 * D * es, (uint32_t)(nrows * D * es));
}

constexpr int kPrefetch = 4;   // rows of x / dt / z in flight per lane (also the unroll factor)
constexpr int kRowBlock = 64;  // rows of B / C staged in LDS at a time

// B_n and C_n are shared by every channel of a row, so the workgroup (all of whose lanes work on
// the same rows) stages them once per block of kRowBlock rows in LDS as fp32, one block ahead of
// use; lanes then read them as broadcasts.
template <int NS, bool READOUT>
struct BCStage {
  static constexpr int PER_ROW = READOUT ? 2 * NS : NS;         // B then C
  static constexpr int PER_BLOCK = kRowBlock * PER_ROW;
  static constexpr int PER_THREAD = (PER_BLOCK + kThreads - 1) / kThreads;
  float v[PER_THREAD];

  // element e of the block: row e / PER_ROW, column e % PER_ROW (B for col < NS, else C)
  template <typename Tin>
  __device__ __forceinline__ void fetch(const SelParams& p, int64_t row0, int64_t nrows, int64_t blk) {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) {
      const int e = q * kThreads + threadIdx.x;
      const int r = e / PER_ROW, col = e - r * PER_ROW;
      const int64_t row = row0 + min(blk * kRowBlock + r, nrows - 1);
      const void* M = col < NS ? p.Bm : p.Cm;
      const int n = col < NS ? col : col - NS;
      v[q] = (e < PER_BLOCK) ? io<Tin>::load(M, row * NS + n) : 0.0f;
    }
  }
  __device__ __forceinline__ void put(float* lds) const {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) {
      const int e = q * kThreads + threadIdx.x;
      if (e < PER_BLOCK) lds[e] = v[q];
    }
  }
};

// ----------------------------------------------------------------------------- the row loop
// How abar_n = exp(min(delta A_n, 20)) is formed (a wave-uniform choice):
//   kClamp: exp of the clamped exponent (any A, any delta);
//   kExp:   exp without the clamp, when delta >= 0 and every A <= 0 (then delta A_n <= 0).
enum Disc { kClamp = 0, kExp = 1 };

// One row of one channel: discretise, advance the N states, optionally read out.
template <typename Tin, int NS, bool SOFTPLUS, int DISC, bool READOUT, bool GATE>
__device__ __forceinline__ float row_step(float xx, float dd, float zz, const float* bc, const float* A2, float dskip,
                                          float* h, float* e, float& sum_delta) {
  const float delta = SOFTPLUS ? softplus_in<Tin>(dd) : dd;
  const float dx = delta * xx;
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    float dA = delta * A2[n];
    if (DISC == kClamp) {
      dA = dA > kClampLog2 ? kClampLog2 : dA;
      if (!READOUT) e[n] += dA;
    }
    h[n] = fmaf(hw_exp2(dA), h[n], dx * bc[n]);
    if (READOUT) acc = fmaf(bc[NS + n], h[n], acc);
    // states in groups of 8: bounds the exponentials held in flight (register pressure)
    if (NS > 8 && (n & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
  if (!READOUT) sum_delta += delta;
  if (READOUT) {
    acc = fmaf(dskip, xx, acc);
    if (GATE) acc *= silu_f(zz);
  }
  return acc;
}

// Runs rows [row0, row1) of one segment for channel dl.  Every lane of the workgroup must call it
// with the same rows (B / C staging uses barriers).  x / dt / z are prefetched kPrefetch rows ahead
// in registers.  Loads and stores are unconditional inside the unrolled groups (indices are
// clamped in range) so the compiler counts outstanding memory operations exactly; a lane without a
// channel of its own recomputes channel D-1 bit for bit and rewrites the same value.
// The workgroup's rows, marked wave-uniform (scalar registers): where the compiler cannot prove it
// (a unit read from a table in a kernel with two roles), it would otherwise keep the windows built
// from them in vector registers and wrap every buffer access in a loop over distinct values.
__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <typename Tin, typename Tout, int NS, bool SOFTPLUS, int DISC, bool READOUT, bool GATE>
__device__ __forceinline__ void run_rows(const SelParams& p, int64_t row0, int64_t row1, int64_t dl,
                                         const float* A2, float bias, float dskip, float* h, float* e,
                                         float& sum_delta, float* lds) {
  row0 = wave_uniform(row0);
  row1 = wave_uniform(row1);
  using W = win<Tin, 1>;
  using Stage = BCStage<NS, READOUT>;
  constexpr int PR = Stage::PER_ROW;
  const int64_t nrows = row1 - row0;
  if (nrows <= 0) return;
  const auto wx = unit_window(p.x, row0, nrows, p.D, sizeof(Tin));
  const auto wd = unit_window(p.dt, row0, nrows, p.D, sizeof(Tin));
  const auto wz = unit_window(GATE ? p.z : p.x, row0, nrows, p.D, sizeof(Tin));
  const auto wy = unit_window(READOUT ? p.y : p.x, row0, nrows, p.D, sizeof(Tout));
  const uint32_t lane_in = (uint32_t)(dl * (int64_t)sizeof(Tin)), row_in = (uint32_t)(p.D * (int64_t)sizeof(Tin));
  const uint32_t lane_out = (uint32_t)(dl * (int64_t)sizeof(Tout)), row_out = (uint32_t)(p.D * (int64_t)sizeof(Tout));
  const int last = (int)nrows - 1;
  typename W::raw rx[kPrefetch], rd[kPrefetch], rz[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    const uint32_t ro = (uint32_t)min(k, last) * row_in;
    rx[k] = W::load(wx, lane_in, ro);
    rd[k] = W::load(wd, lane_in, ro);
    if (GATE) rz[k] = W::load(wz, lane_in, ro);
  }
  Stage st;
  st.template fetch<Tin>(p, row0, nrows, 0);
  st.put(lds);
  const int nblk = (int)((nrows + kRowBlock - 1) / kRowBlock);
  for (int blk = 0; blk < nblk; ++blk) {
    float* cur = lds + (blk & 1) * Stage::PER_BLOCK;
    if (blk + 1 < nblk) st.template fetch<Tin>(p, row0, nrows, blk + 1);
    __syncthreads();  // block blk is in LDS; the other buffer is free
    const int r_begin = blk * kRowBlock;
    const int r_end = min(r_begin + kRowBlock, (int)nrows);
    const int r_full = r_begin + (r_end - r_begin) / kPrefetch * kPrefetch;
    for (int base = r_begin; base < r_full; base += kPrefetch) {
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        // slot of row i in the prefetch ring is i % kPrefetch = k (r_begin is a multiple of it)
        const int i = base + k;
        const float xx = W::get(rx[k], 0);
        const float dd = W::get(rd[k], 0) + bias;
        const float zz = GATE ? W::get(rz[k], 0) : 0.0f;
        const uint32_t ro = (uint32_t)min(i + kPrefetch, last) * row_in;
        rx[k] = W::load(wx, lane_in, ro);
        rd[k] = W::load(wd, lane_in, ro);
        if (GATE) rz[k] = W::load(wz, lane_in, ro);
        float bc[PR];
        if constexpr (PR % 4 == 0) {
          const float4* src = reinterpret_cast<const float4*>(cur + (i - r_begin) * PR);
#pragma unroll
          for (int q = 0; q < PR / 4; ++q) {
            const float4 t = src[q];
            bc[4 * q] = t.x; bc[4 * q + 1] = t.y; bc[4 * q + 2] = t.z; bc[4 * q + 3] = t.w;
          }
        } else {
#pragma unroll
          for (int q = 0; q < PR; ++q) bc[q] = cur[(i - r_begin) * PR + q];
        }
        const float y = row_step<Tin, NS, SOFTPLUS, DISC, READOUT, GATE>(xx, dd, zz, bc, A2, dskip, h, e, sum_delta);
        if (READOUT) win<Tout, 1>::store(wy, lane_out, (uint32_t)i * row_out, &y);
        // keep rows in program order so the B / C of later rows are not all read into registers early
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // rows of this block past the last full group (only in the sequence's final block)
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int i = r_full + k;
      if (i < r_end) {
        float bc[PR];
#pragma unroll
        for (int q = 0; q < PR; ++q) bc[q] = cur[(i - r_begin) * PR + q];
        const float y = row_step<Tin, NS, SOFTPLUS, DISC, READOUT, GATE>(
            W::get(rx[k], 0), W::get(rd[k], 0) + bias, GATE ? W::get(rz[k], 0) : 0.0f, bc, A2, dskip, h, e,
            sum_delta);
        if (READOUT) win<Tout, 1>::store(wy, lane_out, (uint32_t)i * row_out, &y);
      }
    }
    if (blk + 1 < nblk) st.put(lds + ((blk + 1) & 1) * Stage::PER_BLOCK);
  }
}

// Loads the lane's row of A (scaled to base 2) and picks the wave's discretisation (see Disc).
template <int NS, bool SOFTPLUS>
__device__ __forceinline__ int load_A(const SelParams& p, int64_t dl, float* A2) {
  bool nonpos = true;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const float a = p.A[dl * NS + n];
    A2[n] = a * kLog2e;
    nonpos = nonpos && !(a > 0.0f);
  }
  return (SOFTPLUS && __all(nonpos)) ? kExp : kClamp;
}

// ----------------------------------------------------------------------------- pass 1: aggregates
// One aggregate unit of one channel block: the unit's rows from zero, storing prod abar and the state
// reached per state and channel.
template <typename Tin, int NS, bool SOFTPLUS>
__device__ __forceinline__ void agg_unit(const SelParams& p, int64_t u, int64_t cb, float* lds) {
  Unit U;
  if (p.vagg != nullptr) {  // packed plan: aggregate unit u (a middle piece's rows)
    if (u >= (int64_t)p.vcount[1]) return;
    const int4 ve = p.vagg[u];
    U.row0 = (int64_t)p.cu[ve.x] + ve.y;
    U.row1 = U.row0 + ve.z;
  } else {
    U = unit_of(p, u);
    if (!U.valid || U.last) return;
  }
  const int64_t d = cb * kThreads + threadIdx.x;
  const bool active = d < p.D;
  const int64_t dl = active ? d : p.D - 1;  // lanes past D recompute channel D-1, store nothing
  float A2[NS];
  const int disc = load_A<NS, SOFTPLUS>(p, dl, A2);
  const float bias = p.dt_bias ? p.dt_bias[dl] : 0.0f;
  float h[NS], e[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) { h[n] = 0.0f; e[n] = 0.0f; }
  float sum_delta = 0.0f;
  if (disc == kExp)
    run_rows<Tin, float, NS, SOFTPLUS, kExp, false, false>(p, U.row0, U.row1, dl, A2, bias, 0.0f, h, e, sum_delta, lds);
  else
    run_rows<Tin, float, NS, SOFTPLUS, kClamp, false, false>(p, U.row0, U.row1, dl, A2, bias, 0.0f, h, e, sum_delta,
                                                             lds);
  if (!active) return;
  // prod abar = 2^(sum of the exponents): A2 sum(delta) without the clamp (rebuilt from the stored
  // delta sum where it is read), else the clamped sum
  p.sdelta[u * p.D + d] = sum_delta;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if (disc == kClamp) p.aggP[(u * NS + n) * p.D + d] = hw_exp2(e[n]);
    p.aggH[(u * NS + n) * p.D + d] = h[n];
  }
}

// Product of abar over aggregate unit u for state n of channel d: rebuilt from the unit's delta sum
// where the clamp cannot act, else the stored product.  One load either way (decay_src), issued
// with the others before any is used (decay_of).
template <int NS>
__device__ __forceinline__ const float* decay_src(const SelParams& p, int64_t u, int n, int64_t d, bool from_sum) {
  return from_sum ? p.sdelta + u * p.D + d : p.aggP + (u * NS + n) * p.D + d;
}
__device__ __forceinline__ float decay_of(float v, float A2n, bool from_sum) { return from_sum ? hw_exp2(A2n * v) : v; }

template <typename Tin, int NS, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads, 4) void selective_aggregate_kernel(SelParams p) {
  __shared__ float lds[2 * BCStage<NS, false>::PER_BLOCK];
  agg_unit<Tin, NS, SOFTPLUS>(p, blockIdx.x, blockIdx.y, lds);
}

// Packed plan: one workgroup per (piece, channel block) folds the piece's aggregate units in order
// into the piece's aggregate (prod abar and the state reached from zero); units in rounds of JB with
// all their loads in flight together.
template <int NS>
__global__ __launch_bounds__(kThreads) void selective_vpiece_kernel(SelParams p) {
  const int64_t slot = blockIdx.x;
  if (slot >= (int64_t)p.vcount[2]) return;
  const int64_t d = (int64_t)blockIdx.y * kThreads + threadIdx.x;
  if (d >= p.D) return;
  const int2 pc = p.vpiece[slot];
  const int64_t first = pc.x;
  const int q = pc.y;
  if (q == 0) return;  // a first piece's slot: its scan leaves the end state there
  float Pp[NS], Hp[NS], A2[NS];
  bool from_sum[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    Pp[n] = 1.0f;
    Hp[n] = 0.0f;
    const float a = p.A[d * NS + n];
    A2[n] = a * kLog2e;
    from_sum[n] = p.softplus && !(a > 0.0f);
  }
  constexpr int JB = 4;
  for (int j0 = 0; j0 < q; j0 += JB) {
    float Pj[JB][NS], Hj[JB][NS];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int64_t uj = first + min(j0 + jj, q - 1);
      const int64_t base = uj * NS * p.D + d;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        Pj[jj][n] = *decay_src<NS>(p, uj, n, d, from_sum[n]);
        Hj[jj][n] = p.aggH[base + n * p.D];
      }
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
#pragma unroll
      for (int n = 0; n < NS; ++n) Pj[jj][n] = decay_of(Pj[jj][n], A2[n], from_sum[n]);
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      if (j0 + jj < q) {
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          Hp[n] = fmaf(Pj[jj][n], Hp[n], Hj[jj][n]);
          Pp[n] *= Pj[jj][n];
        }
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    p.pieceP[(slot * NS + n) * p.D + d] = Pp[n];
    p.pieceH[(slot * NS + n) * p.D + d] = Hp[n];
  }
}

template <typename Tin, typename Tout, int NS, bool SOFTPLUS, bool GATE>
__device__ __forceinline__ void scan_rows(const SelParams& p, const Unit& U, int disc, int64_t dl, const float* A2,
                                          float bias, float dskip, float* h, float* e, float& sum_delta, float* lds) {
  if (disc == kExp)
    run_rows<Tin, Tout, NS, SOFTPLUS, kExp, true, GATE>(p, U.row0, U.row1, dl, A2, bias, dskip, h, e, sum_delta, lds);
  else
    run_rows<Tin, Tout, NS, SOFTPLUS, kClamp, true, GATE>(p, U.row0, U.row1, dl, A2, bias, dskip, h, e, sum_delta,
                                                          lds);
}

// One scan unit of one channel block: the rows from the unit's carry-in, with readout.
template <typename Tin, typename Tout, int NS, bool SOFTPLUS>
__device__ __forceinline__ void scan_unit(const SelParams& p, int64_t u, int64_t cb, float* lds) {
  const Unit U = unit_of(p, u);
  if (!U.valid) return;
  const int64_t d = cb * kThreads + threadIdx.x;
  const bool active = d < p.D;
  const int64_t dl = active ? d : p.D - 1;  // lanes past D recompute channel D-1 exactly
  float A2[NS];
  const int disc = load_A<NS, SOFTPLUS>(p, dl, A2);
  const float bias = p.dt_bias ? p.dt_bias[dl] : 0.0f;
  const float dskip = p.Dskip ? p.Dskip[dl] : 0.0f;

  // carry-in of this segment: h0 (or zero) for a sequence's first segment, else the carry pass's
  float h[NS], e[NS];
  if (U.seg == 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = p.h0 ? p.h0[(U.seq * p.D + dl) * NS + n] : 0.0f;
  } else if (p.vscan) {
    // packed plan: the first piece's end state folded through the aggregates of the middle pieces
    // before this one
    const int64_t first = p.vseq[U.seq].w;
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = p.pieceH[(first * NS + n) * p.D + dl];
    for (int64_t j = first + 1; j <= U.carry; ++j) {
#pragma unroll
      for (int n = 0; n < NS; ++n)
        h[n] = fmaf(p.pieceP[(j * NS + n) * p.D + dl], h[n], p.pieceH[(j * NS + n) * p.D + dl]);
    }
  } else {
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = p.carry[(u * NS + n) * p.D + dl];
  }
  float sum_delta = 0.0f;
  if (p.z)
    scan_rows<Tin, Tout, NS, SOFTPLUS, true>(p, U, disc, dl, A2, bias, dskip, h, e, sum_delta, lds);
  else
    scan_rows<Tin, Tout, NS, SOFTPLUS, false>(p, U, disc, dl, A2, bias, dskip, h, e, sum_delta, lds);

  if (!active) return;
  if (U.last) {
    if (p.h_last) {
#pragma unroll
      for (int n = 0; n < NS; ++n) p.h_last[(U.seq * p.D + d) * NS + n] = h[n];
    }
  } else if (p.vscan && U.seg == 0) {  // packed plan: a long sequence's first piece
    const int64_t first = p.vseq[U.seq].w;
#pragma unroll
    for (int n = 0; n < NS; ++n) p.pieceH[(first * NS + n) * p.D + d] = h[n];
  }
}

// Batched plan and unpacked varlen: grid (unit, channel block).  Packed plan, phase 2: a
// one-dimensional grid over the scan units after phase 1's, unit-major (a unit's channel blocks are
// dispatched together, longest units first).
template <typename Tin, typename Tout, int NS, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void selective_scan_kernel(SelParams p) {
  __shared__ float lds[2 * BCStage<NS, true>::PER_BLOCK];
  if (p.vscan) {
    const int64_t u = blockIdx.x / p.nblk;
    scan_unit<Tin, Tout, NS, SOFTPLUS>(p, (int64_t)p.vcount[3] + u, (int64_t)blockIdx.x - u * p.nblk, lds);
  } else {
    scan_unit<Tin, Tout, NS, SOFTPLUS>(p, blockIdx.x, blockIdx.y, lds);
  }
}

// Packed plan, phase 1: the first pieces' scan units (longest first), then the aggregate units of the
// middle pieces, in one one-dimensional grid, unit-major.
template <typename Tin, typename Tout, int NS, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void selective_phase1_kernel(SelParams p) {
  __shared__ float lds[2 * BCStage<NS, true>::PER_BLOCK];  // the larger of the two stages
  const int64_t s1 = (int64_t)p.vcount[3] * p.nblk;
  const int64_t b = blockIdx.x;
  if (b < s1) {
    const int64_t u = b / p.nblk;
    scan_unit<Tin, Tout, NS, SOFTPLUS>(p, u, b - u * p.nblk, lds);
  } else {
    const int64_t u = (b - s1) / p.nblk;
    agg_unit<Tin, NS, SOFTPLUS>(p, u, b - s1 - u * p.nblk, lds);
  }
}

// ----------------------------------------------------------------------------- carry pass
// One thread per (sequence, state n, channel d): walks the sequence's segments in order,
// carry[s] = h; h = P[s] h + H[s], starting from h0 (or zero).  The aggregate loads do not depend
// on h, so they are issued ahead of the multiply-add chain.
// (ROLE tells apart, by name, the forward's launches from the backward's at its own segment length)
template <int NS, int ROLE = 0>
__global__ __launch_bounds__(kThreads) void selective_carry_kernel(SelParams p) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_seq = NS * p.D;
  const int64_t seq = gid / per_seq;
  if (seq >= p.nseq) return;
  const int64_t e = gid - seq * per_seq;  // n * D + d
  const int64_t n = e / p.D;
  const int64_t d = e - n * p.D;
  int64_t first, count;
  if (p.cu == nullptr) {
    first = seq * p.nseg;
    count = p.nseg;
  } else {
    const int2 r = p.seq_units[seq];
    first = r.x;
    count = r.y;
  }
  float h = p.h0 ? p.h0[(seq * p.D + d) * NS + n] : 0.0f;
  const float a = p.A[d * NS + n];
  const float A2 = a * kLog2e;
  const bool from_sum = p.softplus && !(a > 0.0f);
  constexpr int K = 32;
  for (int64_t s0 = 0; s0 < count; s0 += K) {
    float P[K], H[K];
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const int64_t s = min(s0 + q, count - 1);
      P[q] = *decay_src<NS>(p, first + s, (int)n, d, from_sum);
      H[q] = p.aggH[((first + s) * NS + n) * p.D + d];
    }
#pragma unroll
    for (int q = 0; q < K; ++q) P[q] = decay_of(P[q], A2, from_sum);
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const int64_t s = s0 + q;
      if (s > 0 && s < count) p.carry[((first + s) * NS + n) * p.D + d] = h;
      if (s + 1 < count) h = fmaf(P[q], h, H[q]);  // a sequence's last segment has no aggregate
    }
  }
}

// Pieces of a packed sequence of `len` rows: unsplit up to F rows; else a first piece of F rows and
// the rest cut into pieces of a multiple of Y rows (all but the last full), as few as keep them
// within P.
struct Pieces {
  int64_t len, first, piece, count;  // rows, rows of the first piece, of every later piece but the last, pieces
  __device__ __forceinline__ int64_t rows(int64_t k) const {
    return k == 0 ? first : (k + 1 < count ? piece : len - first - (k - 1) * piece);
  }
  __device__ __forceinline__ int64_t start(int64_t k) const { return k == 0 ? 0 : first + (k - 1) * piece; }
};
__device__ __forceinline__ Pieces pieces_of(int64_t len, int64_t F, int64_t P, int64_t Y) {
  Pieces r;
  r.len = len;
  r.piece = 0;
  if (len <= F) {
    r.first = len;
    r.count = len > 0 ? 1 : 0;
    return r;
  }
  r.first = F;
  const int64_t rest = len - F;
  const int64_t k = (rest + P - 1) / P;
  r.piece = ((rest + k - 1) / k + Y - 1) / Y * Y;
  r.count = 1 + (rest + r.piece - 1) / r.piece;
  return r;
}

constexpr int kLenBuckets = 256;  // scan units are ordered by floor(8 log2(rows)), longest first
__device__ __forceinline__ int len_bucket(int64_t rows) {
  const int b = (int)(8.0f * __builtin_amdgcn_logf((float)rows));
  return b < 0 ? 0 : (b >= kLenBuckets ? kLenBuckets - 1 : b);
}

// Inclusive sum over the 1024 threads of the workgroup (all threads must call it): within each wave
// by shuffles, then over the 16 wave totals by wave 0.
__device__ __forceinline__ int block_inclusive_sum(int v, int* buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) buf[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? buf[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int t = __shfl_up(w, off);
      if (lane >= off) w += t;
    }
    if (lane < 16) buf[lane] = w;
  }
  __syncthreads();
  const int r = v + (wave > 0 ? buf[wave - 1] : 0);
  __syncthreads();  // buf is reused by the next call
  return r;
}

// Packed plan, one workgroup.  The scan runs in two phases.  Phase 1 scans every sequence's first
// piece from its initial state (a long sequence's first piece leaves its end state in the sequence's
// first piece slot) while the aggregate units cover the middle pieces (every piece but the first and
// the last), Y rows each; phase 2 scans the later pieces, each from the first piece's end state folded
// through the aggregates of the middle pieces before it.  Tables: per sequence, the aggregate units,
// the piece slots (the first piece's is filled by its scan, the others by the piece fold), the scan
// units of phase 1 then of phase 2, each ordered by length (longest first; the order among units of
// one length bucket is not fixed, and no result depends on it), the counts, and the final state of
// zero-length sequences (= their initial state, or zero).
__global__ __launch_bounds__(1024) void selective_vplan_kernel(const int32_t* cu, int64_t nseq, int64_t F, int64_t P,
                                                               int64_t Y, int* count, int4* scan, int4* agg,
                                                               int4* seqtab, int2* piece, int64_t D, int64_t N,
                                                               const float* h0, float* h_last) {
  __shared__ int s_buf[1024];
  __shared__ int s_hist[2 * kLenBuckets];  // phase 1 buckets, then phase 2 buckets
  __shared__ int s_base_agg, s_base_carry, s_units, s_first;
  for (int b = threadIdx.x; b < 2 * kLenBuckets; b += 1024) s_hist[b] = 0;
  if (threadIdx.x == 0) { s_base_agg = 0; s_base_carry = 0; s_units = 0; s_first = 0; }
  __syncthreads();
  // pass 1: slots, per-sequence table, aggregate units, length histogram of the scan units
  for (int64_t blk = 0; blk < nseq; blk += 1024) {
    const int64_t sq = blk + threadIdx.x;
    Pieces pc{0, 0, 0, 0};
    if (sq < nseq) pc = pieces_of((int64_t)cu[sq + 1] - cu[sq], F, P, Y);
    const int q = pc.count > 1 ? (int)(pc.piece / Y) : 0;  // aggregate units per middle piece
    const int nagg = pc.count > 2 ? (int)((pc.count - 2) * q) : 0;
    const int ncarry = pc.count > 1 ? (int)(pc.count - 1) : 0;
    const int ia = block_inclusive_sum(nagg, s_buf);
    const int ic = block_inclusive_sum(ncarry, s_buf);
    const int iu = block_inclusive_sum((int)pc.count, s_buf);
    const int i1 = block_inclusive_sum(pc.count > 0 ? 1 : 0, s_buf);
    const int first_agg = s_base_agg + ia - nagg, first_carry = s_base_carry + ic - ncarry;
    if (sq < nseq) {
      seqtab[sq] = make_int4(first_agg, nagg, q, first_carry);
      for (int j = 0; j < nagg; ++j)
        agg[first_agg + j] = make_int4((int)sq, (int)(pc.first + j * Y), (int)Y, first_carry + 1 + j / q);
      if (ncarry > 0) piece[first_carry] = make_int2(0, 0);  // filled by the first piece's scan
      for (int k = 1; k < ncarry; ++k) piece[first_carry + k] = make_int2(first_agg + (k - 1) * q, q);
      for (int64_t k = 0; k < pc.count; ++k)
        atomicAdd(&s_hist[(k == 0 ? 0 : kLenBuckets) + len_bucket(pc.rows(k))], 1);
    }
    __syncthreads();
    if (threadIdx.x == 1023) { s_base_agg += ia; s_base_carry += ic; s_units += iu; s_first += i1; }
    __syncthreads();
  }
  // bucket offsets, phase 1 first, longest bucket first within a phase: thread t < 2 kLenBuckets holds
  // bucket (t / kLenBuckets) kLenBuckets + kLenBuckets - 1 - t % kLenBuckets
  {
    const int t = (int)threadIdx.x;
    const int b = t < 2 * kLenBuckets ? (t / kLenBuckets) * kLenBuckets + kLenBuckets - 1 - t % kLenBuckets : -1;
    const int c = b >= 0 ? s_hist[b] : 0;
    const int incl = block_inclusive_sum(c, s_buf);
    if (b >= 0) s_hist[b] = incl - c;
    __syncthreads();
  }
  // pass 2: scan units into their buckets; zero-length sequences get h_last = h0 (or zero)
  __shared__ int s_empty[1024];
  __shared__ int s_nempty;
  for (int64_t blk = 0; blk < nseq; blk += 1024) {
    const int64_t sq = blk + threadIdx.x;
    if (threadIdx.x == 0) s_nempty = 0;
    __syncthreads();
    if (sq < nseq) {
      const Pieces pc = pieces_of((int64_t)cu[sq + 1] - cu[sq], F, P, Y);
      if (pc.len == 0 && h_last) s_empty[atomicAdd(&s_nempty, 1)] = (int)sq;
      const int first_carry = seqtab[sq].w;
      for (int64_t k = 0; k < pc.count; ++k) {
        const int64_t rows = pc.rows(k);
        const int pos = atomicAdd(&s_hist[(k == 0 ? 0 : kLenBuckets) + len_bucket(rows)], 1);
        scan[pos] = make_int4((int)sq, (int)pc.start(k), (int)rows, k == 0 ? -1 : first_carry + (int)k - 1);
      }
    }
    __syncthreads();
    for (int k = 0; k < s_nempty; ++k) {
      const int64_t es = s_empty[k];
      for (int64_t e = threadIdx.x; e < D * N; e += 1024) h_last[es * D * N + e] = h0 ? h0[es * D * N + e] : 0.0f;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    count[0] = s_units;
    count[1] = s_base_agg;
    count[2] = s_base_carry;
    count[3] = s_first;
  }
}

// ----------------------------------------------------------------------------- varlen planner
// One workgroup: unit table (seq, seg) in sequence order, unit count, and the final state of
// zero-length sequences (= their initial state, or zero).
__global__ __launch_bounds__(1024) void selective_plan_kernel(const int32_t* cu, int64_t nseq, int64_t T,
                                                              int2* units, int* n_units, int2* seq_units, int64_t D,
                                                              int64_t N, const float* h0, float* h_last) {
  __shared__ int s_scan[1024];
  __shared__ int s_base;
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  for (int64_t blk = 0; blk < nseq; blk += 1024) {
    const int64_t sq = blk + threadIdx.x;
    int cnt = 0;
    if (sq < nseq) {
      const int64_t len = (int64_t)cu[sq + 1] - cu[sq];
      cnt = (int)((len + T - 1) / T);
    }
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = threadIdx.x >= off ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += add;
      __syncthreads();
    }
    const int base = s_base + s_scan[threadIdx.x] - cnt;
    for (int sgi = 0; sgi < cnt; ++sgi) units[base + sgi] = make_int2((int)sq, sgi);
    if (sq < nseq) seq_units[sq] = make_int2(base, cnt);
    __syncthreads();
    if (threadIdx.x == 1023) s_base += s_scan[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_units = s_base;
  if (h_last) {
    for (int64_t sq = 0; sq < nseq; ++sq) {
      if (cu[sq + 1] != cu[sq]) continue;
      for (int64_t e = threadIdx.x; e < D * N; e += 1024)
        h_last[sq * D * N + e] = h0 ? h0[sq * D * N + e] : 0.0f;
    }
  }
}

// ----------------------------------------------------------------------------- decode update
template <typename Tin, typename Tout, int NS, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void selective_update_kernel(
    int64_t B, int64_t D, const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
    const float* Dskip, const void* z, const float* dt_bias, float* state, void* y) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= B * D) return;
  const int64_t b = idx / D;
  const int64_t d = idx - b * D;
  float dd = io<Tin>::load(dt, idx) + (dt_bias ? dt_bias[d] : 0.0f);
  const float delta = SOFTPLUS ? softplus_in<Tin>(dd) : dd;
  const float xx = io<Tin>::load(x, idx);
  const float dx = delta * xx;
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    float dA = delta * A[d * NS + n] * kLog2e;
    dA = dA > kClampLog2 ? kClampLog2 : dA;
    const float ab = hw_exp2(dA);
    const float hn = fmaf(ab, state[idx * NS + n], dx * io<Tin>::load(Bm, b * NS + n));
    state[idx * NS + n] = hn;
    acc = fmaf(io<Tin>::load(Cm, b * NS + n), hn, acc);
  }
  if (Dskip) acc = fmaf(Dskip[d], xx, acc);
  if (z) acc *= silu_f(io<Tin>::load(z, idx));
  io<Tout>::store(y, idx, acc);
}

// ----------------------------------------------------------------------------- dispatch helpers
// Waves the scan pass keeps resident per CU (its register budget allows 3 per SIMD): the plan cuts
// sequences so that all scan waves fit in one resident round.
constexpr int64_t kScanWavesPerCU = 12;

int64_t device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

template <typename Tin, typename Tout, int NS>
hipError_t launch_passes(const SelParams& p, int64_t U, bool softplus, hipStream_t s) {
  const dim3 grid((unsigned)U, (unsigned)((p.D + kThreads - 1) / kThreads));
  const bool split = (p.cu != nullptr) || (p.nseg > 1);
  if (split) {
    if (softplus)
      hipLaunchKernelGGL((selective_aggregate_kernel<Tin, NS, true>), grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((selective_aggregate_kernel<Tin, NS, false>), grid, dim3(kThreads), 0, s, p);
    const int64_t nthreads = p.nseq * NS * p.D;
    hipLaunchKernelGGL((selective_carry_kernel<NS>), dim3((unsigned)((nthreads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, p);
  }
  if (softplus)
    hipLaunchKernelGGL((selective_scan_kernel<Tin, Tout, NS, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((selective_scan_kernel<Tin, Tout, NS, false>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_by_n(const SelParams& p, int64_t U, bool softplus, hipStream_t s) {
  switch (p.N) {
    case 1: return launch_passes<Tin, Tout, 1>(p, U, softplus, s);
    case 2: return launch_passes<Tin, Tout, 2>(p, U, softplus, s);
    case 4: return launch_passes<Tin, Tout, 4>(p, U, softplus, s);
    case 8: return launch_passes<Tin, Tout, 8>(p, U, softplus, s);
    default: return launch_passes<Tin, Tout, 16>(p, U, softplus, s);
  }
}

// Packed plan: phase 1 (first pieces and aggregate units; at most one first piece per sequence), the
// piece fold, phase 2 (the later pieces: at most one per piece slot).
template <typename Tin, typename Tout, int NS>
hipError_t launch_packed(const SelParams& p, int64_t A, int64_t C, bool softplus, hipStream_t s) {
  const dim3 grid1((unsigned)((p.nseq + A) * p.nblk));
  if (softplus) hipLaunchKernelGGL((selective_phase1_kernel<Tin, Tout, NS, true>), grid1, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((selective_phase1_kernel<Tin, Tout, NS, false>), grid1, dim3(kThreads), 0, s, p);
  if (C > 0) {
    if (A > 0)
      hipLaunchKernelGGL((selective_vpiece_kernel<NS>), dim3((unsigned)C, (unsigned)p.nblk), dim3(kThreads), 0, s, p);
    const dim3 grid2((unsigned)(C * p.nblk));
    if (softplus) hipLaunchKernelGGL((selective_scan_kernel<Tin, Tout, NS, true>), grid2, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((selective_scan_kernel<Tin, Tout, NS, false>), grid2, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <typename Tin, typename Tout, int NS>
void launch_update_n(const SelectiveUpdateArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.B * a.D + kThreads - 1) / kThreads));
  if (a.dt_softplus)
    hipLaunchKernelGGL((selective_update_kernel<Tin, Tout, NS, true>), grid, dim3(kThreads), 0, s, a.B, a.D, a.x,
                       a.dt, a.A, a.Bm, a.Cm, a.Dskip, a.z, a.dt_bias, a.state, a.y);
  else
    hipLaunchKernelGGL((selective_update_kernel<Tin, Tout, NS, false>), grid, dim3(kThreads), 0, s, a.B, a.D, a.x,
                       a.dt, a.A, a.Bm, a.Cm, a.Dskip, a.z, a.dt_bias, a.state, a.y);
}

template <typename Tin, typename Tout>
void launch_update_t(const SelectiveUpdateArgs& a, hipStream_t s) {
  switch (a.N) {
    case 1: launch_update_n<Tin, Tout, 1>(a, s); break;
    case 2: launch_update_n<Tin, Tout, 2>(a, s); break;
    case 4: launch_update_n<Tin, Tout, 4>(a, s); break;
    case 8: launch_update_n<Tin, Tout, 8>(a, s); break;
    default: launch_update_n<Tin, Tout, 16>(a, s); break;
  }
}

struct Plan {
  int64_t T, nseg, U;
  // packed varlen forward plan (packed = true): a first piece of F rows, later pieces of at most P
  // rows, aggregate units of Y rows; bounds on aggregate units (A), piece slots (C) and scan units (S)
  bool packed;
  int64_t F, P, Y, A, C, S;
};

// Packed varlen plan.  A sequence is scanned by one workgroup per channel block, from its start to
// its end, unless it is longer than F rows; then its first F rows are scanned in phase 1, beside the
// aggregate units of its middle pieces, and the rest, cut into as few pieces as keep them within P
// rows, in phase 2 (only the middle pieces pass through the aggregate kernel).  F and P are
// fractions of the rows each compute unit scans on average, so that in each phase the longest
// pieces, started first, end with the rest.
constexpr int64_t kFirstNum = 1, kFirstDen = 4;  // F = rows per compute unit * kFirstNum / kFirstDen
constexpr int64_t kLaterNum = 1, kLaterDen = 4;  // P = rows per compute unit * kLaterNum / kLaterDen
constexpr int64_t kAggRows = 256;                 // Y


// Longest segment whose rows span under 2^31 bytes of any activation (buffer windows).
int64_t max_segment(int64_t D) {
  const int64_t m = (((int64_t)1 << 31) - 1) / (D * 4) / 16 * 16;
  return m < 16 ? 16 : m;
}

Plan make_plan(const SelectiveScanArgs& a) {
  Plan pl{};
  const int64_t kTargetWaves = device_cus() * kScanWavesPerCU;
  const int64_t max_T = max_segment(a.D);
  const int64_t waves_per_row = (a.D + 63) / 64;
  if (a.cu_seqlens == nullptr) {
    const int64_t row_waves = a.B * waves_per_row;
    int64_t want = (kTargetWaves + row_waves - 1) / row_waves;  // segments per sequence
    if (want < 1) want = 1;
    int64_t T = (a.L + want - 1) / want;
    T = ((T + 15) / 16) * 16;
    if (T < 16) T = 16;
    if (T > max_T) T = max_T;
    if (T > a.L) T = a.L;
    pl.T = T;
    pl.nseg = (a.L + T - 1) / T;
    pl.U = a.B * pl.nseg;
  } else {
    // Packed sequences end in partial segments of uneven length; spreading the rows over about
    // eight resident rounds of workgroups lets the hardware keep the CUs busy while those finish
    // (measured 4.8 -> 3.3 ms for 32 sequences of 600 to 15500 rows at D = 4096; 16 rounds: no gain).
    constexpr int64_t kVarlenRounds = 8;
    int64_t want = (kVarlenRounds * kTargetWaves + waves_per_row - 1) / waves_per_row;  // units over the packed rows
    if (want < 1) want = 1;
    int64_t T = (a.L + want - 1) / want;
    T = ((T + 15) / 16) * 16;
    if (T < 16) T = 16;
    if (T > max_T) T = max_T;
    pl.T = T;
    pl.nseg = 0;
    pl.U = (a.L + T - 1) / T + a.nseq;  // upper bound on sum of ceil(len / T)
    // the packed plan, when its one-dimensional scan grids fit
    const int64_t nblk = (a.D + kThreads - 1) / kThreads;
    const int64_t per_cu = (a.L * nblk + device_cus() - 1) / device_cus();
    auto rows_of = [&](int64_t num, int64_t den) {
      int64_t r = (per_cu * num / den + kAggRows - 1) / kAggRows * kAggRows;
      if (r < kAggRows) r = kAggRows;
      if (r > max_T) r = max_T / kAggRows * kAggRows;
      return r;
    };
    pl.P = rows_of(kLaterNum, kLaterDen);
    pl.F = rows_of(kFirstNum, kFirstDen);
    pl.Y = kAggRows;
    pl.A = (a.L + pl.Y - 1) / pl.Y;  // aggregate units are whole Y-row blocks inside one sequence
    // a sequence of len > F rows has a slot per piece but its last: ceil((len - F) / P) <=
    // (len - F) / P + 1 <= len / min(F, P) of them
    const int64_t m = pl.F < pl.P ? pl.F : pl.P;  // 0 when a Y-row block spans 2^31 bytes
    pl.C = m > 0 ? (a.L + m - 1) / m : 0;
    pl.S = a.nseq + pl.C;  // scan units: one per sequence plus one per slot
    pl.packed = m >= kAggRows && (a.nseq + pl.A) * nblk * kThreads < ((int64_t)1 << 31) &&
                pl.S * nblk * kThreads < ((int64_t)1 << 31);
  }
  return pl;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

template <typename Tin, typename Tout>
hipError_t launch_packed_by_n(const SelParams& p, const Plan& pl, bool softplus, hipStream_t s) {
  switch (p.N) {
    case 1: return launch_packed<Tin, Tout, 1>(p, pl.A, pl.C, softplus, s);
    case 2: return launch_packed<Tin, Tout, 2>(p, pl.A, pl.C, softplus, s);
    case 4: return launch_packed<Tin, Tout, 4>(p, pl.A, pl.C, softplus, s);
    case 8: return launch_packed<Tin, Tout, 8>(p, pl.A, pl.C, softplus, s);
    default: return launch_packed<Tin, Tout, 16>(p, pl.A, pl.C, softplus, s);
  }
}

// ============================================================================= backward
// Gradients of the batched scan for the loss sum dy y + sum dh_last h_last.  With s_t the readout
// before the gate, ds_t = dy_t silu(z_t) (or dy_t) and the reverse state q (q_L = dh_last,
// g_t = ds_t C_t + q_{t+1}, q_t = abar_t g_t):
//   dh0 = q_0,  dz_t = dy_t s_t silu'(z_t),  dDskip = sum ds x,  dx_t = ds_t Dskip + delta_t sum_n g B,
//   dC_tn = sum_d ds_t h_tn,  dB_tn = sum_d g_tn delta_t x_t,  and with m = [delta A <= 20] (the clamp
//   passes no gradient above 20): d delta_t = x_t sum_n g B + sum_n m g h_{t-1} abar A_n,
//   dA_n = sum m g h_{t-1} abar delta,  d dt = d delta softplus'(dt + bias),  d dt_bias = sum d dt.
// Passes over units of kBU rows (kBS sub-blocks of kBT rows), one lane per channel as in the forward:
//   1. per unit, from zero, in one sweep over its rows: the state it reaches (H), prod abar (P), and
//      q at its first row from q = 0 past its end (Q = sum_t (prod_{s <= t} abar_s) ds_t C_t);
//   2. one thread per (sequence, state, channel): the state entering each unit (forward) and q at
//      each unit's end (reverse);
//   3. per unit: a forward sweep from its entering state gives the states at its sub-block starts
//      (bf16 inputs: its raw dt and x stay in LDS for the rest of the unit); then the sub-blocks
//      from the last to the first, each one state at a time: forward through its rows keeping
//      h_{t-1} and abar, back through them carrying q, accumulating the row gradients; dB and dC
//      are summed over the workgroup's channels by a lane butterfly and across its waves in LDS;
//      dA, dDskip and d dt_bias leave per-unit sums;
//   4. fixed-order sums of the partial results.
constexpr int kBT = 16;         // rows per sub-block (the register tile of pass 3)
constexpr int kBS = 4;          // sub-blocks per unit
constexpr int kBU = kBT * kBS;  // rows per unit

struct SelBwdParams {
  int64_t L, D, nseg, nblk, BL;  // batched: L rows per sequence, nseg units each; BL rows in all
  const int32_t* cu;             // packed varlen: boundaries, or NULL (then the fields below are unused)
  const int2* units;             // (sequence, unit index within it) per unit
  const int* n_units;            // number of units (device)
  const int2* seq_units;         // (first unit, unit count) per sequence
  const void* x;
  const void* dt;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const float* dt_bias;
  const float* h0;
  const void* dy;
  const float* dh_last;
  float* aggP;    // [unit][N][D] prod abar over the unit (pass 1; clamp variant only, see sdelta)
  float* sdelta;  // [unit][D] delta summed over the unit: prod abar = 2^(A log2(e) sdelta) where the clamp
                  // cannot act (softplus steps, A <= 0)
  int softplus;
  float* aggH;  // [unit][N][D] the state the unit reaches from 0
  float* aggQ;  // [unit][N][D] q at the unit's first row from 0 past its end
  float* hin;   // [unit][N][D] the state entering the unit (pass 2)
  float* qend;  // [unit][N][D] q past the unit's last row (pass 2)
  void* dx;
  void* ddt;
  void* dz;
  float* dBm_part;  // [nblk][B L][N] per channel block
  float* dCm_part;
  float* dA_part;     // [unit][N][D]
  float* dD_part;     // [unit][D]
  float* dbias_part;  // [unit][D]
  float* dh0;         // [B][D][N] or NULL
};

// Unit u of the backward passes: its sequence, first row and row count, and whether it is its
// sequence's first and last.
struct BUnit {
  int64_t seq, row0;
  int R;
  bool valid, first, last;
};
__device__ __forceinline__ BUnit bwd_unit(const SelBwdParams& p, int64_t u) {
  BUnit r;
  int64_t seg, end;
  if (p.cu == nullptr) {
    r.seq = u / p.nseg;
    seg = u - r.seq * p.nseg;
    r.row0 = r.seq * p.L + seg * kBU;
    end = (r.seq + 1) * p.L;
    r.valid = true;
  } else {
    r.valid = u < (int64_t)(*p.n_units);
    if (!r.valid) return r;
    const int2 e = p.units[u];
    r.seq = e.x;
    seg = e.y;
    r.row0 = (int64_t)p.cu[r.seq] + seg * kBU;
    end = p.cu[r.seq + 1];
  }
  r.R = (int)min<int64_t>(kBU, end - r.row0);
  r.first = seg == 0;
  r.last = r.row0 + r.R == end;
  return r;
}

// The sigmoid of the backward passes: with fp32 inputs through exp_split (about 1 ulp), for derivatives
// that scale whole gradients; with bf16 inputs (a 2e-2 budget) the plain form.
template <typename Tin>
__device__ __forceinline__ float sigmoid_in(float v) {
  if constexpr (sizeof(Tin) == 2) return sigmoid_f(v);
  else return sigmoid_acc_f(v);
}
template <typename Tin>
__device__ __forceinline__ float silu_in(float z) { return z * sigmoid_in<Tin>(z); }
// The step of row t for the backward passes: v = dt + bias, delta = softplus(v) (or v).  With fp32
// inputs the sum is carried as s + err (a two-sum: err is the exact rounding error of s) and the
// softplus and its derivative take err to first order.  Rounding dt + bias (|dt| of a few units) loses
// up to 2^-24 |dt| of absolute value, which softplus passes on relative to its far smaller result; left
// in, it is the largest error of d dt (a third of the fp32 total in an emulation of these passes).
struct StepIn {
  float s, err;
};
template <typename Tin>
__device__ __forceinline__ StepIn step_in(float dt, float bias) {
  StepIn r;
  r.s = dt + bias;
  if constexpr (sizeof(Tin) == 2) {
    r.err = 0.0f;
  } else {
    const float bb = r.s - dt;
    r.err = (dt - (r.s - bb)) + (bias - bb);
  }
  return r;
}
template <typename Tin, bool SOFTPLUS>
__device__ __forceinline__ float step_delta(StepIn v) {
  if (!SOFTPLUS) return v.s;
  const float sp = softplus_in<Tin>(v.s);
  if constexpr (sizeof(Tin) == 2) {
    return sp;
  } else {
    const float sg = hw_exp2((v.s - sp) * kLog2e);  // softplus'(s) = sigmoid(s) = e^(s - softplus(s))
    return v.s > 20.0f ? sp : fmaf(sg, v.err, sp);
  }
}
// softplus'(v) as torch takes it: sigmoid(v), and 1 above the threshold 20.
template <typename Tin>
__device__ __forceinline__ float step_grad(StepIn v) {
  if (v.s > 20.0f) return 1.0f;
  const float sg = sigmoid_in<Tin>(v.s);
  if constexpr (sizeof(Tin) == 2) return sg;
  else return fmaf(sg * (1.0f - sg), v.err, sg);
}
// silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
template <typename Tin>
__device__ __forceinline__ float silu_grad_in(float z) {
  const float sg = sigmoid_in<Tin>(z);
  return sg * fmaf(z, 1.0f - sg, 1.0f);
}

// The lane's row of A scaled to base 2, and the wave's discretisation (as load_A).
template <int NS, bool SOFTPLUS>
__device__ __forceinline__ int bwd_load_A(const float* A, int64_t dl, float* A2) {
  bool nonpos = true;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const float a = A[dl * NS + n];
    A2[n] = a * kLog2e;
    nonpos = nonpos && !(a > 0.0f);
  }
  return (SOFTPLUS && __all(nonpos)) ? kExp : kClamp;
}

// The unit's rows of B and C, as fp32 [row][n] (rows past the unit read as 0).
template <typename Tin, int NS>
__device__ __forceinline__ void stage_bc(const SelBwdParams& p, int64_t row0, int R, float* sB, float* sC) {
  for (int e = threadIdx.x; e < kBU * NS; e += kThreads) {
    const int t = e / NS;
    const int64_t idx = (row0 + min(t, R - 1)) * NS + (e - t * NS);
    sB[e] = t < R ? io<Tin>::load(p.Bm, idx) : 0.0f;
    sC[e] = t < R ? io<Tin>::load(p.Cm, idx) : 0.0f;
  }
}

// Sum of v[j] over the 64 lanes of the wave, for 16 values j at once: each exchange step halves the
// values a lane keeps (the half picked by one lane bit) and adds its partner's other half.  On return
// lanes with (lane & 3) == 0 hold the total of value (lane >> 2) & 15 in v[0].  All exchanges are VALU
// lane moves: v_permlane32_swap / v_permlane16_swap for partners 32 and 16 lanes apart (the pair
// (v[i], v[i + H]) comes back as (lower half of both, upper half of both), so one add leaves each half
// with the sum of the value it keeps), then DPP within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRor8 = 0x128;        // lane l of a row reads lane (l + 8) mod 16
constexpr int kDppHalfMirror = 0x141;  // lane l of 8 reads lane 7 - l
constexpr int kDppQuad2301 = 0x4E;     // lane l of 4 reads l ^ 2
constexpr int kDppQuad1032 = 0xB1;     // lane l of 4 reads l ^ 1
__device__ __forceinline__ void wave_sum16(float (&v)[16], int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // lanes 32 apart: the lower half keeps v[i], the upper v[i + 8]
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // rows 16 apart: even rows keep v[i], odd rows v[i + 4]
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // lanes 8 apart
    const float lo = v[i] + dpp_mov<kDppRor8>(v[i]), hi = v[i + 2] + dpp_mov<kDppRor8>(v[i + 2]);
    v[i] = b3 ? hi : lo;
  }
  {  // lanes 4 apart (l and 7 - l differ in bit 2 and agree above it)
    const float lo = v[0] + dpp_mov<kDppHalfMirror>(v[0]), hi = v[1] + dpp_mov<kDppHalfMirror>(v[1]);
    v[0] = b2 ? hi : lo;
  }
  v[0] += dpp_mov<kDppQuad2301>(v[0]);
  v[0] += dpp_mov<kDppQuad1032>(v[0]);
}

// ----------------------------------------------------------------------------- pass 1
// Within a unit the rows go in blocks: a block's state from zero (Hk) and its weighted adjoint sum (Qk,
// with the running product of abar restarted at the block) are folded into the unit's with the block's
// decay product applied as one exponential, 2^(A2 sum delta) (2^(sum of the clamped exponents) when the
// clamp can act).  fp32 inputs take blocks of kBT rows, so no product of rounded decays runs longer than
// that; bf16 inputs take the unit as one block (its 64 rounded decays move the sums by a few fp32 ulps,
// far below what the inputs' rounding allows).
template <typename Tin, int NS, bool SOFTPLUS, bool GATE, int DISC>
__device__ __forceinline__ void bwd_agg_rows(const SelBwdParams& p, int64_t row0, int R, int64_t dl,
                                             const float* A2, float bias, const float* sB, const float* sC,
                                             float* P, float* H, float* Q, float& sdelta) {
  using W = win<Tin, 1>;
  constexpr int es = sizeof(Tin);
  constexpr int kBlk = sizeof(Tin) == 2 ? kBU : kBT;  // rows per block
  static_assert(kBlk % kPrefetch == 0, "blocks hold whole prefetch groups");
  const auto wdt = unit_window(p.dt, row0, R, p.D, es), wxx = unit_window(p.x, row0, R, p.D, es);
  const auto wdy = unit_window(p.dy, row0, R, p.D, es), wzz = unit_window(GATE ? p.z : p.dy, row0, R, p.D, es);
  const uint32_t lane_in = (uint32_t)(dl * es), row_in = (uint32_t)(p.D * es);
  typename W::raw rd[kPrefetch], rx[kPrefetch], ry[kPrefetch], rz[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    const uint32_t ro = (uint32_t)min(k, R - 1) * row_in;
    rd[k] = W::load(wdt, lane_in, ro);
    rx[k] = W::load(wxx, lane_in, ro);
    ry[k] = W::load(wdy, lane_in, ro);
    if (GATE) rz[k] = W::load(wzz, lane_in, ro);
  }
  float es_tot[NS];     // the clamped exponents summed over the blocks done (clamp variant)
  float sd_tot = 0.0f;  // delta summed over the blocks done
#pragma unroll
  for (int n = 0; n < NS; ++n) { H[n] = 0.0f; Q[n] = 0.0f; es_tot[n] = 0.0f; }
  const int blk_end = kBlk == kBU ? 1 : R;  // one block when the unit is one (R <= kBU)
  for (int blk0 = 0; blk0 < blk_end; blk0 += kBlk) {
    float hk[NS], qk[NS], cp[NS], es_k[NS];
    float sd_k = 0.0f;
#pragma unroll
    for (int n = 0; n < NS; ++n) { hk[n] = 0.0f; qk[n] = 0.0f; cp[n] = 1.0f; es_k[n] = 0.0f; }
#pragma unroll 1
    for (int base = blk0; base < blk0 + kBlk && base < R; base += kPrefetch) {
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        const int i = base + k;
        const StepIn sv = step_in<Tin>(W::get(rd[k], 0), bias);
        const float xx = W::get(rx[k], 0), dyv = W::get(ry[k], 0);
        const float zz = GATE ? W::get(rz[k], 0) : 0.0f;
        const uint32_t ro = (uint32_t)min(i + kPrefetch, R - 1) * row_in;
        rd[k] = W::load(wdt, lane_in, ro);
        rx[k] = W::load(wxx, lane_in, ro);
        ry[k] = W::load(wdy, lane_in, ro);
        if (GATE) rz[k] = W::load(wzz, lane_in, ro);
        if (i < R) {
          const float delta = step_delta<Tin, SOFTPLUS>(sv);
          const float dxv = delta * xx;
          const float dsv = GATE ? dyv * silu_in<Tin>(zz) : dyv;
          const float* b = sB + i * NS;
          const float* c = sC + i * NS;
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            float e = delta * A2[n];
            if (DISC == kClamp) {
              e = e > kClampLog2 ? kClampLog2 : e;
              es_k[n] += e;
            }
            const float ab = hw_exp2(e);
            hk[n] = fmaf(ab, hk[n], dxv * b[n]);
            cp[n] *= ab;
            qk[n] = fmaf(cp[n], dsv * c[n], qk[n]);
            if (NS > 8 && (n & 7) == 7) __builtin_amdgcn_sched_barrier(0);
          }
          sd_k += delta;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // fold the block: H = P_k H + Hk;  Q += (decay of the blocks before) Qk
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      const float before = DISC == kClamp ? hw_exp2(es_tot[n]) : hw_exp2(A2[n] * sd_tot);
      Q[n] = fmaf(before, qk[n], Q[n]);
      const float Pk = DISC == kClamp ? hw_exp2(es_k[n]) : hw_exp2(A2[n] * sd_k);
      H[n] = fmaf(Pk, H[n], hk[n]);
      es_tot[n] += es_k[n];
    }
    sd_tot += sd_k;
  }
#pragma unroll
  for (int n = 0; n < NS; ++n) P[n] = DISC == kClamp ? hw_exp2(es_tot[n]) : hw_exp2(A2[n] * sd_tot);
  sdelta = sd_tot;
}

template <typename Tin, int NS, bool SOFTPLUS, bool GATE>
__global__ __launch_bounds__(kThreads) void selective_bwd_agg_kernel(SelBwdParams p) {
  const int64_t u = blockIdx.x;
  const BUnit U = bwd_unit(p, u);
  if (!U.valid || (U.first && U.last)) return;  // a sequence of one unit needs no aggregates
  const int64_t d = (int64_t)blockIdx.y * kThreads + threadIdx.x;
  const bool active = d < p.D;
  const int64_t dl = active ? d : p.D - 1;  // lanes past D recompute channel D-1 and store nothing
  __shared__ float sB[kBU * NS], sC[kBU * NS];
  stage_bc<Tin, NS>(p, U.row0, U.R, sB, sC);
  float A2[NS];
  const int disc = bwd_load_A<NS, SOFTPLUS>(p.A, dl, A2);
  const float bias = p.dt_bias ? p.dt_bias[dl] : 0.0f;
  __syncthreads();
  float P[NS], H[NS], Q[NS], sd;
  if (disc == kExp)
    bwd_agg_rows<Tin, NS, SOFTPLUS, GATE, kExp>(p, U.row0, U.R, dl, A2, bias, sB, sC, P, H, Q, sd);
  else
    bwd_agg_rows<Tin, NS, SOFTPLUS, GATE, kClamp>(p, U.row0, U.R, dl, A2, bias, sB, sC, P, H, Q, sd);
  if (!active) return;
  // prod abar is stored only where the carry cannot rebuild it from the delta sum
  p.sdelta[u * p.D + d] = sd;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const int64_t idx = (u * NS + n) * p.D + d;
    if (disc == kClamp) p.aggP[idx] = P[n];
    if (!U.last) p.aggH[idx] = H[n];   // the carry uses H of all units but a sequence's last
    if (!U.first) p.aggQ[idx] = Q[n];  // and Q of all but its first
  }
}

// ----------------------------------------------------------------------------- pass 2
// One thread per (sequence, state, channel): units in order for the entering states, then in reverse
// for q; the aggregates of kCarryBatch units are loaded together ahead of their sequential use.
constexpr int kCarryBatch = 8;
template <int NS>
__global__ __launch_bounds__(kThreads) void selective_bwd_carry_kernel(SelBwdParams p, int64_t nseq) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_seq = NS * p.D;
  const int64_t seq = gid / per_seq;
  if (seq >= nseq) return;
  const int64_t e = gid - seq * per_seq;  // n * D + d
  const int64_t n = e / p.D, d = e - n * p.D;
  int64_t first = seq * p.nseg, count = p.nseg;
  if (p.cu != nullptr) {
    const int2 r = p.seq_units[seq];
    first = r.x;
    count = r.y;
  }
  const int64_t base = (first * NS + n) * p.D + d, stride = NS * p.D;
  // prod abar of unit s: 2^(A log2(e) sdelta) where the clamp cannot act (the aggregate pass computes it
  // the same way there), else the stored product
  const float An = p.A[d * NS + n];
  const bool from_sum = p.softplus && !(An > 0.0f);
  const float A2 = An * kLog2e;
  auto prod_src = [&](int64_t s) {  // one load either way: the delta sum or the product
    return from_sum ? p.sdelta + (first + s) * p.D + d : p.aggP + base + s * stride;
  };
  float h = p.h0 ? p.h0[(seq * p.D + d) * NS + n] : 0.0f;
  for (int64_t s0 = 0; s0 < count; s0 += kCarryBatch) {
    float Pv[kCarryBatch], Hv[kCarryBatch];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) {
      const int64_t s = s0 + k;
      const bool need = s + 1 < count;  // the last unit's aggregate is not used
      Pv[k] = need ? *prod_src(s) : 0.0f;
      Hv[k] = need ? p.aggH[base + s * stride] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) Pv[k] = from_sum ? hw_exp2(A2 * Pv[k]) : Pv[k];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) {
      const int64_t s = s0 + k;
      if (s < count) {
        p.hin[base + s * stride] = h;
        h = fmaf(Pv[k], h, Hv[k]);
      }
    }
  }
  float q = p.dh_last ? p.dh_last[(seq * p.D + d) * NS + n] : 0.0f;
  if (count == 0 && p.dh0) p.dh0[(seq * p.D + d) * NS + n] = q;  // empty sequence: dh0 = dh_last
  for (int64_t s0 = count - 1; s0 >= 0; s0 -= kCarryBatch) {
    float Pv[kCarryBatch], Qv[kCarryBatch];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) {
      const int64_t s = s0 - k;
      const bool need = s > 0;  // the first unit's aggregate is not used
      Pv[k] = need ? *prod_src(s) : 0.0f;
      Qv[k] = need ? p.aggQ[base + s * stride] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) Pv[k] = from_sum ? hw_exp2(A2 * Pv[k]) : Pv[k];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) {
      const int64_t s = s0 - k;
      if (s >= 0) {
        p.qend[base + s * stride] = q;
        q = fmaf(Pv[k], q, Qv[k]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- pass 3
// LDS of one unit.  With bf16 inputs the unit's raw dt and x stay here from the forward sweep to the
// last sub-block; dy and z pass through a two-slot ring (the sub-block being worked on and the next).
template <typename Raw, int NS, bool STASH>
struct BwdLds {
  Raw dt[STASH ? kBU : 1][kThreads];
  Raw x[STASH ? kBU : 1][kThreads];
  Raw dy[2][kBT][kThreads];
  Raw z[2][kBT][kThreads];
  float B[kBU * NS], C[kBU * NS];    // [row][n]
  alignas(16) float Bt[NS][kBU];     // [n][row]: one state's rows of a sub-block are contiguous
  alignas(16) float Ct[NS][kBU];
  float redB[NS][kThreads / 64][kBT], redC[NS][kThreads / 64][kBT];
  // per lane and state: q entering the current sub-block from its end, and dA summed so far.  The
  // state loop indexes them by a loop counter; in registers that would be indexed register access
  // (a mode switch around every read and write)
  float qv[NS][kThreads], dA[NS][kThreads];
};

template <typename Tin, typename Tout, int NS, bool SOFTPLUS, bool GATE, int DISC, typename Lds>
__device__ __forceinline__ void bwd_grad_unit(const SelBwdParams& p, const BUnit& U, int64_t u, int64_t d,
                                              int64_t dl, bool active, Lds& S) {
  constexpr bool STASH = sizeof(Tin) == 2;
  constexpr bool kChainQ = sizeof(Tin) == 2;  // h and q run through the whole unit (bf16 inputs)
  using W = win<Tin, 1>;
  using Raw = typename W::raw;
  constexpr int es = sizeof(Tin);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = U.row0;
  const int R = U.R;
  const int nsb = (R + kBT - 1) / kBT;
  const auto wdt = unit_window(p.dt, row0, R, p.D, es), wxx = unit_window(p.x, row0, R, p.D, es);
  const auto wdy = unit_window(p.dy, row0, R, p.D, es), wzz = unit_window(GATE ? p.z : p.dy, row0, R, p.D, es);
  const uint32_t lane_in = (uint32_t)(dl * es), row_in = (uint32_t)(p.D * es);
  auto ro_of = [&](int r) { return (uint32_t)min(r, R - 1) * row_in; };
  const float bias = p.dt_bias ? p.dt_bias[dl] : 0.0f;
  const float dskip = p.Dskip ? p.Dskip[dl] : 0.0f;

  // dy and z of the last sub-block into its ring slot
  {
    const int j = nsb - 1;
#pragma unroll
    for (int t = 0; t < kBT; ++t) {
      S.dy[j & 1][t][tid] = W::load(wdy, lane_in, ro_of(j * kBT + t));
      if (GATE) S.z[j & 1][t][tid] = W::load(wzz, lane_in, ro_of(j * kBT + t));
    }
  }

#pragma unroll
  for (int n = 0; n < NS; ++n) {
    S.qv[n][tid] = p.qend[(u * NS + n) * p.D + dl];
    S.dA[n][tid] = 0.0f;
  }

  // ---- forward sweep: the states at the sub-block starts.  After it s3 holds the start of sub-block
  // nsb-1, s2 of nsb-2, s1 of nsb-3, s0 of nsb-4 (those that exist).
  float s0[NS], s1[NS], s2[NS], s3[NS];
  {
    float A2[NS], h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      A2[n] = p.A[dl * NS + n] * kLog2e;
      h[n] = p.hin[(u * NS + n) * p.D + dl];
      s0[n] = 0.0f; s1[n] = 0.0f; s2[n] = 0.0f; s3[n] = h[n];
    }
    const int nload = STASH ? nsb : nsb - 1;  // 16-row blocks read here
    Raw rd[kBT], rx[kBT];
    if (nload > 0) {
#pragma unroll
      for (int t = 0; t < kBT; ++t) {
        rd[t] = W::load(wdt, lane_in, ro_of(t));
        rx[t] = W::load(wxx, lane_in, ro_of(t));
      }
    }
    for (int k = 0; k < nload; ++k) {
      Raw nd[kBT], nx[kBT];
      if (k + 1 < nload) {
#pragma unroll
        for (int t = 0; t < kBT; ++t) {
          nd[t] = W::load(wdt, lane_in, ro_of((k + 1) * kBT + t));
          nx[t] = W::load(wxx, lane_in, ro_of((k + 1) * kBT + t));
        }
      }
      if constexpr (STASH) {
#pragma unroll
        for (int t = 0; t < kBT; ++t) {
          S.dt[k * kBT + t][tid] = rd[t];
          S.x[k * kBT + t][tid] = rx[t];
        }
      }
      if (k < nsb - 1) {  // every row of this block is inside the unit
        // fp32 inputs: the block's state from zero, then h = (decay of the block, one exponential) h +
        // that; bf16 inputs: h chained through the block's rows
        float hk[NS], es_k[NS];
        float sd_k = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) { hk[n] = kChainQ ? h[n] : 0.0f; es_k[n] = 0.0f; }
#pragma unroll
        for (int t = 0; t < kBT; ++t) {
          const float delta = step_delta<Tin, SOFTPLUS>(step_in<Tin>(W::get(rd[t], 0), bias));
          const float dxv = delta * W::get(rx[t], 0);
          const float* b = S.B + (k * kBT + t) * NS;
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            float e = delta * A2[n];
            if (DISC == kClamp) {
              e = e > kClampLog2 ? kClampLog2 : e;
              es_k[n] += e;
            }
            hk[n] = fmaf(hw_exp2(e), hk[n], dxv * b[n]);
            if (NS > 8 && (n & 7) == 7) __builtin_amdgcn_sched_barrier(0);
          }
          sd_k += delta;
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (kChainQ) {
            h[n] = hk[n];
          } else {
            const float Pk = DISC == kClamp ? hw_exp2(es_k[n]) : hw_exp2(A2[n] * sd_k);
            h[n] = fmaf(Pk, h[n], hk[n]);
          }
          s0[n] = s1[n]; s1[n] = s2[n]; s2[n] = s3[n]; s3[n] = h[n];
        }
      }
      if (k + 1 < nload) {
#pragma unroll
        for (int t = 0; t < kBT; ++t) { rd[t] = nd[t]; rx[t] = nx[t]; }
      }
    }
  }

  // ---- the sub-blocks, last to first
  using WO = win<Tout, 1>;
  const auto wox = unit_window(p.dx, row0, R, p.D, sizeof(Tout)), wot = unit_window(p.ddt, row0, R, p.D, sizeof(Tout));
  const auto woz = unit_window(GATE ? p.dz : p.dx, row0, R, p.D, sizeof(Tout));
  const uint32_t lane_out = (uint32_t)(dl * (int64_t)sizeof(Tout)), row_out = (uint32_t)(p.D * (int64_t)sizeof(Tout));
  float dsum = 0.0f, bsum = 0.0f;
  for (int j = nsb - 1; j >= 0; --j) {
    const int slot = j & 1;
    const int Rj = min(kBT, R - j * kBT);
    const int r0 = j * kBT;
    // the previous sub-block's dy and z: loaded now, put in the other slot after the state loop
    Raw ny[kBT], nz[kBT];
    if (j > 0) {
#pragma unroll
      for (int t = 0; t < kBT; ++t) {
        ny[t] = W::load(wdy, lane_in, (uint32_t)(r0 - kBT + t) * row_in);
        if (GATE) nz[t] = W::load(wzz, lane_in, (uint32_t)(r0 - kBT + t) * row_in);
      }
    }
    __syncthreads();  // this sub-block's ring slot and the stash are written; red is free again
    auto raw_dt = [&](int t) { return STASH ? S.dt[r0 + t][tid] : W::load(wdt, lane_in, ro_of(r0 + t)); };
    auto raw_x = [&](int t) { return STASH ? S.x[r0 + t][tid] : W::load(wxx, lane_in, ro_of(r0 + t)); };
    // per row: delta, delta x, ds = dy silu(z); rows past the unit and lanes past D: exact zeros
    float delta[kBT], dx_[kBT], ds[kBT];
#pragma unroll
    for (int t = 0; t < kBT; ++t) {
      const bool ok = t < Rj;
      const float xx = W::get(raw_x(t), 0);
      const float dyv = W::get(S.dy[slot][t][tid], 0);
      const float g = GATE ? silu_in<Tin>(W::get(S.z[slot][t][tid], 0)) : 1.0f;
      const float dl_ = step_delta<Tin, SOFTPLUS>(step_in<Tin>(W::get(raw_dt(t), 0), bias));
      delta[t] = ok ? dl_ : 0.0f;
      dx_[t] = ok && active ? dl_ * xx : 0.0f;
      ds[t] = ok && active ? dyv * g : 0.0f;
      if (ok) dsum = fmaf(ds[t], xx, dsum);
    }
    float sd_j = 0.0f;  // delta summed over the sub-block (rows past the unit add 0)
#pragma unroll
    for (int t = 0; t < kBT; ++t) sd_j += delta[t];
    float sacc[kBT], GB[kBT], MA[kBT];
#pragma unroll
    for (int t = 0; t < kBT; ++t) { sacc[t] = 0.0f; GB[t] = 0.0f; MA[t] = 0.0f; }

#pragma unroll 1
    for (int n = 0; n < NS; ++n) {
      const float An = p.A[dl * NS + n];
      const float A2 = An * kLog2e;
      // this state's B and C over the sub-block's rows, read four rows at a time
      const float4* Bn4 = reinterpret_cast<const float4*>(&S.Bt[n][r0]);
      const float4* Cn4 = reinterpret_cast<const float4*>(&S.Ct[n][r0]);
      float h = s3[n];
      const float q_in = S.qv[n][tid];
      float q = q_in;
      // forward through the rows, keeping abar and h_{t-1} for the way back
      float v[16], abr[kBT], hpr[kBT];
      uint32_t live = 0;  // bit t: the clamp does not act at row t
      float es_j = 0.0f;  // the clamped exponents summed (clamp variant, last row first)
#pragma unroll
      for (int t4 = 0; t4 < kBT / 4; ++t4) {
        const float4 b4 = Bn4[t4], c4 = Cn4[t4];
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = 4 * t4 + k;
          float e = delta[t] * A2;
          if (DISC == kClamp) {
            live |= (e <= kClampLog2 ? 1u : 0u) << t;
            e = e > kClampLog2 ? kClampLog2 : e;
          }
          const float ab = hw_exp2(e);
          abr[t] = ab;
          hpr[t] = h;
          h = fmaf(ab, h, dx_[t] * bb[k]);
          sacc[t] = fmaf(cc[k], h, sacc[t]);
          v[t] = ds[t] * h;  // this lane's share of dC_tn
        }
      }
      wave_sum16(v, lane);
      if ((lane & 3) == 0) S.redC[n][wave][(lane >> 2) & 15] = v[0];
      float dA = 0.0f;
      float qz = 0.0f;  // q from zero past the sub-block's end (fp32 inputs)
#pragma unroll
      for (int t4 = kBT / 4 - 1; t4 >= 0; --t4) {
        const float4 b4 = Bn4[t4], c4 = Cn4[t4];
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int k = 3; k >= 0; --k) {
          const int t = 4 * t4 + k;
          const float ab = abr[t], hp = hpr[t];
          const float g = fmaf(ds[t], cc[k], q);
          q = ab * g;
          if (!kChainQ) qz = ab * fmaf(ds[t], cc[k], qz);
          float mab = (g * hp) * ab;  // d abar times abar
          if (DISC == kClamp) {
            mab = (live >> t) & 1u ? mab : 0.0f;  // no gradient through the clamp
            if (!kChainQ) {
              const float e = delta[t] * A2;  // the clamped exponents summed from the sub-block's end
              es_j += e > kClampLog2 ? kClampLog2 : e;
            }
          }
          MA[t] = fmaf(mab, An, MA[t]);
          dA = fmaf(mab, delta[t], dA);
          GB[t] = fmaf(g, bb[k], GB[t]);
          v[t] = g * dx_[t];  // this lane's share of dB_tn
        }
      }
      wave_sum16(v, lane);
      if ((lane & 3) == 0) S.redB[n][wave][(lane >> 2) & 15] = v[0];
      // q entering the earlier sub-block.  fp32 inputs: q from zero plus q_in carried by the sub-block's
      // decay product taken as one exponential, so no chain of rounded decays runs past a sub-block.
      // bf16 inputs: the chained q itself (a unit's 64 rounded decays move it by a few fp32 ulps, far
      // below what the inputs' rounding allows), which saves the second recurrence
      if (kChainQ) {
        S.qv[n][tid] = q;
      } else {
        const float Pj = DISC == kClamp ? hw_exp2(es_j) : hw_exp2(A2 * sd_j);
        S.qv[n][tid] = fmaf(Pj, q_in, qz);
      }
      S.dA[n][tid] += dA;
    }

    // row gradients
#pragma unroll
    for (int t = 0; t < kBT; ++t) {
      if (t < Rj) {
        const float xx = W::get(raw_x(t), 0);
        const float ddelta = fmaf(xx, GB[t], MA[t]);
        const float gdt = SOFTPLUS ? ddelta * step_grad<Tin>(step_in<Tin>(W::get(raw_dt(t), 0), bias)) : ddelta;
        const float gx = fmaf(ds[t], dskip, delta[t] * GB[t]);
        float gz = 0.0f;
        if (GATE) {
          const float dyv = W::get(S.dy[slot][t][tid], 0), zz = W::get(S.z[slot][t][tid], 0);
          gz = dyv * silu_grad_in<Tin>(zz) * fmaf(dskip, xx, sacc[t]);
        }
        bsum += gdt;
        if (active) {
          WO::store(wox, lane_out, (uint32_t)(r0 + t) * row_out, &gx);
          WO::store(wot, lane_out, (uint32_t)(r0 + t) * row_out, &gdt);
          if (GATE) WO::store(woz, lane_out, (uint32_t)(r0 + t) * row_out, &gz);
        }
      }
    }
    if (j > 0) {
#pragma unroll
      for (int t = 0; t < kBT; ++t) {
        S.dy[slot ^ 1][t][tid] = ny[t];
        if (GATE) S.z[slot ^ 1][t][tid] = nz[t];
      }
    }
    // dB / dC of this sub-block's rows for this channel block: the waves' sums, in wave order
    __syncthreads();
    for (int e = tid; e < NS * kBT; e += kThreads) {
      const int n = e / kBT, t = e - n * kBT;
      float sb = 0.0f, sc = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kThreads / 64; ++wv) {
        sb += S.redB[n][wv][t];
        sc += S.redC[n][wv][t];
      }
      if (t < Rj) {
        const int64_t row = (int64_t)blockIdx.y * p.BL + row0 + r0 + t;
        p.dBm_part[row * NS + n] = sb;
        p.dCm_part[row * NS + n] = sc;
      }
    }
    // the next (earlier) sub-block starts where s2 said
#pragma unroll
    for (int n = 0; n < NS; ++n) { s3[n] = s2[n]; s2[n] = s1[n]; s1[n] = s0[n]; }
  }
  if (active) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      p.dA_part[(u * NS + n) * p.D + d] = S.dA[n][tid];
      if (U.first && p.dh0) p.dh0[(U.seq * p.D + d) * NS + n] = S.qv[n][tid];
    }
    p.dD_part[u * p.D + d] = dsum;
    p.dbias_part[u * p.D + d] = bsum;
  }
}

template <typename Tin, typename Tout, int NS, bool SOFTPLUS, bool GATE>
__global__ __launch_bounds__(kThreads, 1) void selective_bwd_kernel(SelBwdParams p) {
  const int64_t u = blockIdx.x;
  const BUnit U = bwd_unit(p, u);
  if (!U.valid) return;
  const int64_t d = (int64_t)blockIdx.y * kThreads + threadIdx.x;
  const bool active = d < p.D;
  const int64_t dl = active ? d : p.D - 1;  // lanes past D recompute channel D-1 and store nothing
  __shared__ BwdLds<typename win<Tin, 1>::raw, NS, sizeof(Tin) == 2> S;
  stage_bc<Tin, NS>(p, U.row0, U.R, S.B, S.C);
  for (int e = threadIdx.x; e < kBU * NS; e += kThreads) {
    const int n = e / kBU, t = e - n * kBU;
    const int64_t idx = (U.row0 + min(t, U.R - 1)) * NS + n;
    S.Bt[n][t] = t < U.R ? io<Tin>::load(p.Bm, idx) : 0.0f;
    S.Ct[n][t] = t < U.R ? io<Tin>::load(p.Cm, idx) : 0.0f;
  }
  bool nonpos = true;
#pragma unroll
  for (int n = 0; n < NS; ++n) nonpos = nonpos && !(p.A[dl * NS + n] > 0.0f);
  __syncthreads();
  if (SOFTPLUS && __all(nonpos))
    bwd_grad_unit<Tin, Tout, NS, SOFTPLUS, GATE, kExp>(p, U, u, d, dl, active, S);
  else
    bwd_grad_unit<Tin, Tout, NS, SOFTPLUS, GATE, kClamp>(p, U, u, d, dl, active, S);
}

// Pass 4: fixed-order sums, in two launches.  dBm, dCm: over channel blocks.  dA [D][N], dDskip and
// d dt_bias: over units in two steps: slice k of S = kSumSlices adds units [k U / S, (k + 1) U / S), then the
// slices are added in order.  The unit sums share one column space: c < N D is column c = n D + d of
// dA's [units][N][D] partials (it goes to dA[d N + n]), then D columns of dDskip's, then D of dt_bias's
// (those present).
constexpr int kSumSlices = 16;
struct BwdSums {
  const float* PB;
  const float* PC;
  int64_t nblk, nbc;  // channel blocks; B L N
  void* dBm;
  void* dCm;
  const float* dA_part;
  const float* dD_part;     // or NULL
  const float* dbias_part;  // or NULL
  int64_t units;
  const int* n_units;  // packed varlen: the units the planner made, else NULL
  int64_t N, D, W;     // W = N D + D (dDskip) + D (d dt_bias)
  float* slices;       // [kSumSlices][W]
  float* dA;
  float* dDskip;
  float* ddt_bias;
};
// the partial buffer, its row width and the column within it of unit-sum column c
__device__ __forceinline__ const float* sum_column(const BwdSums& a, int64_t c, int64_t& width, int64_t& col) {
  const int64_t ND = a.N * a.D;
  if (c < ND) {
    width = ND;
    col = c;
    return a.dA_part;
  }
  width = a.D;
  col = c - ND;
  if (a.dD_part != nullptr) {
    if (col < a.D) return a.dD_part;
    col -= a.D;
  }
  return a.dbias_part;
}
// Threads [0, nbc): dBm / dCm;  then kSumSlices x W threads: the slices.
template <typename Tout>
__global__ __launch_bounds__(kThreads) void selective_bwd_sums_kernel(BwdSums a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < a.nbc) {
    float sb = 0.0f, sc = 0.0f;
    for (int64_t k = 0; k < a.nblk; ++k) {
      sb += a.PB[k * a.nbc + i];
      sc += a.PC[k * a.nbc + i];
    }
    io<Tout>::store(a.dBm, i, sb);
    io<Tout>::store(a.dCm, i, sc);
    return;
  }
  const int64_t j = i - a.nbc;
  if (j >= kSumSlices * a.W) return;
  const int64_t k = j / a.W, c = j - k * a.W;
  const int64_t units = a.n_units ? (int64_t)*a.n_units : a.units;
  const int64_t u0 = k * units / kSumSlices, u1 = (k + 1) * units / kSumSlices;
  int64_t width, col;
  const float* part = sum_column(a, c, width, col);
  float acc = 0.0f;
  for (int64_t u = u0; u < u1; ++u) acc += part[u * width + col];
  a.slices[k * a.W + c] = acc;
}
__global__ __launch_bounds__(kThreads) void selective_bwd_final_kernel(BwdSums a) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= a.W) return;
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < kSumSlices; ++k) acc += a.slices[k * a.W + c];
  const int64_t ND = a.N * a.D;
  if (c < ND) {
    const int64_t n = c / a.D, d = c - n * a.D;
    a.dA[d * a.N + n] = acc;
  } else if (a.dDskip != nullptr && c < ND + a.D) {
    a.dDskip[c - ND] = acc;
  } else {
    a.ddt_bias[c - ND - (a.dDskip != nullptr ? a.D : 0)] = acc;
  }
}

template <typename Tin, typename Tout, int NS, bool SOFTPLUS, bool GATE>
void launch_bwd_g(const SelBwdParams& q, int64_t U, int64_t nseq, hipStream_t s) {
  const dim3 grid((unsigned)U, (unsigned)q.nblk), blk(kThreads);
  hipLaunchKernelGGL((selective_bwd_agg_kernel<Tin, NS, SOFTPLUS, GATE>), grid, blk, 0, s, q);
  const int64_t nthreads = nseq * NS * q.D;
  hipLaunchKernelGGL((selective_bwd_carry_kernel<NS>), dim3((unsigned)((nthreads + kThreads - 1) / kThreads)), blk, 0,
                     s, q, nseq);
  hipLaunchKernelGGL((selective_bwd_kernel<Tin, Tout, NS, SOFTPLUS, GATE>), grid, blk, 0, s, q);
}

template <typename Tin, typename Tout, int NS, bool SOFTPLUS>
void launch_bwd_n(const SelBwdParams& q, int64_t U, int64_t nseq, bool gate, hipStream_t s) {
  if (gate) launch_bwd_g<Tin, Tout, NS, SOFTPLUS, true>(q, U, nseq, s);
  else launch_bwd_g<Tin, Tout, NS, SOFTPLUS, false>(q, U, nseq, s);
}

template <typename Tin, typename Tout, int NS>
void launch_bwd_sp(const SelBwdParams& q, int64_t U, int64_t nseq, bool softplus, bool gate, hipStream_t s) {
  if (softplus) launch_bwd_n<Tin, Tout, NS, true>(q, U, nseq, gate, s);
  else launch_bwd_n<Tin, Tout, NS, false>(q, U, nseq, gate, s);
}

template <typename Tin, typename Tout>
void launch_bwd_t(const SelBwdParams& q, int64_t N, int64_t U, int64_t nseq, bool softplus, bool gate, hipStream_t s) {
  switch (N) {
    case 1: launch_bwd_sp<Tin, Tout, 1>(q, U, nseq, softplus, gate, s); break;
    case 2: launch_bwd_sp<Tin, Tout, 2>(q, U, nseq, softplus, gate, s); break;
    case 4: launch_bwd_sp<Tin, Tout, 4>(q, U, nseq, softplus, gate, s); break;
    case 8: launch_bwd_sp<Tin, Tout, 8>(q, U, nseq, softplus, gate, s); break;
    default: launch_bwd_sp<Tin, Tout, 16>(q, U, nseq, softplus, gate, s); break;
  }
}

}  // namespace

int64_t selective_segment_len(const SelectiveScanArgs& a) { return make_plan(a).T; }

// The packed plan serves bf16 inputs; fp32 inputs keep segments of the first plan.  An fp32
// recurrence advanced row by row loses accuracy on slowly decaying states (abar near 1 is held to
// 2^-24, a relative error of 2^-24 / (1 - abar) in the decay) over long runs, while the aggregate
// and carry passes apply a segment's decay product exp2(A sum delta) in one rounding, so short
// segments keep fp32 results within the fp32-input tolerance.
bool use_packed_plan(const SelectiveScanArgs& a, const Plan& pl) { return a.cu_seqlens && pl.packed && a.in_bf16; }

size_t selective_scan_scratch_bytes(const SelectiveScanArgs& a) {
  const Plan pl = make_plan(a);
  size_t bytes = workspace_head_bytes() + 3 * align256((size_t)pl.U * a.N * a.D * sizeof(float)) +
                 align256((size_t)pl.U * a.D * sizeof(float));
  if (a.cu_seqlens) bytes += align256(256 + (size_t)pl.U * sizeof(int2)) + align256((size_t)a.nseq * sizeof(int2));
  if (a.cu_seqlens && pl.packed) {  // the query does not know the input dtype: room for either plan
    const size_t st = (size_t)a.N * a.D * sizeof(float);
    const size_t packed = workspace_head_bytes() + 2 * align256((size_t)pl.A * st) +
                          align256((size_t)pl.A * a.D * sizeof(float)) + 2 * align256((size_t)pl.C * st) +
                          align256((size_t)pl.C * sizeof(int2)) + 256 +
                          align256((size_t)pl.S * sizeof(int4)) + align256((size_t)pl.A * sizeof(int4)) +
                          align256((size_t)a.nseq * sizeof(int4));
    if (packed > bytes) bytes = packed;
  }
  return bytes;
}

hipError_t launch_selective_scan(const SelectiveScanArgs& a, hipStream_t s) {
  const Plan pl = make_plan(a);
  SelParams p{};
  p.L = a.L; p.D = a.D; p.N = a.N; p.nseq = a.nseq; p.T = pl.T; p.nseg = pl.nseg;
  p.cu = a.cu_seqlens; p.units = nullptr; p.n_units = nullptr; p.seq_units = nullptr;
  p.x = a.x; p.dt = a.dt; p.A = a.A; p.Bm = a.Bm; p.Cm = a.Cm; p.Dskip = a.Dskip; p.z = a.z;
  p.dt_bias = a.dt_bias; p.h0 = a.h0; p.y = a.y; p.h_last = a.h_last;
  p.softplus = a.dt_softplus != 0;
  p.nblk = (a.D + kThreads - 1) / kThreads;
  char* base = static_cast<char*>(a.scratch) + workspace_head_bytes();
  if (use_packed_plan(a, pl)) {
    const size_t st = (size_t)a.N * a.D * sizeof(float);
    char* q = base;
    p.aggP = reinterpret_cast<float*>(q); q += align256((size_t)pl.A * st);
    p.aggH = reinterpret_cast<float*>(q); q += align256((size_t)pl.A * st);
    p.sdelta = reinterpret_cast<float*>(q); q += align256((size_t)pl.A * a.D * sizeof(float));
    p.pieceP = reinterpret_cast<float*>(q); q += align256((size_t)pl.C * st);
    p.pieceH = reinterpret_cast<float*>(q); q += align256((size_t)pl.C * st);
    int2* piece = reinterpret_cast<int2*>(q); q += align256((size_t)pl.C * sizeof(int2));
    int* count = reinterpret_cast<int*>(q); q += 256;
    int4* scan = reinterpret_cast<int4*>(q); q += align256((size_t)pl.S * sizeof(int4));
    int4* aggt = reinterpret_cast<int4*>(q); q += align256((size_t)pl.A * sizeof(int4));
    int4* seqt = reinterpret_cast<int4*>(q);
    p.vcount = count; p.vscan = scan; p.vagg = aggt; p.vseq = seqt; p.vpiece = piece;
    hipLaunchKernelGGL(selective_vplan_kernel, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.nseq, pl.F, pl.P, pl.Y,
                       count, scan, aggt, seqt, piece, a.D, a.N, a.h0, a.h_last);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return a.out_bf16 ? launch_packed_by_n<bf16_t, bf16_t>(p, pl, a.dt_softplus != 0, s)
                      : launch_packed_by_n<bf16_t, float>(p, pl, a.dt_softplus != 0, s);
  }
  const size_t agg = align256((size_t)pl.U * a.N * a.D * sizeof(float));
  p.aggP = reinterpret_cast<float*>(base);
  p.aggH = reinterpret_cast<float*>(base + agg);
  p.carry = reinterpret_cast<float*>(base + 2 * agg);
  p.sdelta = reinterpret_cast<float*>(base + 3 * agg);
  if (a.cu_seqlens) {
    char* tbl = base + 3 * agg + align256((size_t)pl.U * a.D * sizeof(float));
    const size_t tbl_bytes = align256(256 + (size_t)pl.U * sizeof(int2));
    p.n_units = reinterpret_cast<int*>(tbl);
    p.units = reinterpret_cast<const int2*>(tbl + 256);
    p.seq_units = reinterpret_cast<const int2*>(tbl + tbl_bytes);
    hipLaunchKernelGGL(selective_plan_kernel, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.nseq, pl.T,
                       reinterpret_cast<int2*>(tbl + 256), reinterpret_cast<int*>(tbl),
                       reinterpret_cast<int2*>(tbl + tbl_bytes), a.D, a.N, a.h0, a.h_last);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pl.U == 0) return hipSuccess;
  if (!a.in_bf16) return launch_by_n<float, float>(p, pl.U, a.dt_softplus != 0, s);
  return a.out_bf16 ? launch_by_n<bf16_t, bf16_t>(p, pl.U, a.dt_softplus != 0, s)
                    : launch_by_n<bf16_t, float>(p, pl.U, a.dt_softplus != 0, s);
}

namespace {
struct BwdLayout {
  int64_t nseg, U, nblk;          // U: units (packed varlen: an upper bound)
  size_t state, row, bc, slices;  // bytes of one [U][N][D], [U][D], [nblk][B L][N] buffer, and the slices
  size_t tbl, seqtbl;             // packed varlen: unit table (after a 256-byte count), per-sequence table
};
BwdLayout bwd_layout(const SelectiveBwdArgs& a) {
  BwdLayout l;
  if (a.cu_seqlens == nullptr) {
    l.nseg = (a.L + kBU - 1) / kBU;
    l.U = a.B * l.nseg;
    l.tbl = l.seqtbl = 0;
  } else {
    l.nseg = 0;
    l.U = (a.L + kBU - 1) / kBU + a.nseq;  // sum over sequences of ceil(len / kBU)
    l.tbl = align256(256 + (size_t)l.U * sizeof(int2));
    l.seqtbl = align256((size_t)a.nseq * sizeof(int2));
  }
  l.nblk = (a.D + kThreads - 1) / kThreads;
  l.state = align256((size_t)(l.U * a.N * a.D) * sizeof(float));
  l.row = align256((size_t)(l.U * a.D) * sizeof(float));
  l.bc = align256((size_t)(l.nblk * a.B * a.L * a.N) * sizeof(float));
  l.slices = align256((size_t)(kSumSlices * (a.N + 2) * a.D) * sizeof(float));
  return l;
}
}  // namespace

size_t selective_scan_backward_scratch_bytes(const SelectiveBwdArgs& a) {
  const BwdLayout l = bwd_layout(a);
  return workspace_head_bytes() + 6 * l.state + 3 * l.row + 2 * l.bc + l.slices + l.tbl + l.seqtbl;
}

hipError_t launch_selective_scan_backward(const SelectiveBwdArgs& a, hipStream_t s) {
  const BwdLayout l = bwd_layout(a);
  char* q0 = static_cast<char*>(a.scratch) + workspace_head_bytes();
  auto take = [&](size_t bytes) {
    char* r = q0;
    q0 += bytes;
    return reinterpret_cast<float*>(r);
  };
  float* hin = take(l.state);
  float* qend = take(l.state);
  float* aggP = take(l.state);
  float* aggH = take(l.state);
  float* aggQ = take(l.state);
  float* dA_part = take(l.state);
  float* sdelta = take(l.row);
  float* dD_part = take(l.row);
  float* dbias_part = take(l.row);
  float* PB = take(l.bc);
  float* PC = take(l.bc);
  float* slices = take(l.slices);  // kSumSlices x (N D + 2 D)
  char* tbl = q0;
  int* n_units = nullptr;
  int2 *units = nullptr, *seq_units = nullptr;
  const int64_t nseq = a.cu_seqlens ? a.nseq : a.B;
  if (a.cu_seqlens) {  // the forward's planner at the unit length kBU (no h_last to fill)
    n_units = reinterpret_cast<int*>(tbl);
    units = reinterpret_cast<int2*>(tbl + 256);
    seq_units = reinterpret_cast<int2*>(tbl + l.tbl);
    hipLaunchKernelGGL(selective_plan_kernel, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.nseq, (int64_t)kBU, units,
                       n_units, seq_units, a.D, a.N, a.h0, (float*)nullptr);
  }
  // passes 1-3
  SelBwdParams q{};
  q.L = a.L; q.D = a.D; q.nseg = l.nseg; q.nblk = l.nblk; q.BL = a.B * a.L;
  q.cu = a.cu_seqlens; q.units = units; q.n_units = n_units; q.seq_units = seq_units;
  q.x = a.x; q.dt = a.dt; q.A = a.A; q.Bm = a.Bm; q.Cm = a.Cm; q.Dskip = a.Dskip; q.z = a.z; q.dt_bias = a.dt_bias;
  q.h0 = a.h0; q.dy = a.dy; q.dh_last = a.dh_last;
  q.aggP = aggP; q.aggH = aggH; q.aggQ = aggQ; q.hin = hin; q.qend = qend;
  q.sdelta = sdelta; q.softplus = a.dt_softplus != 0;
  q.dx = a.dx; q.ddt = a.ddt; q.dz = a.dz; q.dBm_part = PB; q.dCm_part = PC;
  q.dA_part = dA_part; q.dD_part = dD_part; q.dbias_part = dbias_part; q.dh0 = a.dh0;
  const bool sp = a.dt_softplus != 0, gate = a.z != nullptr;
  if (!a.in_bf16) launch_bwd_t<float, float>(q, a.N, l.U, nseq, sp, gate, s);
  else if (a.out_bf16) launch_bwd_t<bf16_t, bf16_t>(q, a.N, l.U, nseq, sp, gate, s);
  else launch_bwd_t<bf16_t, float>(q, a.N, l.U, nseq, sp, gate, s);
  // pass 4: fixed-order sums
  BwdSums sm{};
  sm.PB = PB; sm.PC = PC; sm.nblk = l.nblk; sm.nbc = a.B * a.L * a.N; sm.dBm = a.dBm; sm.dCm = a.dCm;
  sm.dA_part = dA_part; sm.dD_part = a.dDskip ? dD_part : nullptr; sm.dbias_part = a.ddt_bias ? dbias_part : nullptr;
  sm.units = l.U; sm.n_units = n_units; sm.N = a.N; sm.D = a.D;
  sm.W = a.N * a.D + (a.dDskip ? a.D : 0) + (a.ddt_bias ? a.D : 0);
  sm.slices = slices; sm.dA = a.dA; sm.dDskip = a.dDskip; sm.ddt_bias = a.ddt_bias;
  const int64_t nsum = sm.nbc + kSumSlices * sm.W;
  const dim3 blk(kThreads);
  if (a.out_bf16)
    hipLaunchKernelGGL((selective_bwd_sums_kernel<bf16_t>), dim3((unsigned)((nsum + kThreads - 1) / kThreads)), blk, 0,
                       s, sm);
  else
    hipLaunchKernelGGL((selective_bwd_sums_kernel<float>), dim3((unsigned)((nsum + kThreads - 1) / kThreads)), blk, 0,
                       s, sm);
  hipLaunchKernelGGL(selective_bwd_final_kernel, dim3((unsigned)((sm.W + kThreads - 1) / kThreads)), blk, 0, s, sm);
  return hipGetLastError();
}

hipError_t launch_selective_update(const SelectiveUpdateArgs& a, hipStream_t s) {
  if (!a.in_bf16) launch_update_t<float, float>(a, s);
  else if (a.out_bf16) launch_update_t<bf16_t, bf16_t>(a, s);
  else launch_update_t<bf16_t, float>(a, s);
  return hipGetLastError();
}

}  // namespace ssd
