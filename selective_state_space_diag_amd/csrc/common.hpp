// common.hpp -- device helpers shared by the gfx950 scan kernels.
//
// Number formats: activations arrive as fp32 or bf16 bit patterns; all arithmetic is fp32.
// Transcendentals use the hardware instructions directly (v_exp_f32 = 2^x, v_log_f32 = log2,
// v_rcp_f32, v_sqrt_f32; each about 1 ulp); where a cancellation would cost accuracy the
// formula is rearranged (see one_minus_exp2x and softplus_f).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"  // WaitCfg

namespace ssd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ bf16 <-> fp32
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (the gfx950 conversion instruction; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element access by storage type.
template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};
template <> struct io<bf16_t> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  }
};

// Two consecutive elements (index i even, base 16-byte aligned, row length even).
template <typename T> struct io2;
template <> struct io2<float> {
  using raw = float2;
  static __device__ __forceinline__ raw load(const void* p, int64_t i) {
    return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
  }
  static __device__ __forceinline__ float lo(raw r) { return r.x; }
  static __device__ __forceinline__ float hi(raw r) { return r.y; }
  static __device__ __forceinline__ void store(void* p, int64_t i, float a, float b) {
    *reinterpret_cast<float2*>(static_cast<float*>(p) + i) = make_float2(a, b);
  }
};
template <> struct io2<bf16_t> {
  using raw = uint32_t;
  static __device__ __forceinline__ raw load(const void* p, int64_t i) {
    return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
  }
  static __device__ __forceinline__ float lo(raw r) { return bf16_lo(r); }
  static __device__ __forceinline__ float hi(raw r) { return bf16_hi(r); }
  static __device__ __forceinline__ void store(void* p, int64_t i, float a, float b) {
    uint32_t w = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + i) = w;
  }
};

// Four consecutive elements (index a multiple of 4, base 16-byte aligned).
template <typename T> struct io4;
template <> struct io4<float> {
  static __device__ __forceinline__ void store(void* p, int64_t i, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = make_float4(a, b, c, d);
  }
};
template <> struct io4<bf16_t> {
  static __device__ __forceinline__ void store(void* p, int64_t i, float a, float b, float c, float d) {
    const uint32_t lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = make_uint2(lo, hi);
  }
};

// ------------------------------------------------------------------ buffer windows
// A buffer resource over [p, p + bytes), bytes < 2^31.  Accesses through it take a per-lane byte
// offset (vector register) plus a wave-uniform byte offset (scalar register), so a tile of rows
// costs no per-lane 64-bit address arithmetic.  Callers keep every offset inside the window.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_window(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy operand of the buffer instructions.  kStreaming sets the non-temporal bit: the lines
// are not expected to be touched again, so the caches hold them under their streaming policy instead
// of displacing reused data.  It pays for one-pass streams (input read once, output written once) and
// costs a little where a later pass re-reads the same rows.
constexpr int kCached = 0;
constexpr int kStreaming = 2;

// V consecutive elements of type T per lane through a window, with cache policy P.
template <typename T, int V, int P = kCached> struct win;
template <int P> struct win<float, 1, P> {
  using raw = float;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(w, (int)lane_off, (int)row_off, P));
  }
  static __device__ __forceinline__ float get(raw r, int) { return r; }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off,
                                               const float* v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), w, (int)lane_off, (int)row_off, P);
  }
};
template <int P> struct win<float, 2, P> {
  using raw = u32x2_t;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(w, (int)lane_off, (int)row_off, P);
  }
  static __device__ __forceinline__ float get(raw r, int v) { return __uint_as_float(v == 0 ? r.x : r.y); }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off,
                                               const float* v) {
    u32x2_t d;
    d.x = __float_as_uint(v[0]);
    d.y = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(d, w, (int)lane_off, (int)row_off, P);
  }
};
template <int P> struct win<bf16_t, 1, P> {
  using raw = unsigned short;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off) {
    return __builtin_amdgcn_raw_buffer_load_b16(w, (int)lane_off, (int)row_off, P);
  }
  static __device__ __forceinline__ float get(raw r, int) { return bf16_to_f32(r); }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off,
                                               const float* v) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v[0]), w, (int)lane_off, (int)row_off, P);
  }
};
template <int P> struct win<bf16_t, 2, P> {
  using raw = uint32_t;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off) {
    return __builtin_amdgcn_raw_buffer_load_b32(w, (int)lane_off, (int)row_off, P);
  }
  static __device__ __forceinline__ float get(raw r, int v) { return v == 0 ? bf16_lo(r) : bf16_hi(r); }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t w, uint32_t lane_off, uint32_t row_off,
                                               const float* v) {
    const uint32_t d = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    __builtin_amdgcn_raw_buffer_store_b32(d, w, (int)lane_off, (int)row_off, P);
  }
};
// ------------------------------------------------------------------ hardware transcendentals
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

// e^v with the argument carried past fp32: t = v log2(e) rounds with an absolute error of up to
// half an ulp of |t|, which moves 2^t by that much times ln 2 in relative terms (several ulp once
// |v| is a few units).  The exact rounding error of the product (an fma) and the tail of log2(e)
// beyond fp32 form tl, and 2^(t + tl) = 2^t (1 + tl ln 2) to first order (|tl| < 2^-23 |t|).
constexpr float kLog2eLo = 1.9259629911e-08f;  // log2(e) - (float)log2(e)
// Where the correction is not finite (v = +-inf, or 2^t overflowed) 2^t alone is the answer.
__device__ __forceinline__ float exp_split(float v) {
  const float t = v * kLog2e;
  const float tl = fmaf(v, kLog2eLo, fmaf(v, kLog2e, -t));
  const float e = hw_exp2(t);
  const float c = e * tl;
  return __builtin_isfinite(c) ? fmaf(c, kLn2, e) : e;
}

// sigmoid(v) = 1 / (1 + e^-v); saturates cleanly to 0 / 1 for large |v|.  The plain form rounds
// the exponent (several ulp for |v| of a few units), which the forward gates can afford.
__device__ __forceinline__ float sigmoid_f(float v) { return hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// silu(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// The same with e^-v through exp_split (about 1 ulp): for derivatives that scale a whole gradient,
// such as softplus'(v) = sigmoid(v) in d dt.
__device__ __forceinline__ float sigmoid_acc_f(float v) { return hw_rcp(1.0f + exp_split(-v)); }
__device__ __forceinline__ float silu_acc_f(float z) { return z * sigmoid_acc_f(z); }

// softplus with the usual threshold: v for v > 20, else log(1 + e^v).  log1p is kept accurate
// for small e^v by the correction log1p(e) = log(u) * e / (u - 1), u = 1 + e (u - 1 is exact).
// e^v is formed with exp_split: delta scales every input term and every decay exponent of the scan,
// so its relative error passes straight into the states.
__device__ __forceinline__ float softplus_f(float v) {
  float e = exp_split(v);
  float u = 1.0f + e;
  float um1 = u - 1.0f;
  float lg = hw_log2(u) * kLn2;
  float r = (um1 == 0.0f) ? e : lg * (e * hw_rcp(um1));
  return v > 20.0f ? v : r;
}

// softplus for bf16 inputs: log(1 + e^v) from the hardware exp2 and log2 alone, identity above 20.
// Forming 1 + e^v rounds away up to 2^-24 of absolute value, i.e. 2^-24 / e^v of the result in relative
// terms (6e-5 at delta = 1e-3, the smallest step of the selective workloads; below e^v = 2^-24 the step
// rounds to 0 where it is under 6e-8).  A bf16 dt is itself only known to 2^-9 of its value, which moves
// delta by about |dt| 2^-9 in relative terms, 30 to 200 times more; softplus_f's exponent and log1p
// corrections are kept for fp32 inputs.
__device__ __forceinline__ float softplus_plain_f(float v) {
  const float r = hw_log2(1.0f + hw_exp2(v * kLog2e)) * kLn2;
  return v > 20.0f ? v : r;
}

// The softplus a kernel with input type Tin uses (see softplus_plain_f).
template <typename Tin> __device__ __forceinline__ float softplus_in(float v) { return softplus_f(v); }
template <> __device__ __forceinline__ float softplus_in<bf16_t>(float v) { return softplus_plain_f(v); }

// 1 - 2^x for x <= 0, accurate also near x = 0 (where 1 - 2^x cancels): for |x ln2| < 0.25 the
// Taylor series of -expm1 to degree 6 (truncation < 5e-8 relative), else 1 - 2^x directly.
__device__ __forceinline__ float one_minus_exp2x(float x) {
  float u = x * kLn2;  // natural-log argument
  float p = fmaf(u, 1.0f / 720.0f, 1.0f / 120.0f);
  p = fmaf(u, p, 1.0f / 24.0f);
  p = fmaf(u, p, 1.0f / 6.0f);
  p = fmaf(u, p, 0.5f);
  p = fmaf(u, p, 1.0f);
  float small = -u * p;
  float big = 1.0f - hw_exp2(x);
  return fabsf(u) < 0.25f ? small : big;
}

// ------------------------------------------------------------------ lookback words
// A 64-bit word = (epoch << 32) | float bits.  Written and read with agent-scope relaxed atomics,
// so each word is self-validating and needs no separate flag or fence.
__device__ __forceinline__ void word_store(unsigned long long* p, uint32_t epoch, float v) {
  unsigned long long w = ((unsigned long long)epoch << 32) | (unsigned long long)__float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long word_load(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool word_ready(unsigned long long w, uint32_t epoch) {
  return (uint32_t)(w >> 32) == epoch;
}
__device__ __forceinline__ float word_value(unsigned long long w) { return __uint_as_float((uint32_t)w); }

// Per-launch control block at the head of a lookback scratch buffer.  `tick` packs the number of
// completed launches (high 32 bits; a launch stamps its lookback words with that number + 1) with
// the next work unit of a single-counter kernel (low 32 bits), so one atomic add hands a workgroup
// both; the last workgroup of a launch resets the counters it used and advances the count.  The
// atomics on one address retire one at a time (about 12 ns apiece on gfx950, near 80 units per
// microsecond): enough for a forward scan, whose units are long, while kernels with shorter units
// use kTicketClasses counters, each on a 128-byte line of its own.  Class x owns the sequences whose
// index is x mod kTicketClasses and hands their units out in chunk order, so every unit a lookback
// waits on comes from the same counter and was taken earlier.
constexpr int kTicketClasses = 32;
struct alignas(128) TicketLine {
  unsigned int next;  // next local ticket of the class
  unsigned int done;  // workgroups of this home class that have finished
};
struct LookbackCtl {
  TicketLine cls[kTicketClasses];
  alignas(128) unsigned long long tick;
  unsigned int done;      // workgroups finished (single-counter kernels)
  unsigned int done_all;  // home classes whose workgroups have all finished
  unsigned int error;     // set when a bounded wait expires (read and cleared by the host)
};
constexpr int64_t kCtlBytes = (int64_t)((sizeof(LookbackCtl) + 255) / 256 * 256);

}  // namespace ssd
