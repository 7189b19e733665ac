// api.cpp -- the C ABI declared in include/ssd.h: host-side validation (arguments and the caller's
// workspace) and dispatch to the kernel launchers.  Nothing is enqueued unless every check passes.
// The library allocates nothing and keeps no state between calls besides the process-wide settings
// of the timeout test hook.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <utility>
#include <vector>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int ok() {
  g_last_error.clear();
  return SSD_OK;
}

// ------------------------------------------------------------------ validation helpers
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const char* name;
  const void* p;
  size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), a1 = a0 + a.bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(b.p), b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

int check_alias(const std::vector<Span>& outs, const std::vector<Span>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Span& s : ins)
      if (overlap(outs[i], s))
        return fail(SSD_ERR_ALIAS, std::string(outs[i].name) + " overlaps input " + s.name);
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SSD_ERR_ALIAS, std::string(outs[i].name) + " overlaps output " + outs[j].name);
  }
  return SSD_OK;
}

int check_align(const std::vector<Span>& all) {
  for (const Span& s : all)
    if (s.p && !aligned16(s.p)) return fail(SSD_ERR_ALIGN, std::string(s.name) + " is not 16-byte aligned");
  return SSD_OK;
}

int check_dtypes(int in, int out) {
  if (in != SSD_F32 && in != SSD_BF16) return fail(SSD_ERR_DTYPE, "in_dtype must be SSD_F32 or SSD_BF16");
  if (out != SSD_F32 && out != SSD_BF16) return fail(SSD_ERR_DTYPE, "out_dtype must be SSD_F32 or SSD_BF16");
  if (in == SSD_F32 && out == SSD_BF16) return fail(SSD_ERR_DTYPE, "bf16 output requires bf16 input");
  return SSD_OK;
}

size_t esize(int dtype) { return dtype == SSD_BF16 ? 2 : 4; }
// [B][ceil(L / SSD_SCAN_CHUNK)][D] fp32 chunk states
size_t chunk_bytes(int64_t B, int64_t L, int64_t D) {
  return (size_t)(B * ((L + SSD_SCAN_CHUNK - 1) / SSD_SCAN_CHUNK) * D) * 4;
}

// a*b*c... without signed overflow for the sizes we accept (each factor < 2^40)
bool too_big(std::initializer_list<int64_t> dims) {
  double prod = 1.0;
  for (int64_t d : dims) prod *= (double)d;
  return prod > 9.0e15;
}

// ------------------------------------------------------------------ workspaces
// The timeout test hook (ssd_testing_lookback): 0 = default spin limit; never_ready shifts the epoch
// the waits accept to one no launch writes.
std::atomic<unsigned int> g_spin_limit{0};
std::atomic<int> g_never_ready{0};

ssd::WaitCfg wait_cfg() {
  ssd::WaitCfg w;
  const unsigned int lim = g_spin_limit.load(std::memory_order_relaxed);
  if (lim) w.spin_limit = lim;
  if (g_never_ready.load(std::memory_order_relaxed)) w.skew = 0x80000000u;
  return w;
}

// The caller's workspace against what the call needs; it must not overlap the call's other buffers.
int check_workspace(void* ws, size_t ws_bytes, size_t need, const std::vector<Span>& others) {
  if (need == 0) return SSD_OK;
  if (!ws) return fail(SSD_ERR_NULL, "workspace is required: " + std::to_string(need) + " bytes (see the *_workspace_bytes query)");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(SSD_ERR_ALIGN, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(SSD_ERR_SHAPE, "workspace_bytes = " + std::to_string(ws_bytes) + " is below the " +
                                   std::to_string(need) + " bytes this call needs");
  const Span w{"workspace", ws, ws_bytes};
  for (const Span& o : others)
    if (overlap(w, o)) return fail(SSD_ERR_ALIAS, std::string("workspace overlaps ") + o.name);
  return SSD_OK;
}

int ws_query(size_t* out, size_t bytes) {
  if (!out) return fail(SSD_ERR_NULL, "bytes is NULL");
  *out = bytes;
  return ok();
}

// Shape limits shared by each scan and its workspace query.
int scan1_shape(int64_t B, int64_t L, int64_t D) {
  if (B < 0 || L < 0 || D < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (too_big({B, L, D}) || D >= (int64_t)1 << 22 || B * ((L + 63) / 64) * ((D + 63) / 64) >= (int64_t)1 << 31)
    return fail(SSD_ERR_SHAPE, "problem too large");
  return SSD_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

#define SSD_TRY(expr)          \
  do {                         \
    int _st = (expr);          \
    if (_st != SSD_OK) return _st; \
  } while (0)

}  // namespace

extern "C" {

const char* ssd_status_str(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid or unsupported size";
    case SSD_ERR_DTYPE: return "unsupported dtype";
    case SSD_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SSD_ERR_VALUE: return "scalar argument out of range";
    case SSD_ERR_ALIAS: return "output overlaps another buffer";
    case SSD_ERR_HIP: return "HIP runtime error";
    case SSD_ERR_TIMEOUT: return "a bounded wait between workgroups expired";
    default: return "unknown status";
  }
}

const char* ssd_last_error(void) { return g_last_error.c_str(); }

int ssd_version(void) { return 300; }

int ssd_workspace_check(const void* workspace, void* stream) {
  if (!workspace) return fail(SSD_ERR_NULL, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* word = static_cast<char*>(const_cast<void*>(workspace)) + ssd::workspace_error_offset();
  unsigned int err = 0;
  if (hipMemcpyAsync(&err, word, sizeof(err), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(SSD_ERR_HIP, "reading the workspace's wait record failed");
  if (err == 0) return ok();
  static const unsigned int kZero = 0;
  if (hipMemcpyAsync(word, &kZero, sizeof(kZero), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(SSD_ERR_HIP, "clearing the workspace's wait record failed");
  return fail(SSD_ERR_TIMEOUT, "a bounded wait between workgroups expired; the outputs that depend on it are NaN");
}

void ssd_testing_lookback(unsigned int spin_limit, int never_ready) {
  g_spin_limit.store(spin_limit, std::memory_order_relaxed);
  g_never_ready.store(never_ready ? 1 : 0, std::memory_order_relaxed);
}

// ============================================================================ RG-LRU
int ssd_rglru_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes) {
  SSD_TRY(scan1_shape(B, L, D));
  return ws_query(bytes, B * L * D > 0 ? ssd::scan1_scratch_bytes(B, L, D) : 0);
}

int ssd_rglru_scan(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype, const void* x, const void* r_logit,
                   const void* i_logit, const float* a_log, float c, const float* h0, const void* gate, void* y,
                   float* h_last, float* chunk_states, void* workspace, size_t workspace_bytes, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(scan1_shape(B, L, D));
  if (!std::isfinite(c)) return fail(SSD_ERR_VALUE, "c must be finite");
  const int64_t nact = B * L * D;
  if (nact > 0 && (!x || !r_logit || !i_logit || !y)) return fail(SSD_ERR_NULL, "x, r_logit, i_logit and y are required");
  if (B * D > 0 && !a_log) return fail(SSD_ERR_NULL, "a_log is required");
  const size_t ab = (size_t)nact * esize(in_dtype), yb = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * D) * 4;
  std::vector<Span> ins = {{"x", x, ab}, {"r_logit", r_logit, ab}, {"i_logit", i_logit, ab},
                           {"a_log", a_log, (size_t)D * 4}, {"h0", h0, sb}, {"gate", gate, ab}};
  std::vector<Span> outs = {{"y", y, yb}, {"h_last", h_last, sb}, {"chunk_states", chunk_states, chunk_bytes(B, L, D)}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B * D == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(h_last, h0, B * D, s), "rglru_scan");
  SSD_TRY(check_workspace(workspace, workspace_bytes, ssd::scan1_scratch_bytes(B, L, D), all));
  ssd::RglruScanArgs a{B, L, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, r_logit, i_logit, a_log, c, h0, gate,
                       y, h_last, chunk_states, workspace, wait_cfg()};
  return hip_status(ssd::launch_rglru_scan(a, s), "rglru_scan launch");
}

int ssd_rglru_scan_noalloc(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype, const void* x,
                           const void* r_logit, const void* i_logit, const float* a_log, float c, const float* h0,
                           const void* gate, void* y, float* h_last, float* chunk_states, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(scan1_shape(B, L, D));
  if (!std::isfinite(c)) return fail(SSD_ERR_VALUE, "c must be finite");
  const int64_t nact = B * L * D;
  if (nact > 0 && (!x || !r_logit || !i_logit || !y)) return fail(SSD_ERR_NULL, "x, r_logit, i_logit and y are required");
  if (B * D > 0 && !a_log) return fail(SSD_ERR_NULL, "a_log is required");
  const size_t ab = (size_t)nact * esize(in_dtype), yb = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * D) * 4;
  std::vector<Span> ins = {{"x", x, ab}, {"r_logit", r_logit, ab}, {"i_logit", i_logit, ab},
                           {"a_log", a_log, (size_t)D * 4}, {"h0", h0, sb}, {"gate", gate, ab}};
  std::vector<Span> outs = {{"y", y, yb}, {"h_last", h_last, sb}, {"chunk_states", chunk_states, chunk_bytes(B, L, D)}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B * D == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(h_last, h0, B * D, s), "rglru_scan_noalloc");
  const size_t need = ssd::scan1_scratch_bytes(B, L, D);
  if (need > ssd::kNoAllocScratchBytes)
    return fail(SSD_ERR_SHAPE, "rglru_scan_noalloc: the problem needs " + std::to_string(need) +
                                   " bytes of scratch, above the fixed " +
                                   std::to_string(ssd::kNoAllocScratchBytes) + " (use ssd_rglru_scan)");
  void* scratch = nullptr;
  SSD_TRY(hip_status(ssd::noalloc_scratch(&scratch), "rglru_scan_noalloc scratch address"));
  ssd::RglruScanArgs a{B, L, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, r_logit, i_logit, a_log, c, h0, gate,
                       y, h_last, chunk_states, scratch, wait_cfg()};
  return hip_status(ssd::launch_rglru_scan(a, s), "rglru_scan_noalloc launch");
}

int ssd_rglru_update(int64_t B, int64_t D, int in_dtype, int out_dtype, const void* x, const void* r_logit,
                     const void* i_logit, const float* a_log, float c, const void* gate, float* state, void* y,
                     void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || D < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (too_big({B, D}) || B * D >= (int64_t)1 << 38) return fail(SSD_ERR_SHAPE, "problem too large");
  if (!std::isfinite(c)) return fail(SSD_ERR_VALUE, "c must be finite");
  const int64_t n = B * D;
  if (n > 0 && (!x || !r_logit || !i_logit || !a_log || !state || !y))
    return fail(SSD_ERR_NULL, "x, r_logit, i_logit, a_log, state and y are required");
  const size_t ab = (size_t)n * esize(in_dtype);
  std::vector<Span> ins = {{"x", x, ab}, {"r_logit", r_logit, ab}, {"i_logit", i_logit, ab},
                           {"a_log", a_log, (size_t)D * 4}, {"gate", gate, ab}};
  std::vector<Span> outs = {{"y", y, (size_t)n * esize(out_dtype)}, {"state", state, (size_t)n * 4}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  if (n == 0) return ok();
  ssd::RglruUpdateArgs a{B, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, r_logit, i_logit, a_log, c, gate, state, y};
  return hip_status(ssd::launch_rglru_update(a, static_cast<hipStream_t>(stream)), "rglru_update launch");
}

int ssd_rglru_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes) {
  SSD_TRY(scan1_shape(B, L, D));
  return ws_query(bytes, B * L * D > 0 ? ssd::rglru_bwd_scratch_bytes(B, L, D) : 0);
}

int ssd_rglru_scan_backward(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype, const void* x,
                            const void* r_logit, const void* i_logit, const float* a_log, float c, const float* h0,
                            const void* gate, const float* chunk_states, const void* dy, const float* dh_last,
                            void* dx, void* dr_logit, void* di_logit, float* da_log, float* dh0, void* dgate,
                            void* workspace, size_t workspace_bytes, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(scan1_shape(B, L, D));
  if (!std::isfinite(c)) return fail(SSD_ERR_VALUE, "c must be finite");
  const int64_t nact = B * L * D;
  if (nact > 0 && (!x || !r_logit || !i_logit || !dy || !dx || !dr_logit || !di_logit))
    return fail(SSD_ERR_NULL, "x, r_logit, i_logit, dy, dx, dr_logit and di_logit are required");
  if (D > 0 && (!a_log || !da_log)) return fail(SSD_ERR_NULL, "a_log and da_log are required");
  const size_t ab = (size_t)nact * esize(in_dtype), ob = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * D) * 4;
  std::vector<Span> ins = {{"x", x, ab},           {"r_logit", r_logit, ab}, {"i_logit", i_logit, ab},
                           {"a_log", a_log, (size_t)D * 4}, {"h0", h0, sb}, {"gate", gate, ab},
                           {"dy", dy, ab},         {"dh_last", dh_last, sb},
                           {"chunk_states", chunk_states, chunk_bytes(B, L, D)}};
  std::vector<Span> outs = {{"dx", dx, ob},        {"dr_logit", dr_logit, ob}, {"di_logit", di_logit, ob},
                            {"da_log", da_log, (size_t)D * 4}, {"dh0", dh0, sb}, {"dgate", gate ? dgate : nullptr, ob}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 0) return ok();
  if (nact == 0) {  // no steps: d a_log = 0, dh0 = dh_last
    SSD_TRY(hip_status(ssd::launch_copy_or_zero(da_log, nullptr, D, s), "rglru_scan_backward"));
    return hip_status(ssd::launch_copy_or_zero(dh0, dh_last, B * D, s), "rglru_scan_backward");
  }
  SSD_TRY(check_workspace(workspace, workspace_bytes, ssd::rglru_bwd_scratch_bytes(B, L, D), all));
  ssd::RglruBwdArgs a{B, L, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, r_logit, i_logit, a_log, c, h0, gate,
                      chunk_states, dy, dh_last, dx, dr_logit, di_logit, gate ? dgate : nullptr, da_log, dh0,
                      workspace, wait_cfg()};
  return hip_status(ssd::launch_rglru_scan_backward(a, s), "rglru_scan_backward launch");
}

// ============================================================================ MinMax
int ssd_minmax_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes) {
  SSD_TRY(scan1_shape(B, L, D));
  return ws_query(bytes, B * L * D > 0 ? ssd::scan1_scratch_bytes(B, L, D) : 0);
}

int ssd_minmax_scan(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype, const void* r, const void* s_in,
                    const float* x0, const void* gate, void* y, float* x_last, float* chunk_states, void* workspace,
                    size_t workspace_bytes, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(scan1_shape(B, L, D));
  const int64_t nact = B * L * D;
  if (nact > 0 && (!r || !s_in || !y)) return fail(SSD_ERR_NULL, "r, s and y are required");
  const size_t ab = (size_t)nact * esize(in_dtype), yb = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * D) * 4;
  std::vector<Span> ins = {{"r", r, ab}, {"s", s_in, ab}, {"x0", x0, sb}, {"gate", gate, ab}};
  std::vector<Span> outs = {{"y", y, yb}, {"x_last", x_last, sb}, {"chunk_states", chunk_states, chunk_bytes(B, L, D)}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (B * D == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(x_last, x0, B * D, st), "minmax_scan");
  SSD_TRY(check_workspace(workspace, workspace_bytes, ssd::scan1_scratch_bytes(B, L, D), all));
  ssd::MinmaxScanArgs a{B, L, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, r, s_in, x0, gate, y, x_last,
                        chunk_states, workspace, wait_cfg()};
  return hip_status(ssd::launch_minmax_scan(a, st), "minmax_scan launch");
}

int ssd_minmax_update(int64_t B, int64_t D, int in_dtype, int out_dtype, const void* r, const void* s_in,
                      const void* gate, float* state, void* y, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || D < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (too_big({B, D}) || B * D >= (int64_t)1 << 38) return fail(SSD_ERR_SHAPE, "problem too large");
  const int64_t n = B * D;
  if (n > 0 && (!r || !s_in || !state || !y)) return fail(SSD_ERR_NULL, "r, s, state and y are required");
  const size_t ab = (size_t)n * esize(in_dtype);
  std::vector<Span> ins = {{"r", r, ab}, {"s", s_in, ab}, {"gate", gate, ab}};
  std::vector<Span> outs = {{"y", y, (size_t)n * esize(out_dtype)}, {"state", state, (size_t)n * 4}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  if (n == 0) return ok();
  ssd::MinmaxUpdateArgs a{B, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, r, s_in, gate, state, y};
  return hip_status(ssd::launch_minmax_update(a, static_cast<hipStream_t>(stream)), "minmax_update launch");
}

int ssd_minmax_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes) {
  SSD_TRY(scan1_shape(B, L, D));
  return ws_query(bytes, B * L * D > 0 ? ssd::minmax_bwd_scratch_bytes(B, L, D) : 0);
}

int ssd_minmax_scan_backward(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype, const void* r,
                             const void* s_in, const float* x0, const void* gate, const float* chunk_states,
                             const void* dy, const float* dx_last, void* dr, void* ds, float* dx0, void* dgate,
                             void* workspace, size_t workspace_bytes, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(scan1_shape(B, L, D));
  const int64_t nact = B * L * D;
  if (nact > 0 && (!r || !s_in || !dy || !dr || !ds)) return fail(SSD_ERR_NULL, "r, s, dy, dr and ds are required");
  const size_t ab = (size_t)nact * esize(in_dtype), ob = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * D) * 4;
  std::vector<Span> ins = {{"r", r, ab},   {"s", s_in, ab}, {"x0", x0, sb},
                           {"gate", gate, ab}, {"dy", dy, ab}, {"dx_last", dx_last, sb},
                           {"chunk_states", chunk_states, chunk_bytes(B, L, D)}};
  std::vector<Span> outs = {{"dr", dr, ob}, {"ds", ds, ob}, {"dx0", dx0, sb}, {"dgate", gate ? dgate : nullptr, ob}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (B * D == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(dx0, dx_last, B * D, st), "minmax_scan_backward");
  SSD_TRY(check_workspace(workspace, workspace_bytes, ssd::minmax_bwd_scratch_bytes(B, L, D), all));
  ssd::MinmaxBwdArgs a{B, L, D, in_dtype == SSD_BF16, out_dtype == SSD_BF16, r, s_in, x0, gate, chunk_states, dy,
                       dx_last, dr, ds, gate ? dgate : nullptr, dx0, workspace, wait_cfg()};
  return hip_status(ssd::launch_minmax_scan_backward(a, st), "minmax_scan_backward launch");
}

// ============================================================================ causal conv1d
int ssd_causal_conv1d(int64_t B, int64_t L, int64_t D, int64_t W, int in_dtype, int out_dtype, const void* x,
                      const float* weight, const float* bias, const float* state_in, void* y, float* state_out,
                      void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || L < 0 || D < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (W < 1 || W > 4) return fail(SSD_ERR_SHAPE, "kernel width W must be 1 .. 4");
  if (too_big({B, L, D}) || D >= (int64_t)1 << 22 || B * ((L + 63) / 64) * ((D + 63) / 64) >= (int64_t)1 << 31)
    return fail(SSD_ERR_SHAPE, "problem too large");
  const int64_t nact = B * L * D;
  if (nact > 0 && (!x || !y)) return fail(SSD_ERR_NULL, "x and y are required");
  if (B * D > 0 && !weight) return fail(SSD_ERR_NULL, "weight is required");
  const size_t xb = (size_t)nact * esize(in_dtype), yb = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * D * W) * 4;
  std::vector<Span> ins = {{"x", x, xb}, {"weight", weight, (size_t)(D * W) * 4}, {"bias", bias, (size_t)D * 4},
                           {"state_in", state_in, sb}};
  std::vector<Span> outs = {{"y", y, yb}, {"state_out", state_out, sb}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (B * D == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(state_out, state_in, B * D * W, st), "causal_conv1d");
  ssd::Conv1dArgs a{B, L, D, W, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, weight, bias, state_in, y, state_out};
  return hip_status(ssd::launch_causal_conv1d(a, st), "causal_conv1d launch");
}

int ssd_causal_conv1d_update(int64_t B, int64_t D, int64_t W, int in_dtype, int out_dtype, const void* x,
                             const float* weight, const float* bias, float* state, void* y, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || D < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (W < 1 || W > 4) return fail(SSD_ERR_SHAPE, "kernel width W must be 1 .. 4");
  if (too_big({B, D, W}) || B * D >= (int64_t)1 << 38) return fail(SSD_ERR_SHAPE, "problem too large");
  const int64_t n = B * D;
  if (n > 0 && (!x || !weight || !state || !y)) return fail(SSD_ERR_NULL, "x, weight, state and y are required");
  std::vector<Span> ins = {{"x", x, (size_t)n * esize(in_dtype)}, {"weight", weight, (size_t)(D * W) * 4},
                           {"bias", bias, (size_t)D * 4}};
  std::vector<Span> outs = {{"y", y, (size_t)n * esize(out_dtype)}, {"state", state, (size_t)(n * W) * 4}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  if (n == 0) return ok();
  ssd::Conv1dUpdateArgs a{B, D, W, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, weight, bias, state, y};
  return hip_status(ssd::launch_causal_conv1d_update(a, static_cast<hipStream_t>(stream)), "causal_conv1d_update launch");
}

// ============================================================================ selective
static bool supported_n(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

// Shape limits shared by the selective scans and their workspace queries; *nseq becomes B unless packed.
static int selective_shape(int64_t B, int64_t L, int64_t D, int64_t N, bool packed, int64_t* nseq, bool bwd) {
  if (B < 0 || L < 0 || D < 0 || N < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (!supported_n(N)) return fail(SSD_ERR_SHAPE, "N must be 1, 2, 4, 8 or 16");
  if (packed) {
    if (B != 1) return fail(SSD_ERR_SHAPE, "cu_seqlens requires B == 1");
    if (*nseq < 0) return fail(SSD_ERR_SHAPE, "nseq must be >= 0");
    if (*nseq == 0 && L != 0) return fail(SSD_ERR_SHAPE, "nseq == 0 requires L == 0");
    if (L >= (int64_t)1 << 31 || *nseq >= (int64_t)1 << 30) return fail(SSD_ERR_SHAPE, "packed length too large");
  } else {
    *nseq = B;
  }
  if (too_big({B, L, D}) || too_big({*nseq, D, N}) || (D + 255) / 256 > 65535 ||
      (bwd && B * ((L + 15) / 16) + *nseq >= (int64_t)1 << 31))
    return fail(SSD_ERR_SHAPE, "problem too large");
  return SSD_OK;
}

// Workspace of a selective scan with these sizes (0 when the call launches no scan).  The packed plan
// reads only whether a cu_seqlens table is given, never the table itself.
static size_t selective_ws(int64_t B, int64_t L, int64_t D, int64_t N, bool packed, int64_t nseq) {
  if (D * N == 0 || nseq == 0 || L == 0) return 0;
  ssd::SelectiveScanArgs a{};
  a.B = B; a.L = L; a.D = D; a.N = N; a.nseq = nseq;
  a.cu_seqlens = packed ? reinterpret_cast<const int32_t*>(&a) : nullptr;
  return ssd::selective_scan_scratch_bytes(a);
}
static size_t selective_bwd_ws(int64_t B, int64_t L, int64_t D, int64_t N, bool packed, int64_t nseq) {
  if (D * N == 0 || nseq == 0 || L == 0) return 0;
  ssd::SelectiveBwdArgs a{};
  a.B = B; a.L = L; a.D = D; a.N = N; a.nseq = nseq;
  a.cu_seqlens = packed ? reinterpret_cast<const int32_t*>(&a) : nullptr;
  return ssd::selective_scan_backward_scratch_bytes(a);
}

extern "C" int ssd_selective_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t nseq, int packed,
                                                  size_t* bytes) {
  SSD_TRY(selective_shape(B, L, D, N, packed != 0, &nseq, false));
  return ws_query(bytes, selective_ws(B, L, D, N, packed != 0, nseq));
}

extern "C" int ssd_selective_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t nseq,
                                                           int packed, size_t* bytes) {
  SSD_TRY(selective_shape(B, L, D, N, packed != 0, &nseq, true));
  return ws_query(bytes, selective_bwd_ws(B, L, D, N, packed != 0, nseq));
}

int ssd_selective_scan(int64_t B, int64_t L, int64_t D, int64_t N, int in_dtype, int out_dtype, const void* x,
                       const void* dt, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                       const void* z, const float* dt_bias, int dt_softplus, const int32_t* cu_seqlens, int64_t nseq,
                       const float* h0, void* y, float* h_last, void* workspace, size_t workspace_bytes,
                       void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(selective_shape(B, L, D, N, cu_seqlens != nullptr, &nseq, false));
  const int64_t nact = B * L * D;
  if (nact > 0 && (!x || !dt || !y)) return fail(SSD_ERR_NULL, "x, dt and y are required");
  if (B * L * N > 0 && (!Bm || !Cm)) return fail(SSD_ERR_NULL, "Bm and Cm are required");
  if (D * N > 0 && !A) return fail(SSD_ERR_NULL, "A is required");
  const size_t ab = (size_t)nact * esize(in_dtype);
  const size_t bb = (size_t)(B * L * N) * esize(in_dtype);
  const size_t sb = (size_t)(nseq * D * N) * 4;
  std::vector<Span> ins = {{"x", x, ab}, {"dt", dt, ab}, {"A", A, (size_t)(D * N) * 4}, {"Bm", Bm, bb}, {"Cm", Cm, bb},
                           {"Dskip", Dskip, (size_t)D * 4}, {"z", z, ab}, {"dt_bias", dt_bias, (size_t)D * 4},
                           {"cu_seqlens", cu_seqlens, (size_t)(nseq + 1) * 4}, {"h0", h0, sb}};
  std::vector<Span> outs = {{"y", y, (size_t)nact * esize(out_dtype)}, {"h_last", h_last, sb}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D * N == 0 || nseq == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(h_last, h0, nseq * D * N, s), "selective_scan");
  SSD_TRY(check_workspace(workspace, workspace_bytes, selective_ws(B, L, D, N, cu_seqlens != nullptr, nseq), all));
  ssd::SelectiveScanArgs a{B, L, D, N, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, dt, A, Bm, Cm, Dskip, z,
                           dt_bias, dt_softplus ? 1 : 0, cu_seqlens, nseq, h0, y, h_last, workspace};
  return hip_status(ssd::launch_selective_scan(a, s), "selective_scan launch");
}

int ssd_selective_scan_backward(int64_t B, int64_t L, int64_t D, int64_t N, int in_dtype, int out_dtype,
                                const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                                const float* Dskip, const void* z, const float* dt_bias, int dt_softplus,
                                const int32_t* cu_seqlens, int64_t nseq, const float* h0, const void* dy,
                                const float* dh_last, void* dx, void* ddt, float* dA,
                                void* dBm, void* dCm, float* dDskip, void* dz, float* ddt_bias, float* dh0,
                                void* workspace, size_t workspace_bytes, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(selective_shape(B, L, D, N, cu_seqlens != nullptr, &nseq, true));
  const int64_t nact = B * L * D;
  if (nact > 0 && (!x || !dt || !dy || !dx || !ddt)) return fail(SSD_ERR_NULL, "x, dt, dy, dx and ddt are required");
  if (B * L * N > 0 && (!Bm || !Cm || !dBm || !dCm)) return fail(SSD_ERR_NULL, "Bm, Cm, dBm and dCm are required");
  if (D * N > 0 && (!A || !dA)) return fail(SSD_ERR_NULL, "A and dA are required");
  if (nact > 0 && z && !dz) return fail(SSD_ERR_NULL, "dz is required with z");
  const size_t ab = (size_t)nact * esize(in_dtype), ob = (size_t)nact * esize(out_dtype);
  const size_t bb = (size_t)(B * L * N) * esize(in_dtype), bo = (size_t)(B * L * N) * esize(out_dtype);
  const size_t sb = (size_t)(nseq * D * N) * 4, db = (size_t)D * 4;
  std::vector<Span> ins = {{"x", x, ab},         {"dt", dt, ab},         {"A", A, (size_t)(D * N) * 4},
                           {"Bm", Bm, bb},       {"Cm", Cm, bb},         {"Dskip", Dskip, db},
                           {"z", z, ab},         {"dt_bias", dt_bias, db}, {"h0", h0, sb},
                           {"dy", dy, ab},       {"dh_last", dh_last, sb},
                           {"cu_seqlens", cu_seqlens, (size_t)(nseq + 1) * 4}};
  std::vector<Span> outs = {{"dx", dx, ob},      {"ddt", ddt, ob},       {"dA", dA, (size_t)(D * N) * 4},
                            {"dBm", dBm, bo},    {"dCm", dCm, bo},       {"dDskip", dDskip, db},
                            {"dz", z ? dz : nullptr, ob}, {"ddt_bias", ddt_bias, db}, {"dh0", dh0, sb}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D * N == 0 || nseq == 0) return ok();
  if (L == 0) {  // no steps: parameter gradients are zero, dh0 = dh_last
    SSD_TRY(hip_status(ssd::launch_copy_or_zero(dA, nullptr, D * N, s), "selective_scan_backward"));
    SSD_TRY(hip_status(ssd::launch_copy_or_zero(dDskip, nullptr, D, s), "selective_scan_backward"));
    SSD_TRY(hip_status(ssd::launch_copy_or_zero(ddt_bias, nullptr, D, s), "selective_scan_backward"));
    return hip_status(ssd::launch_copy_or_zero(dh0, dh_last, nseq * D * N, s), "selective_scan_backward");
  }
  SSD_TRY(check_workspace(workspace, workspace_bytes, selective_bwd_ws(B, L, D, N, cu_seqlens != nullptr, nseq), all));
  ssd::SelectiveBwdArgs a{B, L, D, N, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, dt, A, Bm, Cm, Dskip, z,
                          dt_bias, dt_softplus ? 1 : 0, cu_seqlens, nseq, h0, dy, dh_last, dx, ddt, dA, dBm, dCm, dDskip,
                          z ? dz : nullptr, ddt_bias, dh0, workspace};
  return hip_status(ssd::launch_selective_scan_backward(a, s), "selective_scan_backward launch");
}

int ssd_selective_update(int64_t B, int64_t D, int64_t N, int in_dtype, int out_dtype, const void* x, const void* dt,
                         const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                         const float* dt_bias, int dt_softplus, float* state, void* y, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || D < 0 || N < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (!supported_n(N)) return fail(SSD_ERR_SHAPE, "N must be 1, 2, 4, 8 or 16");
  if (too_big({B, D, N}) || B * D >= (int64_t)1 << 38) return fail(SSD_ERR_SHAPE, "problem too large");
  const int64_t n = B * D;
  if (n > 0 && (!x || !dt || !state || !y)) return fail(SSD_ERR_NULL, "x, dt, state and y are required");
  if (B * N > 0 && (!Bm || !Cm)) return fail(SSD_ERR_NULL, "Bm and Cm are required");
  if (D * N > 0 && !A) return fail(SSD_ERR_NULL, "A is required");
  const size_t ab = (size_t)n * esize(in_dtype);
  const size_t bb = (size_t)(B * N) * esize(in_dtype);
  std::vector<Span> ins = {{"x", x, ab}, {"dt", dt, ab}, {"A", A, (size_t)(D * N) * 4}, {"Bm", Bm, bb}, {"Cm", Cm, bb},
                           {"Dskip", Dskip, (size_t)D * 4}, {"z", z, ab}, {"dt_bias", dt_bias, (size_t)D * 4}};
  std::vector<Span> outs = {{"y", y, (size_t)n * esize(out_dtype)}, {"state", state, (size_t)(n * N) * 4}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  if (n == 0 || N == 0) return ok();
  ssd::SelectiveUpdateArgs a{B, D, N, in_dtype == SSD_BF16, out_dtype == SSD_BF16, x, dt, A, Bm, Cm, Dskip, z, dt_bias,
                             dt_softplus ? 1 : 0, state, y};
  return hip_status(ssd::launch_selective_update(a, static_cast<hipStream_t>(stream)), "selective_update launch");
}

// ============================================================================ HGRN2
static bool supported_d(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

static int hgrn2_scan_common(bool key, int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype,
                             const void* q, const void* k, const void* v, const void* g_logit, float lower_bound,
                             const float* S0, void* o, float* S_last, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || L < 0 || H < 0 || d < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (!supported_d(d)) return fail(SSD_ERR_SHAPE, "head dim d must be 16, 32, 64 or 128");
  // (the register sweeps address a stage of a head's rows with 32-bit offsets: H d < 2^24 keeps them small)
  if (too_big({B, L, H, d}) || B * H >= (int64_t)1 << 30 || H * d >= (int64_t)1 << 24)
    return fail(SSD_ERR_SHAPE, "problem too large");
  if (!(lower_bound >= 0.0f && lower_bound <= 1.0f)) return fail(SSD_ERR_VALUE, "lower_bound must be in [0, 1]");
  const int64_t nact = B * L * H * d;
  if (nact > 0 && (!q || !k || !v || !g_logit || !o)) return fail(SSD_ERR_NULL, "q, k, v, g_logit and o are required");
  const size_t ab = (size_t)nact * esize(in_dtype);
  const size_t sb = (size_t)(B * H * d * d) * 4;
  std::vector<Span> ins = {{"q", q, ab}, {"k", k, ab}, {"v", v, ab}, {"g_logit", g_logit, ab}, {"S0", S0, sb}};
  std::vector<Span> outs = {{"o", o, (size_t)nact * esize(out_dtype)}, {"S_last", S_last, sb}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B * H == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(S_last, S0, B * H * d * d, s), "hgrn2_scan");
  ssd::Hgrn2ScanArgs a{B, L, H, d, in_dtype == SSD_BF16, out_dtype == SSD_BF16, q, k, v, g_logit, lower_bound, S0, o,
                       S_last};
  if (key) return hip_status(ssd::launch_hgrn2_key_scan(a, s), "hgrn2_key_scan launch");
  return hip_status(ssd::launch_hgrn2_scan(a, s), "hgrn2_scan launch");
}

int ssd_hgrn2_scan(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype, const void* q,
                   const void* k, const void* v, const void* g_logit, float lower_bound, const float* S0, void* o,
                   float* S_last, void* stream) {
  return hgrn2_scan_common(false, B, L, H, d, in_dtype, out_dtype, q, k, v, g_logit, lower_bound, S0, o, S_last,
                           stream);
}

int ssd_hgrn2_key_scan(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype, const void* q,
                       const void* k, const void* v, const void* g_logit, float lower_bound, const float* S0, void* o,
                       float* S_last, void* stream) {
  return hgrn2_scan_common(true, B, L, H, d, in_dtype, out_dtype, q, k, v, g_logit, lower_bound, S0, o, S_last,
                           stream);
}

static int hgrn2_update_common(bool key, int64_t B, int64_t H, int64_t d, int in_dtype, int out_dtype,
                               const void* q, const void* k, const void* v, const void* g_logit, float lower_bound,
                               float* S, void* o, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (B < 0 || H < 0 || d < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (!supported_d(d)) return fail(SSD_ERR_SHAPE, "head dim d must be 16, 32, 64 or 128");
  if (too_big({B, H, d, d}) || B * H * d >= (int64_t)1 << 33) return fail(SSD_ERR_SHAPE, "problem too large");
  if (!(lower_bound >= 0.0f && lower_bound <= 1.0f)) return fail(SSD_ERR_VALUE, "lower_bound must be in [0, 1]");
  const int64_t n = B * H * d;
  if (n > 0 && (!q || !k || !v || !g_logit || !S || !o)) return fail(SSD_ERR_NULL, "q, k, v, g_logit, S and o are required");
  const size_t ab = (size_t)n * esize(in_dtype);
  std::vector<Span> ins = {{"q", q, ab}, {"k", k, ab}, {"v", v, ab}, {"g_logit", g_logit, ab}};
  std::vector<Span> outs = {{"o", o, (size_t)n * esize(out_dtype)}, {"S", S, (size_t)(n * d) * 4}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  if (n == 0) return ok();
  ssd::Hgrn2UpdateArgs a{B, H, d, in_dtype == SSD_BF16, out_dtype == SSD_BF16, q, k, v, g_logit, lower_bound, S, o};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (key) return hip_status(ssd::launch_hgrn2_key_update(a, s), "hgrn2_key_update launch");
  return hip_status(ssd::launch_hgrn2_update(a, s), "hgrn2_update launch");
}

int ssd_hgrn2_update(int64_t B, int64_t H, int64_t d, int in_dtype, int out_dtype, const void* q, const void* k,
                     const void* v, const void* g_logit, float lower_bound, float* S, void* o, void* stream) {
  return hgrn2_update_common(false, B, H, d, in_dtype, out_dtype, q, k, v, g_logit, lower_bound, S, o, stream);
}

int ssd_hgrn2_key_update(int64_t B, int64_t H, int64_t d, int in_dtype, int out_dtype, const void* q, const void* k,
                         const void* v, const void* g_logit, float lower_bound, float* S, void* o, void* stream) {
  return hgrn2_update_common(true, B, H, d, in_dtype, out_dtype, q, k, v, g_logit, lower_bound, S, o, stream);
}

int ssd_readout_norm(int64_t rows, int64_t width, int in_dtype, int out_dtype, const float* o, const void* gate,
                     const float* weight, const float* bias, float eps, void* y, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  if (rows < 0 || width < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (width > 8192) return fail(SSD_ERR_SHAPE, "width must be at most 8192");
  if (rows >= (int64_t)1 << 31 || too_big({rows, width})) return fail(SSD_ERR_SHAPE, "problem too large");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(SSD_ERR_VALUE, "eps must be finite and >= 0");
  const int64_t n = rows * width;
  if (n > 0 && (!o || !y)) return fail(SSD_ERR_NULL, "o and y are required");
  std::vector<Span> ins = {{"o", o, (size_t)n * 4},
                           {"gate", gate, (size_t)n * esize(in_dtype)},
                           {"weight", weight, (size_t)width * 4},
                           {"bias", bias, (size_t)width * 4}};
  std::vector<Span> outs = {{"y", y, (size_t)n * esize(out_dtype)}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  if (n == 0) return ok();
  ssd::ReadoutNormArgs a{rows, width, in_dtype == SSD_BF16, out_dtype == SSD_BF16, o, gate, weight, bias, eps, y};
  return hip_status(ssd::launch_readout_norm(a, static_cast<hipStream_t>(stream)), "readout_norm launch");
}

static int hgrn2_bwd_shape(int64_t B, int64_t L, int64_t H, int64_t d) {
  if (B < 0 || L < 0 || H < 0 || d < 0) return fail(SSD_ERR_SHAPE, "negative size");
  if (!supported_d(d)) return fail(SSD_ERR_SHAPE, "head dim d must be 16, 32, 64 or 128");
  if (too_big({B, L, H, d}) || B * H >= (int64_t)1 << 30 || H * d >= (int64_t)1 << 24)
    return fail(SSD_ERR_SHAPE, "problem too large");
  return SSD_OK;
}

static size_t hgrn2_bwd_ws(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, bool have_o) {
  if (B * H == 0 || L == 0) return 0;
  ssd::Hgrn2BwdArgs a{};
  a.B = B; a.L = L; a.H = H; a.d = d; a.in_bf16 = in_dtype == SSD_BF16;
  a.o = have_o ? reinterpret_cast<const float*>(&a) : nullptr;  // only whether it is given matters
  return ssd::hgrn2_scan_backward_scratch_bytes(a);
}

int ssd_hgrn2_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int have_o,
                                            size_t* bytes) {
  if (in_dtype != SSD_F32 && in_dtype != SSD_BF16) return fail(SSD_ERR_DTYPE, "in_dtype must be SSD_F32 or SSD_BF16");
  SSD_TRY(hgrn2_bwd_shape(B, L, H, d));
  return ws_query(bytes, hgrn2_bwd_ws(B, L, H, d, in_dtype, have_o != 0));
}

int ssd_hgrn2_scan_backward(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype, const void* q,
                            const void* k, const void* v, const void* g_logit, float lower_bound, const float* S0,
                            const float* o, const void* dO, const float* dS_last, void* dq, void* dk, void* dv,
                            void* dg_logit, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  SSD_TRY(check_dtypes(in_dtype, out_dtype));
  SSD_TRY(hgrn2_bwd_shape(B, L, H, d));
  if (!(lower_bound >= 0.0f && lower_bound <= 1.0f)) return fail(SSD_ERR_VALUE, "lower_bound must be in [0, 1]");
  const int64_t nact = B * L * H * d;
  if (nact > 0 && (!q || !k || !v || !g_logit || !dO))
    return fail(SSD_ERR_NULL, "q, k, v, g_logit and dO are required");
  if (nact > 0 && (!dq || !dk || !dv || !dg_logit))
    return fail(SSD_ERR_NULL, "dq, dk, dv and dg_logit are required");
  const size_t ab = (size_t)nact * esize(in_dtype), ob = (size_t)nact * esize(out_dtype);
  const size_t sb = (size_t)(B * H * d * d) * 4;
  std::vector<Span> ins = {{"q", q, ab},           {"k", k, ab},   {"v", v, ab},
                           {"g_logit", g_logit, ab}, {"S0", S0, sb}, {"o", o, (size_t)nact * 4},
                           {"dO", dO, ab},         {"dS_last", dS_last, sb}};
  std::vector<Span> outs = {{"dq", dq, ob}, {"dk", dk, ob}, {"dv", dv, ob}, {"dg_logit", dg_logit, ob},
                            {"dS0", dS0, sb}};
  std::vector<Span> all = ins;
  all.insert(all.end(), outs.begin(), outs.end());
  SSD_TRY(check_align(all));
  SSD_TRY(check_alias(outs, ins));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B * H == 0) return ok();
  if (L == 0) return hip_status(ssd::launch_copy_or_zero(dS0, dS_last, B * H * d * d, s), "hgrn2_scan_backward");
  SSD_TRY(check_workspace(workspace, workspace_bytes, hgrn2_bwd_ws(B, L, H, d, in_dtype, o != nullptr), all));
  ssd::Hgrn2BwdArgs a{B,  L,  H,  d,  in_dtype == SSD_BF16, out_dtype == SSD_BF16, q, k, v, g_logit, lower_bound,
                      S0, o,  dO, dS_last, dq, dk, dv, dg_logit, dS0, workspace};
  return hip_status(ssd::launch_hgrn2_scan_backward(a, s), "hgrn2_scan_backward launch");
}

}  // extern "C"
