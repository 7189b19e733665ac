// kernels.hpp -- host-side launchers of the gfx950 kernels.  Called by api.cpp after every
// argument has been validated; each returns the hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// ------------------------------------------------------------------ workspaces and bounded waits
// Every workspace starts with a lookback control block (work tickets, the launch counter, and the
// word in which a launch records a bounded wait that expired); the rest is the family's own layout.
size_t workspace_head_bytes();
size_t workspace_error_offset();  // byte offset of the expired-wait word within the head

// How the bounded waits of one launch behave: the polls before a wait gives up (each poll is a
// memory round trip, so the default bounds a wait at about a second), and an offset added to the
// epoch a waiting workgroup accepts (always 0, except from the timeout test hook, which makes every
// wait target words no launch writes).  A wait that gives up records it in the control block and
// hands on NaN as the carry, so every output that depends on it reads NaN.
constexpr unsigned int kSpinLimit = 1u << 20;
struct WaitCfg {
  unsigned int spin_limit = kSpinLimit;
  unsigned int skew = 0;
};

// ------------------------------------------------------------------ state-size-1 scans
// (RG-LRU and MinMax share one kernel template and its lookback scratch layout)
// Lookback scratch (control block + words) of a state-size-1 scan.
size_t scan1_scratch_bytes(int64_t B, int64_t L, int64_t D);

struct RglruScanArgs {
  int64_t B, L, D;
  int in_bf16, out_bf16;
  const void *x, *r_logit, *i_logit;
  const float* a_log;
  float c;
  const float* h0;
  const void* gate;  // y = gelu(gate) * h, or NULL
  void* y;
  float* h_last;
  float* chunk_states;  // [B][ceil(L/64)][D] state entering each 64-step chunk, or NULL
  void* scratch;        // scan1_scratch_bytes
  WaitCfg wait;
};
hipError_t launch_rglru_scan(const RglruScanArgs& a, hipStream_t s);
// The fixed per-device scratch of ssd_rglru_scan_noalloc: its device address on the current device
// (looked up once per device); it holds kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** out);

struct RglruUpdateArgs {
  int64_t B, D;
  int in_bf16, out_bf16;
  const void *x, *r_logit, *i_logit;
  const float* a_log;
  float c;
  const void* gate;
  float* state;
  void* y;
};
hipError_t launch_rglru_update(const RglruUpdateArgs& a, hipStream_t s);

// Gradients of the RG-LRU scan (loss = sum dy * y + sum dh_last * h_last): a forward pass that
// records the chunk carries, a reverse-time pass, and a fixed-order reduction for d a_log.
struct RglruBwdArgs {
  int64_t B, L, D;
  int in_bf16, out_bf16;
  const void *x, *r_logit, *i_logit;
  const float* a_log;
  float c;
  const float* h0;
  const void* gate;
  const float* chunk_states;  // the forward's chunk states, or NULL (then recomputed)
  const void* dy;         // in dtype
  const float* dh_last;   // [B][D] or NULL
  void *dx, *dr_logit, *di_logit, *dgate;  // out dtype; dgate may be NULL
  float* da_log;          // [D]
  float* dh0;             // [B][D] or NULL
  void* scratch;          // rglru_bwd_scratch_bytes
  WaitCfg wait;
};
size_t rglru_bwd_scratch_bytes(int64_t B, int64_t L, int64_t D);
hipError_t launch_rglru_scan_backward(const RglruBwdArgs& a, hipStream_t s);

struct MinmaxScanArgs {
  int64_t B, L, D;
  int in_bf16, out_bf16;
  const void *r, *s;
  const float* x0;
  const void* gate;  // y = x * gate, or NULL
  void* y;
  float* x_last;
  float* chunk_states;  // as RglruScanArgs
  void* scratch;        // scan1_scratch_bytes
  WaitCfg wait;
};
hipError_t launch_minmax_scan(const MinmaxScanArgs& a, hipStream_t s);

struct MinmaxBwdArgs {
  int64_t B, L, D;
  int in_bf16, out_bf16;
  const void *r, *s;
  const float* x0;        // [B][D] or NULL
  const void* gate;       // or NULL
  const float* chunk_states;  // the forward's chunk states, or NULL (then recomputed)
  const void* dy;         // in dtype
  const float* dx_last;   // [B][D] or NULL
  void *dr, *ds, *dgate;  // out dtype; dgate may be NULL
  float* dx0;             // [B][D] or NULL
  void* scratch;          // minmax_bwd_scratch_bytes
  WaitCfg wait;
};
size_t minmax_bwd_scratch_bytes(int64_t B, int64_t L, int64_t D);
hipError_t launch_minmax_scan_backward(const MinmaxBwdArgs& a, hipStream_t s);

struct MinmaxUpdateArgs {
  int64_t B, D;
  int in_bf16, out_bf16;
  const void *r, *s;
  const void* gate;
  float* state;
  void* y;
};
hipError_t launch_minmax_update(const MinmaxUpdateArgs& a, hipStream_t s);

// ------------------------------------------------------------------ causal depthwise conv
struct Conv1dArgs {
  int64_t B, L, D, W;
  int in_bf16, out_bf16;
  const void* x;
  const float* weight;    // [D][W]
  const float* bias;      // [D] or NULL
  const float* state_in;  // [B][D][W] or NULL
  void* y;
  float* state_out;       // [B][D][W] or NULL
};
hipError_t launch_causal_conv1d(const Conv1dArgs& a, hipStream_t s);

struct Conv1dUpdateArgs {
  int64_t B, D, W;
  int in_bf16, out_bf16;
  const void* x;
  const float* weight;
  const float* bias;
  float* state;           // [B][D][W] in / out
  void* y;
};
hipError_t launch_causal_conv1d_update(const Conv1dUpdateArgs& a, hipStream_t s);

// ------------------------------------------------------------------ selective
struct SelectiveScanArgs {
  int64_t B, L, D, N;
  int in_bf16, out_bf16;
  const void *x, *dt;
  const float* A;
  const void *Bm, *Cm;
  const float* Dskip;
  const void* z;
  const float* dt_bias;
  int dt_softplus;
  const int32_t* cu_seqlens;  // device, or NULL (batched)
  int64_t nseq;               // sequences (B when batched)
  const float* h0;
  void* y;
  float* h_last;
  void* scratch;
};
// Segment length the launcher will use, and the scratch it needs.
int64_t selective_segment_len(const SelectiveScanArgs& a);
size_t selective_scan_scratch_bytes(const SelectiveScanArgs& a);
hipError_t launch_selective_scan(const SelectiveScanArgs& a, hipStream_t s);

// Gradients of the selective scan (batched, or packed varlen with B = 1).
struct SelectiveBwdArgs {
  int64_t B, L, D, N;
  int in_bf16, out_bf16;
  const void *x, *dt;
  const float* A;
  const void *Bm, *Cm;
  const float* Dskip;   // or NULL
  const void* z;        // or NULL
  const float* dt_bias; // or NULL
  int dt_softplus;
  const int32_t* cu_seqlens;  // device [nseq + 1] or NULL
  int64_t nseq;
  const float* h0;      // [B or nseq][D][N] or NULL
  const void* dy;       // in dtype
  const float* dh_last; // [B][D][N] or NULL
  void *dx, *ddt;       // out dtype
  float* dA;            // [D][N]
  void *dBm, *dCm;      // out dtype [B][L][N]
  float* dDskip;        // [D] or NULL
  void* dz;             // out dtype, when z is given
  float* ddt_bias;      // [D] or NULL
  float* dh0;           // [B][D][N] or NULL
  void* scratch;        // selective_scan_backward_scratch_bytes
};
size_t selective_scan_backward_scratch_bytes(const SelectiveBwdArgs& a);
hipError_t launch_selective_scan_backward(const SelectiveBwdArgs& a, hipStream_t s);

struct SelectiveUpdateArgs {
  int64_t B, D, N;
  int in_bf16, out_bf16;
  const void *x, *dt;
  const float* A;
  const void *Bm, *Cm;
  const float* Dskip;
  const void* z;
  const float* dt_bias;
  int dt_softplus;
  float* state;
  void* y;
};
hipError_t launch_selective_update(const SelectiveUpdateArgs& a, hipStream_t s);

// ------------------------------------------------------------------ HGRN2
struct Hgrn2ScanArgs {
  int64_t B, L, H, d;
  int in_bf16, out_bf16;
  const void *q, *k, *v, *g_logit;
  float lower_bound;
  const float* S0;
  void* o;
  float* S_last;
};
hipError_t launch_hgrn2_scan(const Hgrn2ScanArgs& a, hipStream_t s);

struct Hgrn2UpdateArgs {
  int64_t B, H, d;
  int in_bf16, out_bf16;
  const void *q, *k, *v, *g_logit;
  float lower_bound;
  float* S;
  void* o;
};
hipError_t launch_hgrn2_update(const Hgrn2UpdateArgs& a, hipStream_t s);
// Key-axis gating (S[i][j] = g_j S[i][j] + v_i k_j): the same arguments.
hipError_t launch_hgrn2_key_scan(const Hgrn2ScanArgs& a, hipStream_t s);
// The row-gated scan as a register sweep (the cases the chunked MFMA kernel does not take).
hipError_t launch_hgrn2_row_sweep(const Hgrn2ScanArgs& a, hipStream_t s);
// The key-axis-gated scan in chunked MFMA form: bf16 inputs, d = 128, any lower bound.
hipError_t launch_hgrn2_key_chunk(const Hgrn2ScanArgs& a, hipStream_t s);
hipError_t launch_hgrn2_key_update(const Hgrn2UpdateArgs& a, hipStream_t s);

// Readout LayerNorm over rows of `width` features (fp32 o), affine, times silu(gate).
struct ReadoutNormArgs {
  int64_t rows, width;
  int in_bf16, out_bf16;  // gate dtype, output dtype
  const float* o;
  const void* gate;
  const float* weight;
  const float* bias;
  float eps;
  void* y;
};
hipError_t launch_readout_norm(const ReadoutNormArgs& a, hipStream_t s);

// Backward of the HGRN2 scan: o is the forward output in fp32 (NULL: recomputed into scratch).
struct Hgrn2BwdArgs {
  int64_t B, L, H, d;
  int in_bf16, out_bf16;
  const void *q, *k, *v, *g_logit;
  float lower_bound;
  const float* S0;
  const float* o;
  const void* dO;
  const float* dS_last;
  void *dq, *dk, *dv, *dg_logit;
  float* dS0;
  void* scratch;
};
size_t hgrn2_scan_backward_scratch_bytes(const Hgrn2BwdArgs& a);
hipError_t launch_hgrn2_scan_backward(const Hgrn2BwdArgs& a, hipStream_t s);
// The backward in chunked MFMA form (bf16 inputs, d = 128, H < 2^16): the cases it takes, its scratch,
// and its launch (launch_hgrn2_scan_backward dispatches to it).
bool hgrn2_backward_chunked(const Hgrn2BwdArgs& a);
size_t hgrn2_backward_chunked_scratch_bytes(const Hgrn2BwdArgs& a);
hipError_t launch_hgrn2_backward_chunked(const Hgrn2BwdArgs& a, hipStream_t s);

// ------------------------------------------------------------------ utilities
// dst[i] = src ? src[i] : 0 for i < n (used for empty problems: final state = initial state).
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s);

}  // namespace ssd
