/*
 * ssd.h -- C ABI of the MI355X (gfx950) gated diagonal linear-recurrence scans.
 *
 * Three forms of h_t = a_t (.) h_{t-1} + b_t, each as a full-sequence scan and a
 * single-step decode update:
 *
 *   RG-LRU        state size 1 per channel          ssd_rglru_scan / ssd_rglru_update
 *                 (gradients)                       ssd_rglru_scan_backward
 *   MinMax        state size 1 per channel          ssd_minmax_scan / ssd_minmax_update
 *                 (gradients)                       ssd_minmax_scan_backward
 *   causal conv   depthwise, width W <= 4           ssd_causal_conv1d / ssd_causal_conv1d_update
 *   selective     N <= 16 states per channel        ssd_selective_scan / ssd_selective_update
 *                 (gradients)                       ssd_selective_scan_backward
 *   HGRN2         d x d matrix state per head       ssd_hgrn2_scan / ssd_hgrn2_update
 *                 (gradients)                       ssd_hgrn2_scan_backward
 *                 (gate on the key axis)            ssd_hgrn2_key_scan / ssd_hgrn2_key_update
 *                 (readout LayerNorm, silu gate)    ssd_readout_norm
 *
 * Conventions (every entry point):
 *   - Sizes are int64_t element counts; every pointer is DEVICE memory owned by
 *     the caller, dense row-major, with the layout given per function.
 *   - Activations are SSD_F32 or SSD_BF16 (the `in` dtype); parameters (a_log,
 *     A, Dskip, dt_bias) and recurrent state are always fp32.  Outputs are fp32
 *     or, when `in` is SSD_BF16, optionally bf16 (round-to-nearest-even).
 *   - The library computes in fp32 from the input bits; state stays fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; the call returns after the launch.
 *   - Every argument is validated on the host before anything is enqueued.  A
 *     non-zero status means nothing was launched and nothing was written;
 *     ssd_last_error() then holds a thread-local message.  Faults during
 *     execution surface at the caller's next synchronisation, as with any HIP
 *     call.
 *   - Base pointers must be 16-byte aligned.  Outputs must not overlap inputs.
 *   - Empty problems (a zero size) launch nothing except copying the initial
 *     state to the final-state output (or zero-filling it).
 *   - The library allocates no memory and keeps no state between calls.  Scans
 *     that pass partial results between workgroups take a caller-owned device
 *     `workspace` (see "Workspaces" below).  The library is reentrant and
 *     thread-safe: calls share nothing but the memory the caller passes.
 *   - NaN / Inf inputs propagate by IEEE rules; nothing is trapped.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

enum {
  SSD_OK = 0,
  SSD_ERR_NULL = 1,   /* a required pointer is NULL                              */
  SSD_ERR_SHAPE = 2,  /* a size is negative or outside the supported range        */
  SSD_ERR_DTYPE = 3,  /* unsupported dtype or dtype combination                   */
  SSD_ERR_ALIGN = 4,  /* a base pointer is not 16-byte aligned                    */
  SSD_ERR_VALUE = 5,  /* a scalar argument is out of range (c, lower_bound, ...)  */
  SSD_ERR_ALIAS = 6,  /* an output overlaps an input                              */
  SSD_ERR_HIP = 7,    /* the HIP runtime reported an error (launch, copy)         */
  SSD_ERR_TIMEOUT = 8 /* a bounded wait between workgroups expired (ssd_workspace_check) */
};

/* Static description of a status code. */
const char* ssd_status_str(int status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* ssd_last_error(void);
/* Library ABI version (major * 10000 + minor * 100 + patch). */
int ssd_version(void);

/* ---------------------------------------------------------------------------------------------
 * Workspaces.  The scans that split one sequence over several workgroups (RG-LRU, MinMax and
 * selective scans and the gradients of those and of HGRN2) hand partial results and work tickets
 * from workgroup to workgroup through device memory the caller owns: the `workspace` argument, of
 * at least the size the matching ssd_*_workspace_bytes query reports for the same sizes on the
 * current device, 256-byte aligned.
 *   - A workspace belongs to one entry point.  It must be zero-filled before its first use; each call
 *     leaves it ready for the next call of the same entry point (it keeps a launch counter, so the
 *     words one launch publishes never validate for another), so it is reused without clearing for
 *     any later sizes.  Passed to a different entry point, it must be zero-filled again first.
 *   - Calls whose work may run at the same time (on different streams, or from threads that do not
 *     order their calls) need distinct workspaces.
 *   - A call that needs no workspace (an empty problem) accepts NULL.
 * Workspace errors: SSD_ERR_NULL (NULL when one is needed), SSD_ERR_SHAPE (workspace_bytes below the
 * query's size), SSD_ERR_ALIGN (not 256-byte aligned), SSD_ERR_ALIAS (overlaps another argument).
 *
 * The workgroups of these scans wait on one another with bounded waits (about a second).  A wait
 * that expires, which a correct launch never sees, does not hang the GPU: the waiting workgroup
 * takes NaN as its incoming state (so every output that depends on it reads NaN) and records the
 * event in the workspace.  ssd_workspace_check reports it.
 * ------------------------------------------------------------------------------------------- */

/* Waits for `stream` to finish its work, then reports whether any launch that used `workspace` since
 * the last check had a bounded wait expire: SSD_ERR_TIMEOUT (and the record is cleared) or SSD_OK.
 * The workspace is one passed to any of the calls that take one.  SSD_ERR_NULL for a NULL workspace,
 * SSD_ERR_HIP if the runtime fails. */
int ssd_workspace_check(const void* workspace, void* stream);

/* Test hook for the timeout path, process-wide: the bounded waits of later launches give up after
 * `spin_limit` polls (0 restores the default), and with `never_ready` nonzero they wait for words no
 * launch ever writes, so every wait expires (then outputs read NaN as described above and
 * ssd_workspace_check reports SSD_ERR_TIMEOUT).  Every kernel still runs to its end. */
void ssd_testing_lookback(unsigned int spin_limit, int never_ready);

/* Steps per chunk of the state-size-1 scans (RG-LRU, MinMax).  Their optional `chunk_states`
 * buffers are [B, ceil(L / SSD_SCAN_CHUNK), D] fp32, entry [b, k, d] being the state entering step
 * k * SSD_SCAN_CHUNK (h0 for k = 0): 1/64 of the per-step states, which a forward pass can save
 * for the backward pass so that the latter need not recompute them. */
#define SSD_SCAN_CHUNK 64

/* ---------------------------------------------------------------------------------------------
 * RG-LRU scan.  Defined by the lrnnx documentation, "lrnnx.models.ltv.rglru" (RGLRU.forward gate
 * computation and RGLRU.step recurrence):  for each batch b, channel d and step t
 *     r = sigmoid(r_logit), i = sigmoid(i_logit), log a_t = c * r * a_log[d],
 *     h_t = a_t * h_{t-1} + sqrt(1 - a_t^2) * (i * x),     y_t = h_t,
 * starting from h0 (or 0).  The base a = exp(a_log) lies in (0, 1) for a_log < 0.  With a gate,
 * y_t = gelu(gate_t) * h_t: the block's output multiply (gelu of its gate projection times the
 * recurrence output), with torch's exact gelu v * Phi(v).
 *   x, r_logit, i_logit : [B, L, D] activations (in dtype)
 *   a_log               : [D] fp32          c : finite scalar (8 in the Griffin block)
 *   h0                  : [B, D] fp32 or NULL (= zeros)
 *   gate                : [B, L, D] (in dtype) or NULL (= no output multiply)
 *   y                   : [B, L, D] (out dtype)
 *   h_last              : [B, D] fp32 or NULL; receives h_{L-1} (h0 when L = 0), never gated
 *   chunk_states        : [B, ceil(L/64), D] fp32 or NULL; receives the state entering each 64-step
 *                         chunk (see SSD_SCAN_CHUNK), the same bits ssd_rglru_scan_backward recomputes
 *   workspace           : see "Workspaces"; size from ssd_rglru_scan_workspace_bytes(B, L, D)
 * Errors: SSD_ERR_NULL (x, r_logit, i_logit, a_log, y when B*L*D > 0), SSD_ERR_SHAPE (negative
 * size, D >= 2^22, or B * ceil(L/64) * ceil(D/64) >= 2^31), SSD_ERR_DTYPE, SSD_ERR_ALIGN,
 * SSD_ERR_VALUE (c not finite), SSD_ERR_ALIAS, and the workspace errors.
 * ------------------------------------------------------------------------------------------- */
int ssd_rglru_scan(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype,
                   const void* x, const void* r_logit, const void* i_logit,
                   const float* a_log, float c, const float* h0, const void* gate,
                   void* y, float* h_last, float* chunk_states,
                   void* workspace, size_t workspace_bytes, void* stream);
/* Workspace size of ssd_rglru_scan for these sizes, in *bytes.  SSD_ERR_NULL (bytes NULL) or
 * SSD_ERR_SHAPE (sizes the scan rejects).  The other queries below follow the same convention. */
int ssd_rglru_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes);

/* ssd_rglru_scan without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The same kernels
 * run on a fixed scratch array the library holds per GPU (SSD_NOALLOC_SCRATCH_BYTES, taken when the
 * library's device code loads on that GPU and kept until the process ends); the call allocates nothing.
 * All calls on one GPU share that array, so calls whose work may overlap on one GPU (different streams,
 * unordered threads) race; calls ordered on one stream do not.  Arguments, results and errors as
 * ssd_rglru_scan, plus SSD_ERR_SHAPE when ssd_rglru_scan_workspace_bytes exceeds the array's size. */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssd_rglru_scan_noalloc(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype,
                           const void* x, const void* r_logit, const void* i_logit,
                           const float* a_log, float c, const float* h0, const void* gate,
                           void* y, float* h_last, float* chunk_states, void* stream);

/* Gradients of ssd_rglru_scan (reverse-time adjoint; the pages train through autograd and print no
 * backward pass, so this is the gradient of the forward definition above) for the loss
 *     sum_{b,t,d} dy * y  +  sum_{b,d} dh_last * h_last:
 *   g_t = dL/dh_t = dy_t G_t + a_{t+1} g_{t+1} (G_t = gelu(gate_t) or 1; g_{L-1} adds dh_last), and
 *   dx = g beta i,  d i_logit = g beta x i (1-i),  with l = log a_t = c r a_log,
 *   dl = g (a h_{t-1} - i x a^2 / beta),  d r_logit = dl c a_log r (1-r),  d a_log = sum_{b,t} dl c r,
 *   dgate = dy h_t gelu'(gate),  dh0 = a_0 g_0.
 *   x, r_logit, i_logit, gate, a_log, c, h0 : as ssd_rglru_scan (the forward's inputs)
 *   chunk_states        : [B, ceil(L/64), D] fp32 from the forward call, or NULL
 *   dy                  : [B, L, D] (in dtype) gradient of y;   dh_last : [B, D] fp32 or NULL (= 0)
 *   dx, dr_logit, di_logit : [B, L, D] (out dtype), overwritten
 *   dgate               : [B, L, D] (out dtype) or NULL; written only when gate is given
 *   da_log              : [D] fp32, overwritten (not accumulated)
 *   dh0                 : [B, D] fp32 or NULL
 * The per-step forward states are rebuilt inside each 64-step chunk from the chunk's incoming state:
 * the forward's chunk_states when given, else a forward pass first records them in the library's
 * workspace (then the call needs no saved activations).  Results are deterministic, and identical
 * with and without chunk_states.
 * workspace: see "Workspaces"; size from ssd_rglru_scan_backward_workspace_bytes(B, L, D).
 * Errors as ssd_rglru_scan, plus SSD_ERR_NULL for missing dy / dx / dr_logit / di_logit / da_log. */
int ssd_rglru_scan_backward(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype,
                            const void* x, const void* r_logit, const void* i_logit,
                            const float* a_log, float c, const float* h0, const void* gate,
                            const float* chunk_states, const void* dy, const float* dh_last,
                            void* dx, void* dr_logit, void* di_logit, float* da_log, float* dh0,
                            void* dgate, void* workspace, size_t workspace_bytes, void* stream);
int ssd_rglru_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes);

/* One RG-LRU decode step (RGLRU.step: single token, state carried by the caller).
 *   x, r_logit, i_logit : [B, D] (in dtype);  a_log : [D] fp32;  gate : [B, D] or NULL
 *   state               : [B, D] fp32, read then overwritten with h_t (in place)
 *   y                   : [B, D] (out dtype), y = h_t, or gelu(gate) * h_t
 * Errors as ssd_rglru_scan; y must not overlap state. */
int ssd_rglru_update(int64_t B, int64_t D, int in_dtype, int out_dtype,
                     const void* x, const void* r_logit, const void* i_logit,
                     const float* a_log, float c, const void* gate, float* state, void* y,
                     void* stream);

/* ---------------------------------------------------------------------------------------------
 * MinMax scan.  Defined by the minmaxrnc package (minmax_neuron.py, MinMaxNeuron: the state update
 * of its docstring and forward(); minmax_operator.py: the operator and its composition):  for each
 * batch b, channel d and step t
 *     x_t = max(min(r_t, x_{t-1}), s_t),      y_t = x_t, or x_t * gate_t with a gate,
 * starting from x0 (or 0, the neuron's default initial state).  min and max order -0 below +0 and
 * return NaN when either operand is NaN, so every state is exactly one input value and the result
 * is identical bit for bit to the sequential loop, however the scan is split.
 *   r, s                : [B, L, D] (in dtype), the per-step upper and lower clamps
 *   x0                  : [B, D] fp32 or NULL (= zeros)
 *   gate                : [B, L, D] (in dtype) or NULL (the neuron's output gate values)
 *   y                   : [B, L, D] (out dtype)
 *   x_last              : [B, D] fp32 or NULL; receives x_{L-1} (x0 when L = 0), never gated
 *   chunk_states        : [B, ceil(L/64), D] fp32 or NULL, as for ssd_rglru_scan
 *   workspace           : see "Workspaces"; size from ssd_minmax_scan_workspace_bytes(B, L, D)
 * Errors: as ssd_rglru_scan (no scalar arguments).
 * ------------------------------------------------------------------------------------------- */
int ssd_minmax_scan(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype,
                    const void* r, const void* s, const float* x0, const void* gate,
                    void* y, float* x_last, float* chunk_states,
                    void* workspace, size_t workspace_bytes, void* stream);
int ssd_minmax_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes);

/* Gradients of ssd_minmax_scan for the loss  sum dy * y + sum dx_last * x_last.  The package trains
 * the neuron through torch autograd, so the derivative of min and max is torch's: the selected operand
 * takes the gradient, equal operands take half each, and a NaN operand passes it to both.  With
 * m_t = min(r_t, x_{t-1}), g_t = dL/dx_t = dy_t G_t + (gradient from step t+1) (G_t = gate_t or 1;
 * g_{L-1} adds dx_last):
 *   dr_t = g_t wM wR,   ds_t = g_t wS,   dgate_t = dy_t x_t,   dx0 = g_0 wM_0 wX_0,
 * where wR, wX are the weights of r_t and x_{t-1} in min(r_t, x_{t-1}) and wM, wS those of m_t and
 * s_t in max(m_t, s_t).
 *   r, s, x0, gate      : as ssd_minmax_scan (the forward's inputs)
 *   chunk_states        : [B, ceil(L/64), D] fp32 from the forward call, or NULL
 *   dy                  : [B, L, D] (in dtype);   dx_last : [B, D] fp32 or NULL (= 0)
 *   dr, ds              : [B, L, D] (out dtype), overwritten
 *   dgate               : [B, L, D] (out dtype) or NULL; written only when gate is given
 *   dx0                 : [B, D] fp32 or NULL
 * The forward states are rebuilt from each 64-step chunk's incoming state (the forward's
 * chunk_states, else recorded by a forward pass first).  Results are deterministic, and identical
 * with and without chunk_states.
 * workspace: see "Workspaces"; size from ssd_minmax_scan_backward_workspace_bytes(B, L, D).
 * Errors as ssd_minmax_scan, plus SSD_ERR_NULL for missing dy / dr / ds. */
int ssd_minmax_scan_backward(int64_t B, int64_t L, int64_t D, int in_dtype, int out_dtype,
                             const void* r, const void* s, const float* x0, const void* gate,
                             const float* chunk_states, const void* dy, const float* dx_last, void* dr, void* ds,
                             float* dx0, void* dgate, void* workspace, size_t workspace_bytes, void* stream);
int ssd_minmax_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t D, size_t* bytes);

/* One MinMax decode step.  r, s, gate : [B, D] (gate may be NULL); state : [B, D] fp32 in/out;
 * y : [B, D].  Errors as ssd_minmax_scan; y must not overlap state. */
int ssd_minmax_update(int64_t B, int64_t D, int in_dtype, int out_dtype,
                      const void* r, const void* s, const void* gate, float* state, void* y,
                      void* stream);

/* ---------------------------------------------------------------------------------------------
 * Causal depthwise convolution in front of the RG-LRU recurrence.  Defined by the lrnnx
 * documentation, "lrnnx.models.ltv.rglru": the block's nn.Conv1d (groups = channels, kernel
 * d_conv = W, padding W - 1, first L outputs kept) and the conv_state window of its step():
 *     y[b, t, d] = bias[d] + sum_{k < W} weight[d][k] * x[b, t - (W-1) + k, d].
 * Inputs before t = 0 come from state_in (entry W + tau of a channel's window holds time tau < 0)
 * or are zero when state_in is NULL.  state_out receives the window after the sequence: the last
 * W inputs (times L-W .. L-1; from state_in or zero where negative), ready for
 * ssd_causal_conv1d_update or a following ssd_causal_conv1d call.
 *   x, y                : [B, L, D] (in / out dtype)
 *   weight              : [D, W] fp32 (nn.Conv1d's [D, 1, W] weight)     bias : [D] fp32 or NULL
 *   state_in, state_out : [B, D, W] fp32 or NULL; they must not overlap
 * Errors: SSD_ERR_NULL (x, y when B*L*D > 0; weight when B*D > 0), SSD_ERR_SHAPE (negative size,
 * W outside 1 .. 4, D >= 2^22, B * ceil(L/64) * ceil(D/64) >= 2^31), SSD_ERR_DTYPE,
 * SSD_ERR_ALIGN, SSD_ERR_ALIAS.
 * ------------------------------------------------------------------------------------------- */
int ssd_causal_conv1d(int64_t B, int64_t L, int64_t D, int64_t W, int in_dtype, int out_dtype,
                      const void* x, const float* weight, const float* bias, const float* state_in,
                      void* y, float* state_out, void* stream);

/* One convolution decode step (the block's step()): state [B, D, W] fp32 shifts left by one, x
 * [B, D] enters last, y [B, D] = bias + sum_k weight[d][k] * state[b][d][k].  In place.
 * Errors as ssd_causal_conv1d; y must not overlap state. */
int ssd_causal_conv1d_update(int64_t B, int64_t D, int64_t W, int in_dtype, int out_dtype,
                             const void* x, const float* weight, const float* bias, float* state,
                             void* y, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Multi-scale selective scan.  Defined by the cortexnet 3.2.1 package, cortexnet/ssm.py,
 * MultiScaleSSM.forward and MultiScaleSSM._selective_scan:  for each sequence, channel d, state
 * n and step t
 *     delta = dt + dt_bias[d], then softplus(delta) if dt_softplus (identity above 20),
 *     abar  = exp(min(delta * A[d][n], 20)),      h_n = abar * h_n + (delta * B_n) * x,
 *     y     = (sum_n C_n * h_n + Dskip[d] * x) * silu(z).
 *   x, dt, z, y  : [B, L, D] (z NULL = no gate)       A : [D, N] fp32
 *   Bm, Cm       : [B, L, N] (in dtype)                Dskip, dt_bias : [D] fp32 or NULL (= 0)
 *   cu_seqlens   : device int32[nseq + 1] or NULL.  With it, B must be 1 and the L rows are
 *                  nseq packed sequences, sequence s = rows [cu_seqlens[s], cu_seqlens[s+1]);
 *                  each starts from its own h0 (or 0).  The table must satisfy cu_seqlens[0] = 0,
 *                  non-decreasing, cu_seqlens[nseq] = L (the caller's duty: it is device memory
 *                  and is not read on the host).  Zero-length sequences are allowed.
 *   h0, h_last   : [B or nseq, D, N] fp32 or NULL.
 *   Supported N : 1, 2, 4, 8, 16.
 *   workspace    : see "Workspaces"; size from ssd_selective_scan_workspace_bytes(B, L, D, N, nseq,
 *                  packed) with packed = (cu_seqlens != NULL) (nseq is ignored when not packed)
 * Errors: SSD_ERR_NULL, SSD_ERR_SHAPE (negative size, unsupported N, cu_seqlens with B != 1,
 * nseq < 0), SSD_ERR_DTYPE, SSD_ERR_ALIGN, SSD_ERR_ALIAS, and the workspace errors.
 * ------------------------------------------------------------------------------------------- */
int ssd_selective_scan(int64_t B, int64_t L, int64_t D, int64_t N, int in_dtype, int out_dtype,
                       const void* x, const void* dt, const float* A,
                       const void* Bm, const void* Cm, const float* Dskip, const void* z,
                       const float* dt_bias, int dt_softplus,
                       const int32_t* cu_seqlens, int64_t nseq,
                       const float* h0, void* y, float* h_last,
                       void* workspace, size_t workspace_bytes, void* stream);
int ssd_selective_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t nseq, int packed,
                                       size_t* bytes);

/* Gradients of ssd_selective_scan (batched, or packed varlen sequences as there) for the loss
 *     sum_{b,t,d} dy * y  +  sum_{sequence,d,n} dh_last * h_last.
 * The pages train through autograd and print no backward pass; this is the gradient of the forward
 * definition above, with the clamp at 20 passing no gradient where delta*A > 20 (torch.clamp).
 * With s_t the readout before the gate, ds_t = dy_t silu(z_t) and g_t = dL/dh_t:
 *   dx = ds Dskip + delta sum_n g B,  dBm_tn = sum_d g delta x,  dCm_tn = sum_d ds h,  dz = dy s silu'(z),
 *   d delta = x sum_n g B + sum_n g h_{t-1} abar A (unclamped entries),  ddt = d delta softplus'(dt + bias)
 *   (or d delta without softplus),  dA = sum_{b,t} g h_{t-1} abar delta,  dDskip = sum ds x,
 *   ddt_bias = sum ddt,  dh0 = abar_0 g_0.
 *   inputs              : as ssd_selective_scan (cu_seqlens, nseq and the state shapes too), plus
 *   dy                  : [B, L, D] (in dtype);   dh_last : [B or nseq, D, N] fp32 or NULL (= 0)
 *   dx, ddt             : [B, L, D] (out dtype);  dz : [B, L, D] (out dtype), required when z is given
 *   dBm, dCm            : [B, L, N] (out dtype)
 *   dA                  : [D, N] fp32;  dDskip, ddt_bias : [D] fp32 or NULL;
 *   dh0                 : [B or nseq, D, N] fp32 or NULL (a zero-length sequence gets its dh_last)
 * Every output is overwritten (not accumulated).  The forward states are recomputed (the workspace
 * holds per-64-row-unit states, about 6 x B * ceil(L/64) * D * N fp32; see "Workspaces", size
 * from ssd_selective_scan_backward_workspace_bytes).  Reductions run in a fixed order: results are
 * deterministic.  Errors as ssd_selective_scan, plus SSD_ERR_NULL for missing dy / dx / ddt / dBm /
 * dCm / dA (or dz with z). */
int ssd_selective_scan_backward(int64_t B, int64_t L, int64_t D, int64_t N, int in_dtype, int out_dtype,
                                const void* x, const void* dt, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip, const void* z,
                                const float* dt_bias, int dt_softplus,
                                const int32_t* cu_seqlens, int64_t nseq, const float* h0,
                                const void* dy, const float* dh_last,
                                void* dx, void* ddt, float* dA, void* dBm, void* dCm,
                                float* dDskip, void* dz, float* ddt_bias, float* dh0,
                                void* workspace, size_t workspace_bytes, void* stream);
int ssd_selective_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t nseq,
                                                int packed, size_t* bytes);

/* One selective decode step (the L == 1 path of MultiScaleSSM.forward with past_state).
 *   x, dt, z, y : [B, D];  Bm, Cm : [B, N];  A : [D, N] fp32;  state : [B, D, N] fp32 in place.
 * Other arguments and errors as ssd_selective_scan. */
int ssd_selective_update(int64_t B, int64_t D, int64_t N, int in_dtype, int out_dtype,
                         const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip,
                         const void* z, const float* dt_bias, int dt_softplus,
                         float* state, void* y, void* stream);

/* ---------------------------------------------------------------------------------------------
 * HGRN2 matrix-state scan.  Defined by the frankenstein-transformer documentation, "HGRN2
 * Attention" (state-update equation and forget gate):  per batch b, head h and step t
 *     g_i  = lower_bound + (1 - lower_bound) * sigmoid(g_logit_i),
 *     S[i][j] = g_i * S[i][j] + v_i * k_j,        o_i = sum_j S[i][j] * q_j,
 * i.e. S_t = diag(g_t) S_{t-1} + v_t k_t^T and o_t = S_t q_t (readout includes token t).
 *   q, k, v, g_logit, o : [B, L, H, d] (in dtype / out dtype)
 *   S0, S_last          : [B, H, d, d] fp32 or NULL; S[i][j] with i = value row, j = key column
 *   lower_bound         : in [0, 1]
 *   Supported d : multiples of 16 up to 128.
 * Errors: SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_DTYPE, SSD_ERR_ALIGN, SSD_ERR_VALUE
 * (lower_bound outside [0, 1]), SSD_ERR_ALIAS.
 * ------------------------------------------------------------------------------------------- */
int ssd_hgrn2_scan(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype,
                   const void* q, const void* k, const void* v, const void* g_logit,
                   float lower_bound, const float* S0, void* o, float* S_last, void* stream);

/* Gradients of ssd_hgrn2_scan for the loss  sum do * o + sum dS_last * S_last.  The page trains
 * through autograd and prints no backward pass; this is the gradient of the definition above.  With
 * R_t = dL/dS_t (R_t = do_t q_t^T + diag(g_{t+1}) R_{t+1}, R_{L-1} = do_{L-1} q_{L-1}^T + dS_last):
 *   dq_t = S_t^T do_t,   dk_t = R_t^T v_t,   dv_t = R_t k_t,   dS0 = diag(g_0) R_0,
 *   dg_logit_t = c_t (1 - lower_bound) sigmoid'(g_logit_t) / g_t  with
 *   c_t[i] = sum_{u >= t} (do_u[i] o_u[i] - v_u[i] dv_u[i]) + sum_j dS_last[i][j] S_last[i][j]
 *   (c_t is the derivative with respect to log g_t; 0 where sigmoid(g_logit) is 0).
 *   inputs            : as ssd_hgrn2_scan (S0 [B, H, d, d] fp32 or NULL), plus
 *   o                 : [B, L, H, d] fp32, the forward output for these inputs, or NULL (then it is
 *                       recomputed into the workspace: B * L * H * d fp32 more)
 *   dO                : [B, L, H, d] (in dtype);  dS_last : [B, H, d, d] fp32 or NULL (= 0)
 *   dq, dk, dv, dg_logit : [B, L, H, d] (out dtype);  dS0 : [B, H, d, d] fp32 or NULL
 *   workspace         : see "Workspaces"; size from ssd_hgrn2_scan_backward_workspace_bytes(B, L, H,
 *                       d, in_dtype, have_o) with have_o = (o != NULL)
 * Any lower_bound in [0, 1].  Every output is overwritten.  With bf16 inputs and d = 128 the adjoint
 * passes run in the chunked matrix form of ssd_hgrn2_scan (dq as the key-axis scan of (dO, v, k) from
 * S0^T; dv as the row-gated scan backward in time of (k, q, dO) with the next token's gate, from dS_last;
 * dk as the key-axis scan backward in time of (v, dO, q) from dS_last^T), and c_t is summed over
 * 64-token segments; the workspace then holds R_0, S0^T, dS_last^T and S_L^T (4 * B * H * d * d fp32),
 * the segment sums (B * H * ceil(L / 64) * d fp32) and dv in fp32 (B * L * H * d fp32, the sums' input
 * when the outputs are bf16).  Otherwise (fp32 inputs, other d) the gradients come from register sweeps
 * and the workspace holds S_last (B * H * d * d fp32) and, for fp32 inputs, the state after every 32nd
 * token (from which the running sum c_t is restarted exactly: B * H * floor((L - 1) / 32) * d * d fp32).
 * Errors as ssd_hgrn2_scan, plus SSD_ERR_NULL for missing dO, dq, dk, dv or dg_logit, and the
 * workspace errors. */
int ssd_hgrn2_scan_backward(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype,
                            const void* q, const void* k, const void* v, const void* g_logit,
                            float lower_bound, const float* S0, const float* o, const void* dO,
                            const float* dS_last, void* dq, void* dk, void* dv, void* dg_logit,
                            float* dS0, void* workspace, size_t workspace_bytes, void* stream);
int ssd_hgrn2_scan_backward_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int have_o,
                                            size_t* bytes);

/* One HGRN2 decode step.  q, k, v, g_logit, o : [B, H, d];  S : [B, H, d, d] fp32 in place.
 * Errors as ssd_hgrn2_scan. */
int ssd_hgrn2_update(int64_t B, int64_t H, int64_t d, int in_dtype, int out_dtype,
                     const void* q, const void* k, const void* v, const void* g_logit,
                     float lower_bound, float* S, void* o, void* stream);

/* ---------------------------------------------------------------------------------------------
 * HGRN2 with the gate on the key axis.  The page defines the state update with the gate scaling
 * the state "per channel" and cites the HGRN2 paper, whose convention (the gate on the key
 * dimension) it does not print; this is that reading:
 *     g_j = lower_bound + (1 - lower_bound) * sigmoid(g_logit_j),
 *     S[i][j] = g_j * S[i][j] + v_i * k_j,        o_i = sum_j S[i][j] * q_j,
 * i.e. S_t = S_{t-1} diag(g_t) + v_t k_t^T.  Arguments, layouts and errors as ssd_hgrn2_scan /
 * ssd_hgrn2_update.
 * ------------------------------------------------------------------------------------------- */
int ssd_hgrn2_key_scan(int64_t B, int64_t L, int64_t H, int64_t d, int in_dtype, int out_dtype,
                       const void* q, const void* k, const void* v, const void* g_logit,
                       float lower_bound, const float* S0, void* o, float* S_last, void* stream);
int ssd_hgrn2_key_update(int64_t B, int64_t H, int64_t d, int in_dtype, int out_dtype,
                         const void* q, const void* k, const void* v, const void* g_logit,
                         float lower_bound, float* S, void* o, void* stream);

/* The HGRN2 layer's readout normalisation and output gate (frankenstein-transformer documentation,
 * "HGRN2 Attention": a LayerNorm on the recurrent readout, before the silu-gated output).  Per row of
 * `width` contiguous features:
 *     y = ((o - mean) / sqrt(var + eps) * weight + bias) * silu(gate),
 * mean and biased variance over the row (torch.nn.LayerNorm).  For the layer's norm over its hidden
 * size, rows = B * L and width = H * d of the scan output [B, L, H, d]; width = d normalises each head.
 *   o      : [rows, width] fp32 (the scan output)
 *   gate   : [rows, width] (in dtype) or NULL (no gate)
 *   weight, bias : [width] fp32 or NULL (1 / 0)
 *   y      : [rows, width] (out dtype)
 *   eps    : finite, >= 0 (torch's default is 1e-5)
 * Errors: SSD_ERR_NULL, SSD_ERR_SHAPE (negative size, width > 8192), SSD_ERR_DTYPE, SSD_ERR_ALIGN,
 * SSD_ERR_VALUE (eps), SSD_ERR_ALIAS. */
int ssd_readout_norm(int64_t rows, int64_t width, int in_dtype, int out_dtype, const float* o,
                     const void* gate, const float* weight, const float* bias, float eps, void* y,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
