/*
 * ssd_oracle.h -- plain sequential fp64 CPU oracle for the gated diagonal
 * linear-recurrence scans (RG-LRU, multi-scale selective scan, HGRN2).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the correctness reference the
 * GPU kernels are checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load or call it; the product path
 * never does.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Every function is a direct, slow transcription of the recurrence as the
 * source pages define it: one loop over time per independent unit, no
 * blocking, no reordering, no fusion.  All arithmetic is IEEE double.
 *
 * Conventions shared by all functions:
 *   - arrays are dense, row-major, host memory, owned by the caller;
 *   - optional inputs are NULL when absent (documented per function);
 *   - return 0 on success, non-zero (and no output written) on an invalid
 *     argument: a negative size, or a NULL pointer that is required.
 *   - NaN/Inf inputs propagate by IEEE rules; nothing is trapped.
 */
#ifndef SSD_ORACLE_H
#define SSD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Plain first-order affine recurrence h_t = a_t * h_{t-1} + b_t over t = 0..L-1,
 * starting from h_{-1} = h0; writes h[t].  The common core of all three forms. */
int oracle_affine_scan(int64_t L, const double* a, const double* b, double h0, double* h);

/* gelu(v) = v * Phi(v) = v/2 * (1 + erf(v / sqrt(2))) (torch's default, exact form). */
double oracle_gelu(double v);

/* RG-LRU scan (lrnnx RGLRU block; recurrence of its step() fallback branch).
 * x, r_logit, i_logit, y: [B,L,D]; a_log: [D]; h0, h_last: [B,D] or NULL;
 * gate: [B,L,D] or NULL (the block's output multiply).
 *   r = sigmoid(r_logit), i = sigmoid(i_logit), lambda = c * r * a_log[d],
 *   a = exp(lambda), beta = sqrt(1 - a^2) (as sqrt(-expm1(2 lambda))),
 *   h = a*h + beta*(i*x), y = h (sum over the single state), times gelu(gate)
 *   when gate is given; h_last is the ungated state. */
int oracle_rglru_scan(int64_t B, int64_t L, int64_t D,
                      const double* x, const double* r_logit, const double* i_logit,
                      const double* a_log, double c, const double* h0, const double* gate,
                      double* y, double* h_last);

/* One RG-LRU decode step.  x, r_logit, i_logit, gate, y: [B,D] (gate may be
 * NULL); state: [B,D] in/out. */
int oracle_rglru_update(int64_t B, int64_t D,
                        const double* x, const double* r_logit, const double* i_logit,
                        const double* a_log, double c, const double* gate, double* state, double* y);

/* Multi-scale selective scan (cortexnet MultiScaleSSM: forward and
 * _selective_scan).
 *   x, dt, y, z: [B,L,D] (z NULL = no silu gate); A: [D,N]; Bm, Cm: [B,L,N];
 *   Dskip, dt_bias: [D] or NULL; dt_softplus: 0/1.
 *   cu_seqlens: host int32[nseq+1] or NULL.  With cu_seqlens, B must be 1 and
 *   sequence s covers rows [cu_seqlens[s], cu_seqlens[s+1]) of the packed L
 *   axis, with the state reset to its own h0 (or zero) at the start; without
 *   it, nseq is ignored and each of the B rows is one sequence.
 *   h0, h_last: [nseq or B, D, N] or NULL.
 * Per step: delta = dt + dt_bias, softplus'd (linear above 20) if dt_softplus;
 *   abar_n = exp(min(delta*A[d][n], 20)); h_n = abar_n*h_n + (delta*B_n)*x;
 *   y = sum_n C_n*h_n + Dskip[d]*x, times z*sigmoid(z) if z is given. */
int oracle_selective_scan(int64_t B, int64_t L, int64_t D, int64_t N,
                          const double* x, const double* dt, const double* A,
                          const double* Bm, const double* Cm, const double* Dskip,
                          const double* z, const double* dt_bias, int dt_softplus,
                          const int32_t* cu_seqlens, int64_t nseq,
                          const double* h0, double* y, double* h_last);

/* One selective-scan decode step.  x, dt, z, y: [B,D]; Bm, Cm: [B,N];
 * state: [B,D,N] in/out.  Other arguments as oracle_selective_scan. */
int oracle_selective_update(int64_t B, int64_t D, int64_t N,
                            const double* x, const double* dt, const double* A,
                            const double* Bm, const double* Cm, const double* Dskip,
                            const double* z, const double* dt_bias, int dt_softplus,
                            double* state, double* y);

/* HGRN2 matrix-state scan (HGRN2 Attention API page, state-update equation),
 * gate on the value (row) index of S.
 *   q, k, v, g_logit, o: [B,L,H,d]; S0, S_last: [B,H,d,d] (S[i][j], i = value
 *   row, j = key column) or NULL.
 * Per step: g_i = lb + (1-lb)*sigmoid(g_logit_i);
 *   S[i][j] = g_i*S[i][j] + v_i*k_j;  o_i = sum_j S[i][j]*q_j. */
int oracle_hgrn2_scan(int64_t B, int64_t L, int64_t H, int64_t d,
                      const double* q, const double* k, const double* v,
                      const double* g_logit, double lower_bound, const double* S0,
                      double* o, double* S_last);

/* One HGRN2 decode step.  q, k, v, g_logit, o: [B,H,d]; S: [B,H,d,d] in/out. */
int oracle_hgrn2_update(int64_t B, int64_t H, int64_t d,
                        const double* q, const double* k, const double* v,
                        const double* g_logit, double lower_bound, double* S, double* o);
int oracle_hgrn2_key_scan(int64_t B, int64_t L, int64_t H, int64_t d,
                          const double* q, const double* k, const double* v,
                          const double* g_logit, double lower_bound, const double* S0,
                          double* o, double* S_last);
int oracle_hgrn2_key_update(int64_t B, int64_t H, int64_t d,
                            const double* q, const double* k, const double* v,
                            const double* g_logit, double lower_bound, double* S, double* o);
int oracle_readout_norm(int64_t rows, int64_t width, const double* o, const double* gate,
                        const double* weight, const double* bias, double eps, double* y);

/* MinMax recurrence (minmaxrnc MinMaxNeuron): x_t = max(min(r_t, x_{t-1}), s_t)
 * from x0 (NULL = zero).  min / max order -0 below +0 and return NaN when an
 * operand is NaN, so every state is one definite input value.
 *   r, s, gate, y: [B,L,D] (gate NULL = none; else y = x * gate, else y = x);
 *   x0, x_last: [B,D] or NULL. */
int oracle_minmax_scan(int64_t B, int64_t L, int64_t D, const double* r, const double* s,
                       const double* x0, const double* gate, double* y, double* x_last);

/* One MinMax step.  r, s, gate, y: [B,D] (gate may be NULL); state: [B,D] in/out. */
int oracle_minmax_update(int64_t B, int64_t D, const double* r, const double* s, const double* gate,
                         double* state, double* y);

/* Causal depthwise convolution of the RG-LRU block (nn.Conv1d, groups = D,
 * kernel W, padding W-1, first L outputs):
 *   y[b,t,d] = bias[d] + sum_{k<W} weight[d][k] * x[b, t-(W-1)+k, d].
 * Inputs before the sequence come from state_in [B,D,W] (entry W+tau holds
 * time tau < 0) or are zero when it is NULL.  state_out [B,D,W] (or NULL)
 * receives the last W inputs (times L-W .. L-1, from state_in or zero where
 * negative).  x, y: [B,L,D]; weight: [D,W]; bias: [D] or NULL. */
int oracle_causal_conv1d(int64_t B, int64_t L, int64_t D, int64_t W, const double* x,
                         const double* weight, const double* bias, const double* state_in,
                         double* y, double* state_out);

/* One decode step of the convolution (the block's step()): the window
 * state [B,D,W] shifts left by one, x [B,D] enters last, and
 * y = bias + sum_k weight[d][k] * window[k]. */
int oracle_causal_conv1d_update(int64_t B, int64_t D, int64_t W, const double* x, const double* weight,
                                const double* bias, double* state, double* y);

#ifdef __cplusplus
}
#endif
#endif
