/*
 * ssd_oracle.c -- plain sequential fp64 CPU oracle.  TEST INFRASTRUCTURE ONLY:
 * loaded by the test suite, the smoke check and the benchmark's CPU-baseline
 * leg; never by the product path.  Shares no code with the HIP library.
 *
 * Sources followed (page title, then the part of it):
 *   [RGLRU]  lrnnx documentation, "lrnnx.models.ltv.rglru": RGLRU.step, the
 *            fallback branch (a_bar = a^(c*r), sqrt(1 - a_bar^2), state update,
 *            sum over the state dimension), with the gate computation of
 *            RGLRU.forward (sigmoid of the two gate projections, delta = c*r,
 *            u = i*x).  The base is read as a = exp(a_log) (see the readings
 *            list of the design notes), so a_bar = exp(c*r*a_log).
 *   [MSSM]   cortexnet 3.2.1 package diff, cortexnet/ssm.py, MultiScaleSSM:
 *            forward (softplus of dt, skip term D*x, silu(z) gate) and
 *            _selective_scan (A_bar = exp(clamp(dt*A, max=20)), B_bar = dt*B,
 *            h = A_bar*h + B_bar*x, y = sum_n h*C).
 *   [HGRN2]  frankenstein-transformer documentation, "HGRN2 Attention": the
 *            state update S_t = diag(g_t) S_{t-1} + v_t k_t^T, forget gate
 *            sigmoid-activated and lower-bounded in [lower_bound, 1], token-by-
 *            token processing; readout o_t = S_t q_t.
 *   [BLOCK]  lrnnx documentation, "lrnnx.models.ltv.rglru", the RG-LRU block
 *            around the recurrence: the causal depthwise nn.Conv1d (groups =
 *            channels, padding d_conv - 1, first L outputs kept) of forward(),
 *            the conv_state window of step() (shift left, newest input last,
 *            sum of window * weight plus bias), and the output multiply
 *            gelu(gate) * y (torch's exact gelu, x * Phi(x)).
 *   [MINMAX] minmaxrnc package diff, minmaxrnc/minmax_neuron.py and
 *            minmax_operator.py: the MinMax recurrence
 *            x_t = max(min(r_t, x_{t-1}), s_t) from the initial state, and the
 *            optional output gate x_t * g_t.
 */
#include "ssd_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* torch.nn.functional.softplus with its default threshold: identity above 20. */
static double softplus(double v) { return v > 20.0 ? v : log1p(exp(v)); }

int oracle_affine_scan(int64_t L, const double* a, const double* b, double h0, double* h) {
  if (L < 0) return 1;
  if (L > 0 && (!a || !b || !h)) return 1;
  double s = h0;
  for (int64_t t = 0; t < L; ++t) {
    s = a[t] * s + b[t];
    h[t] = s;
  }
  return 0;
}

/* [RGLRU] one step of the recurrence for a single channel; returns the new state. */
static double rglru_step(double h, double x, double r_logit, double i_logit, double a_log, double c) {
  double r = sigmoid(r_logit);
  double i = sigmoid(i_logit);
  double lambda = c * r * a_log;          /* log a_bar = c * r * log a */
  double a_bar = exp(lambda);
  double beta = sqrt(-expm1(2.0 * lambda)); /* sqrt(1 - a_bar^2) */
  return a_bar * h + beta * (i * x);
}

/* [BLOCK] torch's default gelu: v * Phi(v) = v/2 * (1 + erf(v / sqrt(2))). */
static double gelu(double v) { return 0.5 * v * (1.0 + erf(v * 0.70710678118654752440)); }

double oracle_gelu(double v) { return gelu(v); }

int oracle_rglru_scan(int64_t B, int64_t L, int64_t D,
                      const double* x, const double* r_logit, const double* i_logit,
                      const double* a_log, double c, const double* h0, const double* gate,
                      double* y, double* h_last) {
  if (B < 0 || L < 0 || D < 0) return 1;
  if (B * L * D > 0 && (!x || !r_logit || !i_logit || !y)) return 1;
  if (B * D > 0 && !a_log) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      double h = h0 ? h0[b * D + d] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t idx = (b * L + t) * D + d;
        h = rglru_step(h, x[idx], r_logit[idx], i_logit[idx], a_log[d], c);
        /* d_state = 1: the sum over the state dimension is h itself */
        y[idx] = gate ? gelu(gate[idx]) * h : h;
      }
      if (h_last) h_last[b * D + d] = h;
    }
  }
  return 0;
}

int oracle_rglru_update(int64_t B, int64_t D,
                        const double* x, const double* r_logit, const double* i_logit,
                        const double* a_log, double c, const double* gate, double* state, double* y) {
  if (B < 0 || D < 0) return 1;
  if (B * D > 0 && (!x || !r_logit || !i_logit || !a_log || !state || !y)) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      int64_t idx = b * D + d;
      double h = rglru_step(state[idx], x[idx], r_logit[idx], i_logit[idx], a_log[d], c);
      state[idx] = h;
      y[idx] = gate ? gelu(gate[idx]) * h : h;
    }
  }
  return 0;
}

/* [MSSM] one time step for channel d: updates h[0..N-1] in place, returns y. */
static double selective_step(double* h, int64_t N, double x, double dt_raw, const double* A_row,
                             const double* Brow, const double* Crow, const double* Dskip_d,
                             const double* z, double bias, int dt_softplus) {
  double delta = dt_raw + bias;
  if (dt_softplus) delta = softplus(delta);
  double acc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double dA = delta * A_row[n];
    if (dA > 20.0) dA = 20.0; /* clamp(max=20); NaN passes through */
    double a_bar = exp(dA);
    double b_bar = delta * Brow[n];
    h[n] = a_bar * h[n] + b_bar * x;
    acc += h[n] * Crow[n];
  }
  if (Dskip_d) acc += x * (*Dskip_d);
  if (z) acc *= (*z) * sigmoid(*z); /* silu(z) */
  return acc;
}

int oracle_selective_scan(int64_t B, int64_t L, int64_t D, int64_t N,
                          const double* x, const double* dt, const double* A,
                          const double* Bm, const double* Cm, const double* Dskip,
                          const double* z, const double* dt_bias, int dt_softplus,
                          const int32_t* cu_seqlens, int64_t nseq,
                          const double* h0, double* y, double* h_last) {
  if (B < 0 || L < 0 || D < 0 || N < 0) return 1;
  if (cu_seqlens) {
    if (B != 1 || nseq < 0) return 1;
    if (cu_seqlens[0] != 0 || cu_seqlens[nseq] != L) return 1;
    for (int64_t s = 0; s < nseq; ++s)
      if (cu_seqlens[s + 1] < cu_seqlens[s]) return 1;
  }
  if (B * L * D > 0 && (!x || !dt || !y)) return 1;
  if (B * L * N > 0 && (!Bm || !Cm)) return 1;
  if (D * N > 0 && !A) return 1;
  int64_t nunits = cu_seqlens ? nseq : B;
  double hbuf[256];
  if (N > 256) return 1;
  for (int64_t s = 0; s < nunits; ++s) {
    int64_t row0 = cu_seqlens ? cu_seqlens[s] : s * L;
    int64_t row1 = cu_seqlens ? cu_seqlens[s + 1] : (s + 1) * L;
    for (int64_t d = 0; d < D; ++d) {
      for (int64_t n = 0; n < N; ++n) hbuf[n] = h0 ? h0[(s * D + d) * N + n] : 0.0;
      for (int64_t row = row0; row < row1; ++row) {
        int64_t idx = row * D + d;
        y[idx] = selective_step(hbuf, N, x[idx], dt[idx], A + d * N, Bm + row * N, Cm + row * N,
                                Dskip ? Dskip + d : NULL, z ? z + idx : NULL,
                                dt_bias ? dt_bias[d] : 0.0, dt_softplus);
      }
      if (h_last)
        for (int64_t n = 0; n < N; ++n) h_last[(s * D + d) * N + n] = hbuf[n];
    }
  }
  return 0;
}

int oracle_selective_update(int64_t B, int64_t D, int64_t N,
                            const double* x, const double* dt, const double* A,
                            const double* Bm, const double* Cm, const double* Dskip,
                            const double* z, const double* dt_bias, int dt_softplus,
                            double* state, double* y) {
  if (B < 0 || D < 0 || N < 0) return 1;
  if (B * D > 0 && (!x || !dt || !state || !y)) return 1;
  if (B * N > 0 && (!Bm || !Cm)) return 1;
  if (D * N > 0 && !A) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      int64_t idx = b * D + d;
      y[idx] = selective_step(state + idx * N, N, x[idx], dt[idx], A + d * N, Bm + b * N, Cm + b * N,
                              Dskip ? Dskip + d : NULL, z ? z + idx : NULL,
                              dt_bias ? dt_bias[d] : 0.0, dt_softplus);
    }
  }
  return 0;
}

/* [HGRN2] one token for one head: S is d x d row-major (row = value index). */
static void hgrn2_step(double* S, int64_t d, const double* q, const double* k, const double* v,
                       const double* g_logit, double lb, double* o) {
  for (int64_t i = 0; i < d; ++i) {
    double g = lb + (1.0 - lb) * sigmoid(g_logit[i]);
    double* row = S + i * d;
    for (int64_t j = 0; j < d; ++j) row[j] = g * row[j] + v[i] * k[j];
  }
  for (int64_t i = 0; i < d; ++i) {
    const double* row = S + i * d;
    double acc = 0.0;
    for (int64_t j = 0; j < d; ++j) acc += row[j] * q[j];
    o[i] = acc;
  }
}

int oracle_hgrn2_scan(int64_t B, int64_t L, int64_t H, int64_t d,
                      const double* q, const double* k, const double* v,
                      const double* g_logit, double lower_bound, const double* S0,
                      double* o, double* S_last) {
  if (B < 0 || L < 0 || H < 0 || d < 0) return 1;
  if (B * L * H * d > 0 && (!q || !k || !v || !g_logit || !o)) return 1;
  double* S = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d * d : 1));
  if (!S) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t hh = 0; hh < H; ++hh) {
      const int64_t sbase = (b * H + hh) * d * d;
      for (int64_t e = 0; e < d * d; ++e) S[e] = S0 ? S0[sbase + e] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t base = ((b * L + t) * H + hh) * d;
        hgrn2_step(S, d, q + base, k + base, v + base, g_logit + base, lower_bound, o + base);
      }
      if (S_last)
        for (int64_t e = 0; e < d * d; ++e) S_last[sbase + e] = S[e];
    }
  }
  free(S);
  return 0;
}

int oracle_hgrn2_update(int64_t B, int64_t H, int64_t d,
                        const double* q, const double* k, const double* v,
                        const double* g_logit, double lower_bound, double* S, double* o) {
  if (B < 0 || H < 0 || d < 0) return 1;
  if (B * H * d > 0 && (!q || !k || !v || !g_logit || !S || !o)) return 1;
  for (int64_t bh = 0; bh < B * H; ++bh) {
    hgrn2_step(S + bh * d * d, d, q + bh * d, k + bh * d, v + bh * d, g_logit + bh * d,
               lower_bound, o + bh * d);
  }
  return 0;
}

/* [HGRN2-KEY] the key-axis reading of the gate (the convention of the HGRN2 paper the page cites,
 * not printed there): the gate scales column j, S[i][j] = g_j S[i][j] + v_i k_j, i.e.
 * S_t = S_{t-1} diag(g_t) + v_t k_t^T; the readout is the same o_i = sum_j S[i][j] q_j. */
static void hgrn2_key_step(double* S, int64_t d, const double* q, const double* k, const double* v,
                           const double* g_logit, double lb, double* o) {
  for (int64_t i = 0; i < d; ++i) {
    double* row = S + i * d;
    for (int64_t j = 0; j < d; ++j) {
      double g = lb + (1.0 - lb) * sigmoid(g_logit[j]);
      row[j] = g * row[j] + v[i] * k[j];
    }
  }
  for (int64_t i = 0; i < d; ++i) {
    const double* row = S + i * d;
    double acc = 0.0;
    for (int64_t j = 0; j < d; ++j) acc += row[j] * q[j];
    o[i] = acc;
  }
}

int oracle_hgrn2_key_scan(int64_t B, int64_t L, int64_t H, int64_t d,
                          const double* q, const double* k, const double* v,
                          const double* g_logit, double lower_bound, const double* S0,
                          double* o, double* S_last) {
  if (B < 0 || L < 0 || H < 0 || d < 0) return 1;
  if (B * L * H * d > 0 && (!q || !k || !v || !g_logit || !o)) return 1;
  double* S = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d * d : 1));
  if (!S) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t hh = 0; hh < H; ++hh) {
      const int64_t sbase = (b * H + hh) * d * d;
      for (int64_t e = 0; e < d * d; ++e) S[e] = S0 ? S0[sbase + e] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t base = ((b * L + t) * H + hh) * d;
        hgrn2_key_step(S, d, q + base, k + base, v + base, g_logit + base, lower_bound, o + base);
      }
      if (S_last)
        for (int64_t e = 0; e < d * d; ++e) S_last[sbase + e] = S[e];
    }
  }
  free(S);
  return 0;
}

int oracle_hgrn2_key_update(int64_t B, int64_t H, int64_t d,
                            const double* q, const double* k, const double* v,
                            const double* g_logit, double lower_bound, double* S, double* o) {
  if (B < 0 || H < 0 || d < 0) return 1;
  if (B * H * d > 0 && (!q || !k || !v || !g_logit || !S || !o)) return 1;
  for (int64_t bh = 0; bh < B * H; ++bh) {
    hgrn2_key_step(S + bh * d * d, d, q + bh * d, k + bh * d, v + bh * d, g_logit + bh * d,
                   lower_bound, o + bh * d);
  }
  return 0;
}

/* [NORM] the HGRN2 layer's readout normalisation and output gate (frankenstein-transformer
 * documentation, "HGRN2 Attention": a LayerNorm applied to the recurrent readout before the
 * silu-gated output): per row of `width` features,
 *   y = ((o - mean) / sqrt(var + eps) * weight + bias) * silu(gate),
 * mean and (biased) variance over the row, as torch.nn.LayerNorm computes them; weight / bias NULL
 * mean 1 / 0, gate NULL means no gate. */
int oracle_readout_norm(int64_t rows, int64_t width, const double* o, const double* gate,
                        const double* weight, const double* bias, double eps, double* y) {
  if (rows < 0 || width < 0) return 1;
  if (rows * width > 0 && (!o || !y)) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    const double* x = o + r * width;
    double mean = 0.0;
    for (int64_t c = 0; c < width; ++c) mean += x[c];
    mean /= (double)width;
    double var = 0.0;
    for (int64_t c = 0; c < width; ++c) var += (x[c] - mean) * (x[c] - mean);
    var /= (double)width;
    const double inv = 1.0 / sqrt(var + eps);
    for (int64_t c = 0; c < width; ++c) {
      double v = (x[c] - mean) * inv * (weight ? weight[c] : 1.0) + (bias ? bias[c] : 0.0);
      if (gate) v *= gate[r * width + c] * sigmoid(gate[r * width + c]);
      y[r * width + c] = v;
    }
  }
  return 0;
}

/* [MINMAX] min and max on the order of the real numbers with -0 placed below +0 (so that every
 * result is one definite input value); a NaN operand gives NaN. */
static double mm_min(double a, double b) {
  if (isnan(a) || isnan(b)) return NAN;
  if (a < b) return a;
  if (b < a) return b;
  return signbit(a) ? a : b;
}
static double mm_max(double a, double b) {
  if (isnan(a) || isnan(b)) return NAN;
  if (a > b) return a;
  if (b > a) return b;
  return signbit(a) ? b : a;
}

int oracle_minmax_scan(int64_t B, int64_t L, int64_t D, const double* r, const double* s,
                       const double* x0, const double* gate, double* y, double* x_last) {
  if (B < 0 || L < 0 || D < 0) return 1;
  if (B * L * D > 0 && (!r || !s || !y)) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      double xv = x0 ? x0[b * D + d] : 0.0; /* the neuron's initial state is zero by default */
      for (int64_t t = 0; t < L; ++t) {
        int64_t idx = (b * L + t) * D + d;
        xv = mm_max(mm_min(r[idx], xv), s[idx]);
        y[idx] = gate ? xv * gate[idx] : xv;
      }
      if (x_last) x_last[b * D + d] = xv;
    }
  }
  return 0;
}

int oracle_minmax_update(int64_t B, int64_t D, const double* r, const double* s, const double* gate,
                         double* state, double* y) {
  if (B < 0 || D < 0) return 1;
  if (B * D > 0 && (!r || !s || !state || !y)) return 1;
  for (int64_t idx = 0; idx < B * D; ++idx) {
    double xv = mm_max(mm_min(r[idx], state[idx]), s[idx]);
    state[idx] = xv;
    y[idx] = gate ? xv * gate[idx] : xv;
  }
  return 0;
}

/* [BLOCK] input at time tau of channel (b, d): x itself for 0 <= tau < L, else the carried window
 * (entry W + tau holds time tau, for -W <= tau < 0), else zero. */
static double conv_input(int64_t b, int64_t d, int64_t tau, int64_t L, int64_t D, int64_t W,
                         const double* x, const double* state_in) {
  if (tau >= 0 && tau < L) return x[(b * L + tau) * D + d];
  if (tau < 0 && tau >= -W && state_in) return state_in[(b * D + d) * W + (W + tau)];
  return 0.0;
}

int oracle_causal_conv1d(int64_t B, int64_t L, int64_t D, int64_t W, const double* x,
                         const double* weight, const double* bias, const double* state_in,
                         double* y, double* state_out) {
  if (B < 0 || L < 0 || D < 0 || W < 1) return 1;
  if (B * L * D > 0 && (!x || !y)) return 1;
  if (D > 0 && !weight) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      for (int64_t t = 0; t < L; ++t) {
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < W; ++k)
          acc += weight[d * W + k] * conv_input(b, d, t - (W - 1) + k, L, D, W, x, state_in);
        y[(b * L + t) * D + d] = acc;
      }
      if (state_out)
        for (int64_t k = 0; k < W; ++k)
          state_out[(b * D + d) * W + k] = conv_input(b, d, L - W + k, L, D, W, x, state_in);
    }
  }
  return 0;
}

int oracle_causal_conv1d_update(int64_t B, int64_t D, int64_t W, const double* x, const double* weight,
                                const double* bias, double* state, double* y) {
  if (B < 0 || D < 0 || W < 1) return 1;
  if (B * D > 0 && (!x || !weight || !state || !y)) return 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      double* win = state + (b * D + d) * W;
      for (int64_t k = 0; k + 1 < W; ++k) win[k] = win[k + 1];
      win[W - 1] = x[b * D + d];
      double acc = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < W; ++k) acc += weight[d * W + k] * win[k];
      y[b * D + d] = acc;
    }
  }
  return 0;
}
