/*
 * oracle.c -- fp64 CPU reference of the selective state-space scan and of
 * sliding-window attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library.
 *
 * What it computes (plain definition, no blocking, no reordering):
 *
 *   Page "SAMBA混合注意力状态空间模型" (metaphor-xennon.pages.dev), section
 *   数学框架 -> Mamba层: the state update h_t = Ā_t h_{t-1} + B̄_t x_t and the
 *   readout y_t = C_t h_t (the readout uses the state *after* the update of the
 *   same step), with B_t, C_t and Δ_t selected from the input (the selection
 *   equations below them).  The same page, section 实现细节 -> 模型配置, gives
 *   an SSM state size of 16; this file accepts any size >= 1.
 *
 *   The pages never define Ā_t, B̄_t or the map τ_Δ, nor a skip or gate; the
 *   paper's own Mamba subsection (hackernoon page, §2.1.1) has no body in the
 *   excerpt.  This library adopts the usual Mamba reading:
 *     Δ      = softplus(dt_raw + dt_bias)            (τ_Δ; dt_raw is given)
 *     Ā[n]   = exp(Δ * A[d][n])                      (zero-order hold, A diagonal, negative real)
 *     B̄x[n]  = Δ * B_t[n] * x_t                      (Euler step for the input)
 *     y_t    = (sum_n C_t[n] h_t[n] + Dskip[d] x_t) * silu(z_t)
 *   B_t and C_t are one vector per token shared by all channels.
 *
 *   Prefill over a packed stream of sequences: each sequence starts from its
 *   own h0 row (zeros when h0 is NULL) and never sees another sequence's
 *   state; its final state goes to its h_last row.  The decode step is the
 *   loop body for a single token, reading and writing the state in place
 *   (page 1, section 推理效率: prefill by forward(prompt), then one constant-
 *   time state update per generated token).
 *
 * The gradients of the prefill (oracle_scan_bwd) are the reverse-mode
 * derivative of exactly that loop; the formulas stand above the function.
 *
 * Gated linear attention (oracle_gla: a decay per key dimension and token) and
 * the Mamba-2 form the pages compare with (oracle_ssd: scalar decay per head,
 * a matrix state per head) are written out the same way, as their recurrences.
 *
 * The other layer of the hybrid, sliding-window attention (oracle_swa), is
 * the definition written out per query: rotate, score the visible keys,
 * softmax, weight the values (its reading stands above the function).
 *
 * Everything is double precision with libm exp / log1p; build without
 * fast-math.  OpenMP runs over independent (sequence, channel) recurrences;
 * time always runs sequentially inside one recurrence.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(v) = log(1 + e^v), evaluated without overflow for large v. */
static double softplus(double v) {
  if (v > 0.0) return v + log1p(exp(-v));
  return log1p(exp(v));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^{-z}). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One token of one channel: update h[0..N) in place and return y.
 *   xv, dtv, zv : this token's x, dt_raw, z at the channel
 *   Bt, Ct      : this token's B and C vectors (length N)
 *   Arow        : A[d][0..N)
 */
static double token_update(double* h, int64_t N, double xv, double dtv, double zv,
                           const double* Bt, const double* Ct, const double* Arow,
                           double dskip, double bias) {
  const double delta = softplus(dtv + bias);
  double acc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    const double abar = exp(delta * Arow[n]);
    const double bbar_x = delta * Bt[n] * xv;
    h[n] = abar * h[n] + bbar_x;
    acc += Ct[n] * h[n];
  }
  return (acc + dskip * xv) * silu(zv);
}

/*
 * Prefill over nseq sequences packed along the token axis, with ngroups groups of (B, C) vectors per token.
 *   seq_start [nseq+1] : token offsets, seq_start[0] = 0, ascending; seq s owns
 *                        tokens [seq_start[s], seq_start[s+1]).
 *   x, dt, z  [T][dim] , B, C [T][ngroups][dstate] , A [dim][dstate], Dskip, dt_bias [dim]
 *   channel d reads the (B, C) of group d / (dim / ngroups): contiguous blocks of channels share a group
 *   (ngroups = 1: one vector per token shared by all channels, the pages' selection)
 *   h0        [nseq][dim][dstate] or NULL (zeros)
 *   y         [T][dim] (written)
 *   h_last    [nseq][dim][dstate] or NULL (not written)
 * Returns 0, or -1 on invalid sizes / allocation failure.
 */
int oracle_scan_fwd_groups(int64_t nseq, const int64_t* seq_start, int64_t dim, int64_t dstate, int64_t ngroups,
                           const double* x, const double* dt, const double* z,
                           const double* B, const double* C,
                           const double* A, const double* Dskip, const double* dt_bias,
                           const double* h0, double* y, double* h_last, int nthreads) {
  if (nseq < 0 || dim < 0 || dstate < 1 || ngroups < 1 || dim % ngroups != 0 || !seq_start) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_start[s + 1] < seq_start[s]) return -1;
  const int64_t per_group = dim / ngroups;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
  for (int64_t s = 0; s < nseq; ++s) {
    for (int64_t d = 0; d < dim; ++d) {
      const int64_t g = d / per_group;
      double* h = (double*)malloc((size_t)dstate * sizeof(double));
      if (!h) { failed = 1; continue; }
      for (int64_t n = 0; n < dstate; ++n)
        h[n] = h0 ? h0[(s * dim + d) * dstate + n] : 0.0;
      for (int64_t t = seq_start[s]; t < seq_start[s + 1]; ++t) {
        y[t * dim + d] = token_update(h, dstate, x[t * dim + d], dt[t * dim + d], z[t * dim + d],
                                      B + (t * ngroups + g) * dstate, C + (t * ngroups + g) * dstate,
                                      A + d * dstate,
                                      Dskip[d], dt_bias[d]);
      }
      if (h_last)
        for (int64_t n = 0; n < dstate; ++n) h_last[(s * dim + d) * dstate + n] = h[n];
      free(h);
    }
  }
  (void)nthreads;
  return failed ? -1 : 0;
}

/* The pages' selection: one (B, C) pair per token shared by all channels. */
int oracle_scan_fwd(int64_t nseq, const int64_t* seq_start, int64_t dim, int64_t dstate,
                    const double* x, const double* dt, const double* z,
                    const double* B, const double* C,
                    const double* A, const double* Dskip, const double* dt_bias,
                    const double* h0, double* y, double* h_last, int nthreads) {
  return oracle_scan_fwd_groups(nseq, seq_start, dim, dstate, 1, x, dt, z, B, C, A, Dskip, dt_bias, h0, y,
                                h_last, nthreads);
}

/*
 * One decode step for `batch` independent sequences.
 *   state [batch][dim][dstate] : read and written in place
 *   x, dt, z [batch][dim], B, C [batch][dstate], A [dim][dstate], Dskip, dt_bias [dim]
 *   y [batch][dim] (written)
 */
int oracle_scan_step(int64_t batch, int64_t dim, int64_t dstate, double* state,
                     const double* x, const double* dt, const double* z,
                     const double* B, const double* C,
                     const double* A, const double* Dskip, const double* dt_bias,
                     double* y, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1) return -1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
#endif
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      y[b * dim + d] = token_update(state + (b * dim + d) * dstate, dstate, x[b * dim + d], dt[b * dim + d],
                                    z[b * dim + d], B + b * dstate, C + b * dstate, A + d * dstate,
                                    Dskip[d], dt_bias[d]);
    }
  }
  (void)nthreads;
  return 0;
}

/*
 * Gradients of the prefill: reverse-mode differentiation of exactly the loop
 * oracle_scan_fwd runs (the pages train Samba with this scan: page
 * "SAMBA混合注意力状态空间模型", 实现细节 -> 训练配置; the hackernoon page,
 * §2.1.2, names Mamba's selective scan as the training-time kernel).  For the
 * loss L = sum_t,d dy[t][d] y[t][d] + sum_s,d,n dh_last[s][d][n] h_last[s][d][n]:
 *
 *   per token t of sequence s, channel d (v = dt_raw + bias, Δ = softplus(v)):
 *     r_t      = sum_n C_t[n] h_t[n] + Dskip x_t          (pre-gate output)
 *     dr_t     = dy_t silu(z_t)
 *     dz_t     = dy_t r_t silu'(z_t),   silu'(z) = σ(z) (1 + z (1 - σ(z)))
 *     g_t[n]   = dr_t C_t[n] + Ā_{t+1}[n] g_{t+1}[n]       (adjoint of h_t; the
 *                term after the last token is dh_last)
 *     dx_t     = dr_t Dskip + Δ_t sum_n g_t[n] B_t[n]
 *     dΔ_t     = sum_n g_t[n] (A[n] Ā_t[n] h_{t-1}[n] + B_t[n] x_t)
 *     ddt_t    = dΔ_t σ(v)                                 (softplus' = σ)
 *     dB_t[n] += g_t[n] Δ_t x_t,   dC_t[n] += dr_t h_t[n]  (summed over d)
 *     dA[d][n]+= g_t[n] Δ_t Ā_t[n] h_{t-1}[n], dDskip[d] += dr_t x_t,
 *     ddt_bias[d] += ddt_t                                 (summed over t, s)
 *   dh0[s][d][n] = Ā_first[n] g_first[n]  (dh_last for an empty sequence).
 *
 *   dy [T][dim]; dh_last [nseq][dim][dstate] or NULL (zeros); h0 as in the
 *   forward.  Outputs: dx, ddt, dz [T][dim]; dB, dC [T][dstate]; dA
 *   [dim][dstate]; dDskip, ddt_bias [dim]; dh0 [nseq][dim][dstate] or NULL.
 * Each (sequence, channel) runs its forward loop (keeping every state) and
 * then the reverse loop.  OpenMP spreads channels; each thread sums its dB and
 * dC into a private buffer, added up in thread order at the end.
 */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_scan_bwd(int64_t nseq, const int64_t* seq_start, int64_t dim, int64_t dstate,
                    const double* x, const double* dt, const double* z,
                    const double* B, const double* C,
                    const double* A, const double* Dskip, const double* dt_bias,
                    const double* h0, const double* dy, const double* dh_last,
                    double* dx, double* ddt, double* dz, double* dB, double* dC,
                    double* dA, double* dDskip, double* ddt_bias, double* dh0, int nthreads) {
  if (nseq < 0 || dim < 0 || dstate < 1 || !seq_start) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_start[s + 1] < seq_start[s]) return -1;
  const int64_t T = seq_start[nseq];
  int64_t maxlen = 0;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_start[s + 1] - seq_start[s] > maxlen) maxlen = seq_start[s + 1] - seq_start[s];
  int nt = 1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  nt = nthreads;
#endif
  double** priv = (double**)calloc((size_t)nt, sizeof(double*));
  if (!priv) return -1;
  int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt) reduction(| : failed)
#endif
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* acc = (double*)calloc((size_t)(2 * T * dstate + 1), sizeof(double));  /* dB, then dC */
    double* hs = (double*)malloc((size_t)((maxlen + 1) * dstate) * sizeof(double));
    double* g = (double*)malloc((size_t)dstate * sizeof(double));
    priv[tid] = acc;
    if (!acc || !hs || !g) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
    for (int64_t d = 0; d < dim; ++d) {
      if (!acc || !hs || !g) continue;
      const double* Arow = A + d * dstate;
      for (int64_t n = 0; n < dstate; ++n) dA[d * dstate + n] = 0.0;
      dDskip[d] = 0.0;
      ddt_bias[d] = 0.0;
      for (int64_t s = 0; s < nseq; ++s) {
        const int64_t t0 = seq_start[s], len = seq_start[s + 1] - t0;
        /* forward: hs[i] = state before token i (hs[0] = h0), hs[i+1] = after it */
        for (int64_t n = 0; n < dstate; ++n) hs[n] = h0 ? h0[(s * dim + d) * dstate + n] : 0.0;
        for (int64_t i = 0; i < len; ++i) {
          const int64_t t = t0 + i;
          const double delta = softplus(dt[t * dim + d] + dt_bias[d]);
          for (int64_t n = 0; n < dstate; ++n)
            hs[(i + 1) * dstate + n] = exp(delta * Arow[n]) * hs[i * dstate + n] +
                                       delta * B[t * dstate + n] * x[t * dim + d];
        }
        /* reverse: g carries Ā_{t+1} g_{t+1} (dh_last after the last token) */
        for (int64_t n = 0; n < dstate; ++n) g[n] = dh_last ? dh_last[(s * dim + d) * dstate + n] : 0.0;
        for (int64_t i = len - 1; i >= 0; --i) {
          const int64_t t = t0 + i;
          const double xv = x[t * dim + d], zv = z[t * dim + d], v = dt[t * dim + d] + dt_bias[d];
          const double delta = softplus(v);
          const double sz = sigmoid(zv);
          const double* hcur = hs + (i + 1) * dstate;
          const double* hprev = hs + i * dstate;
          double r = Dskip[d] * xv;
          for (int64_t n = 0; n < dstate; ++n) r += C[t * dstate + n] * hcur[n];
          const double dyv = dy[t * dim + d];
          const double dr = dyv * zv * sz;
          dz[t * dim + d] = dyv * r * sz * (1.0 + zv * (1.0 - sz));
          double dxv = dr * Dskip[d], ddelta = 0.0;
          for (int64_t n = 0; n < dstate; ++n) {
            const double gt = g[n] + dr * C[t * dstate + n];
            const double abar = exp(delta * Arow[n]);
            acc[t * dstate + n] += gt * delta * xv;
            acc[T * dstate + t * dstate + n] += dr * hcur[n];
            dxv += gt * delta * B[t * dstate + n];
            ddelta += gt * (Arow[n] * abar * hprev[n] + B[t * dstate + n] * xv);
            dA[d * dstate + n] += gt * delta * abar * hprev[n];
            g[n] = abar * gt;
          }
          dx[t * dim + d] = dxv;
          ddt[t * dim + d] = ddelta * sigmoid(v);
          ddt_bias[d] += ddt[t * dim + d];
          dDskip[d] += dr * xv;
        }
        if (dh0)
          for (int64_t n = 0; n < dstate; ++n) dh0[(s * dim + d) * dstate + n] = g[n];
      }
    }
    free(hs);
    free(g);
  }
  if (!failed) {
    for (int64_t i = 0; i < T * dstate; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
    for (int k = 0; k < nt; ++k) {
      if (!priv[k]) continue;
      for (int64_t i = 0; i < T * dstate; ++i) {
        dB[i] += priv[k][i];
        dC[i] += priv[k][T * dstate + i];
      }
    }
  }
  for (int k = 0; k < nt; ++k) free(priv[k]);
  free(priv);
  return failed ? -1 : 0;
}

/*
 * Selection projections (page "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层:
 * B_t, C_t and the argument of τ_Δ are linear maps of x_t).  The three maps are
 * the rows of one matrix W [dim + 2*dstate][dim] (one output feature per row,
 * as a linear layer stores its weight): rows 0..dim-1 give dt_raw (Linear_Δ,
 * full rank), the next dstate rows B_t (Linear_B), the last dstate rows C_t
 * (Linear_C).  No bias: τ_Δ's bias is the scan's dt_bias.
 *   out[t][j] = sum_k x[t][k] * W[j][k];  dt = out[:, :dim], B = out[:, dim:dim+dstate],
 *   C = out[:, dim+dstate:]
 * x [T][dim]; dt [T][dim], B and C [T][dstate] (written).  OpenMP over tokens.
 */
int oracle_proj(int64_t T, int64_t dim, int64_t dstate, const double* x, const double* W,
                double* dt, double* B, double* C, int nthreads) {
  if (T < 0 || dim < 1 || dstate < 1) return -1;
  const int64_t nout = dim + 2 * dstate;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < nout; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < dim; ++k) acc += x[t * dim + k] * W[j * dim + k];
      if (j < dim) dt[t * dim + j] = acc;
      else if (j < dim + dstate) B[t * dstate + (j - dim)] = acc;
      else C[t * dstate + (j - dim - dstate)] = acc;
    }
  }
  (void)nthreads;
  return 0;
}

/*
 * Sliding-window attention (page "SAMBA混合注意力状态空间模型", 数学框架 -> 滑动窗口注意力:
 * softmax(Q K^T / sqrt(d_k) + M) V with the window mask M; the hackernoon page, §2.1.2: window w, RoPE
 * relative positions inside the window).  Reading: causal, query i sees keys j with i - window <= j <= i
 * of its own sequence; RoPE rotates the pairs (c, c + hd/2) of q and k by the token's position inside its
 * sequence with the given tables (cos, sin [positions][hd/2]); NULL tables: no rotation.
 *   q, k, v, o [T][H][hd]; sequences as in oracle_scan_fwd (seq_start [nseq+1]).
 * Each (sequence, head, query) is one plain loop: rotate, score every visible key, softmax (maximum
 * subtracted), weighted sum of v.  OpenMP spreads (head, query) pairs.
 */
static void rope_rotate(const double* x, double* out, int64_t hd, const double* cs, const double* sn) {
  const int64_t half = hd / 2;
  for (int64_t c = 0; c < half; ++c) {
    out[c] = x[c] * cs[c] - x[c + half] * sn[c];
    out[c + half] = x[c + half] * cs[c] + x[c] * sn[c];
  }
}

/* One (head, query) of oracle_swa: the query is row i of the packed stream, t0 its sequence's first row. */
static int swa_query(int64_t i, int64_t t0, int64_t h, int64_t H, int64_t hd, int64_t window, const double* q,
                     const double* k, const double* v, const double* rope_cos, const double* rope_sin, double* o) {
  const int64_t jlo = (i - window > t0) ? i - window : t0;
  const int64_t nkeys = i - jlo + 1;
  double* buf = (double*)malloc((size_t)(2 * hd + nkeys) * sizeof(double));
  if (!buf) return -1;
  double* qr = buf;
  double* kr = buf + hd;
  double* sc = buf + 2 * hd;
  const double* qi = q + (i * H + h) * hd;
  if (rope_cos) rope_rotate(qi, qr, hd, rope_cos + (i - t0) * (hd / 2), rope_sin + (i - t0) * (hd / 2));
  else for (int64_t c = 0; c < hd; ++c) qr[c] = qi[c];
  double mx = -INFINITY;
  for (int64_t j = jlo; j <= i; ++j) {
    const double* kj = k + (j * H + h) * hd;
    if (rope_cos) rope_rotate(kj, kr, hd, rope_cos + (j - t0) * (hd / 2), rope_sin + (j - t0) * (hd / 2));
    else for (int64_t c = 0; c < hd; ++c) kr[c] = kj[c];
    double dot = 0.0;
    for (int64_t c = 0; c < hd; ++c) dot += qr[c] * kr[c];
    sc[j - jlo] = dot / sqrt((double)hd);
    if (sc[j - jlo] > mx) mx = sc[j - jlo];
  }
  double den = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) { sc[j] = exp(sc[j] - mx); den += sc[j]; }
  double* oi = o + (i * H + h) * hd;
  for (int64_t c = 0; c < hd; ++c) oi[c] = 0.0;
  for (int64_t j = jlo; j <= i; ++j) {
    const double w = sc[j - jlo] / den;
    const double* vj = v + (j * H + h) * hd;
    for (int64_t c = 0; c < hd; ++c) oi[c] += w * vj[c];
  }
  free(buf);
  return 0;
}

static int swa_check(int64_t nseq, const int64_t* seq_start, int64_t H, int64_t hd, int64_t window,
                     const double* rope_cos, const double* rope_sin) {
  if (nseq < 0 || H < 1 || hd < 2 || (hd & 1) || window < 0 || !seq_start) return -1;
  if ((rope_cos == NULL) != (rope_sin == NULL)) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_start[s + 1] < seq_start[s]) return -1;
  return 0;
}

static int64_t seq_of_row(const int64_t* seq_start, int64_t i) {
  int64_t s = 0;
  while (seq_start[s + 1] <= i) ++s;
  return s;
}

int oracle_swa(int64_t nseq, const int64_t* seq_start, int64_t H, int64_t hd, int64_t window,
               const double* q, const double* k, const double* v, const double* rope_cos, const double* rope_sin,
               double* o, int nthreads) {
  if (swa_check(nseq, seq_start, H, hd, window, rope_cos, rope_sin) != 0) return -1;
  const int64_t T = seq_start[nseq];
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 16) num_threads(nthreads) reduction(| : failed)
#endif
  for (int64_t h = 0; h < H; ++h) {
    for (int64_t i = 0; i < T; ++i) {
      const int64_t t0 = seq_start[seq_of_row(seq_start, i)];
      if (swa_query(i, t0, h, H, hd, window, q, k, v, rope_cos, rope_sin, o) != 0) failed = 1;
    }
  }
  (void)nthreads;
  return failed ? -1 : 0;
}

/* oracle_swa for the listed query rows only (all heads); other rows of o are left as they are. */
int oracle_swa_rows(int64_t nseq, const int64_t* seq_start, int64_t H, int64_t hd, int64_t window,
                    const double* q, const double* k, const double* v, const double* rope_cos,
                    const double* rope_sin, const int64_t* rows, int64_t nrows, double* o, int nthreads) {
  if (swa_check(nseq, seq_start, H, hd, window, rope_cos, rope_sin) != 0 || nrows < 0 || (nrows && !rows)) return -1;
  const int64_t T = seq_start[nseq];
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= T) return -1;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
  for (int64_t r = 0; r < nrows; ++r) {
    for (int64_t h = 0; h < H; ++h) {
      const int64_t i = rows[r];
      const int64_t t0 = seq_start[seq_of_row(seq_start, i)];
      if (swa_query(i, t0, h, H, hd, window, q, k, v, rope_cos, rope_sin, o) != 0) failed = 1;
    }
  }
  (void)nthreads;
  return failed ? -1 : 0;
}

/* RoPE alone: rotate x [T][H][hd] row t by position pos[t] of the tables (as inside oracle_swa). */
int oracle_rope(int64_t T, int64_t H, int64_t hd, const double* x, const int64_t* pos, const double* rope_cos,
                const double* rope_sin, double* out) {
  if (T < 0 || H < 1 || hd < 2 || (hd & 1) || !pos || !rope_cos || !rope_sin) return -1;
  for (int64_t t = 0; t < T; ++t) {
    if (pos[t] < 0) return -1;
    for (int64_t h = 0; h < H; ++h)
      rope_rotate(x + (t * H + h) * hd, out + (t * H + h) * hd, hd, rope_cos + pos[t] * (hd / 2),
                  rope_sin + pos[t] * (hd / 2));
  }
  return 0;
}

/*
 * State-space duality layer (the Mamba-2 form the pages name for comparison: page 1, 与其他混合架构对比 and
 * 设计哲学对比, SSD / 数学对偶性).  The pages give no formula; this is the usual definition: per head h a
 * scalar decay instead of a diagonal one, a state of P x N per head, (B, C) shared by the heads of a group.
 *   Δ_t = softplus(dt[t][h] + dt_bias[h]),  a_t = exp(Δ_t A[h])                      (A[h] < 0)
 *   H_t[p][n] = a_t H_{t-1}[p][n] + Δ_t x_t[p] B_t[n]                               (outer product)
 *   y_t[p] = (sum_n H_t[p][n] C_t[n] + D[h] x_t[p]) * silu(z_t[p])    (no gate when z is NULL)
 * x, z, y [T][H][P]; dt [T][H]; B, C [T][G][N] with head h reading group h / (H / G); A, D, dt_bias [H];
 * h0, h_last [nseq][H][P][N].  Each (sequence, head) is one sequential loop over its tokens.
 */
int oracle_ssd(int64_t nseq, const int64_t* seq_start, int64_t H, int64_t P, int64_t N, int64_t G,
               const double* x, const double* dt, const double* z, const double* B, const double* C,
               const double* A, const double* D, const double* dt_bias, const double* h0, double* y,
               double* h_last, int nthreads) {
  if (nseq < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0 || !seq_start) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_start[s + 1] < seq_start[s]) return -1;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
  for (int64_t s = 0; s < nseq; ++s) {
    for (int64_t h = 0; h < H; ++h) {
      const int64_t g = h / (H / G);
      double* st = (double*)malloc((size_t)(P * N) * sizeof(double));
      if (!st) { failed = 1; continue; }
      for (int64_t k = 0; k < P * N; ++k) st[k] = h0 ? h0[(s * H + h) * P * N + k] : 0.0;
      for (int64_t t = seq_start[s]; t < seq_start[s + 1]; ++t) {
        const double delta = softplus(dt[t * H + h] + dt_bias[h]);
        const double a = exp(delta * A[h]);
        const double* xt = x + (t * H + h) * P;
        const double* Bt = B + (t * G + g) * N;
        const double* Ct = C + (t * G + g) * N;
        for (int64_t p = 0; p < P; ++p) {
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            st[p * N + n] = a * st[p * N + n] + delta * xt[p] * Bt[n];
            acc += st[p * N + n] * Ct[n];
          }
          const double out = acc + D[h] * xt[p];
          y[(t * H + h) * P + p] = z ? out * silu(z[(t * H + h) * P + p]) : out;
        }
      }
      if (h_last)
        for (int64_t k = 0; k < P * N; ++k) h_last[(s * H + h) * P * N + k] = st[k];
      free(st);
    }
  }
  (void)nthreads;
  return failed ? -1 : 0;
}

/*
 * Gated linear attention (the hackernoon page, §2, names GLA with Multi-Scale Retention as substitutes for
 * the Mamba layer; the recurrence is the GLA paper's): per head h a key-by-value state S with a decay per key
 * dimension that depends on the token,
 *   S_t[n][p] = exp(gk[t][h][n]) S_{t-1}[n][p] + k[t][h][n] v[t][h][p],   o[t][h][p] = sum_n q[t][h][n] S_t[n][p]
 * q, k, gk [T][H][N] (gk = log of the decay, <= 0), v, o [T][H][P], h0, h_last [nseq][H][P][N] (the state
 * stored value-major, S^T).  Each (sequence, head, value column p) is one sequential loop over its tokens.
 */
int oracle_gla(int64_t nseq, const int64_t* seq_start, int64_t H, int64_t P, int64_t N, const double* q,
               const double* k, const double* v, const double* gk, const double* h0, double* o,
               double* h_last, int nthreads) {
  if (nseq < 0 || H < 1 || P < 1 || N < 1 || !seq_start) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_start[s + 1] < seq_start[s]) return -1;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
  for (int64_t s = 0; s < nseq; ++s) {
    for (int64_t h = 0; h < H; ++h) {
      double* st = (double*)malloc((size_t)(P * N) * sizeof(double));
      if (!st) { failed = 1; continue; }
      for (int64_t i = 0; i < P * N; ++i) st[i] = h0 ? h0[(s * H + h) * P * N + i] : 0.0;
      for (int64_t t = seq_start[s]; t < seq_start[s + 1]; ++t) {
        const double* qt = q + (t * H + h) * N;
        const double* kt = k + (t * H + h) * N;
        const double* gt = gk + (t * H + h) * N;
        for (int64_t p = 0; p < P; ++p) {
          const double vp = v[(t * H + h) * P + p];
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            st[p * N + n] = exp(gt[n]) * st[p * N + n] + kt[n] * vp;
            acc += qt[n] * st[p * N + n];
          }
          o[(t * H + h) * P + p] = acc;
        }
      }
      if (h_last)
        for (int64_t i = 0; i < P * N; ++i) h_last[(s * H + h) * P * N + i] = st[i];
      free(st);
    }
  }
  (void)nthreads;
  return failed ? -1 : 0;
}

/* Number of OpenMP threads a call with nthreads <= 0 would use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
