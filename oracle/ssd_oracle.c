/*
 * ssd_oracle.c -- plain, slow, fp64 CPU oracle for the Mamba-2 selective
 * state-space layer (depthwise causal conv + SiLU, selective scan, D skip,
 * SiLU(z) gate) and for its one-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libssd.so and its Python binding) never calls it, links it or includes
 * it, and it shares no code with the GPU kernels.
 *
 * Everything here is the plain definition, evaluated token by token in
 * double precision.  There is no chunking, blocking or reordering: the
 * chunked "state space duality" form that the GPU path uses is an exact
 * re-association of this recurrence, so the recurrence is the oracle.
 *
 * Sources (page title, then section):
 *  - Recurrence h_t = Abar h_{t-1} + Bbar x_t and read-out y_t = C h_t + D x_t,
 *    with input-dependent parameters: "Hybrid Architectures for Language
 *    Models: Systematic Analysis and Design Insights" (Korean summary),
 *    section 2 Background.
 *  - Layer shapes (head_dim 64, d_state 128, conv kernel 4, expand 2,
 *    n_groups 8, SiLU activation, chunk 128): "Nemotron-H style Hybrid
 *    Mamba-Transformer 3B feasibility study", tables 1.4 (Mamba-2 config)
 *    and 1.5 (Nemotron-H 8B).
 *  - The conv runs over the x|B|C channels (its cache holds
 *    N_conv*(2*d_state + d_ssm) values per layer): "Hybrid Architectures ..."
 *    summary, Appendix C (computational and memory costs).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - discretisation: Abar_t = exp(delta_t * A_h) (a scalar per token and
 *    head), Bbar_t = delta_t * B_t; delta_t = softplus(dt_t + dt_bias_h)
 *    when dt_softplus is set, else dt_t (+ dt_bias_h if given);
 *  - the read-out uses h_t after x_t has been added;
 *  - conv: cross-correlation, w[c][K-1] multiplies the current token,
 *    history before the first token comes from conv_state_in (oldest row
 *    first) or is zero;
 *  - head h reads group g = floor(h*G/H);
 *  - gate: out = y * z * sigmoid(z); no gate when z is NULL.
 *
 * Inputs are double.  The Python wrapper rounds the layer's inputs to fp32
 * first (the precision they arrive in); the block composition passes its
 * in_proj output on unrounded.
 *
 * Layouts (all row-major, innermost index contiguous):
 *   xbc  [B][L][Cdim] with a token stride (in elements), Cdim = H*P + 2*G*N,
 *        channel order x (H*P) | B (G*N) | C (G*N)
 *   dt   [B][L][H]        z, y [B][L][H][P]
 *   h0, h_final [B][H][P][N]   conv_state [B][K-1][Cdim] (oldest row first)
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(v) = log(1 + e^v), in the form that neither overflows nor
 * cancels: max(v,0) + log1p(e^{-|v|}). */
static double softplus(double v) {
  return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

/* SiLU(u) = u * sigmoid(u). */
static double silu(double u) { return u / (1.0 + exp(-u)); }

/* The raw conv input of channel c at position tau of sequence b.  tau < 0
 * reads the history: row (K-1)+tau of conv_state_in, or zero. */
static double conv_input(const double* xbc, int64_t tok_stride,
                         const double* hist, int seqlen, int cdim, int width,
                         int b, int tau, int c) {
  if (tau >= 0)
    return (double)xbc[((int64_t)b * seqlen + tau) * tok_stride + c];
  if (hist == NULL) return 0.0;
  return (double)hist[((int64_t)b * (width - 1) + (width - 1) + tau) * cdim + c];
}

/* Depthwise causal conv of channel c at token t, before the activation:
 * u = bias[c] + sum_k w[c][k] * xin[t - (K-1) + k]. */
static double conv_pre(const double* xbc, int64_t tok_stride, const double* hist,
                       const double* w, const double* bias, int seqlen, int cdim,
                       int width, int b, int t, int c) {
  double u = bias ? (double)bias[c] : 0.0;
  for (int k = 0; k < width; ++k)
    u += (double)w[(int64_t)c * width + k] *
         conv_input(xbc, tok_stride, hist, seqlen, cdim, width, b, t - (width - 1) + k, c);
  return u;
}

/* The last K-1 raw inputs of each channel after the sequence, oldest first
 * (taken from the old history when the sequence is shorter than K-1). */
static void conv_history_out(const double* xbc, int64_t tok_stride, const double* hist,
                             double* hist_out, int batch, int seqlen, int cdim,
                             int width) {
  for (int b = 0; b < batch; ++b)
    for (int j = 0; j < width - 1; ++j)
      for (int c = 0; c < cdim; ++c)
        hist_out[((int64_t)b * (width - 1) + j) * cdim + c] =
            conv_input(xbc, tok_stride, hist, seqlen, cdim, width, b,
                       seqlen - (width - 1) + j, c);
}

/*
 * Depthwise causal conv1d over every channel, optionally followed by SiLU.
 *   out [B][L][Cdim] (double, dense), hist_out [B][K-1][Cdim] or NULL.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_causal_conv1d(const double* xbc, int64_t tok_stride, const double* w,
                         const double* bias, const double* conv_state_in,
                         int apply_silu, double* out, double* conv_state_out,
                         int batch, int seqlen, int cdim, int width) {
  if (!xbc || !w || !out || batch < 0 || seqlen < 0 || cdim <= 0 || width < 1 ||
      tok_stride < cdim)
    return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < batch; ++b)
    for (int c = 0; c < cdim; ++c)
      for (int t = 0; t < seqlen; ++t) {
        double u = conv_pre(xbc, tok_stride, conv_state_in, w, bias, seqlen, cdim,
                            width, b, t, c);
        out[((int64_t)b * seqlen + t) * cdim + c] = apply_silu ? silu(u) : u;
      }
  if (conv_state_out)
    conv_history_out(xbc, tok_stride, conv_state_in, conv_state_out, batch, seqlen,
                     cdim, width);
  return 0;
}

/*
 * The whole layer, token by token.
 *
 * When conv_w is non-NULL, xbc holds the raw x|B|C inputs and each value the
 * scan needs is conv'd and SiLU'd on the fly; when it is NULL, xbc already
 * holds the post-conv x|B|C values and is read as is.
 *
 * For each (b, h), with g = floor(h*G/H) and S = h0[b][h] (or 0):
 *   delta = softplus(dt + dt_bias) | dt (+ dt_bias)
 *   a     = exp(delta * A[h])
 *   S[p][n] <- a * S[p][n] + delta * x[t][h][p] * B[t][g][n]
 *   yv[p]   = sum_n S[p][n] * C[t][g][n] + D[h] * x[t][h][p]
 *   y[t][h][p] = z ? yv[p] * silu(z[t][h][p]) : yv[p]
 * and finally h_final[b][h] = S.
 *
 * Any of conv_b, conv_state_in, D, dt_bias, z, h0, h_final, conv_state_out
 * may be NULL.  Returns 0, or -1 on a bad argument.
 */
int oracle_mamba2_fwd(const double* xbc, int64_t xbc_tok_stride, const double* conv_w,
                      const double* conv_b, int width, const double* conv_state_in,
                      const double* dt, const double* A, const double* D,
                      const double* dt_bias, int dt_softplus, const double* z,
                      const double* h0, double* y, double* h_final,
                      double* conv_state_out, int batch, int seqlen, int nheads,
                      int headdim, int ngroups, int dstate) {
  const int H = nheads, P = headdim, G = ngroups, N = dstate;
  if (!xbc || !dt || !A || !y || batch < 0 || seqlen < 0 || H <= 0 || P <= 0 ||
      G <= 0 || N <= 0 || H % G != 0 || (conv_w && width < 1))
    return -1;
  const int HP = H * P, GN = G * N, cdim = HP + 2 * GN;
  if (xbc_tok_stride < cdim) return -1;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < H; ++h) {
      const int g = (int)(((int64_t)h * G) / H);
      double* S = (double*)malloc(sizeof(double) * (size_t)P * N);
      double* xv = (double*)malloc(sizeof(double) * (size_t)(P + 2 * N));
      double* Bv = xv + P;
      double* Cv = Bv + N;
      const double* S0 = h0 ? h0 + ((int64_t)b * H + h) * P * N : NULL;
      for (int64_t i = 0; i < (int64_t)P * N; ++i) S[i] = S0 ? S0[i] : 0.0;

      for (int t = 0; t < seqlen; ++t) {
        /* the post-conv x of this head and B, C of its group at token t */
        for (int j = 0; j < P + 2 * N; ++j) {
          int c = j < P ? h * P + j
                        : (j < P + N ? HP + g * N + (j - P) : HP + GN + g * N + (j - P - N));
          if (conv_w)
            xv[j] = silu(conv_pre(xbc, xbc_tok_stride, conv_state_in, conv_w, conv_b,
                                  seqlen, cdim, width, b, t, c));
          else
            xv[j] = (double)xbc[((int64_t)b * seqlen + t) * xbc_tok_stride + c];
        }
        double v = (double)dt[((int64_t)b * seqlen + t) * H + h];
        if (dt_bias) v += (double)dt_bias[h];
        const double delta = dt_softplus ? softplus(v) : v;
        const double a = exp(delta * (double)A[h]);
        const double Dh = D ? (double)D[h] : 0.0;

        for (int p = 0; p < P; ++p) {
          double acc = 0.0;
          for (int n = 0; n < N; ++n) {
            double* s = &S[(int64_t)p * N + n];
            *s = a * *s + delta * xv[p] * Bv[n];
            acc += *s * Cv[n];
          }
          double yv = acc + Dh * xv[p];
          const int64_t o = (((int64_t)b * seqlen + t) * H + h) * P + p;
          if (z) yv *= silu((double)z[o]);
          y[o] = yv;
        }
      }
      if (h_final)
        memcpy(h_final + ((int64_t)b * H + h) * P * N, S, sizeof(double) * (size_t)P * N);
      free(xv);
      free(S);
    }

  if (conv_w && conv_state_out)
    conv_history_out(xbc, xbc_tok_stride, conv_state_in, conv_state_out, batch, seqlen,
                     cdim, width);
  return 0;
}

/*
 * One decode step for every sequence of the batch: one new token per
 * sequence, the conv ring of the last K-1 raw inputs, and the fp64 state.
 *
 *   state [B][H][P][N] (double, updated in place)
 *   xbc   [B][Cdim]    the new token's raw x|B|C (post-conv if conv_w is NULL)
 *   ring  [B][K-1][Cdim] (double, oldest row first; updated in place; unused
 *                        when conv_w is NULL)
 *   dt [B][H], z [B][H*P] or NULL, y [B][H*P] (double)
 *
 * Conv of channel c: u = bias[c] + sum_{k<K-1} w[c][k] * ring[k][c]
 *                        + w[c][K-1] * xbc[c]; value = silu(u); then the
 * ring drops its oldest row and appends xbc.  The SSM step is the same
 * recurrence as oracle_mamba2_fwd for one token.
 */
int oracle_mamba2_decode_step(double* state, const double* xbc, double* ring,
                              const double* conv_w, const double* conv_b, int width,
                              const double* dt, const double* A, const double* D,
                              const double* dt_bias, int dt_softplus, const double* z,
                              double* y, int batch, int nheads, int headdim,
                              int ngroups, int dstate) {
  const int H = nheads, P = headdim, G = ngroups, N = dstate;
  if (!state || !xbc || !dt || !A || !y || batch < 0 || H <= 0 || P <= 0 || G <= 0 ||
      N <= 0 || H % G != 0 || (conv_w && (!ring || width < 1)))
    return -1;
  const int HP = H * P, GN = G * N, cdim = HP + 2 * GN;
  double* xc = (double*)malloc(sizeof(double) * (size_t)batch * cdim);

  for (int b = 0; b < batch; ++b)
    for (int c = 0; c < cdim; ++c) {
      const double xin = (double)xbc[(int64_t)b * cdim + c];
      if (!conv_w) {
        xc[(int64_t)b * cdim + c] = xin;
        continue;
      }
      double* r = ring + (int64_t)b * (width - 1) * cdim + c; /* r[k*cdim] = row k */
      double u = conv_b ? (double)conv_b[c] : 0.0;
      for (int k = 0; k < width - 1; ++k) u += (double)conv_w[(int64_t)c * width + k] * r[(int64_t)k * cdim];
      u += (double)conv_w[(int64_t)c * width + width - 1] * xin;
      xc[(int64_t)b * cdim + c] = silu(u);
      for (int k = 0; k + 1 < width - 1; ++k) r[(int64_t)k * cdim] = r[(int64_t)(k + 1) * cdim];
      if (width > 1) r[(int64_t)(width - 2) * cdim] = xin;
    }

#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < H; ++h) {
      const int g = (int)(((int64_t)h * G) / H);
      const double* xv = xc + (int64_t)b * cdim + h * P;
      const double* Bv = xc + (int64_t)b * cdim + HP + g * N;
      const double* Cv = xc + (int64_t)b * cdim + HP + GN + g * N;
      double v = (double)dt[(int64_t)b * H + h];
      if (dt_bias) v += (double)dt_bias[h];
      const double delta = dt_softplus ? softplus(v) : v;
      const double a = exp(delta * (double)A[h]);
      const double Dh = D ? (double)D[h] : 0.0;
      double* S = state + ((int64_t)b * H + h) * P * N;
      for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n) {
          double* s = &S[(int64_t)p * N + n];
          *s = a * *s + delta * xv[p] * Bv[n];
          acc += *s * Cv[n];
        }
        double yv = acc + Dh * xv[p];
        const int64_t o = (int64_t)b * HP + h * P + p;
        if (z) yv *= silu((double)z[o]);
        y[o] = yv;
      }
    }
  free(xc);
  return 0;
}

/* d silu(u) / du = sigmoid(u) (1 + u (1 - sigmoid(u))). */
static double silu_grad(double u) {
  const double sg = 1.0 / (1.0 + exp(-u));
  return sg * (1.0 + u * (1.0 - sg));
}

/*
 * The gradient of the layer (reverse-mode differentiation of
 * oracle_mamba2_fwd, token by token in reverse order).
 *
 * Given dout [B][L][H][P] (the gradient of a scalar loss with respect to the
 * layer's output) and dh_final [B][H][P][N] or NULL (with respect to the
 * final state), it returns the loss's gradients with respect to every input:
 *   dxbc [B][L][Cdim] (raw x|B|C when conv_w is given, else the post-conv
 *   values), ddt [B][L][H], dz [B][L][H][P] (when z is given), dA [H],
 *   dD [H], ddt_bias [H], dh0 [B][H][P][N], dconv_w [Cdim][K],
 *   dconv_b [Cdim], dconv_state_in [B][K-1][Cdim]; each output may be NULL
 *   when not wanted (except dxbc, ddt, dA).  Outputs are dense and are
 *   overwritten.
 *
 * For each (b, h), with S_t the state after token t (S_{-1} = h0 or 0),
 * dS the gradient with respect to S_t (dh_final at t = L-1), and
 * yv_t = S_t C_t + D x_t, out_t = yv_t silu(z_t):
 *   dyv = dout silu(z);  dz = dout yv silu'(z)
 *   dD += dyv . x;  dx += D dyv;  dS += dyv C^T;  dC += S_t^T dyv
 *   from S_t = a S_{t-1} + delta x B^T, a = exp(delta A):
 *     dx += delta dS B;  dB += delta dS^T x;  ddelta += x^T dS B
 *     da = <dS, S_{t-1}>;  ddelta += da a A;  dA += da a delta
 *     dS <- a dS
 *   ddt = ddelta softplus'(dt + dt_bias) (= sigmoid) or ddelta;
 *   ddt_bias += ddt;  finally dh0 = dS.
 * B and C gradients of the heads of one group add up.  Then the conv: with
 * du = dpost silu'(u), every tap adds w du to its input (or to the conv
 * history for positions before the sequence), du times the input to dw, and
 * du to db.  Returns 0, or -1 on a bad argument.
 */
int oracle_mamba2_bwd(const double* xbc, int64_t xbc_tok_stride, const double* conv_w,
                      const double* conv_b, int width, const double* conv_state_in,
                      const double* dt, const double* A, const double* D,
                      const double* dt_bias, int dt_softplus, const double* z,
                      const double* h0, const double* dout, const double* dh_final,
                      double* dxbc, double* ddt, double* dz, double* dA, double* dD,
                      double* ddt_bias, double* dh0, double* dconv_w, double* dconv_b,
                      double* dconv_state_in, int batch, int seqlen, int nheads,
                      int headdim, int ngroups, int dstate) {
  const int H = nheads, P = headdim, G = ngroups, N = dstate, L = seqlen;
  if (!xbc || !dt || !A || !dout || !dxbc || !ddt || !dA || batch < 0 || L < 0 || H <= 0 ||
      P <= 0 || G <= 0 || N <= 0 || H % G != 0 || (conv_w && width < 1))
    return -1;
  const int HP = H * P, GN = G * N, cdim = HP + 2 * GN;
  if (xbc_tok_stride < cdim) return -1;
  const int64_t BL = (int64_t)batch * L;

  /* post-conv values (and pre-activations for the conv's gradient) */
  double* post = (double*)malloc(sizeof(double) * (size_t)(BL * cdim + 1));
  double* pre = (double*)malloc(sizeof(double) * (size_t)(BL * cdim + 1));
  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < L; ++t)
      for (int c = 0; c < cdim; ++c) {
        const int64_t o = ((int64_t)b * L + t) * cdim + c;
        if (conv_w) {
          pre[o] = conv_pre(xbc, xbc_tok_stride, conv_state_in, conv_w, conv_b, L, cdim, width,
                            b, t, c);
          post[o] = silu(pre[o]);
        } else {
          pre[o] = 0.0;
          post[o] = xbc[((int64_t)b * L + t) * xbc_tok_stride + c];
        }
      }
  /* gradient with respect to the post-conv values; B and C per head first */
  double* dpost = (double*)calloc((size_t)(BL * cdim + 1), sizeof(double));
  double* dBh = (double*)calloc((size_t)((int64_t)batch * H * L * N + 1), sizeof(double));
  double* dCh = (double*)calloc((size_t)((int64_t)batch * H * L * N + 1), sizeof(double));
  double* dA_bh = (double*)calloc((size_t)(batch * H + 1), sizeof(double));
  double* dD_bh = (double*)calloc((size_t)(batch * H + 1), sizeof(double));
  double* dbias_bh = (double*)calloc((size_t)(batch * H + 1), sizeof(double));

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < H; ++h) {
      const int g = (int)(((int64_t)h * G) / H);
      const int64_t PN = (int64_t)P * N;
      double* S = (double*)malloc(sizeof(double) * (size_t)((L + 1) * PN));  /* S[t+1] = S_t */
      double* delta = (double*)malloc(sizeof(double) * (size_t)(L + 1));
      double* av = (double*)malloc(sizeof(double) * (size_t)(L + 1));
      double* dS = (double*)malloc(sizeof(double) * (size_t)PN);
      const double Ah = A[h], Dh = D ? D[h] : 0.0;
      for (int64_t i = 0; i < PN; ++i) S[i] = h0 ? h0[((int64_t)b * H + h) * PN + i] : 0.0;
      /* forward, keeping every state */
      for (int t = 0; t < L; ++t) {
        const double* row = post + ((int64_t)b * L + t) * cdim;
        const double* xv = row + h * P;
        const double* Bv = row + HP + g * N;
        double v = dt[((int64_t)b * L + t) * H + h];
        if (dt_bias) v += dt_bias[h];
        delta[t] = dt_softplus ? softplus(v) : v;
        av[t] = exp(delta[t] * Ah);
        for (int p = 0; p < P; ++p)
          for (int n = 0; n < N; ++n)
            S[(t + 1) * PN + (int64_t)p * N + n] =
                av[t] * S[t * PN + (int64_t)p * N + n] + delta[t] * xv[p] * Bv[n];
      }
      /* reverse */
      for (int64_t i = 0; i < PN; ++i)
        dS[i] = dh_final ? dh_final[((int64_t)b * H + h) * PN + i] : 0.0;
      for (int t = L - 1; t >= 0; --t) {
        const double* row = post + ((int64_t)b * L + t) * cdim;
        const double* xv = row + h * P;
        const double* Bv = row + HP + g * N;
        const double* Cv = row + HP + GN + g * N;
        double* dxv = dpost + ((int64_t)b * L + t) * cdim + h * P;
        double* dBv = dBh + (((int64_t)b * H + h) * L + t) * N;
        double* dCv = dCh + (((int64_t)b * H + h) * L + t) * N;
        const double* St = S + (t + 1) * PN;
        const double* Sp = S + t * PN;
        double ddelta = 0.0;
        for (int p = 0; p < P; ++p) {
          const int64_t o = (((int64_t)b * L + t) * H + h) * P + p;
          double acc = 0.0;
          for (int n = 0; n < N; ++n) acc += St[(int64_t)p * N + n] * Cv[n];
          const double yv = acc + Dh * xv[p];
          double dyv = dout[o];
          if (z) {
            dyv = dout[o] * silu(z[o]);
            if (dz) dz[o] = dout[o] * yv * silu_grad(z[o]);
          }
          dD_bh[b * H + h] += dyv * xv[p];
          dxv[p] += Dh * dyv;
          for (int n = 0; n < N; ++n) {
            dS[(int64_t)p * N + n] += dyv * Cv[n];
            dCv[n] += dyv * St[(int64_t)p * N + n];
          }
        }
        double da = 0.0;
        for (int p = 0; p < P; ++p)
          for (int n = 0; n < N; ++n) {
            const double d = dS[(int64_t)p * N + n];
            dxv[p] += delta[t] * d * Bv[n];
            dBv[n] += delta[t] * d * xv[p];
            ddelta += d * xv[p] * Bv[n];
            da += d * Sp[(int64_t)p * N + n];
          }
        ddelta += da * av[t] * Ah;
        dA_bh[b * H + h] += da * av[t] * delta[t];
        for (int64_t i = 0; i < PN; ++i) dS[i] *= av[t];
        double v = dt[((int64_t)b * L + t) * H + h];
        if (dt_bias) v += dt_bias[h];
        const double dd = dt_softplus ? ddelta / (1.0 + exp(-v)) : ddelta;
        ddt[((int64_t)b * L + t) * H + h] = dd;
        dbias_bh[b * H + h] += dd;
      }
      if (dh0) memcpy(dh0 + ((int64_t)b * H + h) * PN, dS, sizeof(double) * (size_t)PN);
      free(dS);
      free(av);
      free(delta);
      free(S);
    }

  /* the heads of a group share B and C: their gradients add up */
  for (int b = 0; b < batch; ++b)
    for (int h = 0; h < H; ++h) {
      const int g = (int)(((int64_t)h * G) / H);
      for (int t = 0; t < L; ++t)
        for (int n = 0; n < N; ++n) {
          double* row = dpost + ((int64_t)b * L + t) * cdim;
          row[HP + g * N + n] += dBh[(((int64_t)b * H + h) * L + t) * N + n];
          row[HP + GN + g * N + n] += dCh[(((int64_t)b * H + h) * L + t) * N + n];
        }
    }
  for (int h = 0; h < H; ++h) {
    double sa = 0.0, sd = 0.0, sb = 0.0;
    for (int b = 0; b < batch; ++b) {
      sa += dA_bh[b * H + h];
      sd += dD_bh[b * H + h];
      sb += dbias_bh[b * H + h];
    }
    dA[h] = sa;
    if (dD) dD[h] = sd;
    if (ddt_bias) ddt_bias[h] = sb;
  }

  /* the conv */
  if (conv_w) {
    for (int64_t i = 0; i < BL * cdim; ++i) dxbc[i] = 0.0;
    if (dconv_state_in)
      for (int64_t i = 0; i < (int64_t)batch * (width - 1) * cdim; ++i) dconv_state_in[i] = 0.0;
    if (dconv_w)
      for (int64_t i = 0; i < (int64_t)cdim * width; ++i) dconv_w[i] = 0.0;
    if (dconv_b)
      for (int c = 0; c < cdim; ++c) dconv_b[c] = 0.0;
    for (int b = 0; b < batch; ++b)
      for (int t = 0; t < L; ++t)
        for (int c = 0; c < cdim; ++c) {
          const int64_t o = ((int64_t)b * L + t) * cdim + c;
          const double du = dpost[o] * silu_grad(pre[o]);
          if (dconv_b) dconv_b[c] += du;
          for (int k = 0; k < width; ++k) {
            const int tau = t - (width - 1) + k;
            const double wk = conv_w[(int64_t)c * width + k];
            if (dconv_w)
              dconv_w[(int64_t)c * width + k] +=
                  du * conv_input(xbc, xbc_tok_stride, conv_state_in, L, cdim, width, b, tau, c);
            if (tau >= 0)
              dxbc[((int64_t)b * L + tau) * cdim + c] += wk * du;
            else if (dconv_state_in)
              dconv_state_in[((int64_t)b * (width - 1) + (width - 1) + tau) * cdim + c] += wk * du;
          }
        }
  } else {
    memcpy(dxbc, dpost, sizeof(double) * (size_t)(BL * cdim));
  }
  free(dbias_bh);
  free(dD_bh);
  free(dA_bh);
  free(dCh);
  free(dBh);
  free(dpost);
  free(pre);
  free(post);
  return 0;
}

/*
 * RMSNorm over the last axis of x [ntok][dim] (dense):
 *   out[t][i] = x[t][i] / sqrt(mean_j x[t][j]^2 + eps) * w[i]
 * (no weight when w is NULL).  This is the norm of the pre-norm residual
 * block x + mamba(norm(x)) in "Nemotron-H style Hybrid Mamba-Transformer 3B
 * feasibility study", section 3.2 (approach A); its definition (root mean
 * square over the channels, a learned per-channel scale, eps inside the
 * root) is the standard one.  Returns 0, or -1 on a bad argument.
 */
int oracle_rmsnorm(const double* x, const double* w, double eps, double* out,
                   int64_t ntok, int dim) {
  if (!x || !out || ntok < 0 || dim <= 0 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < ntok; ++t) {
    const double* xr = x + t * dim;
    double ss = 0.0;
    for (int i = 0; i < dim; ++i) ss += xr[i] * xr[i];
    const double r = 1.0 / sqrt(ss / dim + eps);
    for (int i = 0; i < dim; ++i) out[t * dim + i] = xr[i] * r * (w ? w[i] : 1.0);
  }
  return 0;
}

/*
 * Linear map with the weight stored [out][in] (a projection's layout):
 *   out[m][n] = sum_k a[m][k] * w[n][k]  (+ residual[m][n] when given)
 * a [M][K], w [N][K], residual and out [M][N], all dense.  The in_proj and
 * out_proj projections of the Mamba-2 mixer (parameters about
 * 3 * expand * d_model^2 per layer: feasibility study, section 2.4) and the
 * residual add of section 3.2 are this map.  Returns 0, or -1 on a bad
 * argument.
 */
int oracle_linear(const double* a, const double* w, const double* residual, double* out,
                  int64_t M, int N, int K) {
  if (!a || !w || !out || M < 0 || N <= 0 || K <= 0) return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += a[m * K + k] * w[(int64_t)n * K + k];
      out[m * N + n] = residual ? residual[m * N + n] + acc : acc;
    }
  return 0;
}

/* Number of threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
