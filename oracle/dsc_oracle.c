/*
 * CPU oracle for the causal dynamic short convolution.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only users of this file. The GPU
 * library neither links, includes nor calls it, and the two share no source.
 *
 * Every function is the plain definition of its output, evaluated literally
 * with double-precision accumulation, one output element at a time. Inputs
 * are read in their storage type (float32, or bfloat16 bit patterns widened
 * exactly) and every output is double.
 *
 * Source: "Dynamic Short Convolutions Improve Transformers" (technical summary
 * page), section Metodologia:
 *   - Mecanismo: y_t = sum_{k=0}^{W-1} w(t)_k (.) x_{t-k}, the filter being
 *     drawn fresh at every step t;
 *   - Parametrizacao 1 (low-rank factorisation of the filter generator, rank R)
 *     and section "Kernel de Fatoracao de Baixo Posto Fundido": the filter is
 *     the product z.U of the low-rank input z and the projection matrix U;
 *   - Parametrizacao 2 (head-wise tying): one filter shared by H consecutive
 *     channels;
 *   - Posicionamento: the residual form X + dynamicShortConv(X).
 * The page prints no backward pass; the gradients below are the chain rule
 * applied to that forward definition (the page trains with it, section
 * "Implementacao de Treinamento Eficiente").
 *
 * Readings where the page is silent (all are listed with the design notes):
 *   - x at t < 0 is zero for every sequence; nothing carries across the batch;
 *   - tap k = 0 multiplies x_t; (.) is elementwise over channels, a head's
 *     scalar filter tap applied to each of its Hc channels;
 *   - channel c belongs to head h = c / Hc, Hc = D / G;
 *   - the low-rank filter of channel c, tap k is column c*W + k of z.U
 *     (z.U reshaped row-major to [D, W]); no bias or nonlinearity on it.
 *
 * Layouts (all row-major, contiguous):
 *   x, y, dy, dx [B,T,D];  w, dw [B,T,G,W];  z, dz [B,T,R];  U, dU [R, D*W].
 *
 * Packed sequences: every function also takes an optional pos[B*T] (int32,
 * NULL for none), the index of each token within its own sequence. Tap k > 0 of
 * step t is then applied only if k <= pos[b*T+t], so sequences packed into one
 * row do not see each other; NULL keeps every tap (each row is one sequence).
 * This is the convolution of the Mecanismo bullet applied per sequence; the
 * page does not treat packing, the reading is listed with the design notes.
 *
 * Row selection: functions that produce per-token outputs take an optional
 * list of flat token indices rows[n] = b*T + t (NULL means every token in
 * order, nrows = B*T); output row n then belongs to token rows[n].
 *
 * Return value: 0 on success, -1 on an invalid argument.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2 /* only for dy of oracle_bwd_dy64 */

/* One stored element as double, exactly. */
static double ld(const void* p, int64_t i, int dt) {
  if (dt == ORACLE_F64) return ((const double*)p)[i];
  if (dt == ORACLE_F32) return (double)((const float*)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Tap k of step t (flat token index n = b*T + t) exists: inside the row and, with
 * positions, inside the token's own sequence. Taps are a prefix in k for fixed t. */
static int tap_on(const int32_t* pos, int64_t n, int64_t t, int k) {
  return t - k >= 0 && (k == 0 || !pos || k <= pos[n]);
}

static int bad_dims(int64_t B, int64_t T, int64_t D, int W, int dt) {
  return B < 0 || T < 0 || D <= 0 || W < 1 || (dt != ORACLE_F32 && dt != ORACLE_BF16);
}

int oracle_abi_version(void) { return 1; }

void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

int oracle_get_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- head-wise */

/* Forward, head-wise tied filters (Mecanismo + Parametrizacao 2 + Posicionamento):
 *   y[b,t,c] = residual*x[b,t,c] + sum_{k=0}^{W-1} w[b,t,c/Hc,k] * x[b,t-k,c],
 * the terms with t-k < 0 being zero. */
static int fwd_impl(const void* x, const void* w, const int32_t* pos, int64_t B, int64_t T, int64_t D,
                    int64_t G, int W, int residual, int dt, int w_dt, const int64_t* rows, int64_t nrows,
                    double* y) {
  if (bad_dims(B, T, D, W, dt) || G <= 0 || D % G != 0) return -1;
  if (!rows) nrows = B * T;
  const int64_t Hc = D / G;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < nrows; ++n) {
    const int64_t row = rows ? rows[n] : n;
    const int64_t b = row / T, t = row % T;
    for (int64_t c = 0; c < D; ++c) {
      const int64_t h = c / Hc;
      double acc = 0.0;
      for (int k = 0; k < W; ++k) {
        if (!tap_on(pos, b * T + t, t, k)) break;
        acc += ld(w, ((b * T + t) * G + h) * W + k, w_dt) * ld(x, (b * T + (t - k)) * D + c, dt);
      }
      if (residual) acc += ld(x, (b * T + t) * D + c, dt);
      y[n * D + c] = acc;
    }
  }
  return 0;
}

int oracle_fwd(const void* x, const void* w, const int32_t* pos, int64_t B, int64_t T, int64_t D,
               int64_t G, int W, int residual, int dt, const int64_t* rows, int64_t nrows, double* y) {
  return fwd_impl(x, w, pos, B, T, D, G, W, residual, dt, dt, rows, nrows, y);
}

/* oracle_fwd with the filters w given in double (x in storage type dt): filters
 * produced by the generator projection (Parametrizacao, head-wise tying) in
 * exact arithmetic rather than read from a stored tensor. */
int oracle_fwd_w64(const void* x, const double* w, const int32_t* pos, int64_t B, int64_t T, int64_t D,
                   int64_t G, int W, int residual, int dt, const int64_t* rows, int64_t nrows, double* y) {
  return fwd_impl(x, w, pos, B, T, D, G, W, residual, dt, ORACLE_F64, rows, nrows, y);
}

/* Backward of oracle_fwd, by the chain rule:
 *   dx[b,s,c]   = residual*dy[b,s,c] + sum_{k=0}^{W-1} w[b,s+k,c/Hc,k] * dy[b,s+k,c]
 *                 (terms with s+k >= T are zero: no later step exists; with
 *                 positions, only the terms whose tap k exists at step s+k);
 *   dw[b,t,h,k] = sum_{c in head h} dy[b,t,c] * x[b,t-k,c]   (zero when tap k of t does not exist).
 * dx is [nrows, D], dw is [nrows, G, W]; either may be NULL. */
static int bwd_impl(const void* x, const void* w, const void* dy, const int32_t* pos, int64_t B, int64_t T,
                    int64_t D, int64_t G, int W, int residual, int dt, int w_dt, int dy_dt, const int64_t* rows,
                    int64_t nrows, double* dx, double* dw) {
  if (bad_dims(B, T, D, W, dt) || G <= 0 || D % G != 0) return -1;
  if (!rows) nrows = B * T;
  const int64_t Hc = D / G;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < nrows; ++n) {
    const int64_t row = rows ? rows[n] : n;
    const int64_t b = row / T, s = row % T;
    if (dx) {
      for (int64_t c = 0; c < D; ++c) {
        const int64_t h = c / Hc;
        double acc = 0.0;
        for (int k = 0; k < W; ++k) {
          if (s + k >= T) break;
          if (!tap_on(pos, b * T + s + k, s + k, k)) continue;
          acc += ld(w, ((b * T + s + k) * G + h) * W + k, w_dt) * ld(dy, (b * T + s + k) * D + c, dy_dt);
        }
        if (residual) acc += ld(dy, (b * T + s) * D + c, dy_dt);
        dx[n * D + c] = acc;
      }
    }
    if (dw) {
      const int64_t t = s;
      for (int64_t h = 0; h < G; ++h) {
        for (int k = 0; k < W; ++k) {
          double acc = 0.0;
          if (tap_on(pos, b * T + t, t, k)) {
            for (int64_t j = 0; j < Hc; ++j) {
              const int64_t c = h * Hc + j;
              acc += ld(dy, (b * T + t) * D + c, dy_dt) * ld(x, (b * T + (t - k)) * D + c, dt);
            }
          }
          dw[(n * G + h) * W + k] = acc;
        }
      }
    }
  }
  return 0;
}

int oracle_bwd(const void* x, const void* w, const void* dy, const int32_t* pos, int64_t B, int64_t T,
               int64_t D, int64_t G, int W, int residual, int dt, const int64_t* rows, int64_t nrows,
               double* dx, double* dw) {
  return bwd_impl(x, w, dy, pos, B, T, D, G, W, residual, dt, dt, dt, rows, nrows, dx, dw);
}

/* oracle_bwd with dy given in double (x and w in storage type dt): the gradient
 * that reaches the convolution through a rotation applied after it. */
int oracle_bwd_dy64(const void* x, const void* w, const double* dy, const int32_t* pos, int64_t B, int64_t T,
                    int64_t D, int64_t G, int W, int residual, int dt, const int64_t* rows, int64_t nrows,
                    double* dx, double* dw) {
  return bwd_impl(x, w, dy, pos, B, T, D, G, W, residual, dt, dt, ORACLE_F64, rows, nrows, dx, dw);
}

/* oracle_bwd with the filters w given in double (x and dy in storage type dt): the
 * backward of oracle_fwd_w64, for filters produced by the generator projection
 * (Parametrizacao, head-wise tying) in exact arithmetic. */
int oracle_bwd_w64(const void* x, const double* w, const void* dy, const int32_t* pos, int64_t B, int64_t T,
                   int64_t D, int64_t G, int W, int residual, int dt, const int64_t* rows, int64_t nrows,
                   double* dx, double* dw) {
  return bwd_impl(x, w, dy, pos, B, T, D, G, W, residual, dt, ORACLE_F64, dt, rows, nrows, dx, dw);
}

/* ---------------------------------------------------------------- low-rank */

/* The generated filter of token (b,t): omega[c*W+k] = sum_r z[b,t,r] * U[r, c*W+k]
 * (Parametrizacao 1; the product zU of the fused-kernel section). */
static void lowrank_filter(const void* z, const void* U, int64_t b, int64_t t, int64_t T,
                           int64_t D, int R, int W, int dt, double* omega) {
  const int64_t cols = D * W;
  for (int64_t j = 0; j < cols; ++j) {
    double acc = 0.0;
    for (int r = 0; r < R; ++r) acc += ld(z, (b * T + t) * R + r, dt) * ld(U, (int64_t)r * cols + j, dt);
    omega[j] = acc;
  }
}

/* Forward, low-rank filters:
 *   y[b,t,c] = residual*x[b,t,c] + sum_{k=0}^{W-1} omega[b,t][c*W+k] * x[b,t-k,c]. */
int oracle_lowrank_fwd(const void* x, const void* z, const void* U, const int32_t* pos, int64_t B,
                       int64_t T, int64_t D, int R, int W, int residual, int dt, const int64_t* rows,
                       int64_t nrows, double* y) {
  if (bad_dims(B, T, D, W, dt) || R < 1) return -1;
  if (!rows) nrows = B * T;
  int fail = 0;
#pragma omp parallel
  {
    double* omega = (double*)malloc(sizeof(double) * (size_t)(D * W));
    if (!omega) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t n = 0; n < nrows; ++n) {
      if (!omega) continue;
      const int64_t row = rows ? rows[n] : n;
      const int64_t b = row / T, t = row % T;
      lowrank_filter(z, U, b, t, T, D, R, W, dt, omega);
      for (int64_t c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int k = 0; k < W; ++k) {
          if (!tap_on(pos, b * T + t, t, k)) break;
          acc += omega[c * W + k] * ld(x, (b * T + (t - k)) * D + c, dt);
        }
        if (residual) acc += ld(x, (b * T + t) * D + c, dt);
        y[n * D + c] = acc;
      }
    }
    free(omega);
  }
  return fail ? -1 : 0;
}

/* Per-token gradients of oracle_lowrank_fwd, by the chain rule:
 *   dx[b,s,c] = residual*dy[b,s,c] + sum_{k} omega[b,s+k][c*W+k] * dy[b,s+k,c]   (s+k < T, tap k of s+k exists);
 *   dz[b,t,r] = sum_{c,k} dy[b,t,c] * x[b,t-k,c] * U[r, c*W+k]                  (tap k of t exists).
 * dx is [nrows, D], dz is [nrows, R]; either may be NULL. */
int oracle_lowrank_bwd_rows(const void* x, const void* z, const void* U, const void* dy, const int32_t* pos,
                            int64_t B, int64_t T, int64_t D, int R, int W, int residual, int dt,
                            const int64_t* rows, int64_t nrows, double* dx, double* dz) {
  if (bad_dims(B, T, D, W, dt) || R < 1) return -1;
  if (!rows) nrows = B * T;
  const int64_t cols = D * W;
  int fail = 0;
#pragma omp parallel
  {
    double* omega = (double*)malloc(sizeof(double) * (size_t)(cols * W));
    if (!omega) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t n = 0; n < nrows; ++n) {
      if (!omega) continue;
      const int64_t row = rows ? rows[n] : n;
      const int64_t b = row / T, s = row % T;
      if (dx) {
        /* omega of the W tokens s .. s+W-1 that read x[b,s] */
        for (int k = 0; k < W && s + k < T; ++k)
          lowrank_filter(z, U, b, s + k, T, D, R, W, dt, omega + k * cols);
        for (int64_t c = 0; c < D; ++c) {
          double acc = 0.0;
          for (int k = 0; k < W; ++k) {
            if (s + k >= T) break;
            if (!tap_on(pos, b * T + s + k, s + k, k)) continue;
            acc += omega[k * cols + c * W + k] * ld(dy, (b * T + s + k) * D + c, dt);
          }
          if (residual) acc += ld(dy, (b * T + s) * D + c, dt);
          dx[n * D + c] = acc;
        }
      }
      if (dz) {
        const int64_t t = s;
        for (int r = 0; r < R; ++r) {
          double acc = 0.0;
          for (int64_t c = 0; c < D; ++c) {
            for (int k = 0; k < W; ++k) {
              if (!tap_on(pos, b * T + t, t, k)) break;
              acc += ld(dy, (b * T + t) * D + c, dt) * ld(x, (b * T + (t - k)) * D + c, dt) *
                     ld(U, (int64_t)r * cols + c * W + k, dt);
            }
          }
          dz[n * R + r] = acc;
        }
      }
    }
    free(omega);
  }
  return fail ? -1 : 0;
}

/* Gradient of U, summed over every token of every sequence, by the chain rule:
 *   dU[r, c*W+k] = sum_{b,t} z[b,t,r] * dy[b,t,c] * x[b,t-k,c]   (tap k of t exists).
 * Only the columns listed in cols[0..ncols) are produced (NULL: all D*W columns);
 * dU is [R, ncols]. */
int oracle_lowrank_dU(const void* x, const void* z, const void* dy, const int32_t* pos, int64_t B, int64_t T,
                      int64_t D, int R, int W, int dt, const int64_t* cols, int64_t ncols, double* dU) {
  if (bad_dims(B, T, D, W, dt) || R < 1) return -1;
  if (!cols) ncols = D * W;
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < R; ++r) {
    for (int64_t m = 0; m < ncols; ++m) {
      const int64_t j = cols ? cols[m] : m;
      const int64_t c = j / W;
      const int k = (int)(j % W);
      double acc = 0.0;
      for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = k; t < T; ++t) {
          if (!tap_on(pos, b * T + t, t, k)) continue;
          acc += ld(z, (b * T + t) * R + r, dt) * ld(dy, (b * T + t) * D + c, dt) *
                 ld(x, (b * T + (t - k)) * D + c, dt);
        }
      }
      dU[(int64_t)r * ncols + m] = acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------- decode step */

/* Generation appends one token per sequence at a time. The forward definition
 * (Mecanismo) at that token t needs, besides x_t itself, only the W-1 inputs
 * before it, so a sequence carries them from step to step in a ring:
 *   state [B, S, D] with S = W-1; input x_s of sequence b sits in slot s mod S.
 * pos[b] = t is the index of the incoming token in its sequence (0 for the
 * first); a negative pos marks a batch row with no sequence in it.
 * One step, for every row b with t = pos[b] >= 0 and filter f[c,k] of its token:
 *   y[b,c] = residual*x[b,c] + sum_{k=0}^{min(W-1,t)} f[c,k] * x_{t-k}[c],
 *            x_t = x[b,:] and x_{t-k} = state[b, (t-k) mod S, :] for k >= 1;
 *   then slot t mod S, which held x_{t-S} (read by this step, by no later one),
 *            receives x[b,:].
 * Slots of steps before 0 are never read, so a fresh sequence needs no cleared
 * ring. Rows with pos < 0 get y = NaN and keep their ring. state_out starts as
 * a copy of state and receives the updates as stored bits. W = 1 keeps no ring.
 * This is the reading of the pages for generation; they print no decode step. */
static int decode_common(int64_t B, int64_t D, int W, int dt, const int32_t* pos) {
  return B < 0 || D <= 0 || W < 1 || (dt != ORACLE_F32 && dt != ORACLE_BF16) || (B > 0 && !pos);
}

/* y row b from the filter f[c*W+k] of its token (either parametrisation). */
static void decode_row(const void* x, const double* f, const void* state, int64_t b, int64_t D, int W,
                       int residual, int dt, int32_t t, double* yrow) {
  const int64_t S = W - 1;
  for (int64_t c = 0; c < D; ++c) {
    double acc = 0.0;
    for (int k = 0; k < W; ++k) {
      if (t - k < 0) break;
      const double xv = k == 0 ? ld(x, b * D + c, dt) : ld(state, (b * S + (t - k) % S) * D + c, dt);
      acc += f[c * W + k] * xv;
    }
    if (residual) acc += ld(x, b * D + c, dt);
    yrow[c] = acc;
  }
}

static void ring_put(const void* x, int64_t b, int64_t D, int W, int dt, int32_t t, void* state_out) {
  const int64_t S = W - 1;
  if (S == 0) return;
  const size_t e = dt == ORACLE_BF16 ? 2 : 4;
  memcpy((char*)state_out + (size_t)((b * S + t % S) * D) * e, (const char*)x + (size_t)(b * D) * e, (size_t)D * e);
}

static void nan_row(double* yrow, int64_t D) {
  for (int64_t c = 0; c < D; ++c) yrow[c] = __builtin_nan("");
}

/* Head-wise: f[c,k] = w[b, c/Hc, k], w [B,G,W]. */
int oracle_decode_step(const void* x, const void* w, const int32_t* pos, const void* state, int64_t B,
                       int64_t D, int64_t G, int W, int residual, int dt, double* y, void* state_out) {
  if (decode_common(B, D, W, dt, pos) || G <= 0 || D % G != 0) return -1;
  const int64_t Hc = D / G;
  int fail = 0;
#pragma omp parallel
  {
    double* f = (double*)malloc(sizeof(double) * (size_t)(D * W));
    if (!f) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
      if (!f) continue;
      const int32_t t = pos[b];
      if (t < 0) {
        nan_row(y + b * D, D);
        continue;
      }
      for (int64_t c = 0; c < D; ++c)
        for (int k = 0; k < W; ++k) f[c * W + k] = ld(w, (b * G + c / Hc) * W + k, dt);
      decode_row(x, f, state, b, D, W, residual, dt, t, y + b * D);
    }
    free(f);
  }
  if (fail) return -1;
  /* ring updates after every row has read its ring (rows own disjoint slots anyway) */
  for (int64_t b = 0; b < B; ++b)
    if (pos[b] >= 0) ring_put(x, b, D, W, dt, pos[b], state_out);
  return 0;
}

/* Low-rank: f[c,k] = sum_r z[b,r] U[r, c*W+k], z [B,R], U [R, D*W]. */
int oracle_lowrank_decode_step(const void* x, const void* z, const void* U, const int32_t* pos,
                               const void* state, int64_t B, int64_t D, int R, int W, int residual,
                               int dt, double* y, void* state_out) {
  if (decode_common(B, D, W, dt, pos) || R < 1) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* f = (double*)malloc(sizeof(double) * (size_t)(D * W));
    if (!f) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
      if (!f) continue;
      const int32_t t = pos[b];
      if (t < 0) {
        nan_row(y + b * D, D);
        continue;
      }
      lowrank_filter(z, U, b, 0, 1, D, R, W, dt, f); /* z row b of [B,1,R] */
      decode_row(x, f, state, b, D, W, residual, dt, t, y + b * D);
    }
    free(f);
  }
  if (fail) return -1;
  for (int64_t b = 0; b < B; ++b)
    if (pos[b] >= 0) ring_put(x, b, D, W, dt, pos[b], state_out);
  return 0;
}

/* Ring after a prompt: sequence b has consumed its first n = len[b] tokens of
 * x [B,T,D] (n clamped to [0, T]); slot s mod S receives x[b,s,:] for
 * max(0, n-S) <= s < n, the other slots keep their contents. Decoding goes on
 * with pos[b] = n. state_out is updated in place. */
int oracle_decode_state_from_prefill(const void* x, const int32_t* len, int64_t B, int64_t T, int64_t D,
                                     int W, int dt, void* state_out) {
  if (bad_dims(B, T, D, W, dt) || (B > 0 && !len)) return -1;
  const int64_t S = W - 1;
  if (S == 0) return 0;
  const size_t e = dt == ORACLE_BF16 ? 2 : 4;
  for (int64_t b = 0; b < B; ++b) {
    int64_t n = len[b] < 0 ? 0 : len[b];
    if (n > T) n = T;
    for (int64_t s = n - S < 0 ? 0 : n - S; s < n; ++s)
      memcpy((char*)state_out + (size_t)((b * S + s % S) * D) * e, (const char*)x + (size_t)((b * T + s) * D) * e,
             (size_t)D * e);
  }
  return 0;
}
