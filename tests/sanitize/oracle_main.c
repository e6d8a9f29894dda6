/* Every function of the fp64 oracle on small shapes, with each buffer
 * allocated at its exact size, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer: an index past a buffer's end, a use of
 * uninitialised bounds or an integer overflow in the index arithmetic stops
 * the run.  Values are checked elsewhere (the pins); here only that every
 * call returns 0 and its outputs are finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_conv1d_silu(int batch, int L, int CH, int K, const double *x, const double *w, const double *bias,
                       const int *seq_idx, int num_seqs, const double *conv_state_in, double *conv_state_out,
                       double *out);
int oracle_ssd_scan(int batch, int L, int H, int P, int N, int G, const double *x, const double *dt_raw,
                    const double *dt_bias, const double *A, const double *B, const double *C, const double *D,
                    const int *seq_idx, int num_seqs, const double *initial_state, double *final_state, double *y);
int oracle_decode_step(int batch, int H, int P, int N, int G, int K, const double *xBC, const double *dt_raw,
                       const double *dt_bias, const double *A, const double *D, const double *conv_w,
                       const double *conv_bias, double *conv_state, double *ssm_state, double *y);
int oracle_linear(int M, int N, int K, const double *x, const double *w, double *y);
int oracle_gated_rmsnorm(int T, int CH, int group_size, int norm_before_gate, double eps, const double *y,
                         const double *z, const double *w, double *out);
int oracle_decode_step_mimo(int batch, int H, int P, int N, int G, int R, int trapezoid, const double *x,
                            const double *B, const double *C, const double *dt_raw, const double *lam,
                            const double *dt_bias, const double *A, const double *D, double *ssm_state,
                            double *prev_x, double *prev_B, double *y);
int oracle_ssd_scan_bwd(int batch, int L, int H, int P, int N, int G, const double *x, const double *dt_raw,
                        const double *dt_bias, const double *A, const double *B, const double *C, const double *D,
                        const double *initial_state, const double *dy, const double *d_final, double *dx,
                        double *ddt_raw, double *dB, double *dC, double *ddt_bias, double *dA, double *dD,
                        double *dh0);

static unsigned long long rng = 88172645463325252ull;
static double uni(void) {  /* xorshift64, values in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *vec(size_t n) {
  double *p = (double *)malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = 0.5 * uni();
  return p;
}
static double *neg(size_t n) {  /* A < 0 */
  double *p = vec(n);
  for (size_t i = 0; i < n; ++i) p[i] = -0.5 - fabs(p[i]);
  return p;
}
static int failures = 0;
static void check(const char *what, int rc, const double *out, size_t n) {
  int bad = rc != 0;
  for (size_t i = 0; i < n && !bad; ++i) bad = !isfinite(out[i]);
  if (bad) { printf("FAIL %s (rc %d)\n", what, rc); ++failures; }
}

int main(void) {
  const int P = 8, N = 16, K = 4;
  /* conv: batch rows, then a packed stream with conv states */
  {
    const int batch = 2, L = 37, CH = 24;
    double *x = vec((size_t)batch * L * CH), *w = vec((size_t)CH * K), *b = vec(CH);
    double *so = vec((size_t)batch * (K - 1) * CH), *si = vec((size_t)batch * (K - 1) * CH);
    double *out = vec((size_t)batch * L * CH);
    check("conv batch", oracle_conv1d_silu(batch, L, CH, K, x, w, b, NULL, 0, si, so, out), out,
          (size_t)batch * L * CH);
    int seq[37];
    for (int t = 0; t < 37; ++t) seq[t] = t < 2 ? 0 : (t < 20 ? 1 : 2);
    double *si3 = vec((size_t)3 * (K - 1) * CH), *so3 = vec((size_t)3 * (K - 1) * CH);
    check("conv packed", oracle_conv1d_silu(1, L, CH, K, x, w, NULL, seq, 3, si3, so3, out), out, (size_t)L * CH);
    free(x); free(w); free(b); free(so); free(si); free(out); free(si3); free(so3);
  }
  /* scan: batch rows with initial / final states, packed, and L = 0 */
  {
    const int batch = 2, L = 29, H = 4, G = 2;
    double *x = vec((size_t)batch * L * H * P), *dt = vec((size_t)batch * L * H), *dtb = vec(H), *A = neg(H);
    double *B = vec((size_t)batch * L * G * N), *C = vec((size_t)batch * L * G * N), *D = vec(H);
    double *h0 = vec((size_t)batch * H * P * N), *hf = vec((size_t)batch * H * P * N);
    double *y = vec((size_t)batch * L * H * P);
    check("scan batch", oracle_ssd_scan(batch, L, H, P, N, G, x, dt, dtb, A, B, C, D, NULL, 0, h0, hf, y), y,
          (size_t)batch * L * H * P);
    int seq[29];
    for (int t = 0; t < L; ++t) seq[t] = t < 1 ? 0 : (t < 15 ? 1 : 3);  /* sequence 2 is empty */
    double *h04 = vec((size_t)4 * H * P * N), *hf4 = vec((size_t)4 * H * P * N);
    check("scan packed", oracle_ssd_scan(1, L, H, P, N, G, x, dt, dtb, A, B, C, D, seq, 4, h04, hf4, y), hf4,
          (size_t)4 * H * P * N);
    check("scan empty", oracle_ssd_scan(batch, 0, H, P, N, G, x, dt, dtb, A, B, C, D, NULL, 0, h0, hf, y), hf,
          (size_t)batch * H * P * N);
    /* backward */
    double *dy = vec((size_t)batch * L * H * P), *df = vec((size_t)batch * H * P * N);
    double *dx = vec((size_t)batch * L * H * P), *ddt = vec((size_t)batch * L * H);
    double *dB = vec((size_t)batch * L * G * N), *dC = vec((size_t)batch * L * G * N);
    double *ddtb = vec(H), *dA = vec(H), *dD = vec(H), *dh0 = vec((size_t)batch * H * P * N);
    check("scan bwd", oracle_ssd_scan_bwd(batch, L, H, P, N, G, x, dt, dtb, A, B, C, D, h0, dy, df, dx, ddt, dB, dC,
                                          ddtb, dA, dD, dh0), dB, (size_t)batch * L * G * N);
    free(x); free(dt); free(dtb); free(A); free(B); free(C); free(D); free(h0); free(hf); free(y);
    free(h04); free(hf4); free(dy); free(df); free(dx); free(ddt); free(dB); free(dC); free(ddtb); free(dA);
    free(dD); free(dh0);
  }
  /* decode: with and without the conv window */
  {
    const int batch = 3, H = 4, G = 2, CH = H * P + 2 * G * N;
    double *xbc = vec((size_t)batch * CH), *dt = vec((size_t)batch * H), *dtb = vec(H), *A = neg(H), *D = vec(H);
    double *cw = vec((size_t)CH * K), *cb = vec(CH), *cst = vec((size_t)batch * (K - 1) * CH);
    double *st = vec((size_t)batch * H * P * N), *y = vec((size_t)batch * H * P);
    check("decode conv", oracle_decode_step(batch, H, P, N, G, K, xbc, dt, dtb, A, D, cw, cb, cst, st, y), y,
          (size_t)batch * H * P);
    check("decode", oracle_decode_step(batch, H, P, N, G, K, xbc, dt, dtb, A, D, NULL, NULL, NULL, st, y), y,
          (size_t)batch * H * P);
    /* MIMO, rank 3, Euler and trapezoidal */
    const int R = 3;
    double *mx = vec((size_t)batch * H * P * R), *mB = vec((size_t)batch * G * N * R), *mC = vec((size_t)batch * G * N * R);
    double *lam = vec((size_t)batch * H), *px = vec((size_t)batch * H * P * R), *pB = vec((size_t)batch * G * N * R);
    double *my = vec((size_t)batch * H * P * R);
    check("mimo", oracle_decode_step_mimo(batch, H, P, N, G, R, 0, mx, mB, mC, dt, NULL, dtb, A, D, st, NULL, NULL,
                                          my), my, (size_t)batch * H * P * R);
    check("mimo trapezoid", oracle_decode_step_mimo(batch, H, P, N, G, R, 1, mx, mB, mC, dt, lam, dtb, A, D, st, px,
                                                    pB, my), my, (size_t)batch * H * P * R);
    free(xbc); free(dt); free(dtb); free(A); free(D); free(cw); free(cb); free(cst); free(st); free(y);
    free(mx); free(mB); free(mC); free(lam); free(px); free(pB); free(my);
  }
  /* linear and gated norm */
  {
    const int M = 5, Nn = 7, Kk = 9, T = 6, CH = 32;
    double *x = vec((size_t)M * Kk), *w = vec((size_t)Nn * Kk), *y = vec((size_t)M * Nn);
    check("linear", oracle_linear(M, Nn, Kk, x, w, y), y, (size_t)M * Nn);
    double *ny = vec((size_t)T * CH), *nz = vec((size_t)T * CH), *nw = vec(CH), *out = vec((size_t)T * CH);
    check("norm", oracle_gated_rmsnorm(T, CH, 8, 0, 1e-5, ny, nz, nw, out), out, (size_t)T * CH);
    check("norm before gate", oracle_gated_rmsnorm(T, CH, 16, 1, 1e-5, ny, nz, nw, out), out, (size_t)T * CH);
    check("norm no gate", oracle_gated_rmsnorm(T, CH, 32, 0, 1e-5, ny, NULL, nw, out), out, (size_t)T * CH);
    free(x); free(w); free(y); free(ny); free(nz); free(nw); free(out);
  }
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
