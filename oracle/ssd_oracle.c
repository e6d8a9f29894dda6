/*
 * ssd_oracle.c -- plain, slow, sequential fp64 CPU oracle for the Mamba-2
 * selective state-space (SSD) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path never calls, links or includes anything from this directory, and this
 * file includes nothing from the product.
 *
 * What is computed, and where it comes from:
 *
 *  - Mamba-2 mixer order: a depthwise causal conv1d of width 4 with SiLU
 *    runs on the x|B|C channels before the selective scan
 *    ("Nemotron-H style Hybrid Mamba-Transformer 3B feasibility study",
 *    sec. 1.4 "Mamba-2 configuration": conv_kernel 4, activation SiLU;
 *    "Nemotron-Mamba3 architecture" article, sec. 2.2 layer pseudo-code:
 *    Conv1D(kernel 4) before the parallel scan).
 *  - The transition of a Mamba-2 head is a scalar times the identity
 *    ("Mamba-3: an inference-first state space model", the paragraph on
 *    how Mamba-2 simplified the diagonal transition), so each head h has
 *    one decay a_t = exp(dt_t * A_h) per token.
 *  - dt, B and C depend on the input token (selectivity: "AI Engineering
 *    EP6", sec. 6 principle 2).  dt = softplus(dt_raw + dt_bias[h]).
 *  - B and C are shared by the heads of one of n_groups groups
 *    (feasibility study sec. 1.4: n_groups 8); head h uses group
 *    h / (H / G) (contiguous blocks).
 *  - The recurrence per (sequence, head), state S of shape P x N:
 *        S[p][n] <- a_t * S[p][n] + dt_t * x[t][h][p] * B[t][g][n]
 *        y[t][h][p] = sum_n S[p][n] * C[t][g][n] + D[h] * x[t][h][p]
 *    with S = initial_state (or 0) before the first token of a sequence;
 *    the decay of the first token is applied to the initial state.
 *  - The state is fixed-size and carried across calls (resumable prefill,
 *    "Bamba-9B" summary, inference-efficiency section on chunked prefill),
 *    so every entry point takes and returns states.
 *
 * The chunked SSD algorithm the GPU runs reaches exactly this result up to
 * rounding order, so this oracle is the plain definition: one token at a
 * time, in fp64, with no chunking, blocking or reordering.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   x (batch, L, H, P)   B, C (batch, L, G, N)   dt_raw (batch, L, H)
 *   y (batch, L, H, P)   states (rows, H, P, N)
 *   conv input/output (batch, L, CH)   conv weight (CH, K)
 *   conv state (rows, K-1, CH): the K-1 raw inputs that precede the window.
 * Packed mode: batch must be 1 and seq_idx[t] gives the sequence of token
 * t (non-decreasing, values 0..num_seqs-1); rows = num_seqs.  Otherwise
 * every batch row is one sequence and rows = batch.
 *
 * Return value: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* softplus(z) = log(1 + e^z), evaluated without overflow for large z. */
static double softplus(double z) {
    if (z > 30.0) return z + log1p(exp(-z));
    return log1p(exp(z));
}

/* SiLU(u) = u * sigmoid(u) = u / (1 + e^-u). */
static double silu(double u) { return u / (1.0 + exp(-u)); }

/* Sequence boundaries: seq s covers tokens [start[s], end[s]).  In batch
 * mode row b covers [0, L) of its own row.  Returns -1 if seq_idx is not
 * non-decreasing or holds a value outside 0..num_seqs-1. */
static int find_sequences(int L, const int *seq_idx, int num_seqs,
                          int *start, int *end) {
    for (int s = 0; s < num_seqs; ++s) { start[s] = 0; end[s] = 0; }
    for (int t = 0; t < L; ++t) {
        int s = seq_idx[t];
        if (s < 0 || s >= num_seqs) return -1;
        if (t > 0 && seq_idx[t - 1] > s) return -1;
        if (t == 0 || seq_idx[t - 1] != s) start[s] = t;
        end[s] = t + 1;
    }
    return 0;
}

/*
 * Depthwise causal conv1d + SiLU.
 *   u[t][c] = bias[c] + sum_{k=0}^{K-1} w[c][k] * v(t - (K-1) + k, c)
 *   out[t][c] = SiLU(u[t][c])
 * where v(tau, c) is the raw input at tau if tau lies in the same sequence,
 * else conv_state_in[seq][tau - start + K-1][c] if a state is given, else 0.
 * conv_state_out[seq][r][c] = v(end - (K-1) + r, c), r = 0..K-2: the last
 * K-1 inputs of the sequence (falling back on the incoming state / zeros
 * for sequences shorter than K-1).
 */
int oracle_conv1d_silu(int batch, int L, int CH, int K,
                       const double *x, const double *w, const double *bias,
                       const int *seq_idx, int num_seqs,
                       const double *conv_state_in, double *conv_state_out,
                       double *out) {
    if (batch < 1 || L < 0 || CH < 1 || K < 1) return -1;
    if (seq_idx && batch != 1) return -1;
    int rows = seq_idx ? num_seqs : batch;
    if (rows < 1) return -1;
    int *start = (int *)malloc(sizeof(int) * rows);
    int *end = (int *)malloc(sizeof(int) * rows);
    if (seq_idx) {
        if (find_sequences(L, seq_idx, num_seqs, start, end)) {
            free(start); free(end); return -1;
        }
    } else {
        for (int b = 0; b < batch; ++b) { start[b] = 0; end[b] = L; }
    }
    for (int s = 0; s < rows; ++s) {
        const double *xs = x + (seq_idx ? 0 : (size_t)s * L * CH);
        double *os = out + (seq_idx ? 0 : (size_t)s * L * CH);
        const double *st = conv_state_in ? conv_state_in + (size_t)s * (K - 1) * CH : NULL;
        /* channels are independent: OpenMP only splits the channel loop over
         * threads; each output element is computed exactly as in one thread */
#pragma omp parallel for schedule(static)
        for (int c = 0; c < CH; ++c) {
            /* v(tau) for tau relative to the sequence start */
            for (int t = start[s]; t < end[s]; ++t) {
                double u = bias ? bias[c] : 0.0;
                for (int k = 0; k < K; ++k) {
                    int tau = t - (K - 1) + k;
                    double v;
                    if (tau >= start[s]) v = xs[(size_t)tau * CH + c];
                    else if (st) v = st[(size_t)(tau - start[s] + K - 1) * CH + c];
                    else v = 0.0;
                    u += w[(size_t)c * K + k] * v;
                }
                os[(size_t)t * CH + c] = silu(u);
            }
            if (conv_state_out) {
                double *so = conv_state_out + (size_t)s * (K - 1) * CH;
                for (int r = 0; r < K - 1; ++r) {
                    int tau = end[s] - (K - 1) + r;
                    double v;
                    if (tau >= start[s]) v = xs[(size_t)tau * CH + c];
                    else if (st) v = st[(size_t)(tau - start[s] + K - 1) * CH + c];
                    else v = 0.0;
                    so[(size_t)r * CH + c] = v;
                }
            }
        }
    }
    free(start); free(end);
    return 0;
}

/*
 * Selective scan, one token at a time (the plain definition of what the
 * chunked SSD prefill computes).
 */
int oracle_ssd_scan(int batch, int L, int H, int P, int N, int G,
                    const double *x, const double *dt_raw,
                    const double *dt_bias, const double *A,
                    const double *B, const double *C, const double *D,
                    const int *seq_idx, int num_seqs,
                    const double *initial_state, double *final_state,
                    double *y) {
    if (batch < 1 || L < 0 || H < 1 || P < 1 || N < 1 || G < 1) return -1;
    if (H % G != 0) return -1;
    if (seq_idx && batch != 1) return -1;
    int rows = seq_idx ? num_seqs : batch;
    if (rows < 1) return -1;
    int *start = (int *)malloc(sizeof(int) * rows);
    int *end = (int *)malloc(sizeof(int) * rows);
    if (seq_idx) {
        if (find_sequences(L, seq_idx, num_seqs, start, end)) {
            free(start); free(end); return -1;
        }
    } else {
        for (int b = 0; b < batch; ++b) { start[b] = 0; end[b] = L; }
    }
    const int heads_per_group = H / G;
    const long long units = (long long)rows * H;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long unit = 0; unit < units; ++unit) {
        const int s = (int)(unit / H);
        const int h = (int)(unit % H);
        const int g = h / heads_per_group;
        const size_t row_off = seq_idx ? 0 : (size_t)s * L;   /* token offset of this row */
        double *S = (double *)malloc(sizeof(double) * P * N);
        if (initial_state)
            memcpy(S, initial_state + ((size_t)s * H + h) * P * N, sizeof(double) * P * N);
        else
            memset(S, 0, sizeof(double) * P * N);
        const double bias = dt_bias ? dt_bias[h] : 0.0;
        const double d_skip = D ? D[h] : 0.0;
        for (int t = start[s]; t < end[s]; ++t) {
            const size_t tok = row_off + t;
            const double dt = softplus(dt_raw[tok * H + h] + bias);
            const double a = exp(dt * A[h]);
            const double *xt = x + (tok * H + h) * P;
            const double *Bt = B + (tok * G + g) * N;
            const double *Ct = C + (tok * G + g) * N;
            double *yt = y + (tok * H + h) * P;
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];
                    acc += S[p * N + n] * Ct[n];
                }
                yt[p] = acc + d_skip * xt[p];
            }
        }
        if (final_state)
            memcpy(final_state + ((size_t)s * H + h) * P * N, S, sizeof(double) * P * N);
        free(S);
    }
    free(start); free(end);
    return 0;
}

/*
 * Single-token decode: one step of the recurrence above for each batch row.
 * If conv_state is given, xBC is the raw (pre-conv) token: the window
 * [conv_state rows 0..K-2, xBC] goes through the depthwise conv + SiLU, and
 * conv_state becomes the last K-1 rows of that window.  Otherwise xBC is
 * already the post-conv x|B|C.  Channel order of xBC: x (h-major, p-minor),
 * then B (g-major, n-minor), then C.  ssm_state is updated in place.
 */
int oracle_decode_step(int batch, int H, int P, int N, int G, int K,
                       const double *xBC, const double *dt_raw,
                       const double *dt_bias, const double *A, const double *D,
                       const double *conv_w, const double *conv_bias,
                       double *conv_state, double *ssm_state, double *y) {
    if (batch < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    if (conv_state && (!conv_w || K < 1)) return -1;
    const int CH = H * P + 2 * G * N;
    const int heads_per_group = H / G;
    /* batch rows are independent: OpenMP only splits the row loop over
     * threads, each row with its own conv-output buffer v */
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        double *v = (double *)malloc(sizeof(double) * CH);
        const double *tok = xBC + (size_t)b * CH;
        if (conv_state) {
            double *cs = conv_state + (size_t)b * (K - 1) * CH;
            for (int c = 0; c < CH; ++c) {
                double u = conv_bias ? conv_bias[c] : 0.0;
                for (int k = 0; k < K; ++k) {
                    double win = (k < K - 1) ? cs[(size_t)k * CH + c] : tok[c];
                    u += conv_w[(size_t)c * K + k] * win;
                }
                v[c] = silu(u);
            }
            /* shift: drop the oldest row, append the new raw token */
            for (int c = 0; c < CH; ++c) {
                for (int r = 0; r + 1 < K - 1; ++r)
                    cs[(size_t)r * CH + c] = cs[(size_t)(r + 1) * CH + c];
                if (K > 1) cs[(size_t)(K - 2) * CH + c] = tok[c];
            }
        } else {
            memcpy(v, tok, sizeof(double) * CH);
        }
        const double *xv = v;
        const double *Bv = v + H * P;
        const double *Cv = v + H * P + G * N;
        for (int h = 0; h < H; ++h) {
            const int g = h / heads_per_group;
            const double dt = softplus(dt_raw[(size_t)b * H + h] + (dt_bias ? dt_bias[h] : 0.0));
            const double a = exp(dt * A[h]);
            double *S = ssm_state + ((size_t)b * H + h) * P * N;
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    S[p * N + n] = a * S[p * N + n] + dt * xv[h * P + p] * Bv[g * N + n];
                    acc += S[p * N + n] * Cv[g * N + n];
                }
                y[((size_t)b * H + h) * P + p] = acc + (D ? D[h] : 0.0) * xv[h * P + p];
            }
        }
        free(v);
    }
    return 0;
}

/*
 * The mixer's linear projections: in_proj maps each token's d_model
 * features to the conv input x|B|C, the gate z and dt; out_proj maps the
 * gated, normalised y back to d_model ("Nemotron-H style Hybrid
 * Mamba-Transformer 3B feasibility study", the projection parameters of the
 * Mamba-2 block; "Nemotron-Mamba3 architecture" article, sec. 2.2, the
 * layer's projections around the conv and scan).  Both are the plain
 * product with a weight stored like a torch Linear weight, (out, in):
 *   y[m][n] = sum_k x[m][k] * w[n][k]
 * Layouts: x (M, K), w (N, K), y (M, N), row-major.
 */
int oracle_linear(int M, int N, int K, const double *x, const double *w, double *y) {
    if (M < 0 || N < 0 || K < 0 || (M > 0 && N > 0 && (!x || !w || !y))) return -1;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += x[(size_t)m * K + k] * w[(size_t)n * K + k];
            y[(size_t)m * N + n] = acc;
        }
    return 0;
}

/*
 * Gated RMSNorm of the mixer output.  Mamba-2 keeps an RMSNorm together
 * with the output gate z; where the norm sits relative to the gate and
 * whether it is taken per group of channels or over the whole width are
 * model choices ("Mamba-3: an inference-first state space model": the
 * normalization paragraph, which keeps Mamba-2's RMSNorm in hybrid models,
 * and the later remark on the norm's position before or after the gate and
 * its grouped or plain type).  With SiLU(u) = u / (1 + e^-u) and, for each
 * token row and each group of group_size consecutive channels,
 * rms(v) = sqrt(mean over the group of v^2 + eps):
 *   norm after the gate (norm_before_gate = 0):
 *       g = y * SiLU(z);   out = g / rms(g) * w
 *   norm before the gate (norm_before_gate = 1):
 *       out = y / rms(y) * w * SiLU(z)
 * z may be NULL (no gate: out = y / rms(y) * w).
 * Layouts: y, z, out (T, CH) row-major; w (CH); CH a multiple of group_size.
 */
int oracle_gated_rmsnorm(int T, int CH, int group_size, int norm_before_gate,
                         double eps, const double *y, const double *z,
                         const double *w, double *out) {
    if (T < 0 || CH < 1 || group_size < 1 || CH % group_size != 0 || eps < 0.0) return -1;
    const int ngroups = CH / group_size;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int gi = 0; gi < ngroups; ++gi) {
            const size_t base = (size_t)t * CH + (size_t)gi * group_size;
            double ss = 0.0;
            for (int c = 0; c < group_size; ++c) {
                double v = y[base + c];
                if (z && !norm_before_gate) v *= silu(z[base + c]);
                ss += v * v;
            }
            const double rms = sqrt(ss / group_size + eps);
            for (int c = 0; c < group_size; ++c) {
                double v = y[base + c];
                if (z && !norm_before_gate) v *= silu(z[base + c]);
                double o = v / rms * w[(size_t)gi * group_size + c];
                if (z && norm_before_gate) o *= silu(z[base + c]);
                out[base + c] = o;
            }
        }
    }
    return 0;
}

/*
 * MIMO decode step (Mamba-3's multi-input multi-output SSM, optionally with
 * an exponential-trapezoidal input term), one token for every batch row.
 *
 * "Mamba-3: an inference-first state space model" lists the changes: a more
 * general recurrence derived from an exponential-trapezoidal
 * discretization, and MIMO in place of SISO, whose projection widens B and
 * C to the representation the MIMO SSM needs and adds parallel work to each
 * update at almost no extra decode cost.  The page gives no formulas; this
 * is the plainest reading, which reduces to the Mamba-2 step at R = 1 with
 * the Euler form:
 *   per head h (group g = h / (H/G)), rank R, state S (P x N):
 *     dt = softplus(dt_raw + dt_bias[h]),  a = exp(dt A[h])
 *     Euler:        S <- a S + dt X B^T
 *     trapezoidal:  S <- a S + (1 - lam) dt a Xp Bp^T + lam dt X B^T
 *     Y = S C + D[h] X                      (P x R)
 *   with X (P x R) the head's input, B, C (N x R) the group's, and Xp, Bp the
 *   previous token's X and B (kept as decode state, then replaced by X, B).
 *   lam in [0, 1] per (row, head); lam = 1/2 is the trapezoid rule, lam = 1
 *   the Euler form.  The previous-input term is the rule's weight on the
 *   left end of the step, carried through the step's decay.
 * Layouts (row-major, contiguous): x, y, prev_x (batch, H, P, R);
 * B, C, prev_B (batch, G, N, R); dt_raw, lam (batch, H); state
 * (batch, H, P, N).  lam NULL = 1/2.  prev_x / prev_B are read and replaced
 * only when trapezoid != 0.
 */
int oracle_decode_step_mimo(int batch, int H, int P, int N, int G, int R, int trapezoid,
                            const double *x, const double *B, const double *C,
                            const double *dt_raw, const double *lam,
                            const double *dt_bias, const double *A, const double *D,
                            double *ssm_state, double *prev_x, double *prev_B, double *y) {
    if (batch < 1 || H < 1 || P < 1 || N < 1 || G < 1 || R < 1 || H % G != 0) return -1;
    if (trapezoid && (!prev_x || !prev_B)) return -1;
    const int heads_per_group = H / G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / heads_per_group;
            const double dt = softplus(dt_raw[(size_t)b * H + h] + (dt_bias ? dt_bias[h] : 0.0));
            const double a = exp(dt * A[h]);
            const double l = trapezoid ? (lam ? lam[(size_t)b * H + h] : 0.5) : 1.0;
            const double *X = x + ((size_t)b * H + h) * P * R;
            const double *Bm = B + ((size_t)b * G + g) * N * R;
            const double *Cm = C + ((size_t)b * G + g) * N * R;
            const double *Xp = trapezoid ? prev_x + ((size_t)b * H + h) * P * R : NULL;
            const double *Bp = trapezoid ? prev_B + ((size_t)b * G + g) * N * R : NULL;
            double *S = ssm_state + ((size_t)b * H + h) * P * N;
            for (int p = 0; p < P; ++p) {
                for (int n = 0; n < N; ++n) {
                    double cur = 0.0, prev = 0.0;
                    for (int r = 0; r < R; ++r) {
                        cur += X[p * R + r] * Bm[n * R + r];
                        if (trapezoid) prev += Xp[p * R + r] * Bp[n * R + r];
                    }
                    S[p * N + n] = a * S[p * N + n] + l * dt * cur + (1.0 - l) * dt * a * prev;
                }
                for (int r = 0; r < R; ++r) {
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n) acc += S[p * N + n] * Cm[n * R + r];
                    y[(((size_t)b * H + h) * P + p) * R + r] = acc + (D ? D[h] : 0.0) * X[p * R + r];
                }
            }
        }
    }
    if (trapezoid) {
        /* the new token's inputs become the previous ones (after every read) */
        memcpy(prev_x, x, sizeof(double) * (size_t)batch * H * P * R);
        memcpy(prev_B, B, sizeof(double) * (size_t)batch * G * N * R);
    }
    return 0;
}

/*
 * Backward pass of the selective scan (reverse mode of the recurrence in
 * oracle_ssd_scan), batch rows only.  The training workload of the same
 * layer needs the gradients of every input ("Nemotron-H style Hybrid
 * Mamba-Transformer 3B feasibility study": sec. 3.1, its table row on
 * forward/backward verification, and the Phase 2 plan of sec. 7).
 *
 * Forward, per (row, head), g = h / (H/G):
 *   dt_t = softplus(z_t), z_t = dt_raw[t] + dt_bias[h],  a_t = exp(dt_t A[h])
 *   S_t  = a_t S_{t-1} + dt_t x_t B_t^T       (S_{-1} = initial_state or 0)
 *   y_t  = S_t C_t + D[h] x_t
 * Given dy (and d_final = dL/dS_{L-1}, or 0), with Gt = dL/dS_t accumulated
 * from the last token backwards:
 *   Gt  += dy_t C_t^T
 *   dC_t += S_t^T dy_t                   dD += dy_t . x_t
 *   dx_t  = D dy_t + dt_t Gt B_t          dB_t += dt_t Gt^T x_t
 *   ddt_t = x_t^T Gt B_t + A a_t <Gt, S_{t-1}>
 *   dA   += dt_t a_t <Gt, S_{t-1}>
 *   dz_t  = ddt_t sigmoid(z_t)            (d/dz softplus = sigmoid)
 *   ddt_raw_t = dz_t,  ddt_bias += dz_t
 *   G_{t-1} = a_t Gt                      dh0 = G_{-1}
 * dB and dC sum over the heads of a group.  The forward states are
 * recomputed from checkpoints every 64 tokens (the same operations as the
 * forward sweep, so S_t is bit-identical to oracle_ssd_scan's).
 * Outputs (all overwritten): dx (batch,L,H,P), ddt_raw (batch,L,H),
 * dB, dC (batch,L,G,N), ddt_bias, dA, dD (H), dh0 (batch,H,P,N) or NULL.
 */
int oracle_ssd_scan_bwd(int batch, int L, int H, int P, int N, int G,
                        const double *x, const double *dt_raw,
                        const double *dt_bias, const double *A,
                        const double *B, const double *C, const double *D,
                        const double *initial_state, const double *dy,
                        const double *d_final,
                        double *dx, double *ddt_raw, double *dB, double *dC,
                        double *ddt_bias, double *dA, double *dD, double *dh0) {
    if (batch < 1 || L < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    const int heads_per_group = H / G;
    const int K = 64;                                   /* checkpoint interval */
    const int nck = (L + K - 1) / K;
    const size_t PN = (size_t)P * N;
    memset(dB, 0, sizeof(double) * (size_t)batch * L * G * N);
    memset(dC, 0, sizeof(double) * (size_t)batch * L * G * N);
    /* per-(row, head) partial sums, reduced in a fixed order afterwards */
    double *pdA = (double *)calloc((size_t)batch * H, sizeof(double));
    double *pdD = (double *)calloc((size_t)batch * H, sizeof(double));
    double *pdb = (double *)calloc((size_t)batch * H, sizeof(double));
    /* per-(row, head) dB / dC contributions: (batch, H, L, N) */
    double *hB = (double *)calloc((size_t)batch * H * L * N, sizeof(double));
    double *hC = (double *)calloc((size_t)batch * H * L * N, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (long long unit = 0; unit < (long long)batch * H; ++unit) {
        const int b = (int)(unit / H), h = (int)(unit % H);
        const int g = h / heads_per_group;
        const double bias = dt_bias ? dt_bias[h] : 0.0;
        const double dsk = D ? D[h] : 0.0;
        double *ck = (double *)malloc(sizeof(double) * PN * (nck + 1));   /* S before each block */
        double *blk = (double *)malloc(sizeof(double) * PN * (K + 1));    /* S_{t0-1} .. S_{t0+K-1} */
        double *Gt = (double *)malloc(sizeof(double) * PN);
        double *S = (double *)malloc(sizeof(double) * PN);
        if (initial_state) memcpy(S, initial_state + ((size_t)b * H + h) * PN, sizeof(double) * PN);
        else memset(S, 0, sizeof(double) * PN);
        /* forward sweep: checkpoints */
        for (int t = 0; t < L; ++t) {
            if (t % K == 0) memcpy(ck + PN * (t / K), S, sizeof(double) * PN);
            const size_t tok = (size_t)b * L + t;
            const double dt = softplus(dt_raw[tok * H + h] + bias);
            const double a = exp(dt * A[h]);
            const double *xt = x + (tok * H + h) * P, *Bt = B + (tok * G + g) * N;
            for (int p = 0; p < P; ++p)
                for (int n = 0; n < N; ++n) S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bt[n];
        }
        if (d_final) memcpy(Gt, d_final + ((size_t)b * H + h) * PN, sizeof(double) * PN);
        else memset(Gt, 0, sizeof(double) * PN);
        double accA = 0.0, accD = 0.0, accb = 0.0;
        for (int c = nck - 1; c >= 0; --c) {
            const int t0 = c * K, t1 = (t0 + K < L) ? t0 + K : L;
            /* recompute S_{t0-1} .. S_{t1-1} into blk[0 .. t1-t0] */
            memcpy(blk, ck + PN * c, sizeof(double) * PN);
            for (int t = t0; t < t1; ++t) {
                const size_t tok = (size_t)b * L + t;
                const double dt = softplus(dt_raw[tok * H + h] + bias);
                const double a = exp(dt * A[h]);
                const double *xt = x + (tok * H + h) * P, *Bt = B + (tok * G + g) * N;
                const double *Sp = blk + PN * (t - t0);
                double *Sn = blk + PN * (t - t0 + 1);
                for (int p = 0; p < P; ++p)
                    for (int n = 0; n < N; ++n) Sn[p * N + n] = a * Sp[p * N + n] + dt * xt[p] * Bt[n];
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const size_t tok = (size_t)b * L + t;
                const double z = dt_raw[tok * H + h] + bias;
                const double dt = softplus(z);
                const double a = exp(dt * A[h]);
                const double *xt = x + (tok * H + h) * P, *Bt = B + (tok * G + g) * N;
                const double *Ct = C + (tok * G + g) * N, *dyt = dy + (tok * H + h) * P;
                const double *St = blk + PN * (t - t0 + 1), *Sp = blk + PN * (t - t0);
                double *dxt = dx + (tok * H + h) * P;
                double *hBt = hB + (((size_t)b * H + h) * L + t) * N;
                double *hCt = hC + (((size_t)b * H + h) * L + t) * N;
                for (int p = 0; p < P; ++p)
                    for (int n = 0; n < N; ++n) Gt[p * N + n] += dyt[p] * Ct[n];
                for (int n = 0; n < N; ++n) {
                    double s = 0.0;
                    for (int p = 0; p < P; ++p) s += St[p * N + n] * dyt[p];
                    hCt[n] = s;
                }
                double gs = 0.0, xgb = 0.0;
                for (int p = 0; p < P; ++p) {
                    accD += dyt[p] * xt[p];
                    double gb = 0.0;
                    for (int n = 0; n < N; ++n) {
                        gb += Gt[p * N + n] * Bt[n];
                        gs += Gt[p * N + n] * Sp[p * N + n];
                    }
                    dxt[p] = dsk * dyt[p] + dt * gb;
                    xgb += xt[p] * gb;
                }
                for (int n = 0; n < N; ++n) {
                    double s = 0.0;
                    for (int p = 0; p < P; ++p) s += Gt[p * N + n] * xt[p];
                    hBt[n] = dt * s;
                }
                const double ddt = xgb + A[h] * a * gs;
                accA += dt * a * gs;
                const double dz = ddt / (1.0 + exp(-z));
                ddt_raw[tok * H + h] = dz;
                accb += dz;
                for (size_t e = 0; e < PN; ++e) Gt[e] *= a;
            }
        }
        if (dh0) memcpy(dh0 + ((size_t)b * H + h) * PN, Gt, sizeof(double) * PN);
        pdA[unit] = accA;
        pdD[unit] = accD;
        pdb[unit] = accb;
        free(ck); free(blk); free(Gt); free(S);
    }
    for (int h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0, sb = 0.0;
        for (int b = 0; b < batch; ++b) {
            sa += pdA[(size_t)b * H + h];
            sd += pdD[(size_t)b * H + h];
            sb += pdb[(size_t)b * H + h];
        }
        dA[h] = sa;
        if (dD) dD[h] = sd;
        if (ddt_bias) ddt_bias[h] = sb;
    }
    /* dB, dC: sum over the heads of each group, in head order */
#pragma omp parallel for schedule(static)
    for (long long bt = 0; bt < (long long)batch * L; ++bt) {
        const int b = (int)(bt / L), t = (int)(bt % L);
        for (int h = 0; h < H; ++h) {
            const int g = h / heads_per_group;
            const double *sB = hB + (((size_t)b * H + h) * L + t) * N;
            const double *sC = hC + (((size_t)b * H + h) * L + t) * N;
            double *oB = dB + (((size_t)b * L + t) * G + g) * N;
            double *oC = dC + (((size_t)b * L + t) * G + g) * N;
            for (int n = 0; n < N; ++n) { oB[n] += sB[n]; oC[n] += sC[n]; }
        }
    }
    free(pdA); free(pdD); free(pdb); free(hB); free(hC);
    return 0;
}
