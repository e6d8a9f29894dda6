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
    double *v = (double *)malloc(sizeof(double) * CH);
    for (int b = 0; b < batch; ++b) {
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
    }
    free(v);
    return 0;
}
