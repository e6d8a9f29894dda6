"""Test-only fp64 forms of the SSD layer that do NOT share the oracle's code.

They pin the sequential oracle from other directions:

* `quadratic_form`: the "state space duality" view -- the whole causal
  sequence map as one masked matrix, y = (Lmask o C B^T) (dt x) + D x,
  with Lmask[i, j] = exp(sum_{k=j+1..i} dt_k A) for j <= i ("AI Engineering
  EP6", sec. 8 and sec. 10: SSD is mathematically equivalent to (linear)
  attention).  The input scale dt_j and the skip term D x belong to the
  layer's recurrence, so they appear here too.
* `chunked`: the block decomposition the GPU uses (chunk cumsum, intra-chunk
  quadratic block, chunk states, inter-chunk state passing, state->output),
  evaluated in fp64 for any chunk size Q.
* `fir_conv_silu`: the depthwise causal conv as a scipy FIR filter.

softplus here is numpy's logaddexp(0, z); nothing is imported from oracle/.
"""
import numpy as np
from scipy.signal import lfilter
from scipy.special import expit


def softplus(z):
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def _groups(H, G):
    return np.arange(H) // (H // G)


def quadratic_form(x, dt_raw, dt_bias, A, B, C, D, h0=None):
    """One sequence: x (L,H,P), dt_raw (L,H), B/C (L,G,N), h0 (H,P,N) or None."""
    x = np.asarray(x, np.float64)
    L, H, P = x.shape
    G = B.shape[1]
    g_of = _groups(H, G)
    dt = softplus(np.asarray(dt_raw, np.float64) + np.asarray(dt_bias, np.float64)[None, :])
    y = np.zeros((L, H, P))
    tril = np.tril(np.ones((L, L), bool))
    for h in range(H):
        g = g_of[h]
        c = np.cumsum(dt[:, h] * np.float64(A[h]))          # c_t = sum_{k<=t} dt_k A
        seg = c[:, None] - c[None, :]                        # sum_{k=j+1..i} dt_k A
        Lm = np.where(tril, np.exp(np.where(tril, seg, 0.0)), 0.0)
        CB = np.asarray(C[:, g, :], np.float64) @ np.asarray(B[:, g, :], np.float64).T
        y[:, h, :] = (Lm * CB) @ (dt[:, h:h + 1] * x[:, h, :]) + np.float64(D[h]) * x[:, h, :]
        if h0 is not None:
            # contribution of the entering state, decayed through token i inclusive
            y[:, h, :] += np.exp(c)[:, None] * (np.asarray(C[:, g, :], np.float64)
                                                 @ np.asarray(h0[h], np.float64).T)
    return y


def chunked(x, dt_raw, dt_bias, A, B, C, D, Q, h0=None):
    """Chunked SSD evaluation of one sequence in fp64.  Returns (y, final_state)."""
    x = np.asarray(x, np.float64)
    L, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    g_of = _groups(H, G)
    dt = softplus(np.asarray(dt_raw, np.float64) + np.asarray(dt_bias, np.float64)[None, :])
    y = np.zeros((L, H, P))
    finals = np.zeros((H, P, N))
    for h in range(H):
        g = g_of[h]
        state = np.zeros((P, N)) if h0 is None else np.array(h0[h], np.float64)
        for c0 in range(0, L, Q):
            c1 = min(L, c0 + Q)
            n = c1 - c0
            xc = x[c0:c1, h, :]
            Bc = np.asarray(B[c0:c1, g, :], np.float64)
            Cc = np.asarray(C[c0:c1, g, :], np.float64)
            dtc = dt[c0:c1, h]
            cs = np.cumsum(dtc * np.float64(A[h]))            # inclusive, within chunk
            # intra-chunk (diagonal block)
            diff = cs[:, None] - cs[None, :]
            mask = np.tril(np.ones((n, n), bool))
            M = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0) * (Cc @ Bc.T) * dtc[None, :]
            y_diag = M @ xc
            # state entering the chunk -> output
            y_off = np.exp(cs)[:, None] * (Cc @ state.T)
            y[c0:c1, h, :] = y_diag + y_off + np.float64(D[h]) * xc
            # chunk state and inter-chunk passing
            w = np.exp(cs[-1] - cs) * dtc
            S_c = (xc * w[:, None]).T @ Bc                    # (P, N)
            state = np.exp(cs[-1]) * state + S_c
        finals[h] = state
    return y, finals


def fir_conv_silu(x, w, bias=None):
    """Depthwise causal conv as an FIR filter per channel, then SiLU.

    x (L, CH), w (CH, K) with w[:, K-1] on the newest token, zero left padding.
    """
    x = np.asarray(x, np.float64)
    L, CH = x.shape
    K = w.shape[1]
    u = np.zeros((L, CH))
    for c in range(CH):
        u[:, c] = lfilter(np.asarray(w[c, ::-1], np.float64), [1.0], x[:, c])
    if bias is not None:
        u += np.asarray(bias, np.float64)[None, :]
    return u * expit(u)


def rel_err(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(a - ref))) if a.size else 0.0
    return float(np.max(np.abs(a - ref)) / denom)
