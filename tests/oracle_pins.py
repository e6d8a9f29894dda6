"""Pins of the fp64 oracle against things other than itself.

Each `pin_*` takes a loaded oracle library (the real one, or a mutant built
from an edited copy of its source) and raises AssertionError when the
oracle disagrees with the independent fact it is pinned to.  The pins are
run on the real oracle by test_oracle_pins.py and on planted mistakes by
test_oracle_mutants.py (every mutant must fail at least one pin).
"""
import numpy as np

import oracle
from tests.ssd_forms import chunked, fir_conv_silu, quadratic_form, rel_err, softplus


def _rand(seed, H, P, N, G, L, init=False):
    r = np.random.default_rng(seed)
    d = {
        "x": r.standard_normal((1, L, H, P)),
        "dt": r.standard_normal((1, L, H)),
        "dt_bias": np.log(np.expm1(np.exp(r.uniform(np.log(1e-2), np.log(0.5), H)))),
        "A": -np.exp(r.uniform(0, np.log(16), H)),
        "B": r.standard_normal((1, L, G, N)) / np.sqrt(N),
        "C": r.standard_normal((1, L, G, N)) / np.sqrt(N),
        "D": r.standard_normal(H),
    }
    if init:
        d["h0"] = r.standard_normal((1, H, P, N)) * 0.3
    return d


def _scan(lib, d, **kw):
    return oracle.ssd_scan(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"],
                           initial_state=d.get("h0"), want_final_state=True, lib=lib, **kw)


def pin_quadratic_form(lib):
    """Whole map == masked quadratic form (mask orientation, L_ii = 1, groups, D)."""
    for seed, (H, P, N, G, L) in enumerate([(4, 3, 5, 2, 37), (2, 8, 16, 1, 64),
                                            (6, 4, 7, 3, 19)]):
        for init in (False, True):
            d = _rand(seed, H, P, N, G, L, init)
            y, _ = _scan(lib, d)
            ref = quadratic_form(d["x"][0], d["dt"][0], d["dt_bias"], d["A"], d["B"][0],
                                 d["C"][0], d["D"], None if not init else d["h0"][0])
            assert rel_err(y[0], ref) < 1e-11, ("quadratic form", seed, init, rel_err(y[0], ref))


def pin_dt_zero(lib):
    """dt = 0 exactly (dt_raw = -inf): y = D x + C . h0 (state frozen)."""
    H, P, N, G, L = 4, 5, 6, 2, 23
    d = _rand(7, H, P, N, G, L, init=True)
    d["dt"][:] = -np.inf
    y, fs = _scan(lib, d)
    g_of = np.arange(H) // (H // G)
    expect = d["D"][None, :, None] * d["x"][0]
    for h in range(H):
        expect[:, h, :] += d["C"][0][:, g_of[h], :] @ d["h0"][0][h].T
    assert np.max(np.abs(y[0] - expect)) <= 1e-13 * max(1.0, np.max(np.abs(expect))), "dt=0 D path"
    assert np.array_equal(fs, d["h0"]), "dt=0 must freeze the state"


def pin_softplus_large_argument(lib):
    """dt_raw + dt_bias far above 30 (the oracle's overflow-safe softplus branch)
    and just below it: with one token, zero state and P = N = 1,
    y = C dt x B + D x gives dt back, which must equal numpy's logaddexp(0, z).
    A two-head, many-token run against the masked quadratic form follows."""
    z = np.array([45.0, 38.5, 31.0, 30.0, 29.5, 12.0, -3.0])
    for zi in z:
        for bias in (0.0, 40.0, -10.0):
            d = {"x": np.full((1, 1, 1, 1), 1.5), "dt": np.full((1, 1, 1), zi - bias),
                 "dt_bias": np.array([bias]), "A": np.array([-0.7]), "B": np.full((1, 1, 1, 1), 0.5),
                 "C": np.full((1, 1, 1, 1), -2.0), "D": np.array([0.25])}
            y, fs = _scan(lib, d)
            dt = (y[0, 0, 0, 0] - 0.25 * 1.5) / (-2.0 * 1.5 * 0.5)
            assert abs(dt - softplus(zi)) <= 1e-14 * max(1.0, softplus(zi)), ("softplus", zi, bias, dt)
            assert abs(fs[0, 0, 0, 0] - softplus(zi) * 1.5 * 0.5) <= 1e-14 * max(1.0, softplus(zi))
    H, P, N, G, L = 2, 3, 4, 1, 25
    d = _rand(71, H, P, N, G, L)
    d["dt_bias"] = np.array([40.0, 28.0])
    d["A"] = np.array([-1e-3, -2e-3])
    y, _ = _scan(lib, d)
    assert np.all(d["dt"][0, :, 0] + 40.0 > 30.0)
    ref = quadratic_form(d["x"][0], d["dt"][0], d["dt_bias"], d["A"], d["B"][0], d["C"][0], d["D"])
    assert rel_err(y[0], ref) < 1e-11, ("large dt quadratic form", rel_err(y[0], ref))


def pin_linear_attention(lib):
    """A = 0: causal linear attention y_i = sum_{j<=i} (C_i.B_j) dt_j x_j + D x_i,
    computed as a running sum of outer products."""
    H, P, N, G, L = 4, 3, 4, 2, 29
    d = _rand(11, H, P, N, G, L)
    d["A"] = np.zeros(H)
    y, _ = _scan(lib, d)
    dt = softplus(d["dt"][0] + d["dt_bias"][None, :])
    g_of = np.arange(H) // (H // G)
    ref = np.zeros((L, H, P))
    for h in range(H):
        kv = np.cumsum(np.einsum("t,tp,tn->tpn", dt[:, h], d["x"][0][:, h, :],
                                 d["B"][0][:, g_of[h], :]), axis=0)
        ref[:, h, :] = np.einsum("tpn,tn->tp", kv, d["C"][0][:, g_of[h], :]) \
            + d["D"][h] * d["x"][0][:, h, :]
    assert rel_err(y[0], ref) < 1e-12, ("A=0", rel_err(y[0], ref))


def pin_instant_forget(lib):
    """A -> -inf (a = 0 exactly in fp64): only the diagonal term survives."""
    H, P, N, G, L = 4, 3, 4, 4, 17
    d = _rand(13, H, P, N, G, L, init=True)
    d["A"] = np.full(H, -1e6)
    y, fs = _scan(lib, d)
    dt = softplus(d["dt"][0] + d["dt_bias"][None, :])
    ref = np.zeros((L, H, P))
    for h in range(H):
        cb = np.sum(d["C"][0][:, h, :] * d["B"][0][:, h, :], axis=1)
        ref[:, h, :] = (dt[:, h] * cb)[:, None] * d["x"][0][:, h, :] + d["D"][h] * d["x"][0][:, h, :]
    assert rel_err(y[0], ref) < 1e-12, ("A=-inf", rel_err(y[0], ref))


def pin_iir_filter(lib):
    """H=P=N=G=1, constant dt, B, C: a first-order IIR filter (scipy lfilter)."""
    L = 50
    r = np.random.default_rng(17)
    x = r.standard_normal(L)
    zraw, bias, A, Bv, Cv, Dv = 0.3, -1.1, -2.5, 0.7, -1.3, 0.4
    d = {"x": x.reshape(1, L, 1, 1), "dt": np.full((1, L, 1), zraw), "dt_bias": np.array([bias]),
         "A": np.array([A]), "B": np.full((1, L, 1, 1), Bv), "C": np.full((1, L, 1, 1), Cv),
         "D": np.array([Dv])}
    y, _ = _scan(lib, d)
    dt = float(softplus(zraw + bias))
    a = np.exp(dt * A)
    from scipy.signal import lfilter
    ref = Cv * lfilter([dt * Bv], [1.0, -a], x) + Dv * x
    assert rel_err(y[0, :, 0, 0], ref) < 1e-13, ("lfilter", rel_err(y[0, :, 0, 0], ref))


def pin_chunk_invariance(lib):
    """Chunked fp64 evaluation at many chunk sizes (incl. non-divisors) == oracle."""
    H, P, N, G, L = 4, 5, 8, 2, 130
    d = _rand(19, H, P, N, G, L, init=True)
    y, fs = _scan(lib, d)
    for Q in (1, 3, 7, 16, 64, 128, L):
        yc, fc = chunked(d["x"][0], d["dt"][0], d["dt_bias"], d["A"], d["B"][0], d["C"][0],
                         d["D"], Q, d["h0"][0])
        assert rel_err(y[0], yc) < 1e-11, ("chunk", Q, rel_err(y[0], yc))
        assert rel_err(fs[0], fc) < 1e-11, ("chunk state", Q, rel_err(fs[0], fc))


def pin_superposition(lib):
    """y(x, h0) = y(x, 0) + y(0, h0), and y(2x, 0) = 2 y(x, 0)."""
    H, P, N, G, L = 4, 3, 5, 2, 31
    d = _rand(23, H, P, N, G, L, init=True)
    y_full, f_full = _scan(lib, d)
    d0 = dict(d)
    d0["h0"] = None
    y_x, f_x = _scan(lib, d0)
    dz = dict(d)
    dz["x"] = np.zeros_like(d["x"])
    y_h, f_h = _scan(lib, dz)
    assert rel_err(y_full, y_x + y_h) < 1e-12, "superposition"
    assert rel_err(f_full, f_x + f_h) < 1e-12, "state superposition"
    d2 = dict(d0)
    d2["x"] = 2.0 * d["x"]
    y2, _ = _scan(lib, d2)
    assert rel_err(y2, 2.0 * y_x) < 1e-13, "linearity in x"


def pin_packed_equals_separate(lib):
    """Packed sequences (seq_idx) == each sequence run on its own with its h0."""
    H, P, N, G = 4, 3, 6, 2
    lens = [5, 1, 12, 7, 3]
    L = sum(lens)
    d = _rand(29, H, P, N, G, L)
    r = np.random.default_rng(31)
    h0 = r.standard_normal((len(lens), H, P, N)) * 0.3
    seq_idx = np.repeat(np.arange(len(lens)), lens)
    y, fs = oracle.ssd_scan(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"],
                            seq_idx=seq_idx, initial_state=h0, want_final_state=True,
                            num_seqs=len(lens), lib=lib)
    o = 0
    for s, n in enumerate(lens):
        sl = slice(o, o + n)
        ref = quadratic_form(d["x"][0, sl], d["dt"][0, sl], d["dt_bias"], d["A"], d["B"][0, sl],
                             d["C"][0, sl], d["D"], h0[s])
        assert rel_err(y[0, sl], ref) < 1e-11, ("packed", s)
        _, fc = chunked(d["x"][0, sl], d["dt"][0, sl], d["dt_bias"], d["A"], d["B"][0, sl],
                        d["C"][0, sl], d["D"], 4, h0[s])
        assert rel_err(fs[s], fc) < 1e-11, ("packed final", s)
        o += n


def pin_split_continuation(lib):
    """run[0:s] -> final_state -> run[s:L] from it == run[0:L] (y and state)."""
    H, P, N, G, L, s = 4, 4, 6, 2, 41, 17
    d = _rand(37, H, P, N, G, L, init=True)
    y, fs = _scan(lib, d)
    a = {k: (v[:, :s] if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    ya, fa = _scan(lib, a)
    b = {k: (v[:, s:] if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    b["h0"] = fa
    yb, fb = _scan(lib, b)
    assert rel_err(np.concatenate([ya, yb], axis=1), y) < 1e-12, "split y"
    assert rel_err(fb, fs) < 1e-12, "split final state"


def pin_head_permutation(lib):
    """Permuting heads inside a group (with their dt, A, D) permutes y."""
    H, P, N, G, L = 6, 3, 4, 2, 21
    d = _rand(41, H, P, N, G, L)
    y, _ = _scan(lib, d)
    perm = np.array([2, 0, 1, 4, 5, 3])            # stays inside groups {0,1,2}, {3,4,5}
    dp = dict(d)
    dp["x"] = d["x"][:, :, perm]
    dp["dt"] = d["dt"][:, :, perm]
    dp["dt_bias"], dp["A"], dp["D"] = d["dt_bias"][perm], d["A"][perm], d["D"][perm]
    yp, _ = _scan(lib, dp)
    assert rel_err(yp, y[:, :, perm]) < 1e-14, "head permutation"


def pin_state_decay(lib):
    """x = 0 with A < 0, dt > 0: the state norm never grows; it shrinks by exactly
    exp(sum dt A) (the product of the per-token decays)."""
    H, P, N, G, L = 2, 3, 4, 1, 12
    d = _rand(43, H, P, N, G, L, init=True)
    d["x"][:] = 0.0
    prev = np.linalg.norm(d["h0"][0], axis=(1, 2))
    dt = softplus(d["dt"][0] + d["dt_bias"][None, :])
    for t in range(1, L + 1):
        a = {k: (v[:, :t] if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
        _, fs = _scan(lib, a)
        cur = np.linalg.norm(fs[0], axis=(1, 2))
        assert np.all(cur <= prev * (1 + 1e-15)), "state norm grew with x = 0"
        expect = np.linalg.norm(d["h0"][0], axis=(1, 2)) * np.exp(np.sum(dt[:t] * d["A"], axis=0))
        assert np.allclose(cur, expect, rtol=1e-12, atol=0), "decay product"
        prev = cur


def pin_conv_fir(lib):
    """conv + SiLU == scipy FIR filter per channel + expit, with and without bias."""
    r = np.random.default_rng(47)
    for bias in (None, r.standard_normal(12)):
        x = r.standard_normal((2, 33, 12))
        w = r.standard_normal((12, 4)) * 0.5
        out = oracle.conv1d_silu(x, w, bias=bias, lib=lib)
        for b in range(2):
            ref = fir_conv_silu(x[b], w, bias)
            assert rel_err(out[b], ref) < 1e-13, "conv FIR"


def pin_conv_packed_and_state(lib):
    """Packed conv == per-sequence conv; state handoff: conv[0:s] -> state -> conv[s:L]
    == conv[0:L], and the state rows are the last 3 raw inputs."""
    r = np.random.default_rng(53)
    CH = 10
    w = r.standard_normal((CH, 4)) * 0.5
    lens = [6, 2, 9, 1]
    x = r.standard_normal((1, sum(lens), CH))
    seq_idx = np.repeat(np.arange(len(lens)), lens)
    out = oracle.conv1d_silu(x, w, seq_idx=seq_idx, num_seqs=len(lens), lib=lib)
    o = 0
    for n in lens:
        assert rel_err(out[0, o:o + n], fir_conv_silu(x[0, o:o + n], w)) < 1e-13, "packed conv"
        o += n
    L, s = 23, 9
    x = r.standard_normal((2, L, CH))
    full = oracle.conv1d_silu(x, w, lib=lib)
    a, st = oracle.conv1d_silu(x[:, :s], w, want_state_out=True, lib=lib)
    assert np.array_equal(st, x[:, s - 3:s]), "conv state = last 3 raw rows"
    b = oracle.conv1d_silu(x[:, s:], w, conv_state_in=st, lib=lib)
    assert rel_err(np.concatenate([a, b], axis=1), full) < 1e-14, "conv continuation"
    # a sequence shorter than 3 tokens keeps part of the incoming state
    c, st2 = oracle.conv1d_silu(x[:, s:s + 2], w, conv_state_in=st, want_state_out=True, lib=lib)
    assert np.array_equal(st2[:, 0], st[:, 2]) and np.array_equal(st2[:, 1:], x[:, s:s + 2]), \
        "short-sequence conv state"


def pin_prefill_then_decode(lib):
    """prefill(L) (conv + scan, states out) then decode(token L) == prefill(L+1)."""
    H, P, N, G, L = 4, 3, 5, 2, 19
    r = np.random.default_rng(59)
    CH = H * P + 2 * G * N
    xBC = r.standard_normal((1, L + 1, CH)) * 0.7
    w = r.standard_normal((CH, 4)) * 0.5
    cb = r.standard_normal(CH) * 0.1
    dt = r.standard_normal((1, L + 1, H))
    dt_bias = np.log(np.expm1(np.exp(r.uniform(np.log(1e-2), np.log(0.5), H))))
    A = -np.exp(r.uniform(0, np.log(16), H))
    D = r.standard_normal(H)

    def split(v):
        xs = v[..., :H * P].reshape(*v.shape[:-1], H, P)
        Bs = v[..., H * P:H * P + G * N].reshape(*v.shape[:-1], G, N)
        Cs = v[..., H * P + G * N:].reshape(*v.shape[:-1], G, N)
        return xs, Bs, Cs

    v_full = oracle.conv1d_silu(xBC, w, bias=cb, lib=lib)
    y_full, f_full = oracle.ssd_scan(*_xd(split(v_full), dt, dt_bias, A, D), want_final_state=True,
                                     lib=lib)
    v_pre, cst = oracle.conv1d_silu(xBC[:, :L], w, bias=cb, want_state_out=True, lib=lib)
    _, f_pre = oracle.ssd_scan(*_xd(split(v_pre), dt[:, :L], dt_bias, A, D),
                               want_final_state=True, lib=lib)
    y_dec, s_dec, c_dec = oracle.decode_step(xBC[:, L], dt[:, L], dt_bias, A, D, f_pre, H, P, N,
                                             G, conv_w=w, conv_bias=cb, conv_state=cst, lib=lib)
    assert rel_err(y_dec, y_full[:, L]) < 1e-12, "decode y == prefill(L+1) last token"
    assert rel_err(s_dec, f_full) < 1e-12, "decode state == prefill(L+1) state"
    assert np.array_equal(c_dec, xBC[:, L - 2:L + 1]), "decode conv-state shift"


def _xd(xbc, dt, dt_bias, A, D):
    x, B, C = xbc
    return x, dt, dt_bias, A, B, C, D


def pin_decode_closed_form(lib):
    """Decode without conv: y = C.(a h + dt x B^T) + D x, state = a h + dt x B^T."""
    H, P, N, G, Bt = 4, 3, 5, 2, 3
    r = np.random.default_rng(61)
    CH = H * P + 2 * G * N
    v = r.standard_normal((Bt, CH))
    dt = r.standard_normal((Bt, H))
    dt_bias = r.standard_normal(H) * 0.3
    A = -np.exp(r.uniform(0, np.log(16), H))
    D = r.standard_normal(H)
    h = r.standard_normal((Bt, H, P, N))
    y, s, _ = oracle.decode_step(v, dt, dt_bias, A, D, h, H, P, N, G, lib=lib)
    x = v[:, :H * P].reshape(Bt, H, P)
    Bm = v[:, H * P:H * P + G * N].reshape(Bt, G, N)
    Cm = v[:, H * P + G * N:].reshape(Bt, G, N)
    g_of = np.arange(H) // (H // G)
    d = softplus(dt + dt_bias[None, :])
    for b in range(Bt):
        for hh in range(H):
            st = np.exp(d[b, hh] * A[hh]) * h[b, hh] + d[b, hh] * np.outer(x[b, hh], Bm[b, g_of[hh]])
            assert rel_err(s[b, hh], st) < 1e-14
            assert rel_err(y[b, hh], st @ Cm[b, g_of[hh]] + D[hh] * x[b, hh]) < 1e-13


def pin_scalar_golden(lib):
    """Hand-derived 4-token example stored in tests/golden/scalar_recurrence.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "scalar_recurrence.txt")
    rows = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split("=", 1)
        rows[k.strip()] = np.array([float(t) for t in v.split()])
    x = rows["x"]
    L = len(x)
    d = {"x": x.reshape(1, L, 1, 1), "dt": np.full((1, L, 1), rows["dt_raw"][0]),
         "dt_bias": rows["dt_bias"], "A": rows["A"], "B": np.full((1, L, 1, 1), rows["B"][0]),
         "C": np.full((1, L, 1, 1), rows["C"][0]), "D": rows["D"]}
    y, fs = _scan(lib, d)
    expect = rows["y_over_ln2"] * np.log(2.0)
    assert np.allclose(y[0, :, 0, 0], expect, rtol=1e-14, atol=1e-15), "golden y"
    assert np.isclose(fs[0, 0, 0, 0], rows["final_over_ln2"][0] * np.log(2.0), rtol=1e-14), \
        "golden final state"


# ---------------------------------------------------------------------------
# gated RMSNorm of the mixer output
# ---------------------------------------------------------------------------
def _silu(u):
    from scipy.special import expit
    return np.asarray(u, np.float64) * expit(np.asarray(u, np.float64))


def pin_norm_golden(lib):
    """One group of two channels, no gate, eps 0: y = (3, 4) has rms
    sqrt(12.5), so out = (3, 4) sqrt(2) / 5 times the weight; eps = 12.5
    doubles the mean square (out divided by sqrt 2)."""
    y = np.array([[3.0, 4.0]])
    w = np.array([2.0, -1.0])
    out = oracle.gated_rmsnorm(y, None, w, 2, eps=0.0, lib=lib)
    assert np.allclose(out, [[6.0 * np.sqrt(2) / 5, -4.0 * np.sqrt(2) / 5]], rtol=1e-15, atol=0)
    out = oracle.gated_rmsnorm(y, None, w, 2, eps=12.5, lib=lib)
    assert np.allclose(out, [[6.0 / 5, -4.0 / 5]], rtol=1e-15, atol=0)


def pin_norm_unit_rms_per_group(lib):
    """eps 0, unit weight: every group of the output has mean square 1 and
    is a positive multiple of its input group (after the gate: of y SiLU(z),
    with SiLU from scipy's expit); groups are independent of each other."""
    r = np.random.default_rng(73)
    T, CH, gs = 5, 48, 12
    y, z = r.standard_normal((T, CH)), r.standard_normal((T, CH))
    for gate in (False, True):
        out = oracle.gated_rmsnorm(y, z if gate else None, np.ones(CH), gs, eps=0.0, lib=lib)
        v = y * _silu(z) if gate else y
        for gi in range(CH // gs):
            sl = slice(gi * gs, (gi + 1) * gs)
            assert np.allclose(np.mean(out[:, sl] ** 2, axis=1), 1.0, rtol=1e-14, atol=0)
            ratio = out[:, sl] / v[:, sl]
            assert np.all(ratio > 0) and np.allclose(ratio, ratio[:, :1], rtol=1e-13, atol=0)
        # changing one group's input leaves every other group's output unchanged
        y2 = y.copy()
        y2[:, :gs] *= 3.7
        y2[:, gs:2 * gs] = r.standard_normal((T, gs))
        out2 = oracle.gated_rmsnorm(y2, z if gate else None, np.ones(CH), gs, eps=0.0, lib=lib)
        assert np.array_equal(out2[:, 2 * gs:], out[:, 2 * gs:])
        assert np.allclose(out2[:, :gs], out[:, :gs], rtol=1e-13, atol=1e-15)


def pin_norm_gate_placement(lib):
    """Before the gate the output is the plain norm of y times SiLU(z); after
    the gate a gate that is constant over a group cancels in the norm (eps 0).
    The weight multiplies channel by channel."""
    r = np.random.default_rng(79)
    T, CH, gs = 4, 32, 16
    y, z = r.standard_normal((T, CH)), r.standard_normal((T, CH))
    w = r.standard_normal(CH)
    plain = oracle.gated_rmsnorm(y, None, w, gs, eps=1e-3, lib=lib)
    before = oracle.gated_rmsnorm(y, z, w, gs, norm_before_gate=True, eps=1e-3, lib=lib)
    assert np.allclose(before, plain * _silu(z), rtol=1e-14, atol=1e-300)
    zc = np.repeat(r.standard_normal((T, CH // gs)) + 2.0, gs, axis=1)
    after = oracle.gated_rmsnorm(y, zc, w, gs, eps=0.0, lib=lib)
    plain0 = oracle.gated_rmsnorm(y, None, w, gs, eps=0.0, lib=lib)
    assert np.allclose(after, plain0 * np.sign(_silu(zc)), rtol=1e-13, atol=0)
    unit = oracle.gated_rmsnorm(y, z, np.ones(CH), gs, eps=1e-3, lib=lib)
    assert np.allclose(oracle.gated_rmsnorm(y, z, w, gs, eps=1e-3, lib=lib), unit * w[None, :],
                       rtol=1e-14, atol=1e-300)


def pin_norm_scale_and_eps(lib):
    """eps 0: the output does not change when y is scaled by c > 0 and flips
    sign with y; a zero input gives zero (no NaN) when eps > 0, and with eps
    far above the mean square the output tends to y w / sqrt(eps)."""
    r = np.random.default_rng(83)
    y, z, w = r.standard_normal((3, 64)), r.standard_normal((3, 64)), r.standard_normal(64)
    for nbg in (False, True):
        o = oracle.gated_rmsnorm(y, z, w, 64, norm_before_gate=nbg, eps=0.0, lib=lib)
        assert np.allclose(oracle.gated_rmsnorm(7.5 * y, z, w, 64, norm_before_gate=nbg, eps=0.0, lib=lib), o,
                           rtol=1e-14, atol=0)
        assert np.allclose(oracle.gated_rmsnorm(-y, z, w, 64, norm_before_gate=nbg, eps=0.0, lib=lib), -o,
                           rtol=1e-15, atol=0)
    assert np.array_equal(oracle.gated_rmsnorm(np.zeros((2, 8)), None, np.ones(8), 8, eps=1e-6, lib=lib),
                          np.zeros((2, 8)))
    small = 1e-6 * y
    o = oracle.gated_rmsnorm(small, None, w, 64, eps=1e4, lib=lib)
    assert np.allclose(o, small * w / 100.0, rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# MIMO decode step with the optional exponential-trapezoidal input term
# ---------------------------------------------------------------------------
def _mimo_rand(seed, batch, H, P, N, G, R):
    r = np.random.default_rng(seed)
    return {"x": r.standard_normal((batch, H, P, R)), "B": r.standard_normal((batch, G, N, R)) / np.sqrt(N),
            "C": r.standard_normal((batch, G, N, R)) / np.sqrt(N), "dt": r.standard_normal((batch, H)),
            "dt_bias": r.standard_normal(H) * 0.3 - 1.0, "A": -np.exp(r.uniform(0, np.log(16), H)),
            "D": r.standard_normal(H), "S": r.standard_normal((batch, H, P, N)),
            "px": r.standard_normal((batch, H, P, R)), "pB": r.standard_normal((batch, G, N, R)) / np.sqrt(N),
            "lam": r.uniform(0, 1, (batch, H))}


def _siso_decode(lib, x, B, C, dt, d, S):
    """Mamba-2 decode oracle (no conv) on one-column inputs: x (b,H,P), B/C (b,G,N)."""
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    xbc = np.concatenate([x.reshape(b, H * P), B.reshape(b, G * N), C.reshape(b, G * N)], axis=1)
    y, s, _ = oracle.decode_step(xbc, dt, d["dt_bias"], d["A"], d["D"], S, H, P, N, G, lib=lib)
    return y, s


def pin_mimo_rank1_is_mamba2_decode(lib):
    """Rank 1 with the Euler form is the Mamba-2 decode step (its own oracle,
    pinned separately)."""
    d = _mimo_rand(97, 3, 4, 5, 6, 2, 1)
    y, s, _, _ = oracle.decode_step_mimo(d["x"], d["B"], d["C"], d["dt"], d["dt_bias"], d["A"], d["D"], d["S"],
                                         lib=lib)
    ys, ss = _siso_decode(lib, d["x"][..., 0], d["B"][..., 0], d["C"][..., 0], d["dt"], d, d["S"])
    assert rel_err(y[..., 0], ys) < 1e-13 and rel_err(s, ss) < 1e-14


def pin_mimo_superposition_of_siso_steps(lib):
    """A rank-R Euler step: the new state is the Mamba-2 step on column 0 plus
    Mamba-2 steps of columns 1..R-1 from a zero state; output column r is
    the Mamba-2 readout of the new state with C's column r (a step with
    dt = 0: x enters nothing and nothing decays) plus D x_r."""
    d = _mimo_rand(101, 2, 4, 3, 5, 2, 3)
    y, s, _, _ = oracle.decode_step_mimo(d["x"], d["B"], d["C"], d["dt"], d["dt_bias"], d["A"], d["D"], d["S"],
                                         lib=lib)
    _, expect = _siso_decode(lib, d["x"][..., 0], d["B"][..., 0], d["C"][..., 0], d["dt"], d, d["S"])
    for r in (1, 2):
        _, part = _siso_decode(lib, d["x"][..., r], d["B"][..., r], d["C"][..., r], d["dt"], d,
                               np.zeros_like(d["S"]))
        expect = expect + part
    assert rel_err(s, expect) < 1e-13
    frozen = np.full_like(d["dt"], -np.inf)
    for r in range(3):
        yr, s_same = _siso_decode(lib, np.zeros_like(d["x"][..., r]), d["B"][..., r], d["C"][..., r], frozen,
                                  d, s)
        assert np.array_equal(s_same, s)
        assert rel_err(y[..., r], yr + d["D"][None, :, None] * d["x"][..., r]) < 1e-13


def pin_mimo_column_permutation(lib):
    """Permuting the R columns of X, B and C together permutes Y's columns and
    leaves the state as it was (also with the trapezoidal term)."""
    d = _mimo_rand(103, 2, 4, 3, 5, 4, 4)
    perm = np.array([2, 0, 3, 1])
    for trap in (False, True):
        kw = dict(trapezoid=trap, lam=d["lam"], prev_x=d["px"], prev_B=d["pB"]) if trap else {}
        y, s, px, pb = oracle.decode_step_mimo(d["x"], d["B"], d["C"], d["dt"], d["dt_bias"], d["A"], d["D"],
                                               d["S"], lib=lib, **kw)
        kwp = dict(trapezoid=trap, lam=d["lam"], prev_x=d["px"][..., perm], prev_B=d["pB"][..., perm]) \
            if trap else {}
        yp, sp, _, _ = oracle.decode_step_mimo(d["x"][..., perm], d["B"][..., perm], d["C"][..., perm], d["dt"],
                                               d["dt_bias"], d["A"], d["D"], d["S"], lib=lib, **kwp)
        assert rel_err(yp, y[..., perm]) < 1e-13 and rel_err(sp, s) < 1e-13
        if trap:
            assert np.array_equal(px, d["x"]) and np.array_equal(pb, d["B"]), "prev inputs replaced"


def pin_trapezoid_limits(lib):
    """lam = 1 is the Euler form whatever the previous inputs are; lam = 0
    keeps only the previous inputs, decayed over the step."""
    d = _mimo_rand(107, 2, 2, 3, 4, 1, 2)
    ye, se, _, _ = oracle.decode_step_mimo(d["x"], d["B"], d["C"], d["dt"], d["dt_bias"], d["A"], d["D"], d["S"],
                                           lib=lib)
    y1, s1, _, _ = oracle.decode_step_mimo(d["x"], d["B"], d["C"], d["dt"], d["dt_bias"], d["A"], d["D"], d["S"],
                                           trapezoid=True, lam=np.ones_like(d["lam"]), prev_x=d["px"],
                                           prev_B=d["pB"], lib=lib)
    assert np.array_equal(s1, se) and np.array_equal(y1, ye)
    _, s0, _, _ = oracle.decode_step_mimo(d["x"], d["B"], d["C"], d["dt"], d["dt_bias"], d["A"], d["D"], d["S"],
                                          trapezoid=True, lam=np.zeros_like(d["lam"]), prev_x=d["px"],
                                          prev_B=d["pB"], lib=lib)
    dt = softplus(d["dt"] + d["dt_bias"][None, :])
    a = np.exp(dt * d["A"][None, :])
    for b in range(2):
        for h in range(2):
            expect = a[b, h] * d["S"][b, h] + dt[b, h] * a[b, h] * d["px"][b, h] @ d["pB"][b, 0].T
            assert rel_err(s0[b, h], expect) < 1e-13


def pin_trapezoid_second_order(lib):
    """Scalar system h' = A h + x(t), x(t) = sin(w t), h(0) = h0, stepped
    with decode steps of size dt: against the exact solution at T, the
    trapezoidal rule (lam = 1/2) converges at second order in dt and the
    Euler form at first order (error ratios near 4 and 2 when dt halves)."""
    A, w, h0, T = -1.3, 2.0, 0.7, 2.0

    def exact(t):
        # h(t) = e^{At} h0 + int_0^t e^{A(t-s)} sin(w s) ds
        integral = (np.exp(A * t) * w + (-A) * np.sin(w * t) - w * np.cos(w * t)) / (A * A + w * w)
        return np.exp(A * t) * h0 + integral

    def run(n, trap):
        dt = T / n
        z = np.log(np.expm1(dt))            # softplus(z) = dt
        S = np.full((1, 1, 1, 1), h0)
        px, pb = np.zeros((1, 1, 1, 1)), np.ones((1, 1, 1, 1))
        for k in range(1, n + 1):
            xk = np.full((1, 1, 1, 1), np.sin(w * k * dt))
            if k == 1:
                px = np.zeros((1, 1, 1, 1))            # x(0) = sin(0) = 0
            kw = dict(trapezoid=True, lam=np.full((1, 1), 0.5), prev_x=px, prev_B=pb) if trap else {}
            _, S, px2, pb2 = oracle.decode_step_mimo(xk, np.ones((1, 1, 1, 1)), np.ones((1, 1, 1, 1)),
                                                     np.full((1, 1), z), np.zeros(1), np.array([A]), None, S,
                                                     lib=lib, **kw)
            if trap:
                px, pb = px2, pb2
        return abs(S[0, 0, 0, 0] - exact(T))

    et = [run(n, True) for n in (40, 80, 160)]
    ee = [run(n, False) for n in (40, 80, 160)]
    for e1, e2 in zip(et, et[1:]):
        assert 3.6 < e1 / e2 < 4.4, ("trapezoid order", et)
    for e1, e2 in zip(ee, ee[1:]):
        assert 1.8 < e1 / e2 < 2.2, ("Euler order", ee)
    assert et[-1] < ee[-1] / 20


# ---------------------------------------------------------------------------
# backward pass: against finite differences of the forward oracle
# ---------------------------------------------------------------------------
_BWD_INPUTS = ("x", "dt", "dt_bias", "A", "B", "C", "D", "h0")
_BWD_GRAD = {"x": "dx", "dt": "ddt_raw", "dt_bias": "ddt_bias", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "h0": "dh0"}


def _bwd_problem(seed, batch, L, H, P, N, G):
    r = np.random.default_rng(seed)
    d = {"x": r.standard_normal((batch, L, H, P)), "dt": r.standard_normal((batch, L, H)),
         "dt_bias": r.standard_normal(H) * 0.5 - 1.0, "A": -np.exp(r.uniform(0, np.log(4), H)),
         "B": r.standard_normal((batch, L, G, N)) / np.sqrt(N), "C": r.standard_normal((batch, L, G, N)) / np.sqrt(N),
         "D": r.standard_normal(H), "h0": r.standard_normal((batch, H, P, N)) * 0.5}
    w = {"dy": r.standard_normal((batch, L, H, P)), "df": r.standard_normal((batch, H, P, N))}
    return d, w


def _loss(lib, d, w):
    y, fs = oracle.ssd_scan(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"],
                            initial_state=d["h0"], want_final_state=True, lib=lib)
    return float(np.sum(w["dy"] * y) + np.sum(w["df"] * fs))


def _grads(lib, d, w):
    return oracle.ssd_scan_bwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], w["dy"],
                               initial_state=d["h0"], d_final_state=w["df"], lib=lib)


def pin_backward_finite_differences(lib):
    """Every gradient entry against a central difference of the forward
    oracle's loss <dy, y> + <df, final_state> (step 1e-6, fp64)."""
    d, w = _bwd_problem(109, 2, 7, 4, 3, 5, 2)
    g = _grads(lib, d, w)
    eps = 1e-6
    for k in _BWD_INPUTS:
        fd = np.zeros_like(d[k])
        flat = d[k].reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + eps
            lp = _loss(lib, d, w)
            flat[idx] = old - eps
            lm = _loss(lib, d, w)
            flat[idx] = old
            fd.reshape(-1)[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(g[_BWD_GRAD[k]] - fd)) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-6, ("finite difference", k, err)


def pin_backward_directional_across_checkpoints(lib):
    """Sequences longer than the oracle's 64-token checkpoint interval: the
    gradient's inner product with a random direction of every input at once
    equals the loss's central difference along it."""
    d, w = _bwd_problem(113, 2, 150, 2, 3, 4, 1)
    g = _grads(lib, d, w)
    r = np.random.default_rng(127)
    v = {k: r.standard_normal(np.shape(d[k])) for k in _BWD_INPUTS}
    eps = 1e-6
    dp = {k: d[k] + eps * v[k] for k in _BWD_INPUTS}
    dm = {k: d[k] - eps * v[k] for k in _BWD_INPUTS}
    fd = (_loss(lib, dp, w) - _loss(lib, dm, w)) / (2 * eps)
    an = sum(float(np.sum(g[_BWD_GRAD[k]] * v[k])) for k in _BWD_INPUTS)
    assert abs(an - fd) < 1e-6 * max(1.0, abs(fd)), ("directional derivative", an, fd)


def pin_backward_linear_parts(lib):
    """y is linear in x and in h0: the gradients for x and h0 do not change
    when x or h0 change, and with dy = 0, df = 0 every gradient is zero."""
    d, w = _bwd_problem(131, 1, 20, 2, 3, 4, 1)
    g1 = _grads(lib, d, w)
    d2 = dict(d)
    d2["x"] = d["x"] * -2.5 + 1.0
    d2["h0"] = d["h0"] * 3.0
    g2 = _grads(lib, d2, w)
    assert rel_err(g2["dx"], g1["dx"]) < 1e-13 and rel_err(g2["dh0"], g1["dh0"]) < 1e-13
    z = _grads(lib, d, {"dy": np.zeros_like(w["dy"]), "df": np.zeros_like(w["df"])})
    assert all(np.all(v == 0) for v in z.values())


# ---------------------------------------------------------------------------
# the mixer's projections: y = x w^T
# ---------------------------------------------------------------------------
def _linear(lib, x, w):
    return oracle.linear(x, w, lib=lib)


def pin_linear_identity(lib):
    """w = I: y = x exactly."""
    x = np.random.default_rng(41).standard_normal((5, 33))
    assert np.array_equal(_linear(lib, x, np.eye(33)), x)


def pin_linear_integer_closed_form(lib):
    """x[m][k] = 1000 + m, w[n][k] = 1000 + n: y = K (1000 + m)(1000 + n), exact in
    fp64 and beyond fp32's 24-bit integers; N != K so a transposed w cannot pass."""
    M, N, K = 3, 5, 4096
    x = np.repeat(1000.0 + np.arange(M)[:, None], K, axis=1)
    w = np.repeat(1000.0 + np.arange(N)[:, None], K, axis=1)
    want = K * np.outer(1000.0 + np.arange(M), 1000.0 + np.arange(N))
    assert np.array_equal(_linear(lib, x, w), want)


def pin_linear_one_hot_rows(lib):
    """x = e_j picks column j of w: y[n] = w[n][j] for every n (rectangular w)."""
    r = np.random.default_rng(42)
    N, K = 7, 11
    w = r.standard_normal((N, K))
    x = np.eye(K)[[0, 3, 10]]
    assert np.array_equal(_linear(lib, x, w), w[:, [0, 3, 10]].T)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
