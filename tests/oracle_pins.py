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


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
