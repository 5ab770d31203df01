"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each function takes an ``Oracle`` and raises ``AssertionError`` when the
oracle disagrees with what the pages or the mathematics fix: hand-derived
golden values (``tests/golden``), closed-form error bounds, exact identities,
invariants, special cases that reduce to a textbook formula, and brute force
on tiny inputs.  ``test_oracle.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on altered copies and requires that each
alteration is caught by at least one of them.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Slack on top of half a quantization step: three binary32 roundings (the
# reciprocal, the scale and the product x*r) each perturb x/s by at most
# 2^-24 relative, and |x| <= amax = 127*s, so the extra error is below
# 3 * 127 * 2^-24 * s ~= 2.3e-5 * s < 2^-14 * s.
HALF_STEP_SLACK = 2.0 ** -14


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(rows):
    return np.asarray(rows, dtype=np.float64).astype(np.float16)


def _mask(K, chans):
    m = np.zeros(K, np.uint8)
    m[list(chans)] = 1
    return m


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def _tiny_case(seed, M, K, n_out, scale=30.0):
    r = _rng(seed, M, K, n_out)
    X = r.standard_normal((M, K)).astype(np.float32)
    ch = np.sort(r.choice(K, n_out, replace=False)) if n_out else np.zeros(0, int)
    if n_out:
        X[:, ch] *= np.float32(scale)
    return X.astype(np.float16), ch


TINY_SHAPES = [(1, 64, 0), (3, 64, 2), (7, 128, 5), (16, 256, 9), (33, 192, 1), (5, 64, 64)]


# ----------------------------------------------------------------------------
# golden, hand-derived
# ----------------------------------------------------------------------------
def pin_golden_act(o):
    for c in _golden("act_quant_cases.json")["cases"]:
        X = _f16(c["x"])
        M, K = X.shape
        new_set, cnt, flag = o.update_outlier_set(X, c["tau"], _mask(K, c["prev"]), k_cap=K)
        got_set = list(np.nonzero(new_set)[0])
        assert got_set == c["expect_set"], (c["name"], got_set)
        assert (flag == 1) == c["expect_fired"], (c["name"], flag)
        assert cnt == len(c["expect_set"])
        assert list(o.outlier_list(new_set)) == c["expect_set"], c["name"]
        ldo = max(1, len(c["expect_set"]))
        Xq, s_x, X_out = o.quantize_act(X, new_set, ldo)
        assert Xq.tolist() == c["expect_q"], (c["name"], Xq.tolist())
        assert s_x.tolist() == c["expect_s"], (c["name"], s_x.tolist())
        got_out = X_out.view(np.float16).astype(np.float64)[:, :len(c["expect_set"])]
        assert got_out.tolist() == [[float(v) for v in r] for r in c["expect_xout"]], c["name"]
        assert not X_out[:, len(c["expect_set"]):].any(), c["name"]


def pin_golden_weight(o):
    for c in _golden("weight_quant_cases.json")["cases"]:
        Wq, s_w = o.quantize_weight(_f16(c["w"]), c["bits"])
        assert Wq.tolist() == c["expect_q"], (c["name"], Wq.tolist())
        assert s_w.tolist() == c["expect_s"], (c["name"], s_w.tolist())


def golden_layer_inputs():
    g = _golden("layer_worked_example.json")
    Kt = g["k_total"]
    X = np.zeros((len(g["X"]), Kt), np.float16)
    W = np.zeros((len(g["W"]), Kt), np.float16)
    X[:, :len(g["X"][0])] = _f16(g["X"])
    W[:, :len(g["W"][0])] = _f16(g["W"])
    return g, X, W


def pin_golden_layer(o):
    g, X, W = golden_layer_inputs()
    K = X.shape[1]
    k0 = len(g["X"][0])
    new_set, cnt, flag = o.update_outlier_set(X, g["tau"], np.zeros(K, np.uint8), k_cap=K)
    assert list(np.nonzero(new_set)[0]) == g["expect_set"] and flag == 1
    Xq, s_x, X_out = o.quantize_act(X, new_set, 32)
    Wq, s_w = o.quantize_weight(W, 8)
    W_out = o.gather_weight_cols(W, new_set, 32)
    assert Xq[:, :k0].tolist() == g["expect_q_x"] and not Xq[:, k0:].any()
    assert Wq[:, :k0].tolist() == g["expect_q_w"] and not Wq[:, k0:].any()
    assert s_x.tolist() == g["expect_s_x"] and s_w.tolist() == g["expect_s_w"]
    assert X_out.view(np.float16)[:, :cnt].astype(float).tolist() == g["expect_x_out"]
    assert W_out.view(np.float16)[:, :cnt].astype(float).tolist() == g["expect_w_out"]
    acc = o.int_gemm(Xq, Wq)
    assert acc.tolist() == g["expect_acc"], acc.tolist()
    Y = o.output(acc, s_x, s_w, X_out, W_out, cnt)
    assert Y.tolist() == g["expect_y"], Y.tolist()


# ----------------------------------------------------------------------------
# closed forms, bounds and brute force
# ----------------------------------------------------------------------------
def pin_half_decode(o):
    """Every binary16 pattern decodes as NumPy's (independent) conversion."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    sample = np.concatenate([bits[:2048], bits[0x3000:0x3400], bits[0x7800:0x8800],
                             bits[-2048:], bits[::97]])
    for b in sample:
        got = o.half_to_float(int(b))
        want = ref[b]
        if np.isnan(want):
            assert np.isnan(got), hex(b)
        else:
            assert got == want, (hex(b), got, want)


def pin_set_bruteforce(o):
    """Gate + union against a direct column scan (all tokens, all channels)."""
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        X, _ = _tiny_case(seed, M, K, n_out)
        Xa = np.abs(X.astype(np.float64))
        r = _rng(99, seed)
        prev = (r.random(K) < 0.05).astype(np.uint8)
        for tau in (6.0, 3.0, 1e9):
            uncached_over = (Xa[:, prev == 0] > tau).any()
            want = prev.copy()
            if uncached_over:
                want |= (Xa > tau).any(axis=0).astype(np.uint8)
            got, cnt, flag = o.update_outlier_set(X, tau, prev, k_cap=K)
            assert (got == want).all(), (seed, tau)
            assert flag == (1 if uncached_over else 0)
            assert cnt == int(want.sum())
            idx = o.outlier_list(got)
            assert (idx == np.nonzero(want)[0]).all() and (np.diff(idx) > 0).all()


def pin_quant_error_bound(o):
    """|x - q*s| <= s*(1/2 + slack) off the set; q = 0 on it; the row's amax
    maps to +-127; every uncached channel is at or under tau afterwards."""
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        X, _ = _tiny_case(seed, M, K, n_out)
        tau = 6.0
        s_set, _, _ = o.update_outlier_set(X, tau, np.zeros(K, np.uint8), k_cap=K)
        Xq, s_x, _ = o.quantize_act(X, s_set, max(1, K))
        x = X.astype(np.float64)
        s = s_x.astype(np.float64)[:, None]
        off = s_set == 0
        err = np.abs(x - Xq.astype(np.float64) * s)[:, off]
        assert (err <= (s * (0.5 + HALF_STEP_SLACK))).all() if off.any() else True
        assert not Xq[:, ~off].any()
        assert (np.abs(x[:, off]) <= tau).all() if off.any() else True
        amax = np.abs(x[:, off]).max(axis=1) if off.any() else np.zeros(M)
        for m in range(M):
            if amax[m] > 0:
                assert np.abs(Xq[m, off]).max() == 127, (seed, m)
                assert s_x[m] == np.float32(amax[m]) / np.float32(127)
            else:
                assert s_x[m] == 1.0 and not Xq[m].any()


def pin_nearest_code(o):
    """Brute force over all 255 codes with exact rationals: the code is the
    nearest level x / (a/127) (checked where no tie is within 1e-4)."""
    for seed in range(4):
        X, _ = _tiny_case(100 + seed, 4, 64, 0)
        Xq, s_x, _ = o.quantize_act(X, np.zeros(64, np.uint8), 1)
        for m in range(X.shape[0]):
            row = [Fraction(float(v)) for v in X[m].astype(np.float64)]
            a = max(abs(v) for v in row)
            for k, v in enumerate(row):
                t = v * 127 / a
                best = min(range(-127, 128), key=lambda q: abs(t - q))
                frac = abs(t - int(t)) if t >= 0 else abs(t - int(t))
                if abs(frac - Fraction(1, 2)) > Fraction(1, 10000):
                    assert Xq[m, k] == best, (seed, m, k, float(t), int(Xq[m, k]), best)


def pin_weight_bound(o):
    for bits, qmax in ((8, 127), (4, 7)):
        r = _rng(7, bits)
        W = (r.standard_normal((24, 128)) * 0.02).astype(np.float16)
        W[3] = 0
        Wq, s_w = o.quantize_weight(W, bits)
        w = W.astype(np.float64)
        s = s_w.astype(np.float64)[:, None]
        assert (np.abs(w - Wq * s) <= s * (0.5 + HALF_STEP_SLACK)).all()
        assert np.abs(Wq).max() <= qmax
        for n in range(W.shape[0]):
            if np.abs(w[n]).max() > 0:
                assert np.abs(Wq[n]).max() == qmax
            else:
                assert s_w[n] == 1.0 and not Wq[n].any()


def pin_int_gemm_bruteforce(o):
    """Integer product against an int64 matrix product, incl. extreme codes."""
    for seed, (M, N, K) in enumerate([(1, 1, 64), (5, 7, 64), (17, 9, 320), (4, 4, 8192)]):
        r = _rng(11, seed)
        A = r.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
        B = r.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
        if seed == 3:
            A[:] = 127
            B[0] = 127
            B[1] = -127
        acc = o.int_gemm(A, B)
        want = A.astype(np.int64) @ B.astype(np.int64).T
        assert (acc.astype(np.int64) == want).all(), seed


def _layer(o, X, W, tau, bits=8, prev=None, ldo=None):
    M, K = X.shape
    prev = np.zeros(K, np.uint8) if prev is None else prev
    s_set, cnt, flag = o.update_outlier_set(X, tau, prev, k_cap=K)
    ldo = ldo or max(1, K)
    Xq, s_x, X_out = o.quantize_act(X, s_set, ldo)
    Wq, s_w = o.quantize_weight(W, bits)
    W_out = o.gather_weight_cols(W, s_set, ldo)
    acc = o.int_gemm(Xq, Wq)
    Y = o.output(acc, s_x, s_w, X_out, W_out, cnt)
    return dict(set=s_set, cnt=cnt, flag=flag, Xq=Xq, s_x=s_x, X_out=X_out, Wq=Wq,
                s_w=s_w, W_out=W_out, acc=acc, Y=Y)


def _wcase(seed, N, K, std=0.05):
    return (_rng(21, seed, N, K).standard_normal((N, K)) * std).astype(np.float16)


def pin_split_identity(o):
    """Exact split in FP64 on the raw operands:
    X W^T = (X with outlier channels zeroed) W^T + X_out W_out^T.
    A misplaced, dropped or misordered outlier column breaks it."""
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        X, _ = _tiny_case(seed, M, K, n_out)
        W = _wcase(seed, 11, K)
        L = _layer(o, X, W, 6.0)
        x = X.astype(np.float64)
        w = W.astype(np.float64)
        keep = (L["set"] == 0).astype(np.float64)
        c = L["cnt"]
        xo = L["X_out"].view(np.float16).astype(np.float64)[:, :c]
        wo = L["W_out"].view(np.float16).astype(np.float64)[:, :c]
        lhs = x @ w.T
        rhs = (x * keep) @ w.T + xo @ wo.T
        assert np.allclose(lhs, rhs, rtol=0, atol=1e-12 * max(1.0, np.abs(lhs).max())), seed


def pin_output_vs_dequant(o):
    """Y against a brute-force FP64 sum over dequantized operands:
    sum_{k not in I} (q_x s_x)(q_w s_w) + sum_j X_out W_out."""
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        for bits in (8, 4):
            X, _ = _tiny_case(seed, M, K, n_out)
            W = _wcase(seed, 13, K)
            L = _layer(o, X, W, 6.0, bits=bits)
            xd = L["Xq"].astype(np.float64) * L["s_x"].astype(np.float64)[:, None]
            wd = L["Wq"].astype(np.float64) * L["s_w"].astype(np.float64)[:, None]
            c = L["cnt"]
            xo = L["X_out"].view(np.float16).astype(np.float64)[:, :c]
            wo = L["W_out"].view(np.float16).astype(np.float64)[:, :c]
            want = np.zeros((M, W.shape[0]))
            for m in range(M):
                for n in range(W.shape[0]):
                    want[m, n] = sum(xd[m, k] * wd[n, k] for k in range(K)) + \
                        sum(xo[m, j] * wo[n, j] for j in range(c))
            scale = max(1.0, np.abs(want).max())
            assert np.abs(L["Y"] - want).max() <= 1e-12 * scale, (seed, bits)


def pin_output_vs_truth_bound(o):
    """|Y - X W^T| <= sum_{k not in I} (|x| e_w + |w| e_x + e_x e_w), with
    e = s (1/2 + slack): the closed-form quantization error bound."""
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        for bits in (8, 4):
            X, _ = _tiny_case(seed, M, K, n_out)
            W = _wcase(seed, 9, K)
            L = _layer(o, X, W, 6.0, bits=bits)
            x = X.astype(np.float64)
            w = W.astype(np.float64)
            truth = x @ w.T
            ex = L["s_x"].astype(np.float64) * (0.5 + HALF_STEP_SLACK)
            ew = L["s_w"].astype(np.float64) * (0.5 + HALF_STEP_SLACK)
            off = (L["set"] == 0).astype(np.float64)
            bound = (np.abs(x) * off) @ np.ones((K, 1)) * ew[None, :] \
                + ex[:, None] * ((np.abs(w) * off[None, :]).sum(axis=1))[None, :] \
                + ex[:, None] * ew[None, :] * off.sum()
            slack = 1e-9 * (np.abs(x) @ np.abs(w).T + 1.0)
            assert (np.abs(L["Y"] - truth) <= bound + slack).all(), (seed, bits)


def pin_no_outlier_textbook(o):
    """Nothing above the threshold: the layer is plain W8A8 with per-token and
    per-channel scales, Y = (q_x q_w^T) * (s_x s_w^T)."""
    X, _ = _tiny_case(5, 9, 128, 0)
    W = _wcase(5, 10, 128)
    L = _layer(o, X, W, float("inf"))
    assert L["cnt"] == 0 and L["flag"] == 0
    want = (L["Xq"].astype(np.int64) @ L["Wq"].astype(np.int64).T).astype(np.float64)
    want = want * L["s_x"].astype(np.float64)[:, None] * L["s_w"].astype(np.float64)[None, :]
    assert np.abs(L["Y"] - want).max() <= 1e-12 * np.abs(want).max()


def pin_all_outlier(o):
    """tau = 0: every nonzero channel is an outlier, all codes are 0 with unit
    scales, and Y is the plain FP16-input product X W^T."""
    X, _ = _tiny_case(6, 6, 64, 0)
    X[:, 5] = 0
    W = _wcase(6, 8, 64)
    L = _layer(o, X, W, 0.0)
    assert L["cnt"] == 63 and not L["Xq"].any() and (L["s_x"] == 1.0).all()
    truth = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.abs(L["Y"] - truth).max() <= 1e-12 * np.abs(truth).max()


def pin_sign_symmetry(o):
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        X, _ = _tiny_case(seed, M, K, n_out)
        s1, c1, _ = o.update_outlier_set(X, 6.0, np.zeros(K, np.uint8), K)
        s2, c2, _ = o.update_outlier_set(-X, 6.0, np.zeros(K, np.uint8), K)
        assert (s1 == s2).all() and c1 == c2
        q1, sx1, xo1 = o.quantize_act(X, s1, K)
        q2, sx2, xo2 = o.quantize_act(-X, s2, K)
        assert (q1 == -q2).all() and (sx1 == sx2).all()
        assert (xo1.view(np.float16) == -xo2.view(np.float16)).all()


def pin_pow2_scaling(o):
    """X*2^p with tau*2^p: same set and codes, scales times 2^p (binary
    scaling commutes with every rounding when nothing over/underflows)."""
    for seed, (M, K, n_out) in enumerate(TINY_SHAPES):
        X, _ = _tiny_case(seed, M, K, n_out, scale=10.0)
        for p in (1, 3):
            Xs = (X.astype(np.float32) * np.float32(2.0 ** p)).astype(np.float16)
            assert (Xs.astype(np.float64) == X.astype(np.float64) * 2.0 ** p).all()
            s1, _, _ = o.update_outlier_set(X, 6.0, np.zeros(K, np.uint8), K)
            s2, _, _ = o.update_outlier_set(Xs, 6.0 * 2 ** p, np.zeros(K, np.uint8), K)
            assert (s1 == s2).all()
            q1, sx1, _ = o.quantize_act(X, s1, 1)
            q2, sx2, _ = o.quantize_act(Xs, s2, 1)
            assert (q1 == q2).all()
            # rows whose amax is 0 keep the unit scale of the zero-scale rule
            live = np.abs(X.astype(np.float64))[:, s1 == 0].max(axis=1, initial=0) > 0
            assert (sx2[live].astype(np.float64) == sx1[live].astype(np.float64) * 2.0 ** p).all()
            assert (sx1[~live] == 1).all() and (sx2[~live] == 1).all()


def pin_permutation(o):
    """Permuting channels of X and W together permutes the set and leaves the
    integer product and Y unchanged."""
    X, _ = _tiny_case(8, 12, 192, 6)
    W = _wcase(8, 7, 192)
    perm = _rng(8, 1).permutation(192)
    A = _layer(o, X, W, 6.0)
    B = _layer(o, np.ascontiguousarray(X[:, perm]), np.ascontiguousarray(W[:, perm]), 6.0)
    assert (B["set"] == A["set"][perm]).all()
    assert (A["acc"] == B["acc"]).all()
    assert np.abs(A["Y"] - B["Y"]).max() <= 1e-12 * np.abs(A["Y"]).max()


def pin_overflow(o):
    """More outliers than k_cap: flag 2 and the set is left as it was; exactly
    k_cap outliers still fit."""
    X, ch = _tiny_case(9, 8, 128, 6, scale=40.0)
    need = int((np.abs(X.astype(np.float64)) > 6.0).any(axis=0).sum())
    s_ok, c_ok, f_ok = o.update_outlier_set(X, 6.0, np.zeros(128, np.uint8), k_cap=need)
    assert f_ok == 1 and c_ok == need
    s_no, c_no, f_no = o.update_outlier_set(X, 6.0, np.zeros(128, np.uint8), k_cap=need - 1)
    assert f_no == 2 and c_no == 0 and not s_no.any()


def pin_decode_sequence(o):
    """A short decode run with a persistent set and planted transient
    channels: the gate fires on exactly the steps that hold an uncached value
    above tau, and after every step the set equals the union of everything
    seen so far (the gated set equals the ungated one)."""
    M, K, steps = 8, 256, 12
    r = _rng(31)
    pers = np.sort(r.choice(K, 5, replace=False))
    rest = np.setdiff1d(np.arange(K), pers)
    events = {2: r.choice(rest, 2, replace=False), 7: r.choice(rest, 1, replace=False),
              8: r.choice(rest, 3, replace=False)}
    cur = np.zeros(K, np.uint8)
    seen = np.zeros(K, bool)
    for st in range(steps):
        X = r.standard_normal((M, K)).astype(np.float32)
        X[:, pers] = r.uniform(20, 100, (M, pers.size)) * np.where(r.random((M, pers.size)) < .5, -1, 1)
        if st in events:
            e = events[st]
            X[:, e] = r.uniform(20, 100, (M, e.size))
        X = X.astype(np.float16)
        over = (np.abs(X.astype(np.float64)) > 6.0).any(axis=0)
        expect_fire = bool((over & (cur == 0)).any())
        seen |= over
        cur_new, cnt, flag = o.update_outlier_set(X, 6.0, cur, k_cap=K)
        assert flag == (1 if expect_fire else 0), st
        assert (cur_new.astype(bool) == seen).all(), st
        cur = cur_new


def pin_layer_driver(o, layer_cls=None):
    """The decode driver every GPU comparison runs as its checker
    (OracleLayer.step, and run_layer for a single call): over a planted
    multi-step run -- persistent outlier channels, transient ones on some
    steps, a step where nothing exceeds tau -- after every step the set is
    the union of every channel seen above tau so far (brute-force column
    scan, carried across steps here), the flag is the brute-force gate on the
    channels not yet cached, the ids are that set ascending, and Xq, s_x,
    X_out, acc and Y equal the single oracle calls (each pinned above)
    composed here by hand with that set: weight columns gathered for the
    current set, the current set size passed to the output.  MixQ article,
    "MixQ的解决方案": Fig. 9 (outliers recur in fixed channels) and the amax
    paragraph (re-detect only when the amax of the uncached channels exceeds
    the threshold)."""
    from oracle.mixq_oracle import OracleLayer, run_layer
    layer_cls = layer_cls or OracleLayer
    M, K, N, steps, tau, ldo = 6, 192, 40, 9, 6.0, 32
    r = _rng(41)
    W = _wcase(41, N, K)
    pers = np.sort(r.choice(K, 4, replace=False))
    rest = np.setdiff1d(np.arange(K), pers)
    events = {1: r.choice(rest, 2, replace=False), 4: r.choice(rest, 3, replace=False),
              6: r.choice(rest, 1, replace=False)}
    quiet = {3, 5}  # steps on which the persistent channels stay below tau
    layer = layer_cls(W=W, bits=8, tau=tau, k_cap=ldo, ldo=ldo, oracle=o)
    Wq, s_w = o.quantize_weight(W, 8)
    seen = np.zeros(K, bool)
    fires = []
    for st in range(steps):
        X = np.clip(r.standard_normal((M, K)), -4, 4).astype(np.float32)
        if st not in quiet:
            X[:, pers] = r.uniform(20, 100, (M, pers.size)) * np.where(
                r.random((M, pers.size)) < .5, -1, 1)
        if st in events:
            e = events[st]
            X[:, e] = r.uniform(20, 100, (M, e.size))
        X = X.astype(np.float16)
        over = (np.abs(X.astype(np.float64)) > tau).any(axis=0)
        fire = bool((over & ~seen).any())
        seen |= over
        res = layer.step(X)
        assert res.flag == int(fire), st
        assert (res.in_set.astype(bool) == seen).all(), st
        assert res.count == int(seen.sum()), st
        assert np.array_equal(res.idx, np.flatnonzero(seen)), st
        cur = seen.astype(np.uint8)
        Xq, s_x, X_out = o.quantize_act(X, cur, ldo)
        W_out = o.gather_weight_cols(W, cur, ldo)
        acc = o.int_gemm(Xq, Wq)
        Y = o.output(acc, s_x, s_w, X_out, W_out, int(seen.sum()))
        assert np.array_equal(res.Xq, Xq) and np.array_equal(res.s_x, s_x), st
        assert np.array_equal(res.X_out, X_out), st
        assert np.array_equal(res.acc, acc), st
        assert np.array_equal(res.Y, Y), st
        fires.append(fire)
    assert fires == [True, True, False, False, True, False, True, False, False], fires
    # run_layer: one call on an empty set is that same composition
    X = X.astype(np.float16)
    one = run_layer(X, W, bits=8, tau=tau, k_cap=ldo, ldo=ldo, oracle=o)
    cur = (np.abs(X.astype(np.float64)) > tau).any(axis=0).astype(np.uint8)
    Xq, s_x, X_out = o.quantize_act(X, cur, ldo)
    Y = o.output(o.int_gemm(Xq, Wq), s_x, s_w, X_out, o.gather_weight_cols(W, cur, ldo),
                 int(cur.sum()))
    assert one.count == int(cur.sum()) and np.array_equal(one.Y, Y)


def pin_sampled_output(o):
    """The per-pair entry point against an int64 matrix product and an FP64
    sum over the outlier columns, at random (row, col) pairs."""
    X, _ = _tiny_case(12, 19, 320, 7)
    W = _wcase(12, 23, 320)
    L = _layer(o, X, W, 6.0, ldo=32)
    r = _rng(12, 5)
    rows = r.integers(0, 19, 40)
    cols = r.integers(0, 23, 40)
    acc, Y = o.sampled_output(L["Xq"], L["Wq"], L["s_x"], L["s_w"], L["X_out"], L["W_out"],
                              L["cnt"], rows, cols)
    full = L["Xq"].astype(np.int64) @ L["Wq"].astype(np.int64).T
    assert (acc == full[rows, cols]).all()
    c = L["cnt"]
    xo = L["X_out"].view(np.float16).astype(np.float64)[:, :c]
    wo = L["W_out"].view(np.float16).astype(np.float64)[:, :c]
    want = full[rows, cols] * L["s_x"].astype(np.float64)[rows] * L["s_w"].astype(np.float64)[cols] \
        + (xo[rows] * wo[cols]).sum(axis=1)
    assert np.abs(Y - want).max() <= 1e-12 * np.abs(want).max()


# ----------------------------------------------------------------------------
# the RMSNorm before the layer (fused with the amax pass on the GPU)
# ----------------------------------------------------------------------------
def _norm_rows(seed, M, K, wide=True):
    """fp16 rows; ``wide`` mixes values near the fp16 maximum, subnormals and
    N(0,1) draws in one row, where a rounded running sum of squares would lose
    the small terms."""
    r = _rng(seed, M, K, 77)
    H = r.standard_normal((M, K))
    if wide:
        kind = r.integers(0, 4, (M, K))
        H = np.where(kind == 0, r.uniform(1000, 60000, (M, K)) * r.choice([-1, 1], (M, K)), H)
        H = np.where(kind == 1, r.integers(1, 1024, (M, K)) * 2.0 ** -24, H)
    return H.astype(np.float16)


def _gamma(seed, K):
    return (1.0 + 0.25 * _rng(seed, K, 78).standard_normal(K)).astype(np.float16)


def pin_rmsnorm_fsum(o):
    """rstd against a second route to the exactly rounded sum of squares:
    math.fsum returns the correctly rounded sum of the (exact) binary64
    squares, whatever their order."""
    import math
    for seed, (M, K) in enumerate([(5, 64), (4, 256), (3, 1024), (2, 4096)]):
        for wide in (False, True):
            H = _norm_rows(seed, M, K, wide)
            X, rstd = o.rmsnorm(H, _gamma(seed, K), 1e-5)
            for m in range(M):
                S = math.fsum(float(h) ** 2 for h in H[m].astype(np.float64))
                ms = np.float32(S / K)
                want = np.float32(1.0) / np.sqrt(ms + np.float32(1e-5))
                assert rstd[m].view(np.uint32) == want.view(np.uint32), (seed, wide, m)


def pin_rmsnorm_bound(o):
    """Each x within the rounding bound of h * gamma / sqrt(mean(h^2) + eps)
    computed in FP64: two fp16 roundings (2^-11 each), a few binary32 ones,
    plus fp16 subnormal spacing."""
    for seed, (M, K) in enumerate([(6, 64), (4, 512), (2, 2048)]):
        for wide in (False, True):
            H = _norm_rows(seed + 10, M, K, wide)
            g = _gamma(seed, K)
            X, _ = o.rmsnorm(H, g, 1e-5)
            h = H.astype(np.float64)
            true = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + float(np.float32(1e-5)))
            true *= g.astype(np.float64)
            err = np.abs(X.astype(np.float64) - true)
            tol = np.abs(true) * (2.0 ** -10 + 2.0 ** -18) + 2.0 ** -24 * (np.abs(g) + 1.0)
            assert (err <= tol).all(), (seed, wide, (err / tol).max())


def pin_rmsnorm_invariants(o):
    """With eps = 0: scaling a row by 2^p leaves x unchanged (every rounding
    commutes with binary scaling); negating it negates x; permuting channels
    of H and gamma together permutes x (the sum of squares is exact, so its
    order does not matter -- also on the wide rows)."""
    for seed, (M, K) in enumerate([(4, 64), (3, 512), (2, 2048)]):
        H = _norm_rows(seed + 20, M, K, wide=False).astype(np.float64)
        H = (np.sign(H) * np.maximum(np.abs(H), 2.0 ** -8)).astype(np.float16)  # no subnormals
        g = _gamma(seed, K)
        X, rstd = o.rmsnorm(H, g, 0.0)
        for p in (-3, 2):
            Hs = (H.astype(np.float64) * 2.0 ** p).astype(np.float16)
            assert (Hs.astype(np.float64) == H.astype(np.float64) * 2.0 ** p).all()
            Xs, rs = o.rmsnorm(Hs, g, 0.0)
            assert (Xs.view(np.uint16) == X.view(np.uint16)).all()
            assert (rs.astype(np.float64) == rstd.astype(np.float64) * 2.0 ** -p).all()
        Xn, rn = o.rmsnorm(-H, g, 0.0)
        assert (Xn.astype(np.float64) == -X.astype(np.float64)).all() and (rn == rstd).all()
        for wide in (False, True):
            Hw = _norm_rows(seed + 30, M, K, wide)
            perm = _rng(seed, 79).permutation(K)
            A, ra = o.rmsnorm(Hw, g, 1e-5)
            B, rb = o.rmsnorm(np.ascontiguousarray(Hw[:, perm]), np.ascontiguousarray(g[perm]),
                              1e-5)
            assert (ra.view(np.uint32) == rb.view(np.uint32)).all()
            assert (B.view(np.uint16) == A[:, perm].view(np.uint16)).all()


def _round_fmt(q, p, emin):
    """Nearest binary floating-point value to the rational q (ties to even),
    p significand bits, minimum normal exponent emin; no overflow."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sgn, a = (-1 if q < 0 else 1), abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - (p - 1))
    k = a / ulp
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * ulp


def _r64(q):
    return _round_fmt(q, 53, -1022)


def _r32(q):
    return _round_fmt(q, 24, -126)


def _r16(q):
    return _round_fmt(q, 11, -14)


def _sqrt32(t):
    """Correctly rounded binary32 square root of the binary32 value t >= 0,
    decided by exact comparisons of t with squared midpoints."""
    t = Fraction(t)
    if t == 0:
        return Fraction(0)
    y = Fraction(float(np.sqrt(np.float32(float(t)))))  # a guess; checked below
    while True:
        up = Fraction(float(np.nextafter(np.float32(float(y)), np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(np.float32(float(y)), np.float32(0))))
        if ((y + up) / 2) ** 2 < t:
            y = up
        elif ((y + dn) / 2) ** 2 > t:
            y = dn
        else:
            # ties cannot occur: a midpoint squared has more bits than t
            return y


def pin_rmsnorm_exact_rationals(o):
    """Every step of the normalisation redone with exact rationals and the
    IEEE round-to-nearest-even rule written out: the exact sum of squares
    rounded to binary64, the division by K, the binary32 mean square, eps,
    square root and reciprocal, the binary32 product with h rounded to fp16,
    then the product with gamma rounded to fp16."""
    for seed, (M, K, eps) in enumerate([(3, 64, 1e-5), (2, 64, 0.0), (2, 128, 1e-6)]):
        H = _norm_rows(seed + 40, M, K, wide=(seed != 1))
        g = _gamma(seed + 40, K)
        X, rstd = o.rmsnorm(H, g, eps)
        e32 = Fraction(float(np.float32(eps)))
        for m in range(M):
            hs = [Fraction(float(h)) for h in H[m].astype(np.float64)]
            S = _r64(sum(h * h for h in hs))
            ms = _r32(_r64(S / K))
            t = _r32(ms + e32)
            r = Fraction(0) if t == 0 else _r32(1 / _sqrt32(t))
            assert Fraction(float(rstd[m])) == r, (seed, m)
            for k in range(K):
                n = _r16(_r32(hs[k] * r))
                x = _r16(n * Fraction(float(g[k])))
                assert Fraction(float(X[m, k])) == x, (seed, m, k)


def pin_rmsnorm_closed_form(o):
    """A row of one power of two c (any sign) has mean square c^2 exactly,
    so with eps = 0 rstd = 1/|c| and x = sign(c) * gamma; an all-zero row
    gives rstd = 0 and x = 0."""
    K = 128
    g = _gamma(3, K)
    rows = [np.full(K, c) for c in (2.0 ** -20, -0.5, 1.0, 64.0, -1024.0)]
    H = np.array(rows + [np.zeros(K)]).astype(np.float16)
    X, rstd = o.rmsnorm(H, g, 0.0)
    for m, c in enumerate((2.0 ** -20, -0.5, 1.0, 64.0, -1024.0)):
        assert float(rstd[m]) == 1.0 / abs(c)
        assert (X[m].astype(np.float64) == np.sign(c) * g.astype(np.float64)).all()
    assert rstd[-1] == 0 and not X[-1].astype(np.float64).any()


def pin_residual_add(o):
    """H = R + D against exact rationals rounded to fp16 by the rule written
    out (ties to even, subnormals included), on random pairs, pairs built to
    land exactly halfway between fp16 values, and pairs with subnormal sums;
    plus x + (-x) = +0, x + 0 = x and commutativity, bit for bit."""
    r = _rng(91)
    R = (r.standard_normal((6, 64)) * 4.0).astype(np.float16)
    D = (r.standard_normal((6, 64)) * 0.5).astype(np.float16)
    # halfway cases: a value of magnitude in [1, 2) (fp16 step 2^-10) plus 2^-11 or 3*2^-11
    base = (1.0 + r.integers(0, 1024, 64) * 2.0 ** -10).astype(np.float16)
    half = np.where(r.random(64) < 0.5, 2.0 ** -11, 3 * 2.0 ** -11).astype(np.float16)
    sub = (r.integers(-1023, 1024, (2, 64)) * 2.0 ** -24).astype(np.float16)
    cases = [(R, D), (base[None], half[None]), (sub[:1], sub[1:]),
             (R, -R), (R, np.zeros_like(R))]
    for a, b in cases:
        got = o.residual_add(a, b)
        for x, y, h in zip(a.ravel().astype(np.float64), b.ravel().astype(np.float64),
                           got.ravel().astype(np.float64)):
            assert Fraction(float(h)) == _r16(Fraction(x) + Fraction(y)), (x, y, h)
        assert (o.residual_add(b, a).view(np.uint16) == got.view(np.uint16)).all()
    z = o.residual_add(R, -R)
    assert (z.view(np.uint16) == 0).all()  # +0, not -0
    assert (o.residual_add(R, np.zeros_like(R)).view(np.uint16) == R.view(np.uint16)).all()
    # the halfway cases do round to even: about half of them round up
    hb = o.residual_add(base[None], half[None]).astype(np.float64)
    assert 0 < (hb > base.astype(np.float64) + half.astype(np.float64)).sum() < 64


def pin_round_16bit(o):
    """The 16-bit output rule: fp16 against NumPy's (independent) float64 ->
    float16 conversion, bf16 against torch's float32 -> bfloat16 conversion
    on values exact in float32, and both against exact rationals on values
    built to fall on, just beside and halfway between representable values
    (ties to even), subnormal fp16 values and powers of two."""
    import torch
    r = _rng(77)
    y = np.concatenate([r.standard_normal(4000) * 10.0 ** r.integers(-6, 4, 4000),
                        [0.0, -0.0, 1.0, -1.0, 65504.0, 2.0 ** -24, 3 * 2.0 ** -25, 2.0 ** -14]])
    assert np.array_equal(o.round_16bit(y, "f16"), y.astype(np.float16).astype(np.float64))
    y32 = y.astype(np.float32).astype(np.float64)
    tb = torch.from_numpy(y32.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(o.round_16bit(y32, "bf16"), tb)
    # exact rationals: k halfway points between neighbours q*n and q*(n+1)
    for kind, p in (("f16", 11), ("bf16", 8)):
        for E in (-3, 0, 5):
            q = Fraction(2) ** (E - (p - 1))
            for n in (2 ** (p - 1), 2 ** (p - 1) + 1, 2 ** p - 2, 2 ** p - 1):
                for num, want in ((Fraction(1, 2), n + (n % 2)),      # a tie: to the even one
                                  (Fraction(1, 2) - Fraction(1, 2 ** 20), n),
                                  (Fraction(1, 2) + Fraction(1, 2 ** 20), n + 1)):
                    v = (n + num) * q
                    got = Fraction(float(o.round_16bit(np.array([float(v)]), kind)[0]))
                    assert got == want * q, (kind, E, n, num)
    # a value that rounds up into the next binade keeps the even rule
    assert o.round_16bit(np.array([2047.5]), "f16")[0] == 2048.0
    assert o.round_16bit(np.array([255.5]), "bf16")[0] == 256.0


def pin_swiglu(o):
    """silu(g) * u against SciPy's logistic function (an independent
    routine): silu(g) = g * expit(g); plus silu(0) = 0, up = 0 gives 0,
    silu(g) - silu(-g) = g, large negative gates give -0 and no NaN, and the
    halves are taken in the documented order (gate first)."""
    from scipy.special import expit
    r = _rng(93)
    Y = r.standard_normal((7, 64)) * 4.0
    Y[0, :32] = 0.0
    Y[1, 32:] = 0.0
    Y[2, :4] = [-1000.0, -80.0, 80.0, 1000.0]
    got = o.swiglu(Y)
    g, u = Y[:, :32], Y[:, 32:]
    want = g * expit(g) * u
    assert np.isfinite(got).all()
    assert np.allclose(got, want, rtol=1e-13, atol=1e-300)
    assert (got[0] == 0).all() and (got[1] == 0).all()
    x = r.standard_normal(50) * 5
    s1 = o.swiglu(np.stack([x, np.ones(50)], axis=1).reshape(50, 2))[:, 0]
    s2 = o.swiglu(np.stack([-x, np.ones(50)], axis=1).reshape(50, 2))[:, 0]
    assert np.allclose(s1 - s2, x, rtol=1e-12, atol=1e-12)
    # gate first: swapping the halves changes the result
    assert not np.allclose(o.swiglu(np.concatenate([u, g], axis=1)), got)


def _progressive_rows(seed):
    """Weight rows for the progressive pins: N(0, 0.02) rows, a row with one
    large value (most groups then use a few codes), rows of constants (all
    groups identical, one positive and one negative), and rows built so that
    groups hit both ends of the first-level range."""
    r = _rng(seed, 95)
    K = 256
    W = r.standard_normal((6, K)) * 0.02
    W[1, 5] = 0.9
    W[2, :] = 0.01
    W[3, :] = -0.013
    W[4, ::2] = 0.05
    W[4, 1::2] = -0.05
    W[5, :128] = np.linspace(-0.07, 0.07, 128)
    return W.astype(np.float16)


def pin_progressive_levels(o):
    """Progressive INT4.  Level 1: the codes meet the quantization bound
    |w - q8 * s1| <= s1 (1/2 + slack) with the range 119, which each nonzero
    row's maximum reaches.  Level 2, by brute force on every group of those
    codes: s2 is the smallest integer >= 1 whose 15 steps span
    [min(0, min q8), max(0, max q8)]; z is the zero point in [0, 15] nearest
    to -min/s2 (ties to even); each u is the 4-bit value whose rebuilt code
    (u - z) * s2 is nearest to q8, ties to the even (u - z); rebuilt codes stay
    within INT8."""
    for seed in range(3):
        W = _progressive_rows(seed)
        q8p, s1, u, s2, z, q8 = o.progressive_quantize_weight(W)
        N, K = W.shape
        w = W.astype(np.float64)
        q8 = q8.astype(np.int64)
        for n in range(N):
            assert np.abs(q8[n]).max() <= 119
            if np.abs(w[n]).max() == 0:
                assert (q8[n] == 0).all() and s1[n] == 1
                continue
            err = np.abs(w[n] - q8[n] * float(s1[n]))
            assert err.max() <= float(s1[n]) * (0.5 + HALF_STEP_SLACK)
            assert np.abs(q8[n]).max() == 119
            for gi in range(K // 128):
                sl = slice(gi * 128, (gi + 1) * 128)
                S2, Z = int(s2[n, gi]), int(z[n, gi])
                rec = q8p[n, sl].astype(np.int64)
                uu = u[n, sl].astype(np.int64)
                assert 0 <= Z <= 15 and 1 <= S2 <= 16 and (uu >= 0).all() and (uu <= 15).all()
                assert (rec == (uu - Z) * S2).all() and np.abs(rec).max() <= 127
                lo = min(0, int(q8[n, sl].min()))
                hi = max(0, int(q8[n, sl].max()))
                best_s = next(t for t in range(1, 17) if 15 * t >= hi - lo)
                assert S2 == best_s, (n, gi, S2, best_s)
                cands = [(abs(Fraction(-lo, S2) - zz), zz % 2, zz) for zz in range(16)]
                assert Z == min(cands)[2], (n, gi)
                for k, qv in zip(range(128), q8[n, sl]):
                    cu = [(abs((c - Z) * S2 - int(qv)), (c - Z) % 2, c) for c in range(16)]
                    assert uu[k] == min(cu)[2], (n, gi, k, int(qv))


def pin_progressive_no_overflow(o):
    """Groups at both ends of the first-level range, for every scale the range
    allows: no rebuilt code leaves [-127, 127], and the maximum reaches 119 +
    s2/2 rounded to a multiple of s2 at most."""
    r = _rng(96)
    worst = 0
    for trial in range(40):
        W = (r.standard_normal((2, 128)) * 0.01).astype(np.float64)
        W[:, 0] = 0.1 * r.choice([-1, 1], 2)
        W[:, 1] = -W[:, 0] * r.uniform(0, 1, 2)
        q8p = o.progressive_quantize_weight(W.astype(np.float16))[0]
        worst = max(worst, int(np.abs(q8p.astype(np.int64)).max()))
    assert worst <= 127


def pin_mixed_feature(o):
    """Output-feature mixed precision: all rows salient gives the INT8 weight
    quantizer, no row salient gives progressive INT4, and in between every
    row carries exactly its own kind (rows are quantized independently, so
    permuting rows together with the mask permutes codes and scales)."""
    W = _progressive_rows(4)
    N = W.shape[0]
    q8, s8 = o.quantize_weight(W, 8)
    q4p, s4, *_ = o.progressive_quantize_weight(W)
    c, sc = o.mixed_feature_quantize_weight(W, np.ones(N, bool))
    assert (c == q8).all() and (sc.view(np.uint32) == s8.view(np.uint32)).all()
    c, sc = o.mixed_feature_quantize_weight(W, np.zeros(N, bool))
    assert (c == q4p).all() and (sc.view(np.uint32) == s4.view(np.uint32)).all()
    mask = np.array([True, False, True, False, False, True])
    c, sc = o.mixed_feature_quantize_weight(W, mask)
    for n in range(N):
        assert (c[n] == (q8[n] if mask[n] else q4p[n])).all()
        assert sc[n] == (s8[n] if mask[n] else s4[n])
    perm = np.array([3, 0, 5, 1, 4, 2])
    cp, scp = o.mixed_feature_quantize_weight(np.ascontiguousarray(W[perm]), mask[perm])
    assert (cp == c[perm]).all() and (scp == sc[perm]).all()
    # the 8-bit rows really are finer than their 4-bit versions
    err8 = np.abs(q8[mask].astype(np.float64) * s8[mask, None] - W[mask].astype(np.float64)).max()
    err4 = np.abs(q4p[mask].astype(np.float64) * s4[mask, None] - W[mask].astype(np.float64)).max()
    assert err8 < err4


ALL_PINS = [pin_golden_act, pin_golden_weight, pin_golden_layer, pin_half_decode,
            pin_set_bruteforce, pin_quant_error_bound, pin_nearest_code, pin_weight_bound,
            pin_int_gemm_bruteforce, pin_split_identity, pin_output_vs_dequant,
            pin_output_vs_truth_bound, pin_no_outlier_textbook, pin_all_outlier,
            pin_sign_symmetry, pin_pow2_scaling, pin_permutation, pin_overflow,
            pin_decode_sequence, pin_layer_driver, pin_sampled_output, pin_rmsnorm_fsum, pin_rmsnorm_bound,
            pin_rmsnorm_invariants, pin_rmsnorm_closed_form, pin_rmsnorm_exact_rationals,
            pin_residual_add, pin_round_16bit, pin_swiglu, pin_progressive_levels, pin_progressive_no_overflow,
            pin_mixed_feature]
