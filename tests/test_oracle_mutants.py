"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a dropped term, a
wrong comparison, a wrong index, a wrong constant, ...), builds the copy into
a temporary directory and runs every pin on it: at least one pin must fail.
The mistakes are planted in the oracle only, on the CPU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle_pins
from oracle import Oracle
from oracle.mixq_oracle import CFLAGS, _SRC

# (name, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("gate_ge", "if (g > tau) fired = 1;", "if (g >= tau) fired = 1;", 0),
    ("detect_ge", "> tau) hit = 1;", ">= tau) hit = 1;", 0),
    ("gate_ignores_cache", "if (in_set[k]) continue;", ";", 0),
    ("fresh_set_not_union", "int hit = in_set[k] ? 1 : 0;", "int hit = 0;", 0),
    ("overflow_ge", "if (after > k_cap)", "if (after >= k_cap)", 0),
    ("round_half_away", "nearbyintf(x * recip)", "roundf(x * recip)", 0),
    ("scale_off_by_one", "*scale = amax / (float)qmax;", "*scale = amax / (float)(qmax + 1);", 0),
    ("recip_off_by_one", "*recip = (float)qmax / amax;", "*recip = (float)(qmax - 1) / amax;", 0),
    ("zero_scale_rule", "*scale = 1.0f;", "*scale = 0.0f;", 0),
    ("act_amax_includes_outliers", "if (in_set[k]) continue;", ";", 1),
    ("outlier_code_not_zeroed", "Xq[m * K + k] = in_set[k] ? 0", "Xq[m * K + k] = 0 ? 0", 0),
    ("list_descending", "for (k = 0; k < K; ++k)\n        if (in_set[k]) idx[n++] = (int32_t)k;",
     "for (k = K - 1; k >= 0; --k)\n        if (in_set[k]) idx[n++] = (int32_t)k;", 0),
    ("xout_wrong_column", "X_out[m * ldo + j++] = row[k];", "X_out[m * ldo + j++] = row[K - 1 - k];", 0),
    ("wout_wrong_column", "W_out[n * ldo + j++] = W[n * K + k];",
     "W_out[n * ldo + j++] = W[n * K + (K - 1 - k)];", 0),
    ("gemm_reversed_k", "s += (int64_t)Xq[m * K + k] * (int64_t)Wq[n * K + k];",
     "s += (int64_t)Xq[m * K + k] * (int64_t)Wq[n * K + (K - 1 - k)];", 0),
    ("gemm_narrow_accumulator", "int64_t s = 0;", "int16_t s = 0;", 0),
    ("output_drops_outliers", "y += (double)orc_half_to_float(X_out[m * ldxo + j]) *",
     "y += 0.0 * (double)orc_half_to_float(X_out[m * ldxo + j]) *", 0),
    ("output_drops_weight_scale",
     "double y = (double)acc[m * N + n] * (double)s_x[m] * (double)s_w[n];",
     "double y = (double)acc[m * N + n] * (double)s_x[m];", 0),
    ("output_sign", "double y = (double)acc[m * N + n] * (double)s_x[m] * (double)s_w[n];",
     "double y = -(double)acc[m * N + n] * (double)s_x[m] * (double)s_w[n];", 0),
    ("sampled_reversed_k", "s += (int64_t)Xq[m * K + kk] * (int64_t)Wq[n * K + kk];",
     "s += (int64_t)Xq[m * K + kk] * (int64_t)Wq[n * K + (K - 1 - kk)];", 0),
    ("sampled_drops_outliers", "y += (double)orc_half_to_float(X_out[m * ldxo + j]) *",
     "y += 0.0 * (double)orc_half_to_float(X_out[m * ldxo + j]) *", 1),
    ("int4_range", "return (1 << (bits - 1)) - 1;", "return (1 << bits) - 1;", 0),
    ("half_exponent_bias", "expo - 25", "expo - 24", 0),
    ("half_subnormal", "ldexpf((float)mant, -24)", "ldexpf((float)mant, -25)", 0),
]


def _apply(src, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation site not found: {old!r} #{occ}"
    return src[:pos] + new + src[pos + len(old):]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="mixq_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new, occ):
    with open(_SRC) as f:
        src = f.read()
    mutated = _apply(src, old, new, occ)
    assert mutated != src
    c_path = os.path.join(workdir, f"{name}.c")
    so_path = os.path.join(workdir, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", *CFLAGS, c_path, "-o", so_path, "-lm"], check=True)
    o = Oracle(so_path)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"


# Mistakes planted in the oracle's RMSNorm (Python source of
# ``oracle.mixq_oracle.rmsnorm``): (name, text to replace, replacement)
RMS_MUTANTS = [
    ("norm_fp32_running_sum", "S = float(s_units) * 2.0 ** -48",
     "S = float((Hh[m].astype(np.float32) ** 2).sum(dtype=np.float32))"),
    ("norm_limb_shift", "(int(B[m]) << 21)", "(int(B[m]) << 20)"),
    ("norm_mean_over_k_plus_1", "ms = np.float32(S / K)", "ms = np.float32(S / (K + 1))"),
    ("norm_eps_outside_sqrt", "np.float32(1.0) / np.sqrt(t)",
     "np.float32(1.0) / (np.sqrt(ms) + e32)"),
    ("norm_no_sqrt", "np.float32(1.0) / np.sqrt(t)", "np.float32(1.0) / t"),
    ("norm_zero_row_rule", "np.float32(0.0) if t == 0", "np.float32(1.0) if t == 0"),
    ("norm_single_rounding", "n = (Hh.astype(np.float32) * rstd[:, None]).astype(np.float16)",
     "n = Hh.astype(np.float32) * rstd[:, None]"),
    ("norm_no_gamma", "X = (n.astype(np.float32) * g.astype(np.float32)).astype(np.float16)",
     "X = n.astype(np.float16)"),
]


_SUM = "return (r.astype(np.float64) + d.astype(np.float64)).astype(np.float16)"
RES_MUTANTS = [
    ("add_truncates", _SUM,
     "s = r.astype(np.float64) + d.astype(np.float64)\n    t = s.astype(np.float16)\n"
     "    return np.where(np.abs(t.astype(np.float64)) > np.abs(s), "
     "np.nextafter(t, np.float16(0)), t)"),
    ("add_ties_away", _SUM,
     "s = r.astype(np.float64) + d.astype(np.float64)\n"
     "    return (s + np.sign(s) * 2.0 ** -40).astype(np.float16)"),
    ("add_flushes_subnormals", _SUM,
     "t = (r.astype(np.float64) + d.astype(np.float64)).astype(np.float16)\n"
     "    return np.where(np.abs(t) < 2.0 ** -14, t * np.float16(0), t)"),
]


SWIGLU_MUTANTS = [
    ("swiglu_halves_swapped", "g, u = Y[:, : N2 // 2], Y[:, N2 // 2:]",
     "u, g = Y[:, : N2 // 2], Y[:, N2 // 2:]"),
    ("swiglu_sign", "return g / (1.0 + np.exp(-g)) * u", "return g / (1.0 + np.exp(g)) * u"),
    ("swiglu_no_gate_factor", "return g / (1.0 + np.exp(-g)) * u",
     "return 1.0 / (1.0 + np.exp(-g)) * u"),
]


PROG_MUTANTS = [
    ("prog_range_127", "Q1 = Q1_PROGRESSIVE", "Q1 = 127"),
    ("prog_zero_not_in_range", "lo = np.minimum(g8.min(axis=2), 0)", "lo = g8.min(axis=2)"),
    ("prog_scale_floor", "s2 = np.maximum(1, -((lo - hi) // 15))",
     "s2 = np.maximum(1, (hi - lo) // 15)"),
    ("prog_code_floor", "u = np.clip(_rne_div(g8, s2[:, :, None]) + z[:, :, None], 0, 15)",
     "u = np.clip(g8 // s2[:, :, None] + z[:, :, None], 0, 15)"),
    ("prog_zero_sign", "z = _rne_div(-lo, s2)", "z = _rne_div(lo, s2) % 16"),
]

MIXED_MUTANTS = [
    ("mixed_mask_inverted", "codes = np.where(sal[:, None], q8, q4p)",
     "codes = np.where(~sal[:, None], q8, q4p)"),
    ("mixed_scales_swapped", "scales = np.where(sal, s8, s4)", "scales = np.where(sal, s4, s8)"),
    ("mixed_int4_rows_symmetric", "q4p, s4, *_ = progressive_quantize_weight(Wh, group)",
     "q4p, s4 = o.quantize_weight(Wh, 4)"),
    ("mixed_int4_values_not_rebuilt", "q4p, s4, *_ = progressive_quantize_weight(Wh, group)",
     "_, s4, q4p, *_ = progressive_quantize_weight(Wh, group)"),
]
ROUND16_MUTANTS = [
    ("round16_ties_away", "out[nz] = np.rint(y[nz] / q) * q",
     "out[nz] = np.sign(y[nz]) * np.floor(np.abs(y[nz] / q) + 0.5) * q"),
    ("round16_truncates", "out[nz] = np.rint(y[nz] / q) * q", "out[nz] = np.trunc(y[nz] / q) * q"),
    ("round16_fp16_precision", '"f16": (11, -14)', '"f16": (10, -14)'),
    ("round16_bf16_as_f16", '"bf16": (8, -126)', '"bf16": (11, -14)'),
]
PIN_KEY = {"progressive_quantize_weight": "progressive",
           "mixed_feature_quantize_weight": "mixed_feature"}


@pytest.mark.parametrize("fn,name,old,new",
                         [("rmsnorm", *m) for m in RMS_MUTANTS] +
                         [("residual_add", *m) for m in RES_MUTANTS] +
                         [("swiglu", *m) for m in SWIGLU_MUTANTS] +
                         [("progressive_quantize_weight", *m) for m in PROG_MUTANTS] +
                         [("mixed_feature_quantize_weight", *m) for m in MIXED_MUTANTS] +
                         [("round_16bit", *m) for m in ROUND16_MUTANTS],
                         ids=[m[0] for m in RMS_MUTANTS] + [m[0] for m in RES_MUTANTS] +
                         [m[0] for m in SWIGLU_MUTANTS] + [m[0] for m in PROG_MUTANTS] +
                         [m[0] for m in MIXED_MUTANTS] + [m[0] for m in ROUND16_MUTANTS])
def test_prologue_mutant_is_caught(fn, name, old, new):
    import inspect
    import textwrap

    import numpy as np

    from oracle import mixq_oracle

    src = textwrap.dedent(inspect.getsource(getattr(mixq_oracle, fn)))
    assert src.count(old) == 1, f"mutation site not found: {old!r}"
    ns = {"np": np, "Q1_PROGRESSIVE": mixq_oracle.Q1_PROGRESSIVE, "_rne_div": mixq_oracle._rne_div,
          "GROUP": mixq_oracle.GROUP, "Oracle": Oracle,
          "progressive_quantize_weight": mixq_oracle.progressive_quantize_weight}
    exec(compile(src.replace(old, new), f"<{name}>", "exec"), ns)

    class Mutant(Oracle):
        pass

    setattr(Mutant, fn, lambda self, *args: ns[fn](*args))
    o = Mutant()
    failed = []
    for pin in oracle_pins.ALL_PINS:
        key = PIN_KEY.get(fn, fn)
        if key not in pin.__name__:
            continue
        try:
            pin(o)
        except (AssertionError, OverflowError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"


# Mistakes planted in the decode driver (``OracleLayer.step``): the set not
# carried from call to call, the weight's outlier columns gathered for the
# previous set, a wrong set size passed to the output.
DRIVER_MUTANTS = [
    ("driver_set_not_persisted",
     "o.update_outlier_set(X, self.tau, before, self.k_cap)",
     "o.update_outlier_set(X, self.tau, np.zeros_like(before), self.k_cap)"),
    ("driver_wout_previous_set",
     "W_out = o.gather_weight_cols(self.W, self.in_set, self.ldo)",
     "W_out = o.gather_weight_cols(self.W, before, self.ldo)"),
    ("driver_wrong_count",
     "res.Y = o.output(res.acc, s_x, self.s_w, X_out, W_out, count)",
     "res.Y = o.output(res.acc, s_x, self.s_w, X_out, W_out, max(count - 1, 0))"),
]


@pytest.mark.parametrize("name,old,new", DRIVER_MUTANTS, ids=[m[0] for m in DRIVER_MUTANTS])
def test_driver_mutant_is_caught(name, old, new):
    import inspect
    import textwrap

    import numpy as np

    from oracle import mixq_oracle

    src = textwrap.dedent(inspect.getsource(mixq_oracle.OracleLayer.step))
    assert src.count(old) == 1, f"mutation site not found: {old!r}"
    ns = {"np": np, "LayerResult": mixq_oracle.LayerResult}
    exec(compile(src.replace(old, new), f"<{name}>", "exec"), ns)

    class Mutant(mixq_oracle.OracleLayer):
        step = ns["step"]

    with pytest.raises(AssertionError):
        oracle_pins.pin_layer_driver(Oracle(), layer_cls=Mutant)


def test_driver_unmutated_copy_passes():
    """The copy mechanism itself leaves a working driver: the same source
    recompiled without a change passes the pin."""
    import inspect
    import textwrap

    import numpy as np

    from oracle import mixq_oracle

    src = textwrap.dedent(inspect.getsource(mixq_oracle.OracleLayer.step))
    ns = {"np": np, "LayerResult": mixq_oracle.LayerResult}
    exec(compile(src, "<copy>", "exec"), ns)

    class Copy(mixq_oracle.OracleLayer):
        step = ns["step"]

    oracle_pins.pin_layer_driver(Oracle(), layer_cls=Copy)
