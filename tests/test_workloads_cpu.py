"""The synthetic inputs against their stated recipe, on the CPU: shapes and
dtypes, outlier fractions, the planted channels being exactly the channels
above the threshold, magnitudes and signs of the planted values, the decode
sequence's transient events, the weight spread, the salient fraction of a
mixed-precision weight, and seeding."""
import numpy as np
import pytest

from mixed_precision_quantized_amax_amd import workloads

W8 = workloads.WORKLOADS


@pytest.mark.parametrize("name", list(W8))
def test_planted_channels_are_the_channels_above_the_threshold(name):
    wl = W8[name]
    M = min(wl.M, 64)
    X = workloads.make_activation(wl, M=M)
    assert X.dtype == np.float16 and X.shape == (M, wl.K)
    ch = workloads.outlier_channels(wl)
    assert ch.size == wl.n_outliers and np.all(np.diff(ch) > 0)
    above = np.nonzero((np.abs(X.astype(np.float32)) > wl.tau).any(axis=0))[0]
    assert np.array_equal(above, ch)
    rest = np.delete(X.astype(np.float32), ch, axis=1)
    assert abs(float(rest.mean())) < 0.01 and abs(float(rest.std()) - 1.0) < 0.01
    planted = X[:, ch].astype(np.float32)
    if wl.outlier_kind == "uniform":
        assert np.all(np.abs(planted) >= wl.lo) and np.all(np.abs(planted) <= wl.hi)
        frac_neg = float((planted < 0).mean())
        assert 0.4 < frac_neg < 0.6
    else:
        assert abs(float(planted.std()) / wl.factor - 1.0) < 0.1


def test_outlier_fractions():
    assert W8["llama70b_up"].n_outliers == round(0.01 * 8192)
    assert W8["prefill_w8"].n_outliers == round(0.01 * 8192)
    assert W8["prefill_w4"].n_outliers == round(0.005 * 8192)
    assert W8["prefill_w4"].factor == 60.0 and W8["tiny"].factor == 50.0
    assert (W8["tiny"].M, W8["tiny"].K, W8["tiny"].N, W8["tiny"].n_outliers) == (16, 512, 512, 4)


def test_decode_plan():
    wl = W8["decode_seq"]
    plan = workloads.decode_plan(wl)
    assert plan.persistent.size == 40
    assert len(plan.events) == round(0.05 * wl.steps)
    for st, ids in plan.events.items():
        assert 0 <= st < wl.steps and 1 <= ids.size <= 4
        assert np.intersect1d(ids, plan.persistent).size == 0
    st = min(plan.events)
    X = workloads.decode_step(wl, st, plan).astype(np.float32)
    above = np.nonzero((np.abs(X) > wl.tau).any(axis=0))[0]
    assert np.array_equal(above, np.union1d(plan.persistent, plan.events[st]))
    quiet = next(s for s in range(wl.steps) if s not in plan.events)
    X = workloads.decode_step(wl, quiet, plan).astype(np.float32)
    assert np.array_equal(np.nonzero((np.abs(X) > wl.tau).any(axis=0))[0], plan.persistent)


def test_weight_spread_and_seeding():
    wl = W8["tiny"]
    W = workloads.make_weight(wl)
    assert W.dtype == np.float16 and W.shape == (wl.N, wl.K)
    assert abs(float(W.astype(np.float64).std()) / wl.w_std - 1.0) < 0.01
    assert np.array_equal(W, workloads.make_weight(wl))
    assert not np.array_equal(W, workloads.make_weight(wl, seed=1))
    X = workloads.make_activation(wl)
    assert np.array_equal(X, workloads.make_activation(wl))
    assert not np.array_equal(X, workloads.make_activation(wl, seed=1))


def test_salient_fraction():
    for N in (8192, 1000, 7):
        sal = workloads.make_salient(N)
        assert sal.dtype == bool and sal.shape == (N,)
        assert int(sal.sum()) == int(round(0.1 * N))
        assert np.array_equal(sal, workloads.make_salient(N))
