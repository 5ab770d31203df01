"""The layer step replayed from a captured HIP graph (``mixq.LayerGraph``)
computes exactly what the eager calls compute: every replay, with eager work
between replays, including replays in which the outlier gate fires and the
set grows.  Compared bit for bit with an eager twin layer on the same inputs
(the eager path itself is pinned to the oracle by the parity tests)."""
import numpy as np
import pytest
import torch

from gpu_util import GpuLayer, say, to_dev
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu


def snapshot(g: GpuLayer):
    torch.cuda.synchronize()
    return dict(Xq=g.Xq.cpu().numpy().copy(), s_x=g.s_x.cpu().numpy().view(np.uint32).copy(),
                X_out=(g.X_out.view(torch.int16).cpu().numpy().copy() if g.X_out is not None
                       else None),
                Y=g.Y.cpu().numpy().view(np.uint32).copy(), count=g.count(), flag=g.flag(),
                idx=g.idx().copy())


def assert_same(a, b, tag):
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), f"{tag}: {k} differs"


def run_pair(inputs, W, bits, tau, k_cap):
    M, K = inputs[0].shape
    eager = GpuLayer(W, bits, tau, k_cap, M)
    graphed = GpuLayer(W, bits, tau, k_cap, M)
    Xd = torch.empty(M, K, dtype=torch.float16, device="cuda")
    lg = mixq.LayerGraph(Xd, tau, graphed.state, graphed.Wd, graphed.pw, graphed.Xq,
                         graphed.s_x, graphed.X_out, graphed.Y, ws=graphed.ws)
    flags = []
    for t, X in enumerate(inputs):
        say(f"[graph] replay {t} M={M} K={K} N={W.shape[0]}")
        eager.step(X)
        Xd.copy_(to_dev(X.view(np.float16)))  # eager work between replays
        lg.replay()
        a, b = snapshot(eager), snapshot(graphed)
        assert_same(a, b, f"replay {t}")
        flags.append(b["flag"])
    return flags, graphed


def test_graph_replays_match_eager_small():
    M, K, N = 48, 1024, 256
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    pers = np.sort(rng.choice(K, 6, replace=False))
    inputs = []
    for t in range(5):
        X = rng.standard_normal((M, K)).astype(np.float32)
        X[:, pers] = rng.uniform(20, 100, (M, pers.size))
        if t == 2:
            X[:, rng.integers(0, K, 3)] = 40.0  # new channels: the gate fires in a replay
        inputs.append(X.astype(np.float16))
    flags, g = run_pair(inputs, W, 8, 6.0, 64)
    assert flags[0] == mixq.FLAG_FIRED and flags[1] == 0 and flags[2] == mixq.FLAG_FIRED
    # the set the replays built is the oracle's
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=Oracle())
    for X in inputs:
        r = o.step(X, products=False)
    assert g.count() == r.count and np.array_equal(g.idx(), np.flatnonzero(r.in_set))


def test_graph_replays_match_eager_int4():
    M, K, N = 40, 512, 160
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    inputs = []
    for t in range(3):
        X = rng.standard_normal((M, K)).astype(np.float32)
        X[:, [5, 77, 300]] = 30.0
        inputs.append(X.astype(np.float16))
    run_pair(inputs, W, 4, 6.0, 32)


def test_graph_replays_match_eager_full_size():
    """The timed configuration: M=2048, K=N=8192, INT8 weights."""
    wl = workloads.WORKLOADS["prefill_w8"]
    W = workloads.make_weight(wl)
    X = workloads.make_activation(wl)
    run_pair([X, X, X], W, wl.bits, wl.tau, 256)
