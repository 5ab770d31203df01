"""Many tokens (M = 16385, one past a multiple of every tile height): the
activation pass walks several token rounds per block (its grid is capped),
the re-quantize pass of the first call loops over many rows per block, and
the product covers many row tiles with a ragged last one.  A first call
(the gate fires and forms the set) and a steady call on the cached set, both
against the oracle: the activation side bit for bit, acc and Y at sampled
positions."""
import numpy as np
import pytest
import torch

from gpu_util import GpuLayer, compare_quant, say
from mixed_precision_quantized_amax_amd import workloads
from oracle import Oracle, OracleLayer
from test_gpu_parity import sample_positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return Oracle()


@pytest.mark.parametrize("bits", [8, 4])
def test_many_tokens(orc, bits):
    M, K, N = 16385, 4096, 1000
    X, W, ch = workloads.random_case(seed=11, M=M, K=K, N=N, n_out=40)
    # the same channels at half the size, rows in another order: the cached
    # set covers them and the rest stays under the threshold
    perm = np.random.default_rng(12).permutation(M)
    X2 = (X[perm].astype(np.float32) * np.float32(0.5)).astype(np.float16)
    g = GpuLayer(W, bits, 6.0, 256, M)
    o = OracleLayer(W=W, bits=bits, tau=6.0, k_cap=256, ldo=g.ld, oracle=orc)
    rows, cols = sample_positions(M, N, n=2000)
    for step, Xs in enumerate([X, X2]):
        say(f"[large-m] bits={bits} step {step}: M={M} K={K} N={N}")
        g.step(Xs)
        r = o.step(Xs, products=False)
        compare_quant(g, Xs, r)
        assert r.flag == (1 if step == 0 else 0)
        W_out = orc.gather_weight_cols(W, r.in_set, g.ld)
        a_s, y_s = orc.sampled_output(r.Xq, o.Wq, r.s_x, o.s_w, r.X_out, W_out, r.count,
                                      rows, cols)
        dbg = torch.zeros(M, N, dtype=torch.int32, device="cuda")
        g.gemm(dbg)
        torch.cuda.synchronize()
        assert np.array_equal(dbg.cpu().numpy()[rows, cols], a_s)
        Y = g.Y.cpu().numpy()
        err = float(np.abs(Y[rows, cols] - y_s).max()) / float(np.abs(Y).max())
        assert err <= 1e-3, err
        say(f"[large-m] ok: count={r.count} flag={r.flag} max|dY|/max|Y|={err:.2e}")
