"""The largest supported K (65536): the activation pass then walks each token
in several register segments, and an INT8 accumulator can reach
K * 127 * 127 = 1 057 030 144, just under 2^31.  Everything against the
oracle: quantized data and accumulators bit for bit, Y within tolerance."""
import numpy as np
import pytest

from gpu_util import check_y, say
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer
from test_gpu_parity import full_compare
from test_gpu_progressive import check_codes, run_progressive

pytestmark = pytest.mark.gpu

K = 65536


@pytest.fixture(scope="module")
def orc():
    return Oracle()


@pytest.mark.parametrize("bits", [8, 4])
def test_max_k_random(orc, bits):
    X, W, _ = workloads.random_case(seed=bits, M=70, K=K, N=200, n_out=12)
    full_compare(orc, X, W, bits, 6.0, 64, tag=f"K={K}")


def test_max_k_extreme_accumulators(orc):
    """Every activation and weight equal: every code is +-127, every
    accumulator -K * 127 * 127 (compared element by element inside
    full_compare) and every output X . W = -K * 1.5 * 0.25."""
    X = np.full((40, K), 1.5, np.float16)
    W = np.full((130, K), -0.25, np.float16)
    g, o = full_compare(orc, X, W, 8, 6.0, 0, tag="extreme")
    assert (o.Wq == -127).all() and (g.Xq.cpu().numpy() == 127).all()
    Y = g.Y.cpu().numpy()
    assert np.abs(Y / (-K * 0.375) - 1).max() < 1e-5


def test_max_k_progressive(orc):
    X, W, _ = workloads.random_case(seed=3, M=70, K=K, N=200, n_out=12)
    g = run_progressive(X, W, 6.0, 64)
    q8p, s1 = check_codes(orc, g, W)
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    acc = orc.int_gemm(r.Xq, q8p)
    assert np.array_equal(g["acc"], acc)
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(64))
    err = check_y(g["Y"], orc.output(acc, r.s_x, s1, r.X_out, W_out, r.count))
    say(f"[maxk] progressive ok, max|dY|/max|Y|={err:.2e}")
