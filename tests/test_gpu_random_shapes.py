"""A seeded sweep of random shapes through the automatic launch choice: M,
N and K drawn independently (K a multiple of 64), INT8 and INT4 weights,
outlier capacities from none to 256, planted channels from none to more than
the capacity; and progressive INT4 weights (K a multiple of 128).
Everything against the oracle, element by element."""
import numpy as np
import pytest

from gpu_util import check_y
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer
from test_gpu_parity import full_compare
from test_gpu_progressive import check_codes, run_progressive

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 600))
        N = int(rng.integers(1, 600))
        K = 64 * int(rng.integers(1, 33))
        bits = int(rng.choice([8, 4]))
        k_cap = int(rng.choice([0, 8, 64, 256]))
        n_out = int(rng.integers(0, min(K, 40) + 1))
        out.append((i, M, K, N, bits, min(k_cap, K), n_out))
    return out


@pytest.fixture(scope="module")
def orc():
    return Oracle()


@pytest.mark.parametrize("i,M,K,N,bits,k_cap,n_out", _cases())
def test_random_shape(orc, i, M, K, N, bits, k_cap, n_out):
    X, W, _ = workloads.random_case(seed=100 + i, M=M, K=K, N=N, n_out=n_out)
    full_compare(orc, X, W, bits, 6.0, k_cap, tag=f"rand{i}")


def _prog_cases(n=12, seed=2025):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 600)), 128 * int(rng.integers(1, 17)), int(rng.integers(1, 600)),
             int(rng.integers(0, 30))) for i in range(n)]


@pytest.mark.parametrize("i,M,K,N,n_out", _prog_cases())
def test_random_shape_progressive(orc, i, M, K, N, n_out):
    """Progressive group-wise INT4 weights: 4-bit values, group table and
    scales bit for bit, accumulators of the rebuilt INT8 codes bit for bit,
    Y within tolerance."""
    X, W, _ = workloads.random_case(seed=300 + i, M=M, K=K, N=N, n_out=n_out)
    g = run_progressive(X, W, 6.0, 64)
    q8p, s1 = check_codes(orc, g, W)
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    acc = orc.int_gemm(r.Xq, q8p)
    assert np.array_equal(g["acc"], acc)
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(64))
    check_y(g["Y"], orc.output(acc, r.s_x, s1, r.X_out, W_out, r.count))
