"""A seeded sweep of random shapes through the automatic launch choice: M,
N and K drawn independently (K a multiple of 64), INT8 and INT4 weights,
outlier capacities from none to 256, planted channels from none to more than
the capacity.  Everything against the oracle, element by element."""
import numpy as np
import pytest

from mixed_precision_quantized_amax_amd import workloads
from oracle import Oracle
from test_gpu_parity import full_compare

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
