"""Products whose 256 x 256 tiles come to one round of the device plus a short
second round: the library then runs the columns that fill one round with
256 x 256 tiles and the rest as a second launch of 128 x 128 tiles.  Every
weight format through that path against the oracle: quantized data, all
int32 accumulators bit for bit, Y within 1e-3 * max|Y|, every column
written."""
import numpy as np
import pytest
import torch

from gpu_util import GpuLayer, check_y, say
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer
from test_gpu_mixed import check_pack, run_mixed, salient_set
from test_gpu_parity import full_compare
from test_gpu_progressive import check_codes, run_progressive

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return Oracle()


def splits(M, N):
    """The host's rule: 256 x 256 tiles beyond one round, a tail of at most
    half the device in 256 x 256 tiles."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm, tn = -(-M // 256), -(-N // 256)
    fit = cus // tm
    return fit > 0 and tn > fit and 2 * (tn - fit) * tm <= cus


@pytest.mark.parametrize("M,K,N,bits", [(2048, 1024, 8448, 8), (1024, 512, 16520, 8),
                                        (2048, 1024, 8448, 4), (1800, 512, 8300, 4)])
def test_tail_split(orc, M, K, N, bits):
    """With a workspace the tail's K is split too (last arriver adds the
    partials): everything equals the oracle, and Y equals the run without a
    workspace bit for bit; the tile counters are left at zero."""
    assert splits(M, N), "shape expected to split off a tail"
    X, W, _ = workloads.random_case(seed=M + N + bits, M=M, K=K, N=N, n_out=6)
    g, _ = full_compare(orc, X, W, bits, 6.0, 64, tag=f"tail bits={bits}")
    assert g.ws is not None, "the tail's K is expected to split"
    y = g.Y.cpu().numpy()
    assert not np.isnan(y).any()
    h = GpuLayer(W, bits, 6.0, 64, M, split=False)
    h.step(X)
    assert np.array_equal(h.Y.cpu().numpy().view(np.uint32), y.view(np.uint32))
    for _ in range(2):  # repeated calls reuse the counters
        g.gemm()
    torch.cuda.synchronize()
    assert np.array_equal(g.Y.cpu().numpy().view(np.uint32), y.view(np.uint32))
    assert int(g.ws[:1024].abs().sum().cpu()) == 0, "tile counters not cleared"


def test_tail_split_progressive(orc):
    M, K, N = 2048, 1024, 8448
    assert splits(M, N)
    X, W, _ = workloads.random_case(seed=5, M=M, K=K, N=N, n_out=4)
    g = run_progressive(X, W, 6.0, 64, ws=True)
    assert g["ws"] is not None, "the tail's K is expected to split"
    q8p, s1 = check_codes(orc, g, W)
    h = run_progressive(X, W, 6.0, 64, acc=False)
    assert np.array_equal(h["Y"].view(np.uint32), g["Y"].view(np.uint32))
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=orc)
    r = o.step(X, products=False)
    acc = orc.int_gemm(r.Xq, q8p)
    assert np.array_equal(g["acc"], acc)
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(64))
    err = check_y(g["Y"], orc.output(acc, r.s_x, s1, r.X_out, W_out, r.count))
    say(f"[tail] progressive ok, max|dY|/max|Y|={err:.2e}")


@pytest.mark.parametrize("N,S", [(8548, 100), (8704, 300), (8600, 8500)])
def test_tail_split_mixed(orc, N, S):
    """Output-feature mixed precision with a part of more than 8192 rows: the
    4-bit part (8448 or 8404 rows), or the 8-bit part (8500 rows), splits
    off a tail."""
    M, K = 2048, 512
    X, W, _ = workloads.random_case(seed=S, M=M, K=K, N=N, n_out=4)
    sal = salient_set(N, S, S)
    g = run_mixed(X, W, sal, 6.0, 64, ws=True)
    big = max(g["mw"].parts(), key=lambda p: p.N)
    assert splits(M, big.N), "a part expected to split off a tail"
    h = run_mixed(X, W, sal, 6.0, 64, acc=False)
    assert np.array_equal(h["Y"].view(np.uint32), g["Y"].view(np.uint32))
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=orc)
    r = o.step(X, products=False)
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(64))
    codes, scales = check_pack(orc, g, W, sal, W_out)
    acc = orc.int_gemm(r.Xq, codes)
    a4, a8 = g["acc"]
    assert np.array_equal(a4, acc[:, ~sal]) and np.array_equal(a8, acc[:, sal])
    assert not np.isnan(g["Y"]).any(), "an output feature was not written"
    err = check_y(g["Y"], orc.output(acc, r.s_x, scales, r.X_out, W_out, r.count))
    say(f"[tail] mixed S={S} ok, max|dY|/max|Y|={err:.2e}")
