"""16-bit output modes (MIXQ_OUT_F16, MIXQ_OUT_BF16) of mixq_gemm_ex against
the oracle.  Each 16-bit value must be the kernel's own fp32 output rounded
to nearest even (bit for bit against torch's conversion of the fp32 output
of the same product), and must equal the oracle's float64 Y rounded by the
oracle's pinned rule, except where that Y lies so close to a rounding
midpoint that the fp32 output's own distance from the oracle (itself
within 1e-3 * max|Y|) covers both neighbours; there the result must be one
of the two."""
import numpy as np
import pytest
import torch

from gpu_util import GpuLayer, say
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu

KINDS = {"f16": (mixq.OUT_F16, torch.float16), "bf16": (mixq.OUT_BF16, torch.bfloat16)}


@pytest.fixture(scope="module")
def orc():
    return Oracle()


def check16(orc, X, W, bits, kind, tag):
    M, K = X.shape
    N = W.shape[0]
    mode, dt = KINDS[kind]
    g = GpuLayer(W, bits, 6.0, 64, M)
    g.step(X)
    Y16 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    mixq.gemm_ex(g.Xq, g.s_x, g.X_out, g.state, g.pw, Y16, mode, None, g.ws)
    torch.cuda.synchronize()
    # the kernel's own fp32 output rounded to nearest even, bit for bit
    assert torch.equal(Y16.view(torch.int16), g.Y.to(dt).view(torch.int16)), tag
    r = OracleLayer(W=W, bits=bits, tau=6.0, k_cap=64, ldo=g.ld, oracle=orc).step(X)
    ref = orc.round_16bit(r.Y, kind)
    got = Y16.to(torch.float64).cpu().numpy()
    # the fp32 output's own distance from the oracle (within 1e-3 * max|Y|)
    delta = float(np.abs(g.Y.cpu().numpy().astype(np.float64) - r.Y).max())
    assert delta <= 1e-3 * float(np.abs(r.Y).max()), tag
    # so each 16-bit value lies within half its own quantum (its rounding) plus
    # delta of the oracle's Y; it equals the oracle's rounded Y wherever no
    # rounding boundary lies within delta of the oracle's value
    p, qmin = (11, 2.0 ** -24) if kind == "f16" else (8, 2.0 ** -133)
    e = np.frexp(np.abs(got))[1]                   # |got| = m * 2^e, m in [0.5, 1)
    q = np.maximum(np.ldexp(1.0, e - p), qmin)     # quantum of got's binade
    assert (np.abs(got - r.Y) <= q / 2 + delta).all(), tag
    bad = got != ref
    if bad.any():
        mid = (got[bad] + ref[bad]) / 2
        assert np.abs(r.Y[bad] - mid).max() <= delta, tag
    say(f"[out16] {tag} {kind}: {int(bad.sum())} of {bad.size} within {delta:.1e} of a "
        f"rounding midpoint")


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("M,K,N,n_out,bits", [(37, 256, 80, 3, 8), (300, 1024, 520, 9, 8),
                                               (257, 2048, 300, 5, 4), (513, 1088, 129, 2, 8)])
def test_out16_random(orc, kind, M, K, N, n_out, bits):
    X, W, _ = workloads.random_case(seed=M + N + bits, M=M, K=K, N=N, n_out=n_out)
    check16(orc, X, W, bits, kind, f"M={M} K={K} N={N} bits={bits}")


@pytest.mark.parametrize("kind", list(KINDS))
def test_out16_llama7b_up(orc, kind):
    wl = workloads.WORKLOADS["llama7b_up"]
    check16(orc, workloads.make_activation(wl), workloads.make_weight(wl), 8, kind, "llama7b_up")


@pytest.mark.parametrize("kind", list(KINDS))
def test_out16_prefill(orc, kind):
    """The headline shape (256 x 256 tiles): whole tiles take the packed
    two-values-per-store path."""
    wl = workloads.WORKLOADS["prefill_w8"]
    check16(orc, workloads.make_activation(wl), workloads.make_weight(wl), 8, kind, "prefill_w8")


@pytest.mark.parametrize("kind", list(KINDS))
def test_out16_odd_row_stride(orc, kind):
    """A row stride of an odd number of 16-bit values: whole tiles cannot
    take 4-byte stores and use the one-value path; the columns past N stay
    untouched."""
    M, K, N = 300, 1024, 256
    mode, dt = KINDS[kind]
    X, W, _ = workloads.random_case(seed=8, M=M, K=K, N=N, n_out=3)
    g = GpuLayer(W, 8, 6.0, 64, M)
    g.step(X)
    Yw = torch.full((M, N + 41), 7.0, dtype=dt, device="cuda")
    mixq.gemm_ex(g.Xq, g.s_x, g.X_out, g.state, g.pw, Yw[:, :N], mode, None, g.ws)
    torch.cuda.synchronize()
    assert torch.equal(Yw[:, :N].contiguous().view(torch.int16), g.Y.to(dt).view(torch.int16))
    assert bool((Yw[:, N:] == 7.0).all())


def test_out16_ldy_and_errors(orc):
    """A row stride above N leaves the columns past N untouched; a 16-bit
    output with a row-subset weight is refused."""
    M, K, N = 70, 512, 96
    X, W, _ = workloads.random_case(seed=4, M=M, K=K, N=N, n_out=2)
    g = GpuLayer(W, 8, 6.0, 64, M)
    g.step(X)
    Yw = torch.full((M, N + 40), 7.0, dtype=torch.float16, device="cuda")
    mixq.gemm_ex(g.Xq, g.s_x, g.X_out, g.state, g.pw, Yw[:, :N], mixq.OUT_F16, None, g.ws)
    torch.cuda.synchronize()
    assert torch.equal(Yw[:, :N], g.Y.half())
    assert bool((Yw[:, N:] == 7.0).all())
    rows = np.arange(N, dtype=np.int32)
    pr = mixq.PackedWeight.create_rows(rows, N, K, 8, 64)
    with pytest.raises(mixq.MixqError) as e:
        mixq.gemm_ex(g.Xq, g.s_x, g.X_out, g.state, pr, Yw[:, :N], mixq.OUT_F16, None, None)
    assert e.value.code == 1
