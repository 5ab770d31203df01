"""The fused gate-and-up GEMM with the SwiGLU epilogue (mixq_gemm_ex,
MIXQ_OUT_SWIGLU_F16) against the oracle: the gated weight's packed codes,
scales and outlier columns equal the oracle's rows in the documented
interleaved order, the int32 accumulators are bit-exact in that order, and
the fp16 silu(gate) * up is within 1e-3 * max of the oracle's float64 SwiGLU
of its Y (fp16 rounding alone is 2^-11 relative)."""

import numpy as np
import pytest
import torch

from gpu_util import check_y, say, to_dev
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def orc():
    return Oracle()



def packed_order(N):
    """Source row of each packed row of a gated weight (32-row blocks of gate
    and up rows interleaved), written out from the documented layout."""
    I = N // 2
    p = np.arange(N)
    blk, within = p // 64, p % 64
    return np.where(within < 32, blk * 32 + within, I + blk * 32 + within - 32)


def run_gated(X, W, bits, tau, k_cap, ws=False, acc=True):
    """Everything through the C ABI: pack gated, quantize, re-gather, and the
    product both ways (SwiGLU fp16 and plain fp32 on the same gated weight)."""
    M, K = X.shape
    N = W.shape[0]
    Wd = to_dev(W.view(np.float16))
    st = mixq.OutlierState.create(K, k_cap)
    pw = mixq.PackedWeight.create(N, K, bits, k_cap, gated=True)
    mixq.pack_weight(Wd, st, pw, mixq.PACK_FULL)
    ld = mixq.outlier_ld(k_cap)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(max(M * ld, 1), dtype=torch.float16, device="cuda") if ld else None
    mixq.quantize_act(to_dev(X.view(np.float16)), tau, st, Xq, sx, Xo)
    mixq.pack_weight(Wd, st, pw, mixq.PACK_OUTLIER_COLS)
    wsb = mixq.gemm_workspace(M, N, K, bits) if ws else None
    Yh = torch.full((M, N // 2), float("nan"), dtype=torch.float16, device="cuda")
    dbg = torch.zeros(M, N, dtype=torch.int32, device="cuda") if acc else None
    mixq.gemm_ex(Xq, sx, Xo, st, pw, Yh, mixq.OUT_SWIGLU_F16, dbg, wsb)
    Y32 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mixq.gemm_ex(Xq, sx, Xo, st, pw, Y32, mixq.OUT_F32, None, wsb)
    torch.cuda.synchronize()
    return dict(pw=pw, Yh=Yh.cpu().numpy().astype(np.float64), Y32=Y32.cpu().numpy(),
                acc=None if dbg is None else dbg.cpu().numpy(), count=int(st.count.cpu()[0]),
                ws=wsb)


def check_swiglu(orc, X, W, bits=8, tau=6.0, k_cap=64, ws=False, tag=""):
    M, K = X.shape
    N = W.shape[0]
    say(f"[swiglu] {tag} M={M} K={K} N={N} bits={bits} ws={ws}")
    g = run_gated(X, W, bits, tau, k_cap, ws=ws)
    o = OracleLayer(W=W, bits=bits, tau=tau, k_cap=k_cap, ldo=mixq.outlier_ld(k_cap), oracle=orc)
    r = o.step(X)
    perm = packed_order(N)
    pw = g["pw"]
    assert g["count"] == r.count
    if bits == 8:
        codes = pw.codes_view().cpu().numpy().view(np.int8)
        assert np.array_equal(codes, o.Wq[perm])
    assert np.array_equal(pw.s_w.cpu().numpy().view(np.uint32), o.s_w[perm].view(np.uint32))
    ld = mixq.outlier_ld(k_cap)
    if ld and r.count:
        wo = pw.w_out_view().view(torch.int16).cpu().numpy().view(np.uint16)
        wref = orc.gather_weight_cols(W, r.in_set, ld)
        kp = (r.count + 31) // 32 * 32
        assert np.array_equal(wo[:, :kp], wref[perm][:, :kp])
    assert np.array_equal(g["acc"], r.acc[:, perm])
    check_y(g["Y32"], r.Y[:, perm])
    ref = orc.swiglu(r.Y)
    err = np.abs(g["Yh"] - ref).max() / (np.abs(ref).max() or 1.0)
    assert np.isfinite(g["Yh"]).all()
    assert err <= TOL, err
    say(f"[swiglu] {tag} ok: count={r.count} max|dY|/max|Y| = {err:.2e}")
    return g


@pytest.mark.parametrize("tile", ["auto", "256x256", "128x128", "256x256_kpair", "128x128_kpair"], indirect=True)
@pytest.mark.parametrize("M,K,N,n_out", [(37, 512, 128, 3), (130, 1024, 384, 9),
                                         (257, 2048, 512, 0)])
def test_swiglu_random(orc, tile, M, K, N, n_out):
    X, W, _ = workloads.random_case(seed=M + K + N, M=M, K=K, N=N, n_out=n_out)
    check_swiglu(orc, X, W, tag=f"tile{tile}")


@pytest.mark.parametrize("tile", ["auto", "256x256_swp"], indirect=True)
def test_swiglu_int4(orc, tile):
    X, W, _ = workloads.random_case(seed=44, M=100, K=1024, N=512, n_out=5)
    check_swiglu(orc, X, W, bits=4, tag=f"int4 tile{tile}")


def test_swiglu_split_k(orc):
    """A thin product takes the split-K path; the finishing block runs the
    SwiGLU epilogue."""
    M, K, N = 64, 4096, 1024
    assert mixq.gemm_workspace_bytes(M, N, K, 8) > 0
    X, W, _ = workloads.random_case(seed=55, M=M, K=K, N=N, n_out=4)
    g = check_swiglu(orc, X, W, ws=True, tag="split-k")
    assert g["ws"] is not None
    assert int(g["ws"][:1024].abs().sum().cpu()) == 0


def test_swiglu_full_size(orc):
    """The prefill shape as a fused gate-and-up projection (M = 2048,
    K = 8192, I = 4096): SwiGLU outputs at sampled positions (both halves of
    each computed by the oracle's per-pair entry point)."""
    wl = workloads.WORKLOADS["prefill_w8"]
    X = workloads.make_activation(wl)
    W = workloads.make_weight(wl)
    M, K, N = wl.M, wl.K, wl.N
    I = N // 2
    g = run_gated(X, W, 8, wl.tau, 256, acc=False)
    o = OracleLayer(W=W, bits=8, tau=wl.tau, k_cap=256, ldo=mixq.outlier_ld(256), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(256))
    rng = np.random.default_rng(3)
    rows = np.concatenate([rng.integers(0, M, 1500), [0, M - 1, 255, 256]])
    cols = np.concatenate([rng.integers(0, I, 1500), [0, I - 1, 31, 32]])
    _, yg = orc.sampled_output(r.Xq, o.Wq, r.s_x, o.s_w, r.X_out, W_out, r.count, rows, cols)
    _, yu = orc.sampled_output(r.Xq, o.Wq, r.s_x, o.s_w, r.X_out, W_out, r.count, rows, cols + I)
    ref = yg / (1.0 + np.exp(-yg)) * yu
    got = g["Yh"][rows, cols]
    err = np.abs(got - ref).max() / np.abs(ref).max()
    say(f"[swiglu] full: max|dY|/max|Y| = {err:.2e} over {rows.size} samples")
    assert err <= TOL, err
    assert np.isfinite(g["Yh"]).all()


def _random_cases(n=10, seed=77):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 500)), 64 * int(rng.integers(1, 25)), 64 * int(rng.integers(1, 11)),
             int(rng.integers(0, 20)), int(rng.choice([8, 4])), bool(rng.integers(0, 2)))
            for i in range(n)]


@pytest.mark.parametrize("i,M,K,N,n_out,bits,ws", _random_cases())
def test_swiglu_random_shapes(orc, i, M, K, N, n_out, bits, ws):
    """Seeded random shapes through the automatic launch choice (N a
    multiple of 64, as a gated weight requires), INT8 and INT4, with and
    without a split-K workspace."""
    X, W, _ = workloads.random_case(seed=500 + i, M=M, K=K, N=N, n_out=n_out)
    check_swiglu(orc, X, W, bits=bits, ws=ws, tag=f"rand{i}")
