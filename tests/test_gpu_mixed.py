"""Output-feature mixed precision (MixLLM page: the salient output features
keep 8-bit weights, the rest 4-bit, all products on INT8 units) against the
oracle.  A salient row's INT8 code is split into a high and a low
progressive 4-bit plane; the product adds the two planes' accumulators.
Checked: every plane's 4-bit values, group entries and scales bit for bit
against the oracle's codes, the outlier columns, the int32 accumulators per
plane and of each output feature, and Y within 1e-3 * max|Y|."""
import os

import numpy as np
import pytest
import torch

from gpu_util import check_y, say, to_dev
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu

MASK = 0x3FFFFFFF


@pytest.fixture(scope="module")
def orc():
    return Oracle()


@pytest.fixture
def tile(request):
    old = os.environ.get("MIXQ_GEMM_TILE")
    os.environ["MIXQ_GEMM_TILE"] = request.param
    yield request.param
    if old is None:
        del os.environ["MIXQ_GEMM_TILE"]
    else:
        os.environ["MIXQ_GEMM_TILE"] = old


def unpack_u4(packed: np.ndarray, K: int) -> np.ndarray:
    """The documented nibble layout, unsigned: per 32-bit word (8
    consecutive k), byte j holds k+j low and k+j+4 high."""
    N = packed.shape[0]
    b = packed.reshape(N, K // 8, 4).astype(np.uint8)
    return np.concatenate([b & 0xF, b >> 4], axis=2).reshape(N, K)


def salient_set(N, S, seed):
    rng = np.random.default_rng(seed)
    sal = np.zeros(N, bool)
    sal[rng.choice(N, S, replace=False)] = True
    return sal


def run_mixed(X, W, sal, tau, k_cap, acc=True, ws=False):
    M, K = X.shape
    Wd = to_dev(W.view(np.float16))
    st = mixq.OutlierState.create(K, k_cap)
    pw = mixq.PackedWeight.create_mixed(sal, K, k_cap)
    mixq.pack_weight(Wd, st, pw, mixq.PACK_FULL)
    ld = mixq.outlier_ld(k_cap)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(max(M * ld, 1), dtype=torch.float16, device="cuda") if ld else None
    mixq.quantize_act(to_dev(X.view(np.float16)), tau, st, Xq, sx, Xo)
    mixq.pack_weight(Wd, st, pw, mixq.PACK_OUTLIER_COLS)
    Y = torch.full((M, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    dbg = torch.zeros(M, pw.N, dtype=torch.int32, device="cuda") if acc else None
    wsb = mixq.gemm_workspace(M, pw.N, K, 4) if ws else None
    mixq.gemm(Xq, sx, Xo, st, pw, Y, dbg, wsb)
    torch.cuda.synchronize()
    return dict(pw=pw, Y=Y.cpu().numpy(), acc=None if dbg is None else dbg.cpu().numpy(),
                count=int(st.count.cpu()[0]), ws=wsb)


def packed_values(pw):
    """The INT8 value (u - z) * s2 of every packed row and channel."""
    K = pw.K
    u = unpack_u4(pw.codes_view().cpu().numpy(), K).astype(np.int32)
    gsz = pw.gsz.view(torch.int16).cpu().numpy().view(np.uint16).reshape(pw.N, K // 128)
    s2 = np.repeat((gsz & 0xFF).astype(np.int32), 128, axis=1)
    z = np.repeat((gsz >> 8).astype(np.int32), 128, axis=1)
    return (u - z) * s2, gsz


def layout(pw):
    rm = pw.rmap.cpu().numpy()
    src = rm & MASK
    plane = rm.astype(np.uint32) >> 30
    live = src < pw.n_out
    return src, plane, live


def check_pack(orc, g, W, sal, W_out):
    """The packed planes against the oracle's codes and scales."""
    pw = g["pw"]
    codes, scales = orc.mixed_feature_quantize_weight(W, sal)
    v, gsz = packed_values(pw)
    src, plane, live = layout(pw)
    s_w = pw.s_w.cpu().numpy()
    hi = np.flatnonzero((plane == 1) & live)
    lo = hi + 32
    assert np.array_equal(src[lo], src[hi]) and (plane[lo] == 2).all()
    # an 8-bit row: high plane 16 h (h in [-8, 7]), low plane l in [0, 15]
    assert np.array_equal(v[hi] + v[lo], codes[src[hi]].astype(np.int32))
    assert ((v[hi] % 16) == 0).all() and (v[lo] >= 0).all() and (v[lo] <= 15).all()
    assert ((gsz[hi] == (16 | 8 << 8)).all()) and (gsz[lo] == 1).all()
    p4 = np.flatnonzero(plane == 0)
    assert np.array_equal(v[p4], codes[src[p4]].astype(np.int32))
    for rows in (hi, lo, p4):
        assert np.array_equal(s_w[rows].view(np.uint32), scales[src[rows]].view(np.uint32))
    pad = np.flatnonzero(~live)
    assert (v[pad] == 0).all() and (s_w[pad] == 1.0).all()
    # outlier columns ride on the high plane and the 4-bit rows only
    wo = pw.w_out_view().cpu().numpy().view(np.uint16)
    carry = np.concatenate([hi, p4])
    assert np.array_equal(wo[carry], W_out[src[carry]])
    zero = np.concatenate([lo, pad])
    assert (wo[zero] == 0).all()
    return codes, scales, hi, lo, p4, src


@pytest.mark.parametrize("tile", ["0", "1", "2", "4", "6", "8", "10", "11", "15"], indirect=True)
@pytest.mark.parametrize("M,K,N,S,n_act", [(37, 256, 128, 5, 3), (130, 1024, 384, 100, 9),
                                           (257, 2048, 520, 129, 0), (64, 1024, 256, 0, 40),
                                           (100, 512, 300, 300, 4)])
def test_mixed_random(orc, tile, M, K, N, S, n_act):
    X, W, _ = workloads.random_case(seed=M + K + N + S, M=M, K=K, N=N, n_out=n_act)
    sal = salient_set(N, S, M + S)
    say(f"[mixed] tile{tile} M={M} K={K} N={N} S={S}")
    g = run_mixed(X, W, sal, 6.0, 64)
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(64))
    codes, scales, hi, lo, p4, src = check_pack(orc, g, W, sal, W_out)
    acc = orc.int_gemm(r.Xq, codes)
    got = g["acc"]
    # per plane, then per output feature
    hi_codes = ((codes.astype(np.int32) + 128) >> 4) * 16 - 128
    lo_codes = (codes.astype(np.int32) + 128) & 15
    if hi.size:
        assert np.array_equal(got[:, hi], orc.int_gemm(r.Xq, hi_codes[src[hi]].astype(np.int8)))
        assert np.array_equal(got[:, lo], orc.int_gemm(r.Xq, lo_codes[src[lo]].astype(np.int8)))
        assert np.array_equal(got[:, hi] + got[:, lo], acc[:, src[hi]])
    assert np.array_equal(got[:, p4], acc[:, src[p4]])
    Y = orc.output(acc, r.s_x, scales, r.X_out, W_out, r.count)
    assert not np.isnan(g["Y"]).any(), "an output feature was not written"
    err = check_y(g["Y"], Y)
    say(f"[mixed] ok count={r.count} max|dY|/max|Y|={err:.2e}")


def test_mixed_full_size(orc):
    """The INT4 prefill shape (M = 2048, K = N = 8192) with 10% of the output
    features at 8 bits: every plane's values, group entries and scales; the
    accumulators and Y at sampled positions."""
    wl = workloads.WORKLOADS["prefill_w4"]
    X = workloads.make_activation(wl)
    W = workloads.make_weight(wl)
    sal = workloads.make_salient(wl.N)
    g = run_mixed(X, W, sal, wl.tau, 256, ws=True)
    o = OracleLayer(W=W, bits=8, tau=wl.tau, k_cap=256, ldo=mixq.outlier_ld(256), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(256))
    codes, scales, hi, lo, p4, src = check_pack(orc, g, W, sal, W_out)
    rng = np.random.default_rng(11)
    rows = np.concatenate([rng.integers(0, wl.M, 2000), [0, wl.M - 1]])
    cols = np.concatenate([rng.integers(0, wl.N, 2000), np.flatnonzero(sal)[:8],
                           np.flatnonzero(~sal)[-8:]])
    rows = np.resize(rows, cols.shape[0])
    acc, Y = orc.sampled_output(r.Xq, codes, r.s_x, scales, r.X_out, W_out, r.count, rows, cols)
    # the accumulator of an output feature: its 4-bit row, or its two planes
    where = np.empty(wl.N, np.int64)
    where[src[p4]] = p4
    where[src[hi]] = hi
    lo_of = np.where(sal[cols], where[cols] + 32, where[cols])
    got = g["acc"][rows, where[cols]] + np.where(sal[cols], g["acc"][rows, lo_of], 0)
    assert np.array_equal(got, acc)
    assert not np.isnan(g["Y"]).any(), "an output feature was not written"
    ref = np.abs(Y).max()
    err = np.abs(g["Y"][rows, cols].astype(np.float64) - Y).max() / ref
    say(f"[mixed] full: max|dY|/max|Y| = {err:.2e}")
    assert err <= 1e-3
