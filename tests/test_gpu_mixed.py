"""Output-feature mixed precision (MixLLM page: the salient output features
keep 8-bit weights, the rest 4-bit, all products on INT8 units) against the
oracle.  The salient rows form an INT8 row-subset weight and the others a
progressive INT4 one; each product writes its own columns of Y.  Checked:
every row's codes, group entries and scales bit for bit against the oracle's
mixed codes, the outlier columns, both products' int32 accumulators bit for
bit, every Y column written, Y within 1e-3 * max|Y|."""

import numpy as np
import pytest
import torch

from gpu_util import check_y, say, to_dev
from mixed_precision_quantized_amax_amd import mixq, workloads
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return Oracle()



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
    mw = mixq.MixedWeight.create(sal, K, k_cap)
    mw.pack(Wd, st, mixq.PACK_FULL)
    ld = mixq.outlier_ld(k_cap)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(max(M * ld, 1), dtype=torch.float16, device="cuda") if ld else None
    mixq.quantize_act(to_dev(X.view(np.float16)), tau, st, Xq, sx, Xo)
    mw.pack(Wd, st, mixq.PACK_OUTLIER_COLS)
    Y = torch.full((M, W.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    dbg = tuple(torch.zeros(M, p.N, dtype=torch.int32, device="cuda")
                if (acc and p is not None) else None for p in (mw.w4, mw.w8))
    wsb = mw.workspaces(M) if ws else (None, None)
    mw.gemm(Xq, sx, Xo, st, Y, dbg, wsb)
    torch.cuda.synchronize()
    return dict(mw=mw, Y=Y.cpu().numpy(), count=int(st.count.cpu()[0]), ws=wsb,
                acc=tuple(None if d is None else d.cpu().numpy() for d in dbg))


def packed_values(pw):
    """The INT8 code of every packed row and channel: bits 8 directly, bits 4
    rebuilt as (u - z) * s2."""
    if pw.bits == 8:
        return pw.codes_view().cpu().numpy().astype(np.int32), None
    K = pw.K
    u = unpack_u4(pw.codes_view().cpu().numpy(), K).astype(np.int32)
    gsz = pw.gsz.view(torch.int16).cpu().numpy().view(np.uint16).reshape(K // 128, pw.N).T
    s2 = np.repeat((gsz & 0xFF).astype(np.int32), 128, axis=1)
    z = np.repeat((gsz >> 8).astype(np.int32), 128, axis=1)
    return (u - z) * s2, gsz


def check_pack(orc, g, W, sal, W_out):
    """Both parts against the oracle's mixed codes and scales."""
    codes, scales = orc.mixed_feature_quantize_weight(W, sal)
    _, _, u, s2, z, _ = orc.progressive_quantize_weight(W)
    mw = g["mw"]
    for p, rows in ((mw.w8, np.flatnonzero(sal)), (mw.w4, np.flatnonzero(~sal))):
        if p is None:
            assert rows.size == 0
            continue
        assert np.array_equal(p.rmap.cpu().numpy(), rows)
        v, gsz = packed_values(p)
        assert np.array_equal(v, codes[rows].astype(np.int32))
        if gsz is not None:  # the stored 4-bit values and group entries themselves
            got_u = unpack_u4(p.codes_view().cpu().numpy(), p.K)
            assert np.array_equal(got_u, u[rows])
            assert np.array_equal(gsz & 0xFF, s2[rows]) and np.array_equal(gsz >> 8, z[rows])
        assert np.array_equal(p.s_w.cpu().numpy().view(np.uint32), scales[rows].view(np.uint32))
        wo = p.w_out_view().cpu().numpy().view(np.uint16)
        assert np.array_equal(wo, W_out[rows])
    return codes, scales


@pytest.mark.parametrize("tile", ["auto", "256x256", "128x128", "256x256_swp", "256x256_kpair", "128x128_kpair", "128x128_swp"],
                         indirect=True)
@pytest.mark.parametrize("M,K,N,S,n_act", [(37, 256, 128, 5, 3), (130, 1024, 384, 100, 9),
                                           (257, 2048, 520, 129, 0), (64, 1024, 256, 0, 40),
                                           (100, 512, 300, 300, 4)])
def test_mixed_random(orc, tile, M, K, N, S, n_act):
    X, W, _ = workloads.random_case(seed=M + K + N + S, M=M, K=K, N=N, n_out=n_act)
    sal = salient_set(N, S, M + S)
    check_mixed(orc, X, W, sal, tag=f"tile{tile}")


def check_mixed(orc, X, W, sal, ws=False, tag=""):
    """Both parts' codes, scales and outlier columns, both products' int32
    accumulators bit for bit, every Y column written, Y within tolerance."""
    M, K = X.shape
    N = W.shape[0]
    say(f"[mixed] {tag} M={M} K={K} N={N} S={int(sal.sum())} ws={ws}")
    g = run_mixed(X, W, sal, 6.0, 64, ws=ws)
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=mixq.outlier_ld(64), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(64))
    codes, scales = check_pack(orc, g, W, sal, W_out)
    acc = orc.int_gemm(r.Xq, codes)
    a4, a8 = g["acc"]
    if a4 is not None:
        assert np.array_equal(a4, acc[:, ~sal])
    if a8 is not None:
        assert np.array_equal(a8, acc[:, sal])
    Y = orc.output(acc, r.s_x, scales, r.X_out, W_out, r.count)
    assert not np.isnan(g["Y"]).any(), "an output feature was not written"
    err = check_y(g["Y"], Y)
    say(f"[mixed] ok count={r.count} max|dY|/max|Y|={err:.2e}")


def _random_cases(n=10, seed=91):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 600))
        out.append((i, int(rng.integers(1, 600)), 128 * int(rng.integers(1, 17)), N,
                    int(rng.integers(0, N + 1)), int(rng.integers(0, 30)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,M,K,N,S,n_act,ws", _random_cases())
def test_mixed_random_shapes(orc, i, M, K, N, S, n_act, ws):
    """Seeded random shapes and salient counts (none to all output features)
    through the automatic launch choice, with and without workspaces."""
    X, W, _ = workloads.random_case(seed=700 + i, M=M, K=K, N=N, n_out=n_act)
    check_mixed(orc, X, W, salient_set(N, S, 800 + i), ws=ws, tag=f"rand{i}")


def test_mixed_full_size(orc):
    """The INT4 prefill shape (M = 2048, K = N = 8192) with 10% of the output
    features at 8 bits (split-K workspaces given): every code, group entry
    and scale; the accumulators and Y at sampled positions."""
    wl = workloads.WORKLOADS["prefill_w4"]
    X = workloads.make_activation(wl)
    W = workloads.make_weight(wl)
    sal = workloads.make_salient(wl.N)
    g = run_mixed(X, W, sal, wl.tau, 256, ws=True)
    o = OracleLayer(W=W, bits=8, tau=wl.tau, k_cap=256, ldo=mixq.outlier_ld(256), oracle=orc)
    r = o.step(X, products=False)
    assert g["count"] == r.count
    W_out = orc.gather_weight_cols(W, r.in_set, mixq.outlier_ld(256))
    codes, scales = check_pack(orc, g, W, sal, W_out)
    rng = np.random.default_rng(11)
    cols = np.concatenate([rng.integers(0, wl.N, 2000), np.flatnonzero(sal)[:8],
                           np.flatnonzero(~sal)[-8:]])
    rows = np.resize(np.concatenate([rng.integers(0, wl.M, 2000), [0, wl.M - 1]]), cols.shape[0])
    acc, Y = orc.sampled_output(r.Xq, codes, r.s_x, scales, r.X_out, W_out, r.count, rows, cols)
    # the accumulator of an output feature sits in its part's packed column
    pos = np.empty(wl.N, np.int64)
    pos[sal] = np.arange(sal.sum())
    pos[~sal] = np.arange((~sal).sum())
    a4, a8 = g["acc"]
    got = np.where(sal[cols], a8[rows, pos[cols] * sal[cols]], a4[rows, pos[cols] * ~sal[cols]])
    assert np.array_equal(got, acc)
    assert not np.isnan(g["Y"]).any(), "an output feature was not written"
    ref = np.abs(Y).max()
    err = np.abs(g["Y"][rows, cols].astype(np.float64) - Y).max() / ref
    say(f"[mixed] full: max|dY|/max|Y| = {err:.2e}")
    assert err <= 1e-3


@pytest.mark.parametrize("bits", [8, 4])
def test_row_subset_entries_outside_w(orc, bits):
    """Row-map entries outside [0, n_out) pack zero codes with scale 1 and
    zero outlier columns, and write no Y column; the other rows are exact
    and every unnamed Y column keeps its old contents."""
    M, K, n_out = 70, 256, 300
    X, W, _ = workloads.random_case(seed=bits, M=M, K=K, N=n_out, n_out=3)
    rows = np.array([5, -1, 299, n_out, 17, 2**31 - 1], np.int32)
    Wd = to_dev(W.view(np.float16))
    st = mixq.OutlierState.create(K, 64)
    pw = mixq.PackedWeight.create_rows(rows, n_out, K, bits, 64,
                                       group=mixq.PROGRESSIVE_GROUP if bits == 4 else 0)
    mixq.pack_weight(Wd, st, pw, mixq.PACK_FULL)
    ld = mixq.outlier_ld(64)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(M * ld, dtype=torch.float16, device="cuda")
    mixq.quantize_act(to_dev(X.view(np.float16)), 6.0, st, Xq, sx, Xo)
    mixq.pack_weight(Wd, st, pw, mixq.PACK_OUTLIER_COLS)
    Y = torch.full((M, n_out), float("nan"), dtype=torch.float32, device="cuda")
    dbg = torch.zeros(M, pw.N, dtype=torch.int32, device="cuda")
    mixq.gemm(Xq, sx, Xo, st, pw, Y, dbg)
    torch.cuda.synchronize()
    live = (rows >= 0) & (rows < n_out)
    v, _ = packed_values(pw)
    s_w = pw.s_w.cpu().numpy()
    wo = pw.w_out_view().cpu().numpy().view(np.uint16)
    assert (v[~live] == 0).all() and (s_w[~live] == 1.0).all() and (wo[~live] == 0).all()
    assert (dbg.cpu().numpy()[:, ~live] == 0).all()
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=64, ldo=ld, oracle=orc)
    r = o.step(X, products=False)
    W_out = orc.gather_weight_cols(W, r.in_set, ld)
    if bits == 8:
        codes, scales = orc.quantize_weight(W, 8)
    else:
        codes, scales, *_ = orc.progressive_quantize_weight(W)
    sel = rows[live]
    assert np.array_equal(v[live], codes[sel].astype(np.int32))
    acc = orc.int_gemm(r.Xq, codes[sel])
    assert np.array_equal(dbg.cpu().numpy()[:, live], acc)
    Yref = orc.output(acc, r.s_x, scales[sel], r.X_out, W_out[sel], r.count)
    y = Y.cpu().numpy()
    check_y(y[:, sel], Yref)
    others = np.setdiff1d(np.arange(n_out), sel)
    assert np.isnan(y[:, others]).all(), "a column no row names was written"
