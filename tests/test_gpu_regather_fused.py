"""mixq_quantize_act_regather (one call, two launches) against
mixq_quantize_act followed by mixq_pack_weight(PACK_OUTLIER_COLS) (three
launches), step by step over a sequence whose gate fires, stands and
overflows: the state (flag, count, ids, bitmap), Xq, s_x, X_out and the
weight's outlier columns bit for bit, the int32 accumulators against the
oracle and Y within 1e-3 * max|Y|.  Weights: INT8, INT4, gated, and a row
subset; a second weight packed for another state (stale columns) is
re-gathered by the fused call on a step where the set stands."""
import numpy as np
import pytest
import torch

from gpu_util import check_y, say, set_from_bitmap, to_dev
from mixed_precision_quantized_amax_amd import mixq
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu


def _seq(seed, M, K, steps):
    """Tokens with persistent channels, new ones on some steps, a quiet step."""
    r = np.random.default_rng(seed)
    pers = np.sort(r.choice(K, 5, replace=False))
    rest = np.setdiff1d(np.arange(K), pers)
    new = {1: r.choice(rest, 3, replace=False), 4: r.choice(rest, 2, replace=False),
           6: r.choice(rest, 40, replace=False)}  # step 6 overflows k_cap = 32
    out = []
    for st in range(steps):
        X = np.clip(r.standard_normal((M, K)), -4, 4).astype(np.float32)
        if st != 3:
            X[:, pers] = r.uniform(20, 100, (M, pers.size)) * np.where(
                r.random((M, pers.size)) < .5, -1, 1)
        if st in new:
            X[:, new[st]] = r.uniform(20, 100, (M, new[st].size))
        out.append(X.astype(np.float16))
    return out


class Side:
    def __init__(self, W, bits, k_cap, M, gated=False, rows=None):
        N, K = W.shape if rows is None else (len(rows), W.shape[1])
        self.Wd = to_dev(W)
        self.st = mixq.OutlierState.create(K, k_cap)
        if rows is None:
            self.pw = mixq.PackedWeight.create(N, K, bits, k_cap, gated=gated)
        else:
            self.pw = mixq.PackedWeight.create_rows(rows, W.shape[0], K, 8, k_cap)
        mixq.pack_weight(self.Wd, self.st, self.pw, mixq.PACK_FULL)
        ld = mixq.outlier_ld(k_cap)
        self.ld = ld
        self.Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        self.sx = torch.empty(M, dtype=torch.float32, device="cuda")
        self.Xo = torch.full((M * ld,), float("nan"), dtype=torch.float16, device="cuda")
        ycols = W.shape[0]
        self.Y = torch.zeros(M, ycols, dtype=torch.float32, device="cuda")

    def host(self):
        torch.cuda.synchronize()
        c = int(self.st.count.cpu()[0])
        kp = (c + 31) // 32 * 32
        M = self.Xq.shape[0]
        return dict(flag=int(self.st.flag.cpu()[0]), count=c,
                    idx=self.st.idx.cpu().numpy()[:c].copy(),
                    bitmap=self.st.bitmap.cpu().numpy().copy(),
                    Xq=self.Xq.cpu().numpy(), sx=self.sx.cpu().numpy().view(np.uint32),
                    Xo=self.Xo.view(torch.int16).cpu().numpy()[:M * self.ld].reshape(M, self.ld)[:, :kp],
                    wo=self.pw.w_out_view().view(torch.int16).cpu().numpy()[:, :kp])


@pytest.mark.parametrize("kind", ["int8", "int4", "gated", "rows"])
def test_fused_equals_separate(kind):
    orc = Oracle()
    M, K, N, k_cap, steps = 64, 1024, 192, 32, 8
    W = (np.random.default_rng(7).standard_normal((N, K)) * 0.05).astype(np.float16)
    bits = 4 if kind == "int4" else 8
    rows = np.random.default_rng(8).permutation(N)[:150].astype(np.int32) if kind == "rows" else None
    a = Side(W, bits, k_cap, M, gated=kind == "gated", rows=rows)
    b = Side(W, bits, k_cap, M, gated=kind == "gated", rows=rows)
    o = OracleLayer(W=W, bits=8, tau=6.0, k_cap=k_cap, ldo=a.ld, oracle=orc)
    flags = []
    for st, X in enumerate(_seq(3, M, K, steps)):
        Xd = to_dev(X)
        mixq.quantize_act_regather(Xd, 6.0, a.st, a.Xq, a.sx, a.Xo, a.Wd, a.pw)
        mixq.quantize_act(Xd, 6.0, b.st, b.Xq, b.sx, b.Xo)
        mixq.pack_weight(b.Wd, b.st, b.pw, mixq.PACK_OUTLIER_COLS)
        ha, hb = a.host(), b.host()
        for k in ha:
            assert np.array_equal(ha[k], hb[k]), (kind, st, k)
        r = o.step(X, products=False)
        assert ha["flag"] == r.flag and ha["count"] == r.count, (st, ha["flag"], r.flag)
        assert np.array_equal(set_from_bitmap(ha["bitmap"], K), r.in_set)
        flags.append(r.flag)
        if kind in ("int8", "gated"):
            acc = torch.zeros(M, a.pw.N, dtype=torch.int32, device="cuda")
            mixq.gemm(a.Xq, a.sx, a.Xo, a.st, a.pw, a.Y, acc, None)
            torch.cuda.synchronize()
            Wq, s_w = orc.quantize_weight(W, 8)
            order = np.array([32 * (p // 64) + p % 64 if p % 64 < 32 else N // 2 + 32 * (p // 64) + p % 64 - 32
                              for p in range(N)]) if kind == "gated" else np.arange(N)
            ref_acc = orc.int_gemm(r.Xq, Wq[order])
            assert np.array_equal(acc.cpu().numpy(), ref_acc), st
            W_out = orc.gather_weight_cols(W, r.in_set, a.ld)
            Yref = orc.output(ref_acc, r.s_x, s_w[order], r.X_out, W_out[order], r.count)
            err = check_y(a.Y.cpu().numpy(), Yref)
            say(f"[fused] {kind} step {st}: flag {r.flag} count {r.count} err {err:.1e}")
    assert flags == [1, 1, 0, 0, 1, 0, mixq.FLAG_OVERFLOW, 0], flags


def test_fused_regathers_stale_weight():
    """A weight packed for another state: on a step where the set stands,
    the fused call finds its columns stale and re-gathers them."""
    orc = Oracle()
    M, K, N, k_cap = 48, 512, 96, 32
    W = (np.random.default_rng(11).standard_normal((N, K)) * 0.05).astype(np.float16)
    Wd = to_dev(W)
    X = _seq(12, M, K, 1)[0]
    st = mixq.OutlierState.create(K, k_cap)
    other = mixq.OutlierState.create(K, k_cap)
    pw = mixq.PackedWeight.create(N, K, 8, k_cap)
    ld = mixq.outlier_ld(k_cap)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(M * ld, dtype=torch.float16, device="cuda")
    mixq.quantize_act(to_dev(X), 6.0, st, Xq, sx, Xo)            # st's set is formed
    Xb = _seq(13, M, K, 1)[0]
    mixq.quantize_act(to_dev(Xb), 6.0, other, Xq, sx, Xo)        # another set
    mixq.pack_weight(Wd, other, pw, mixq.PACK_FULL)              # columns of the other set
    mixq.quantize_act_regather(to_dev(X), 6.0, st, Xq, sx, Xo, Wd, pw)  # st stands: flag 0
    torch.cuda.synchronize()
    assert int(st.flag.cpu()[0]) == 0
    in_set = set_from_bitmap(st.bitmap.cpu().numpy(), K)
    kp = (int(st.count.cpu()[0]) + 31) // 32 * 32
    wo = pw.w_out_view().view(torch.int16).cpu().numpy()[:, :kp]
    assert np.array_equal(wo, orc.gather_weight_cols(W, in_set, ld)[:, :kp].view(np.int16))
