"""One activation state feeding several weights, as the projections that read
the same tokens do: each weight re-gathers its outlier columns when the set
has changed since its last gather.  Three weights (INT8, INT4, progressive
INT4; different output sizes) over a sequence in which the set is formed,
then grows, then stays; every product against the oracle (int32
accumulators bit for bit, Y within 1e-3 * max|Y|)."""
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


def test_one_state_three_weights(orc):
    M, K, k_cap = 300, 2048, 64
    X1, _, ch = workloads.random_case(seed=21, M=M, K=K, N=8, n_out=5)
    new_ch = next(c for c in range(7, K, 97) if c not in set(ch.tolist()))
    X2 = X1.astype(np.float32)
    X2[:, new_ch] *= np.float32(30.0)       # one more outlier channel: the set grows
    X2 = X2.astype(np.float16)
    X3 = (X1.astype(np.float32) * np.float32(0.5)).astype(np.float16)  # covered by the set
    kinds = [(384, 8, 0), (200, 4, 0), (520, 4, mixq.PROGRESSIVE_GROUP)]
    rng = np.random.default_rng(22)
    Ws = [(rng.standard_normal((n, K)) * 0.05).astype(np.float16) for n, _, _ in kinds]

    st = mixq.OutlierState.create(K, k_cap)
    ld = mixq.outlier_ld(k_cap)
    pws = []
    for W, (n, bits, group) in zip(Ws, kinds):
        pw = mixq.PackedWeight.create(n, K, bits, k_cap, group=group)
        mixq.pack_weight(to_dev(W.view(np.float16)), st, pw, mixq.PACK_FULL)
        pws.append(pw)
    ref_w = []
    for W, (n, bits, group) in zip(Ws, kinds):
        if group:
            q, s, *_ = orc.progressive_quantize_weight(W)
        else:
            q, s = orc.quantize_weight(W, bits)
        ref_w.append((q, s))
    o = OracleLayer(W=Ws[0], bits=8, tau=6.0, k_cap=k_cap, ldo=ld, oracle=orc)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(M * ld, dtype=torch.float16, device="cuda")
    for step, (X, flag) in enumerate([(X1, 1), (X2, 1), (X3, 0)]):
        mixq.quantize_act(to_dev(X.view(np.float16)), 6.0, st, Xq, sx, Xo)
        r = o.step(X, products=False)
        assert r.flag == flag
        torch.cuda.synchronize()
        assert int(st.count.cpu()[0]) == r.count
        assert np.array_equal(Xq.cpu().numpy(), r.Xq)
        for W, pw, (q, s), (n, bits, group) in zip(Ws, pws, ref_w, kinds):
            mixq.pack_weight(to_dev(W.view(np.float16)), st, pw, mixq.PACK_OUTLIER_COLS)
            Y = torch.full((M, n), float("nan"), dtype=torch.float32, device="cuda")
            dbg = torch.zeros(M, n, dtype=torch.int32, device="cuda")
            ws = mixq.gemm_workspace(M, n, K, bits)
            mixq.gemm(Xq, sx, Xo, st, pw, Y, dbg, ws)
            torch.cuda.synchronize()
            acc = orc.int_gemm(r.Xq, q)
            assert np.array_equal(dbg.cpu().numpy(), acc), (step, n, bits, group)
            W_out = orc.gather_weight_cols(W, r.in_set, ld)
            err = check_y(Y.cpu().numpy(), orc.output(acc, r.s_x, s, r.X_out, W_out, r.count))
            say(f"[shared] step {step} N={n} bits={bits} group={group} count={r.count} "
                f"max|dY|/max|Y|={err:.2e}")
    assert r.count == 6


def _planted(seed, M, K, chans):
    """N(0,1) tokens (clipped below the threshold) with the given channels
    planted at U(20, 100) * sign: exactly those channels exceed tau."""
    r = np.random.default_rng(seed)
    X = np.clip(r.standard_normal((M, K)), -4, 4).astype(np.float32)
    X[:, chans] = r.uniform(20, 100, (M, len(chans))) * np.where(r.random((M, len(chans))) < .5, -1, 1)
    return X.astype(np.float16)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("how", ["reset", "second_state"])
def test_same_size_set_regathers(orc, bits, how):
    """A weight whose outlier columns were gathered for one set, then used
    with a set of the same size but other channels -- after the state is
    reset, or through a second state -- must re-gather them (MixQ article,
    Fig. 11: the outlier columns are those of the current set, in order).
    Y and the int32 accumulators against the oracle for both sets."""
    M, K, N, k_cap = 96, 1024, 320, 32
    ld = mixq.outlier_ld(k_cap)
    set_a = [5, 77, 300, 901]
    set_b = [6, 78, 301, 902]  # same size, other channels
    XA, XB = _planted(31, M, K, set_a), _planted(32, M, K, set_b)
    W = (np.random.default_rng(33).standard_normal((N, K)) * 0.05).astype(np.float16)
    Wd = to_dev(W)
    q, s = orc.quantize_weight(W, bits)
    pw = mixq.PackedWeight.create(N, K, bits, k_cap)
    st_a = mixq.OutlierState.create(K, k_cap)
    st_b = st_a if how == "reset" else mixq.OutlierState.create(K, k_cap)
    mixq.pack_weight(Wd, st_a, pw, mixq.PACK_FULL)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    Xo = torch.zeros(M * ld, dtype=torch.float16, device="cuda")
    for X, st, chans in ((XA, st_a, set_a), (XB, st_b, set_b)):
        if st is st_a and X is XB:
            st.reset()
        mixq.quantize_act(to_dev(X), 6.0, st, Xq, sx, Xo)
        mixq.pack_weight(Wd, st, pw, mixq.PACK_OUTLIER_COLS)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        dbg = torch.zeros(M, N, dtype=torch.int32, device="cuda")
        mixq.gemm(Xq, sx, Xo, st, pw, Y, dbg, None)
        torch.cuda.synchronize()
        r = OracleLayer(W=W, bits=bits, tau=6.0, k_cap=k_cap, ldo=ld, oracle=orc).step(X)
        assert r.idx.tolist() == chans and int(st.count.cpu()[0]) == len(chans)
        wo = pw.w_out_view().cpu().numpy().view(np.uint16)
        assert np.array_equal(wo, orc.gather_weight_cols(W, r.in_set, ld)), how
        assert np.array_equal(dbg.cpu().numpy(), r.acc)
        err = check_y(Y.cpu().numpy(), r.Y)
        say(f"[regather] {how} bits={bits} set={chans} max|dY|/max|Y|={err:.2e}")
