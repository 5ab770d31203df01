"""The RMSNorm fused into the activation pass (mixq_rmsnorm_quantize_act)
against the oracle's RMSNorm followed by its activation side, bit for bit:
rstd, the set (gate, detection, union, overflow), Xq, s_x and X_out; and the
layer's product from those buffers against the oracle's Y."""
import numpy as np
import pytest
import torch

from gpu_util import GpuLayer, check_y, compare_quant, say, to_dev
from mixed_precision_quantized_amax_amd import mixq
from oracle import Oracle, OracleLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return Oracle()


class NormLayer(GpuLayer):
    """GpuLayer whose activation side is the fused RMSNorm + quantize call."""

    def __init__(self, W, gamma, eps, bits, tau, k_cap, M, ldh=None):
        self.gamma = to_dev(gamma.view(np.float16))
        self.eps = eps
        self.ldh = ldh
        super().__init__(W, bits, tau, k_cap, M)

    def alloc(self, M):
        super().alloc(M)
        self.rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")

    def quantize(self, H: np.ndarray):
        M, K = H.shape
        if self.ldh:
            wide = np.zeros((M, self.ldh), np.float16)
            wide[:, :K] = H
            Hd = to_dev(wide)[:, :K]
        else:
            Hd = to_dev(H.view(np.float16))
        mixq.rmsnorm_quantize_act(Hd, self.gamma, self.eps, self.tau, self.state, self.Xq,
                                  self.s_x, self.X_out, self.rstd)


def make_case(seed, M, K, n_out, wide=False):
    """Hidden states N(0,1) with n_out planted channels U(20,100)*sign, and a
    gamma around the expected root mean square of such a token, so that the
    normalised values have the spread of the layer's usual inputs (unit scale,
    the planted channels above the threshold)."""
    r = np.random.default_rng(seed)
    H = r.standard_normal((M, K))
    ch = np.sort(r.choice(K, n_out, replace=False)) if n_out else np.zeros(0, int)
    if n_out:
        H[:, ch] = r.uniform(20, 100, (M, n_out)) * r.choice([-1, 1], (M, n_out))
    if wide:
        kind = r.integers(0, 5, (M, K))
        H = np.where(kind == 0, r.integers(1, 1024, (M, K)) * 2.0 ** -24, H)
        H = np.where(kind == 1, r.uniform(1000, 60000, (M, K)) * r.choice([-1, 1], (M, K)), H)
    g0 = np.sqrt(1.0 + n_out / K * (100.0 ** 3 - 20.0 ** 3) / (3 * 80.0))
    gamma = (g0 * (1.0 + 0.1 * r.standard_normal(K))).astype(np.float16)
    return H.astype(np.float16), gamma


def compare_norm(orc, g: NormLayer, o: OracleLayer, H, gamma, eps, products=True, tag=""):
    M, K = H.shape
    say(f"[norm] {tag} M={M} K={K} eps={eps} k_cap={g.k_cap} ldh={g.ldh}")
    if products:
        acc = g.step(H, acc=True)
    else:
        g.quantize(H)
        torch.cuda.synchronize()
    X, rstd = orc.rmsnorm(H, gamma, eps)
    r = o.step(X, products=products)
    got = g.rstd.cpu().numpy()
    bad = np.nonzero(got.view(np.uint32) != rstd.view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} rstd mismatches, first token {bad[:4].tolist()}"
    compare_quant(g, X, r)
    if products:
        a = acc.cpu().numpy()
        assert np.array_equal(a, r.acc)
        err = check_y(g.Y.cpu().numpy(), r.Y)
        say(f"[norm] {tag} ok: count={r.count} flag={r.flag} max|dY|/max|Y|={err:.2e}")
    else:
        say(f"[norm] {tag} ok: count={r.count} flag={r.flag}")
    return r


def layer_pair(orc, W, gamma, eps, tau, k_cap, M, ldh=None):
    g = NormLayer(W, gamma, eps, 8, tau, k_cap, M, ldh=ldh)
    o = OracleLayer(W=W, bits=8, tau=tau, k_cap=k_cap, ldo=mixq.outlier_ld(k_cap), oracle=orc)
    return g, o


@pytest.mark.parametrize("M,K,N,n_out,eps,wide", [
    (1, 64, 32, 0, 1e-5, False), (37, 512, 96, 3, 1e-5, False), (130, 4096, 256, 20, 1e-6, False),
    (64, 8192, 128, 82, 1e-5, False), (5, 32768, 64, 10, 1e-5, False),
    (300, 1024, 200, 0, 0.0, False), (40, 2048, 64, 4, 1e-5, True), (3, 32768, 32, 0, 0.0, True),
    (4097, 1024, 64, 6, 1e-5, False),  # several tokens per block, an odd count for some
])
def test_norm_random(orc, M, K, N, n_out, eps, wide):
    H, gamma = make_case(M * 7 + K + n_out, M, K, n_out, wide)
    W = (np.random.default_rng(K + N).standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = layer_pair(orc, W, gamma, eps, 6.0, min(K, 128), M)
    compare_norm(orc, g, o, H, gamma, eps, tag=f"rand{'-wide' if wide else ''}")


def test_norm_zero_rows(orc):
    """All-zero tokens: with eps = 0 the denominator is 0 and rstd is 0; with
    eps > 0 rstd = 1/sqrt(eps); either way the codes are 0 and the scale 1."""
    H, gamma = make_case(3, 9, 256, 2)
    H[[0, 4, 8]] = 0
    W = (np.random.default_rng(3).standard_normal((48, 256)) * 0.05).astype(np.float16)
    for eps in (0.0, 1e-5):
        g, o = layer_pair(orc, W, gamma, eps, 6.0, 32, 9)
        compare_norm(orc, g, o, H, gamma, eps, tag=f"zero-rows eps={eps}")
        r = g.rstd.cpu().numpy()
        assert (r[[0, 4, 8]] == (0.0 if eps == 0 else np.float32(1) / np.sqrt(np.float32(eps)))).all()
        assert (g.s_x.cpu().numpy()[[0, 4, 8]] == 1.0).all()


def test_norm_sequence(orc):
    """Decode-like steps through one state: persistent channels, planted
    transient ones (the gate fires and the fused re-quantize pass runs),
    quiet steps; every step compared in full."""
    M, K, N = 24, 1024, 64
    rng = np.random.default_rng(11)
    pers = np.sort(rng.choice(K, 6, replace=False))
    gamma = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = layer_pair(orc, W, gamma, 1e-5, 6.0, 64, M)
    flags = []
    for st in range(8):
        H = rng.standard_normal((M, K))
        H[:, pers] = rng.uniform(20, 100, (M, pers.size))
        if st in (2, 5):
            H[rng.integers(0, M, 3), rng.integers(0, K, 3)] = 90.0
        compare_norm(orc, g, o, H.astype(np.float16), gamma, 1e-5, tag=f"step{st}")
        flags.append(g.flag())
    assert flags[0] == 1 and flags[1] == 0 and flags[2] == 1 and flags[5] == 1


def test_norm_overflow(orc):
    """More outliers than k_cap: flag 2, the set unchanged, the call
    quantized with the old set."""
    H, gamma = make_case(21, 16, 512, 12)
    W = (np.random.default_rng(21).standard_normal((32, 512)) * 0.05).astype(np.float16)
    g, o = layer_pair(orc, W, gamma, 1e-5, 6.0, 4, 16)
    r = compare_norm(orc, g, o, H, gamma, 1e-5, tag="overflow")
    assert r.flag == 2 and g.flag() == 2 and g.count() == 0


def test_norm_row_stride(orc):
    H, gamma = make_case(31, 50, 640, 5)
    W = (np.random.default_rng(31).standard_normal((40, 640)) * 0.05).astype(np.float16)
    g, o = layer_pair(orc, W, gamma, 1e-5, 6.0, 64, 50, ldh=1024)
    compare_norm(orc, g, o, H, gamma, 1e-5, tag="ldh")


def test_norm_full_size(orc):
    """The prefill shape (M = 2048, K = 8192, 82 planted channels): the whole
    activation side in the launch configuration the benchmark uses."""
    H, gamma = make_case(0, 2048, 8192, 82)
    W = (np.random.default_rng(0).standard_normal((64, 8192)) * 0.02).astype(np.float16)
    g, o = layer_pair(orc, W, gamma, 1e-5, 6.0, 256, 2048)
    r = compare_norm(orc, g, o, H, gamma, 1e-5, products=False, tag="full")
    assert r.count >= 60
    # second call: the set is cached, the gate stays closed
    r = compare_norm(orc, g, o, H, gamma, 1e-5, products=False, tag="full-cached")
    assert r.flag == 0


# ---- the residual add before the norm (mixq_add_rmsnorm_quantize_act) ----------------
class ResLayer(NormLayer):
    """The activation side is the fused residual add + RMSNorm + quantize
    call; ``quantize`` takes the pair (R, D) and H is written to ``self.H``."""

    def __init__(self, *args, lds=None, **kw):
        self.lds = lds  # (ldr, ldd, ldh) or None for K
        super().__init__(*args, **kw)

    def quantize(self, RD):
        R, D = RD
        M, K = R.shape
        ldr, ldd, ldh = self.lds or (K, K, K)

        def dev(a, ld):
            wide = np.zeros((M, ld), np.float16)
            wide[:, :K] = a
            return to_dev(wide)[:, :K]

        Rd, Dd = dev(R, ldr), dev(D, ldd)
        self.Hbuf = torch.full((M, ldh), float("nan"), dtype=torch.float16, device="cuda")
        H = self.Hbuf[:, :K]
        mixq.add_rmsnorm_quantize_act(Rd, Dd, H, self.gamma, self.eps, self.tau, self.state,
                                      self.Xq, self.s_x, self.X_out, self.rstd)


def compare_res(orc, g: ResLayer, o: OracleLayer, R, D, gamma, eps, products=True, tag=""):
    M, K = R.shape
    say(f"[res] {tag} M={M} K={K} eps={eps} k_cap={g.k_cap} lds={g.lds}")
    if products:
        acc = g.step((R, D), acc=True)
    else:
        g.quantize((R, D))
        torch.cuda.synchronize()
    H = orc.residual_add(R, D)
    got_h = g.Hbuf[:, :K].cpu().numpy()
    bad = np.argwhere(got_h.view(np.uint16) != H.view(np.uint16))
    assert bad.shape[0] == 0, f"{bad.shape[0]} H mismatches, first {bad[:4].tolist()}"
    if g.lds:  # the padding of H's rows is not written
        assert np.isnan(g.Hbuf[:, K:].cpu().numpy().astype(np.float32)).all()
    X, rstd = orc.rmsnorm(H, gamma, eps)
    r = o.step(X, products=products)
    assert np.array_equal(g.rstd.cpu().numpy().view(np.uint32), rstd.view(np.uint32))
    compare_quant(g, X, r)
    if products:
        assert np.array_equal(acc.cpu().numpy(), r.acc)
        err = check_y(g.Y.cpu().numpy(), r.Y)
        say(f"[res] {tag} ok: count={r.count} flag={r.flag} max|dY|/max|Y|={err:.2e}")
    return r


def res_pair(orc, W, gamma, eps, tau, k_cap, M, lds=None):
    g = ResLayer(W, gamma, eps, 8, tau, k_cap, M, lds=lds)
    o = OracleLayer(W=W, bits=8, tau=tau, k_cap=k_cap, ldo=mixq.outlier_ld(k_cap), oracle=orc)
    return g, o


def split_case(H, seed):
    """R and D whose fp16 sum is near H: D is a small update, R = H - D in fp16;
    some entries of D cancel R exactly (H = 0) and some sums are subnormal."""
    r = np.random.default_rng(seed)
    D = (r.standard_normal(H.shape) * 0.3).astype(np.float16)
    R = (H.astype(np.float64) - D.astype(np.float64)).astype(np.float16)
    cancel = r.random(H.shape) < 0.01
    D[cancel] = -R[cancel]
    tiny = r.random(H.shape) < 0.01
    R[tiny] = (r.integers(-512, 512, tiny.sum()) * 2.0 ** -24).astype(np.float16)
    D[tiny] = (r.integers(-512, 512, tiny.sum()) * 2.0 ** -24).astype(np.float16)
    return R, D


@pytest.mark.parametrize("M,K,N,n_out,lds", [
    (1, 64, 32, 0, None), (37, 512, 96, 3, None), (130, 4096, 256, 20, (4104, 4096, 4112)),
    (64, 8192, 128, 82, None), (5, 32768, 64, 10, None),
    (2049, 1024, 64, 6, None),  # two and three tokens per block
])
def test_res_random(orc, M, K, N, n_out, lds):
    Hs, gamma = make_case(M * 5 + K + n_out, M, K, n_out)
    R, D = split_case(Hs, M + K)
    W = (np.random.default_rng(K + N + 1).standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = res_pair(orc, W, gamma, 1e-5, 6.0, min(K, 128), M, lds=lds)
    compare_res(orc, g, o, R, D, gamma, 1e-5, tag="rand")


def test_res_sequence(orc):
    """Decode-like steps through one state with row strides above K: the gate
    fires on planted transients, so the re-quantize pass reads the written H."""
    M, K, N = 24, 1024, 64
    rng = np.random.default_rng(17)
    pers = np.sort(rng.choice(K, 6, replace=False))
    gamma = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = res_pair(orc, W, gamma, 1e-5, 6.0, 64, M, lds=(1032, 1040, 1096))
    flags = []
    for st in range(6):
        H = rng.standard_normal((M, K))
        H[:, pers] = rng.uniform(20, 100, (M, pers.size))
        if st in (2, 4):
            H[rng.integers(0, M, 3), rng.integers(0, K, 3)] = 90.0
        R, D = split_case(H.astype(np.float16), st)
        compare_res(orc, g, o, R, D, gamma, 1e-5, tag=f"step{st}")
        flags.append(g.flag())
    assert flags[0] == 1 and flags[1] == 0 and flags[2] == 1 and flags[4] == 1


def test_res_full_size(orc):
    """The prefill shape, set detected then cached, activation side only."""
    Hs, gamma = make_case(0, 2048, 8192, 82)
    R, D = split_case(Hs, 5)
    W = (np.random.default_rng(0).standard_normal((64, 8192)) * 0.02).astype(np.float16)
    g, o = res_pair(orc, W, gamma, 1e-5, 6.0, 256, 2048)
    r = compare_res(orc, g, o, R, D, gamma, 1e-5, products=False, tag="full")
    assert r.count >= 60
    r = compare_res(orc, g, o, R, D, gamma, 1e-5, products=False, tag="full-cached")
    assert r.flag == 0
