"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the CPU oracle on the same seeded inputs and compare them."""
from __future__ import annotations

import sys

import numpy as np
import torch

from mixed_precision_quantized_amax_amd import mixq
from oracle import Oracle

# Y tolerance: max |dY| <= 1e-3 * max |Y| (the integer part is exact; the
# rest is fp32 rounding of the dequantize/scale/add and of the fp16 outlier
# product, about 1e-6 relative).
Y_RTOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def set_from_bitmap(bitmap: np.ndarray, K: int) -> np.ndarray:
    bits = np.unpackbits(bitmap.view(np.uint8), bitorder="little")[:K]
    return bits.astype(np.uint8)


class GpuLayer:
    """One layer on the GPU: state, packed weight and output buffers."""

    def __init__(self, W: np.ndarray, bits: int, tau: float, k_cap: int, M: int,
                 split: bool = True):
        self.N, self.K = W.shape
        self.split = split  # pass a split-K workspace to the GEMM when the shape uses one
        self.bits, self.tau, self.k_cap = bits, tau, k_cap
        self.Wd = to_dev(W.view(np.float16))
        self.state = mixq.OutlierState.create(self.K, k_cap)
        self.pw = mixq.PackedWeight.create(self.N, self.K, bits, k_cap)
        self.ld = mixq.outlier_ld(k_cap)
        self.alloc(M)
        mixq.pack_weight(self.Wd, self.state, self.pw, mixq.PACK_FULL)

    def alloc(self, M):
        self.M = M
        self.Xq = torch.empty(M, self.K, dtype=torch.int8, device="cuda")
        self.s_x = torch.empty(M, dtype=torch.float32, device="cuda")
        self.X_out = torch.full((max(M * self.ld, 1),), float("nan"), dtype=torch.float16,
                                device="cuda") if self.ld else None
        self.Y = torch.full((M, self.N), float("nan"), dtype=torch.float32, device="cuda")
        self.ws = mixq.gemm_workspace(M, self.N, self.K, self.bits) if self.split else None

    def quantize(self, X: np.ndarray):
        Xd = to_dev(X.view(np.float16))
        mixq.quantize_act(Xd, self.tau, self.state, self.Xq, self.s_x, self.X_out)

    def regather(self):
        mixq.pack_weight(self.Wd, self.state, self.pw, mixq.PACK_OUTLIER_COLS)

    def gemm(self, acc_debug=None):
        mixq.gemm(self.Xq, self.s_x, self.X_out, self.state, self.pw, self.Y, acc_debug, self.ws)

    def step(self, X, acc=False):
        self.quantize(X)
        self.regather()
        dbg = torch.zeros(self.M, self.N, dtype=torch.int32, device="cuda") if acc else None
        self.gemm(dbg)
        torch.cuda.synchronize()
        return dbg

    # -- host copies -------------------------------------------------------------
    def count(self) -> int:
        return int(self.state.count.cpu()[0])

    def flag(self) -> int:
        return int(self.state.flag.cpu()[0])

    def idx(self) -> np.ndarray:
        return self.state.idx.cpu().numpy()[: self.count()]

    def in_set(self) -> np.ndarray:
        return set_from_bitmap(self.state.bitmap.cpu().numpy(), self.K)

    def x_out(self) -> np.ndarray:
        return self.X_out.view(torch.int16).cpu().numpy().view(np.uint16)[: self.M * self.ld] \
            .reshape(self.M, self.ld)

    def w_codes(self) -> np.ndarray:
        """Unpacked int8 codes of the packed weight, decoded here in NumPy."""
        raw = self.pw.codes_view().cpu().numpy()
        if self.bits == 8:
            return raw.view(np.int8)
        return unpack_int4(raw, self.K)


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    """Decode the documented nibble layout: per 32-bit word (8 consecutive k),
    byte j holds k+j in its low nibble and k+j+4 in its high nibble."""
    N = packed.shape[0]
    b = packed.reshape(N, K // 8, 4).astype(np.uint8)
    lo = (b & 0xF).astype(np.int8)
    hi = (b >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.concatenate([lo, hi], axis=2)  # [N, K/8, 8] = k+0..3, k+4..7
    return out.reshape(N, K).astype(np.int8)


def kpad(count: int) -> int:
    return (count + 31) // 32 * 32


def compare_quant(g: GpuLayer, X: np.ndarray, o_res) -> None:
    """Bit-exact comparison of everything the activation side produces."""
    assert g.flag() == o_res.flag, (g.flag(), o_res.flag)
    assert g.count() == o_res.count, (g.count(), o_res.count)
    assert np.array_equal(g.idx(), o_res.idx)
    assert np.array_equal(g.in_set(), o_res.in_set)
    Xq = g.Xq.cpu().numpy()
    s_x = g.s_x.cpu().numpy()
    bad = np.nonzero(Xq != o_res.Xq)
    assert bad[0].size == 0, f"{bad[0].size} Xq mismatches, first at {bad[0][0]},{bad[1][0]}"
    assert np.array_equal(s_x.view(np.uint32), o_res.s_x.view(np.uint32))
    if g.ld:
        kp = kpad(g.count())
        got, want = g.x_out()[:, :kp], o_res.X_out[:, :kp]
        bad = np.argwhere(got != want)
        assert bad.shape[0] == 0, (f"{bad.shape[0]} X_out mismatches, first (row, col) "
                                   f"{bad[:6].tolist()}: got {got[tuple(bad[:6].T)].tolist()} "
                                   f"want {want[tuple(bad[:6].T)].tolist()}; rows "
                                   f"{np.unique(bad[:, 0]).size}, cols {np.unique(bad[:, 1]).tolist()[:20]}")


def check_y(Y: np.ndarray, Yref: np.ndarray) -> float:
    scale = float(np.abs(Yref).max()) or 1.0
    err = float(np.abs(Y.astype(np.float64) - Yref).max()) / scale
    assert np.isfinite(Y).all()
    assert err <= Y_RTOL, err
    return err
