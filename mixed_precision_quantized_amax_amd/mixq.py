"""Python binding of ``libmixq.so`` (the C ABI declared in ``include/mixq.h``).

Argument marshalling only: torch tensors supply device memory and the
current stream; every step of the layer runs in the library's HIP kernels.
There is no fallback -- if the library is missing or the device is not a
gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmixq.so")

MIXQ_OK = 0
STATUS = {0: "MIXQ_OK", 1: "MIXQ_ERR_INVALID_ARG", 2: "MIXQ_ERR_UNSUPPORTED_SHAPE",
          3: "MIXQ_ERR_UNSUPPORTED_DEVICE", 4: "MIXQ_ERR_NO_DEVICE", 5: "MIXQ_ERR_HIP",
          6: "MIXQ_ERR_WORKSPACE"}
FLAG_FIRED = 1
FLAG_OVERFLOW = 2
PACK_FULL = 0
PACK_OUTLIER_COLS = 1
OUT_F32 = 0
OUT_SWIGLU_F16 = 1
OUT_F16 = 2
OUT_BF16 = 3
PROGRESSIVE_GROUP = 128
OUTLIER_ALIGN = 32
K_MULTIPLE = 64
GATHER_SLOTS = 256


class MixqError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({msg})")
        self.code = code


class ActState(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("count", ctypes.c_void_p),
                ("flag", ctypes.c_void_p), ("bitmap", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("k_cap", ctypes.c_int32)]


class Weight(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("s_w", ctypes.c_void_p), ("w_out", ctypes.c_void_p),
                ("k_out", ctypes.c_void_p), ("bits", ctypes.c_int32), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("k_cap", ctypes.c_int32), ("gated", ctypes.c_int32), ("group", ctypes.c_int32),
                ("gsz", ctypes.c_void_p), ("rmap", ctypes.c_void_p), ("n_out", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m mixed_precision_quantized_amax_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.mixq_outlier_ld.argtypes = [I32]
        L.mixq_outlier_ld.restype = I64
        L.mixq_bitmap_words.argtypes = [I64]
        L.mixq_bitmap_words.restype = I64
        L.mixq_state_work_words.argtypes = [I64]
        L.mixq_state_work_words.restype = I64
        L.mixq_packed_weight_bytes.argtypes = [I64, I64, I32]
        L.mixq_packed_weight_bytes.restype = ctypes.c_size_t
        L.mixq_quantize_act.argtypes = [P, I64, I64, I64, ctypes.c_float,
                                        ctypes.POINTER(ActState), P, P, P, P]
        L.mixq_quantize_act.restype = ctypes.c_int
        L.mixq_quantize_act_regather.argtypes = [P, I64, I64, I64, ctypes.c_float,
                                                 ctypes.POINTER(ActState), P, P, P, P,
                                                 ctypes.POINTER(Weight), P]
        L.mixq_quantize_act_regather.restype = ctypes.c_int
        L.mixq_rmsnorm_quantize_act.argtypes = [P, I64, I64, I64, P, ctypes.c_float,
                                                ctypes.c_float, ctypes.POINTER(ActState), P, P,
                                                P, P, P]
        L.mixq_rmsnorm_quantize_act.restype = ctypes.c_int
        L.mixq_add_rmsnorm_quantize_act.argtypes = [P, I64, P, I64, P, I64, I64, I64, P,
                                                    ctypes.c_float, ctypes.c_float,
                                                    ctypes.POINTER(ActState), P, P, P, P, P]
        L.mixq_add_rmsnorm_quantize_act.restype = ctypes.c_int
        L.mixq_pack_weight.argtypes = [P, I64, I64, I32, ctypes.POINTER(ActState), I32,
                                       ctypes.POINTER(Weight), P]
        L.mixq_pack_weight.restype = ctypes.c_int
        L.mixq_gemm.argtypes = [P, P, P, ctypes.POINTER(ActState), ctypes.POINTER(Weight), I64,
                                P, I64, P, P]
        L.mixq_gemm.restype = ctypes.c_int
        L.mixq_gemm_ws.argtypes = [P, P, P, ctypes.POINTER(ActState), ctypes.POINTER(Weight), I64,
                                   P, I64, P, P, ctypes.c_size_t, P]
        L.mixq_gemm_ws.restype = ctypes.c_int
        L.mixq_gemm_ex.argtypes = [P, P, P, ctypes.POINTER(ActState), ctypes.POINTER(Weight), I64,
                                   P, I64, I32, P, P, ctypes.c_size_t, P]
        L.mixq_gemm_ex.restype = ctypes.c_int
        L.mixq_gemm_workspace_bytes.argtypes = [I64, I64, I64, I32]
        L.mixq_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.mixq_status_string.argtypes = [ctypes.c_int]
        L.mixq_status_string.restype = ctypes.c_char_p
        L.mixq_check_device.argtypes = []
        L.mixq_check_device.restype = ctypes.c_int
        L.mixq_version.argtypes = []
        L.mixq_version.restype = ctypes.c_int
        L.mixq_gemm_noalloc.argtypes = [P, P, P, ctypes.POINTER(ActState),
                                        ctypes.POINTER(Weight), I64, P, I64, I32, P, P]
        L.mixq_gemm_noalloc.restype = ctypes.c_int
        L.mixq_gemm_scratch_bytes.argtypes = []
        L.mixq_gemm_scratch_bytes.restype = ctypes.c_size_t
        L.mixq_set_clock_record.argtypes = [P, I32]
        L.mixq_set_clock_record.restype = ctypes.c_int
        L.mixq_set_gemm_variant.argtypes = [I32]
        L.mixq_set_gemm_variant.restype = ctypes.c_int
        L.mixq_mfma_probe.argtypes = [P, I64, P, I64, I32, I32, P, P, P]
        L.mixq_mfma_probe.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != MIXQ_OK:
        raise MixqError(fn, rc, lib().mixq_status_string(rc).decode())


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def gemm_noalloc(Xq: torch.Tensor, s_x: torch.Tensor, X_out: torch.Tensor | None,
                 state: OutlierState, pw: PackedWeight, Y: torch.Tensor,
                 out_mode: int = OUT_F32, acc_debug: torch.Tensor | None = None) -> None:
    """mixq_gemm_noalloc: mixq_gemm_ex with the library's own device
    workspace (no workspace argument, nothing allocated)."""
    M = Xq.shape[0]
    st = state.c()
    w = pw.c()
    rc = lib().mixq_gemm_noalloc(_ptr(Xq), _ptr(s_x), _ptr(X_out), ctypes.byref(st),
                                 ctypes.byref(w), M, _ptr(Y), Y.stride(0), int(out_mode),
                                 _ptr(acc_debug), _stream(Y.device))
    _check("mixq_gemm_noalloc", rc)


# GEMM kernel variants (ids of mixq_set_gemm_variant; testing hook)
GEMM_VARIANTS = {"auto": 0, "256x256": 1, "128x128": 2, "256x256_swp": 3, "256x256_kpair": 4,
                 "128x128_kpair": 5, "128x128_swp": 6}


def set_gemm_variant(variant: int | str) -> None:
    """Force one GEMM kernel variant for every later call (0 / "auto" =
    the automatic choice); for tests that cover each variant."""
    v = GEMM_VARIANTS[variant] if isinstance(variant, str) else int(variant)
    _check("mixq_set_gemm_variant", lib().mixq_set_gemm_variant(v))


def mfma_probe(a: torch.Tensor, b: torch.Tensor, iters: int, blocks: int,
               out: torch.Tensor, clk: torch.Tensor | None = None, stream=None) -> None:
    """Measurement aid (mixq_mfma_probe): ``blocks`` x 4 waves run ``iters``
    rounds of the GEMM main loop's 32 INT8 MFMAs on operand bytes taken from
    ``a`` and ``b`` (int8 device tensors, any shape), with no memory traffic
    in the timed part.  ``out``: int32 [256 * blocks], each lane's sum of its
    accumulators; ``clk``: int64 [4 * blocks] clock stamps, or None."""
    assert a.dtype == torch.int8 and b.dtype == torch.int8 and a.is_contiguous() and b.is_contiguous()
    assert out.dtype == torch.int32 and out.numel() >= 256 * blocks
    assert clk is None or (clk.dtype == torch.int64 and clk.numel() >= 4 * blocks)
    s = stream if stream is not None else torch.cuda.current_stream(a.device).cuda_stream
    na = a.numel() // 16 * 16
    nb = b.numel() // 16 * 16
    _check("mixq_mfma_probe", lib().mixq_mfma_probe(
        _ptr(a), na, _ptr(b), nb, iters, blocks, _ptr(out),
        _ptr(clk), ctypes.c_void_p(s)))


def set_clock_record(buf: torch.Tensor | None) -> None:
    """Measurement hook: while ``buf`` (int64 device tensor of 4 * n) is
    set, GEMM blocks b < n write their entry/exit shader-clock and 100 MHz
    real-time stamps to buf[4b:4b+4]; None turns it off."""
    if buf is None:
        _check("mixq_set_clock_record", lib().mixq_set_clock_record(None, 0))
    else:
        assert buf.dtype == torch.int64 and buf.numel() % 4 == 0
        _check("mixq_set_clock_record",
               lib().mixq_set_clock_record(ctypes.c_void_p(buf.data_ptr()), buf.numel() // 4))


def outlier_ld(k_cap: int) -> int:
    return int(lib().mixq_outlier_ld(k_cap))


def bitmap_words(K: int) -> int:
    return int(lib().mixq_bitmap_words(K))


@dataclass
class OutlierState:
    """Device memory of one cached outlier-channel set (zero = empty)."""
    K: int
    k_cap: int
    idx: torch.Tensor
    count: torch.Tensor
    flag: torch.Tensor
    bitmap: torch.Tensor
    work: torch.Tensor

    @classmethod
    def create(cls, K: int, k_cap: int, device="cuda") -> "OutlierState":
        w = bitmap_words(K)
        ww = int(lib().mixq_state_work_words(K))
        z = lambda n, dt: torch.zeros(max(n, 1), dtype=dt, device=device)  # noqa: E731
        return cls(K=K, k_cap=k_cap, idx=z(k_cap, torch.int32), count=z(1, torch.int32),
                   flag=z(1, torch.int32), bitmap=z(w, torch.int32), work=z(ww, torch.int32))

    def c(self) -> ActState:
        return ActState(self.idx.data_ptr(), self.count.data_ptr(), self.flag.data_ptr(),
                        self.bitmap.data_ptr(), self.work.data_ptr(), self.k_cap)

    def reset(self):
        for t in (self.idx, self.count, self.flag, self.bitmap, self.work):
            t.zero_()


@dataclass
class PackedWeight:
    N: int
    K: int
    bits: int
    k_cap: int
    wq: torch.Tensor
    s_w: torch.Tensor
    w_out: torch.Tensor
    k_out: torch.Tensor
    gated: int = 0  # 1: W = [W_gate; W_up], packed with 32-row blocks interleaved
    group: int = 0  # PROGRESSIVE_GROUP: progressive group-wise INT4
    gsz: torch.Tensor | None = None  # [K/group, N] uint16: s2 | z << 8
    # row subset: packed row -> W row (= Y column); int32 [N] on the device
    rmap: torch.Tensor | None = None
    n_out: int = 0  # rows of W (columns of Y) when rmap is set

    @classmethod
    def create(cls, N: int, K: int, bits: int, k_cap: int, device="cuda",
               gated: bool = False, group: int = 0) -> "PackedWeight":
        nbytes = int(lib().mixq_packed_weight_bytes(N, K, bits))
        if nbytes == 0:
            raise ValueError("invalid weight shape or bits")
        ld = outlier_ld(k_cap)
        return cls(N=N, K=K, bits=bits, k_cap=k_cap,
                   wq=torch.empty(nbytes, dtype=torch.uint8, device=device),
                   s_w=torch.empty(N, dtype=torch.float32, device=device),
                   w_out=torch.zeros(max(N * ld, 1), dtype=torch.float16, device=device),
                   k_out=torch.zeros(GATHER_SLOTS, dtype=torch.int32, device=device),
                   gated=int(bool(gated)), group=int(group),
                   gsz=(torch.zeros(N * (K // group), dtype=torch.int16, device=device)
                        if group else None))

    @classmethod
    def create_rows(cls, rows, n_out: int, K: int, bits: int, k_cap: int, device="cuda",
                    group: int = 0) -> "PackedWeight":
        """A weight over a subset of W's rows: packed row n quantizes W row
        rows[n] and the product writes Y column rows[n]."""
        rm = torch.as_tensor(np.asarray(rows, dtype=np.int32))
        pw = cls.create(int(rm.shape[0]), K, bits, k_cap, device=device, group=group)
        pw.rmap = rm.to(device)
        pw.n_out = int(n_out)
        return pw

    def c(self) -> Weight:
        return Weight(self.wq.data_ptr(), self.s_w.data_ptr(), self.w_out.data_ptr(),
                      self.k_out.data_ptr(), self.bits, self.N, self.K, self.k_cap, self.gated,
                      self.group, None if self.gsz is None else self.gsz.data_ptr(),
                      None if self.rmap is None else self.rmap.data_ptr(), self.n_out)

    def codes_view(self) -> torch.Tensor:
        """int8 [N, K] (bits 8) or packed uint8 [N, K/2] (bits 4) view of wq."""
        if self.bits == 8:
            return self.wq.view(torch.int8).view(self.N, self.K)
        # K-tile-major inside 32-row blocks: [N/32][K/64][32 rows][32 bytes]
        nb = (self.N + 31) // 32
        t = self.wq.view(nb, self.K // 64, 32, 32).permute(0, 2, 1, 3)
        return t.reshape(nb * 32, self.K // 2)[: self.N]

    def w_out_view(self) -> torch.Tensor:
        return self.w_out[: self.N * outlier_ld(self.k_cap)].view(self.N, outlier_ld(self.k_cap))


def quantize_act(X: torch.Tensor, tau: float, state: OutlierState, Xq: torch.Tensor,
                 s_x: torch.Tensor, X_out: torch.Tensor | None) -> None:
    """mixq_quantize_act on the current stream.  X: fp16 [M, ldx] (row-major,
    the first K columns used)."""
    assert X.dtype == torch.float16 and X.dim() == 2 and X.stride(1) == 1
    M = X.shape[0]
    st = state.c()
    rc = lib().mixq_quantize_act(_ptr(X), M, state.K, X.stride(0), float(tau), ctypes.byref(st),
                                 _ptr(Xq), _ptr(s_x), _ptr(X_out), _stream(X.device))
    _check("mixq_quantize_act", rc)


def quantize_act_regather(X: torch.Tensor, tau: float, state: OutlierState, Xq: torch.Tensor,
                          s_x: torch.Tensor, X_out: torch.Tensor | None, W: torch.Tensor,
                          pw: PackedWeight) -> None:
    """mixq_quantize_act followed by mixq_pack_weight(PACK_OUTLIER_COLS) for
    one weight, in two kernel launches instead of three."""
    M, K = X.shape
    st = state.c()
    w = pw.c()
    rc = lib().mixq_quantize_act_regather(_ptr(X), M, K, X.stride(0), ctypes.c_float(tau),
                                          ctypes.byref(st), _ptr(Xq), _ptr(s_x), _ptr(X_out),
                                          _ptr(W), ctypes.byref(w), _stream(X.device))
    _check("mixq_quantize_act_regather", rc)


def rmsnorm_quantize_act(H: torch.Tensor, gamma: torch.Tensor, eps: float, tau: float,
                         state: OutlierState, Xq: torch.Tensor, s_x: torch.Tensor,
                         X_out: torch.Tensor | None, rstd: torch.Tensor) -> None:
    """mixq_rmsnorm_quantize_act on the current stream: the RMSNorm of H
    (fp16 [M, ldh], gamma fp16 [K]) fused into the activation pass; rstd fp32
    [M] receives each token's 1/sqrt(mean square + eps)."""
    assert H.dtype == torch.float16 and H.dim() == 2 and H.stride(1) == 1
    assert gamma.dtype == torch.float16 and gamma.is_contiguous()
    assert rstd.dtype == torch.float32
    M = H.shape[0]
    st = state.c()
    rc = lib().mixq_rmsnorm_quantize_act(_ptr(H), M, state.K, H.stride(0), _ptr(gamma),
                                         float(eps), float(tau), ctypes.byref(st), _ptr(Xq),
                                         _ptr(s_x), _ptr(X_out), _ptr(rstd), _stream(H.device))
    _check("mixq_rmsnorm_quantize_act", rc)


def add_rmsnorm_quantize_act(R: torch.Tensor, D: torch.Tensor, H: torch.Tensor,
                             gamma: torch.Tensor, eps: float, tau: float, state: OutlierState,
                             Xq: torch.Tensor, s_x: torch.Tensor, X_out: torch.Tensor | None,
                             rstd: torch.Tensor) -> None:
    """mixq_add_rmsnorm_quantize_act on the current stream: H = R + D (fp16,
    written; it must not overlap R or D), then the RMSNorm of H fused into the
    activation pass."""
    for t in (R, D, H):
        assert t.dtype == torch.float16 and t.dim() == 2 and t.stride(1) == 1
    assert gamma.dtype == torch.float16 and gamma.is_contiguous()
    assert rstd.dtype == torch.float32
    M = R.shape[0]
    st = state.c()
    rc = lib().mixq_add_rmsnorm_quantize_act(
        _ptr(R), R.stride(0), _ptr(D), D.stride(0), _ptr(H), H.stride(0), M, state.K,
        _ptr(gamma), float(eps), float(tau), ctypes.byref(st), _ptr(Xq), _ptr(s_x), _ptr(X_out),
        _ptr(rstd), _stream(R.device))
    _check("mixq_add_rmsnorm_quantize_act", rc)


def pack_weight(W: torch.Tensor, state: OutlierState, pw: PackedWeight,
                mode: int = PACK_FULL) -> None:
    """mixq_pack_weight.  W: fp16 [N, K], or [n_out, K] for a row subset."""
    assert W.dtype == torch.float16 and W.is_contiguous()
    assert W.shape[0] == (pw.n_out if pw.rmap is not None else pw.N)
    K = W.shape[1]
    st = state.c()
    w = pw.c()
    rc = lib().mixq_pack_weight(_ptr(W), pw.N, K, pw.bits, ctypes.byref(st), mode, ctypes.byref(w),
                                _stream(W.device))
    _check("mixq_pack_weight", rc)


def gemm_workspace_bytes(M: int, N: int, K: int, bits: int) -> int:
    return int(lib().mixq_gemm_workspace_bytes(M, N, K, bits))


def gemm_workspace(M: int, N: int, K: int, bits: int, device=None) -> torch.Tensor | None:
    """Zero-filled split-K workspace for ``gemm(..., ws=...)``, or None when
    the product is not split (then no workspace is needed)."""
    n = gemm_workspace_bytes(M, N, K, bits)
    if n == 0:
        return None
    return torch.zeros((n + 15) // 16 * 4, dtype=torch.int32, device=device or "cuda")


def gemm(Xq: torch.Tensor, s_x: torch.Tensor, X_out: torch.Tensor | None, state: OutlierState,
         pw: PackedWeight, Y: torch.Tensor, acc_debug: torch.Tensor | None = None,
         ws: torch.Tensor | None = None) -> None:
    M = Xq.shape[0]
    st = state.c()
    w = pw.c()
    if ws is None:
        rc = lib().mixq_gemm(_ptr(Xq), _ptr(s_x), _ptr(X_out), ctypes.byref(st), ctypes.byref(w),
                             M, _ptr(Y), Y.stride(0), _ptr(acc_debug), _stream(Y.device))
        _check("mixq_gemm", rc)
    else:
        rc = lib().mixq_gemm_ws(_ptr(Xq), _ptr(s_x), _ptr(X_out), ctypes.byref(st),
                                ctypes.byref(w), M, _ptr(Y), Y.stride(0), _ptr(acc_debug),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(Y.device))
        _check("mixq_gemm_ws", rc)


def gemm_ex(Xq: torch.Tensor, s_x: torch.Tensor, X_out: torch.Tensor | None,
            state: OutlierState, pw: PackedWeight, Y: torch.Tensor, out_mode: int,
            acc_debug: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> None:
    """mixq_gemm_ex: OUT_F32 (Y fp32 [M, >= N]), OUT_F16 / OUT_BF16 (Y fp16 /
    bf16 [M, >= N], the fp32 output rounded to nearest even) or
    OUT_SWIGLU_F16 (a gated weight; Y fp16 [M, >= N/2] = silu(gate) * up)."""
    M = Xq.shape[0]
    st = state.c()
    w = pw.c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().mixq_gemm_ex(_ptr(Xq), _ptr(s_x), _ptr(X_out), ctypes.byref(st), ctypes.byref(w),
                            M, _ptr(Y), Y.stride(0), int(out_mode), _ptr(acc_debug), _ptr(ws),
                            nbytes, _stream(Y.device))
    _check("mixq_gemm_ex", rc)


class LayerStep:
    """One layer step (quantize, outlier-column gather, GEMM) with every
    ctypes argument built once, so that a hot loop pays only the foreign
    calls and their kernel launches.  ``fused`` (the default) quantizes and
    re-gathers the weight's outlier columns in one call
    (mixq_quantize_act_regather: two launches); otherwise mixq_quantize_act
    and mixq_pack_weight(PACK_OUTLIER_COLS) run separately (three)."""

    def __init__(self, X: torch.Tensor, tau: float, state: OutlierState, W: torch.Tensor,
                 pw: PackedWeight, Xq: torch.Tensor, s_x: torch.Tensor,
                 X_out: torch.Tensor | None, Y: torch.Tensor,
                 acc_debug: torch.Tensor | None = None, stream=None,
                 ws: torch.Tensor | None = None, fused: bool = True):
        L = lib()
        dev = X.device
        s = ctypes.c_void_p(stream if stream is not None
                            else torch.cuda.current_stream(dev).cuda_stream)
        self._keep = (X, W, Xq, s_x, X_out, Y, acc_debug, state, pw, ws)
        self._st = state.c()
        self._w = pw.c()
        M = X.shape[0]
        if fused:
            self._act = [
                ("mixq_quantize_act_regather", L.mixq_quantize_act_regather,
                 (_ptr(X), M, state.K, X.stride(0), ctypes.c_float(tau), ctypes.byref(self._st),
                  _ptr(Xq), _ptr(s_x), _ptr(X_out), _ptr(W), ctypes.byref(self._w), s))]
        else:
            self._act = [
                ("mixq_quantize_act", L.mixq_quantize_act,
                 (_ptr(X), M, state.K, X.stride(0), ctypes.c_float(tau), ctypes.byref(self._st),
                  _ptr(Xq), _ptr(s_x), _ptr(X_out), s)),
                ("mixq_pack_weight", L.mixq_pack_weight,
                 (_ptr(W), pw.N, pw.K, pw.bits, ctypes.byref(self._st), PACK_OUTLIER_COLS,
                  ctypes.byref(self._w), s))]
        self._gemm = (
            ("mixq_gemm", L.mixq_gemm,
             (_ptr(Xq), _ptr(s_x), _ptr(X_out), ctypes.byref(self._st), ctypes.byref(self._w),
              M, _ptr(Y), Y.stride(0), _ptr(acc_debug), s)) if ws is None else
            ("mixq_gemm_ws", L.mixq_gemm_ws,
             (_ptr(Xq), _ptr(s_x), _ptr(X_out), ctypes.byref(self._st), ctypes.byref(self._w),
              M, _ptr(Y), Y.stride(0), _ptr(acc_debug), _ptr(ws),
              ws.numel() * ws.element_size(), s)))
        self._calls = self._act + [self._gemm]

    def act(self):
        """The activation side and the gather: everything before the GEMM."""
        for name, fn, args in self._act:
            rc = fn(*args)
            if rc:
                _check(name, rc)

    def gemm(self):
        name, fn, args = self._gemm
        rc = fn(*args)
        if rc:
            _check(name, rc)

    def __call__(self):
        for name, fn, args in self._calls:
            rc = fn(*args)
            if rc:
                _check(name, rc)


class LayerGraph:
    """One layer step captured into a HIP graph: a replay launches the step's
    kernels without a host round trip per kernel.  Nothing is cached in the
    graph but the launches -- every kernel reads the outlier state and the
    activations from device memory on each replay, so a replay computes what
    the same three eager calls would (a gate firing during a replay included).
    The step allocates nothing and records no memory fills, so it captures
    as is.  Arguments are those of ``LayerStep`` (without ``stream``)."""

    def __init__(self, *args, **kwargs):
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            # built inside the capture so that it binds the capture stream
            self.step = LayerStep(*args, **kwargs)
            self.step()

    def replay(self):
        self.graph.replay()

    __call__ = replay


class MixQLinear:
    """Y = X W^T through the three library calls, with the outlier set cached
    across calls (the layer the MixQ article describes)."""

    def __init__(self, W: torch.Tensor, bits: int = 8, tau: float = 6.0, k_cap: int = 256):
        N, K = W.shape
        self.W = W.contiguous()
        self.N, self.K, self.bits, self.tau = N, K, bits, float(tau)
        self.k_cap = min(k_cap, K)
        self.state = OutlierState.create(K, self.k_cap, W.device)
        self.pw = PackedWeight.create(N, K, bits, self.k_cap, W.device)
        pack_weight(self.W, self.state, self.pw, PACK_FULL)
        self._bufs = {}

    def buffers(self, M: int):
        if M not in self._bufs:
            dev = self.W.device
            ld = outlier_ld(self.k_cap)
            self._bufs[M] = (torch.empty(M, self.K, dtype=torch.int8, device=dev),
                             torch.empty(M, dtype=torch.float32, device=dev),
                             torch.zeros(max(M * ld, 1), dtype=torch.float16, device=dev),
                             gemm_workspace(M, self.N, self.K, self.bits, dev))
        return self._bufs[M]

    def forward(self, X: torch.Tensor, Y: torch.Tensor | None = None,
                acc_debug: torch.Tensor | None = None) -> torch.Tensor:
        M = X.shape[0]
        Xq, s_x, X_out, ws = self.buffers(M)
        if Y is None:
            Y = torch.empty(M, self.N, dtype=torch.float32, device=X.device)
        quantize_act(X, self.tau, self.state, Xq, s_x, X_out)
        pack_weight(self.W, self.state, self.pw, PACK_OUTLIER_COLS)
        gemm(Xq, s_x, X_out, self.state, self.pw, Y, acc_debug, ws)
        return Y

    __call__ = forward


@dataclass
class MixedWeight:
    """Output-feature mixed precision (MixLLM page): the salient output
    features of W keep 8-bit weights and the others get progressive 4-bit
    ones, as two row-subset weights whose products write disjoint columns of
    one Y."""
    w8: PackedWeight | None  # None when no feature is salient
    w4: PackedWeight | None  # None when every feature is

    @classmethod
    def create(cls, salient, K: int, k_cap: int, device="cuda") -> "MixedWeight":
        sal = np.asarray(salient, dtype=bool)
        n = int(sal.shape[0])
        r8, r4 = np.flatnonzero(sal), np.flatnonzero(~sal)
        return cls(w8=PackedWeight.create_rows(r8, n, K, 8, k_cap, device) if r8.size else None,
                   w4=PackedWeight.create_rows(r4, n, K, 4, k_cap, device,
                                               group=PROGRESSIVE_GROUP) if r4.size else None)

    def parts(self):
        return [p for p in (self.w4, self.w8) if p is not None]

    def pack(self, W: torch.Tensor, state: OutlierState, mode: int = PACK_FULL) -> None:
        for p in self.parts():
            pack_weight(W, state, p, mode)

    def workspaces(self, M: int, device=None):
        """Split-K workspaces, (4-bit, 8-bit)."""
        return tuple(None if p is None else gemm_workspace(M, p.N, p.K, p.bits, device)
                     for p in (self.w4, self.w8))

    def gemm(self, Xq, s_x, X_out, state, Y, acc_debug=(None, None), ws=(None, None)) -> None:
        """Both products into Y; acc_debug and ws are (4-bit, 8-bit) pairs."""
        for p, dbg, w in zip((self.w4, self.w8), acc_debug, ws):
            if p is not None:
                gemm(Xq, s_x, X_out, state, p, Y, dbg, w)
