"""The C-ABI library on the CPU: it loads, exports every declared symbol, its
size helpers are right, and argument validation answers before any HIP call.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

from mixed_precision_quantized_amax_amd import mixq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mixq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mixq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("mixq_quantize_act", "mixq_pack_weight", "mixq_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = mixq.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_size_helpers():
    L = mixq.lib()
    assert [L.mixq_outlier_ld(k) for k in (0, 1, 31, 32, 33, 82, 96)] == [0, 32, 32, 32, 64, 96, 96]
    assert L.mixq_bitmap_words(8192) == 256 and L.mixq_bitmap_words(64) == 2
    assert L.mixq_state_work_words(8192) == 2 * 256 + 4
    assert L.mixq_packed_weight_bytes(8192, 8192, 8) == 8192 * 8192
    assert L.mixq_packed_weight_bytes(8192, 8192, 4) == 8192 * 4096
    assert L.mixq_packed_weight_bytes(40, 128, 4) == 64 * 64          # whole 32-row blocks
    assert L.mixq_packed_weight_bytes(8, 64, 5) == 0
    assert L.mixq_version() >= 100
    for c in range(6):
        assert L.mixq_status_string(c)


def _state(k_cap=8, null=None):
    vals = dict(idx=0x1000, count=0x2000, flag=0x3000, bitmap=0x4000, work=0x5000)
    if null:
        vals[null] = 0
    return mixq.ActState(vals["idx"], vals["count"], vals["flag"], vals["bitmap"],
                         vals["work"], k_cap)


def _quant(X=0x10000, M=4, K=64, ldx=64, tau=6.0, st=None, Xq=0x20000, sx=0x30000, xo=0x40000):
    st = st or _state()
    return mixq.lib().mixq_quantize_act(ctypes.c_void_p(X), M, K, ldx, tau, ctypes.byref(st),
                                        ctypes.c_void_p(Xq), ctypes.c_void_p(sx),
                                        ctypes.c_void_p(xo), None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=0), 1), (dict(Xq=0), 1), (dict(sx=0), 1), (dict(M=0), 1), (dict(K=0), 1),
    (dict(ldx=32), 1), (dict(tau=float("nan")), 1), (dict(tau=float("inf")), 1),
    (dict(tau=-1.0), 1), (dict(st=_state(k_cap=65)), 1), (dict(st=_state(k_cap=-1)), 1),
    (dict(st=_state(null="work")), 1), (dict(xo=0), 1),
    (dict(K=96, ldx=96), 2), (dict(K=65536 + 64, ldx=65536 + 64), 2), (dict(X=0x10008), 2),
    (dict(ldx=68), 2),
])
def test_quantize_act_validation(kw, code):
    assert _quant(**kw) == code


def _norm(H=0x10000, M=4, K=64, ldh=64, gamma=0x50000, eps=1e-5, tau=6.0, st=None, Xq=0x20000,
          sx=0x30000, xo=0x40000, rstd=0x60000):
    st = st or _state()
    return mixq.lib().mixq_rmsnorm_quantize_act(
        ctypes.c_void_p(H), M, K, ldh, ctypes.c_void_p(gamma), eps, tau, ctypes.byref(st),
        ctypes.c_void_p(Xq), ctypes.c_void_p(sx), ctypes.c_void_p(xo), ctypes.c_void_p(rstd), None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), 1), (dict(gamma=0), 1), (dict(rstd=0), 1), (dict(eps=float("nan")), 1),
    (dict(eps=float("inf")), 1), (dict(eps=-1e-6), 1), (dict(tau=-1.0), 1), (dict(ldh=32), 1),
    (dict(st=_state(k_cap=65)), 1), (dict(xo=0), 1),
    (dict(K=32768 + 64, ldh=32768 + 64, st=_state(k_cap=8)), 2), (dict(gamma=0x50008), 2),
    (dict(K=96, ldh=96), 2), (dict(H=0x10008), 2),
])
def test_rmsnorm_quantize_act_validation(kw, code):
    assert _norm(**kw) == code


def _addnorm(R=0x10000, ldr=64, D=0x70000, ldd=64, H=0x80000, ldh=64, M=4, K=64, gamma=0x50000,
             eps=1e-5, tau=6.0, st=None, Xq=0x20000, sx=0x30000, xo=0x40000, rstd=0x60000):
    st = st or _state()
    v = ctypes.c_void_p
    return mixq.lib().mixq_add_rmsnorm_quantize_act(
        v(R), ldr, v(D), ldd, v(H), ldh, M, K, v(gamma), eps, tau, ctypes.byref(st), v(Xq), v(sx),
        v(xo), v(rstd), None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), 1), (dict(D=0), 1), (dict(H=0), 1), (dict(gamma=0), 1), (dict(rstd=0), 1),
    (dict(ldd=32), 1), (dict(ldh=32), 1), (dict(eps=-1.0), 1),
    (dict(H=0x10000), 1), (dict(H=0x10000 + 4 * 64 * 2 - 16), 1), (dict(H=0x70000), 1),
    (dict(D=0x70008), 2), (dict(H=0x80008), 2), (dict(ldd=68), 2), (dict(ldh=68), 2),
    (dict(K=32768 + 64, ldr=32768 + 64, ldd=32768 + 64, ldh=32768 + 64, D=0x100000, H=0x200000), 2),
])
def test_add_rmsnorm_quantize_act_validation(kw, code):
    assert _addnorm(**kw) == code


def test_valid_arguments_need_a_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _quant() == 4                       # MIXQ_ERR_NO_DEVICE, nothing launched
    assert _norm() == 4 and _norm(K=32768, ldh=32768) == 4 and _norm(eps=0.0) == 4
    assert _addnorm() == 4 and _addnorm(H=0x10000 + 4 * 64 * 2) == 4  # adjacent, not overlapping
    assert mixq.lib().mixq_check_device() == 4


def _weight(N=16, K=64, bits=8, k_cap=8, gated=0, group=0, n_out=0, **null):
    vals = dict(wq=0x100000, s_w=0x200000, w_out=0x300000, k_out=0x400000, gsz=0x500000, rmap=0)
    vals.update(null)
    return mixq.Weight(vals["wq"], vals["s_w"], vals["w_out"], vals["k_out"], bits, N, K, k_cap,
                       gated, group, vals["gsz"], vals["rmap"] or None, n_out)


def _rows(N=512, n_out=3000, bits=4, group=128, **kw):
    """A row-subset descriptor (K = 128: one progressive group)."""
    kw.setdefault("rmap", 0x600000)
    return _weight(N=N, K=128, bits=bits, group=group if bits == 4 else 0, n_out=n_out, **kw)


@pytest.mark.parametrize("args,code", [
    (dict(bits=5), 1), (dict(mode=7), 1), (dict(N=0), 1), (dict(w=_weight(N=8)), 1),
    (dict(w=_weight(bits=4)), 1), (dict(w=_weight(k_cap=4)), 1), (dict(w=_weight(wq=0)), 1),
    (dict(w=_weight(k_out=0)), 1), (dict(K=96, w=_weight(K=96)), 2),
    (dict(w=_weight(gated=2)), 1), (dict(w=_weight(gated=1)), 2),          # gated: N % 64
    (dict(w=_weight(group=64, bits=4), bits=4), 1),                        # group size
    (dict(w=_weight(group=128), bits=8), 1),                               # groups need INT4
    (dict(w=_weight(group=128, bits=4, gsz=0), bits=4), 1),                # no group table
    (dict(w=_weight(group=128, bits=4), bits=4), 2),                       # K = 64 < 128
    (dict(w=_rows(group=0), N=512, K=128, bits=4), 1),                     # INT4 rows: groups
    (dict(w=_rows(n_out=0), N=512, K=128, bits=4), 1),                     # no output rows
    (dict(w=_rows(gated=1), N=512, K=128, bits=4), 1),                     # not with gated
    (dict(w=_rows(bits=8, n_out=0), N=512, K=128, bits=8), 1),
])
def test_pack_weight_validation(args, code):
    N = args.get("N", 16)
    K = args.get("K", 64)
    bits = args.get("bits", 8)
    mode = args.get("mode", 0)
    w = args.get("w", _weight(N=N or 16, K=K, bits=bits if bits in (4, 8) else 8))
    st = _state()
    rc = mixq.lib().mixq_pack_weight(ctypes.c_void_p(0x900000), N, K, bits, ctypes.byref(st), mode,
                                     ctypes.byref(w), None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(M=0), 1), (dict(Y=0), 1), (dict(ldy=8), 1), (dict(Xq=0), 1),
    (dict(w=_weight(k_cap=3)), 1), (dict(w=_weight(bits=6)), 1), (dict(xo=0), 1),
    (dict(w=_weight(K=100)), 2), (dict(Xq=0x20004), 2),
])
def test_gemm_validation(args, code):
    w = args.get("w", _weight())
    st = _state()
    rc = mixq.lib().mixq_gemm(ctypes.c_void_p(args.get("Xq", 0x20000)), ctypes.c_void_p(0x30000),
                              ctypes.c_void_p(args.get("xo", 0x40000)), ctypes.byref(st),
                              ctypes.byref(w), args.get("M", 4), ctypes.c_void_p(args.get("Y", 0x50000)),
                              args.get("ldy", 16), None, None)
    assert rc == code


def _gemm(**args):
    w = args.get("w", _weight())
    st = _state()
    return mixq.lib().mixq_gemm(ctypes.c_void_p(args.get("Xq", 0x20000)), ctypes.c_void_p(0x30000),
                                ctypes.c_void_p(args.get("xo", 0x40000)), ctypes.byref(st),
                                ctypes.byref(w), args.get("M", 4),
                                ctypes.c_void_p(args.get("Y", 0x50000)), args.get("ldy", 16), None,
                                None)


def test_gemm_32bit_offsets():
    """Y stores take 32-bit byte offsets within a tile of at most 256 rows,
    and the grid is one dimension: sizes beyond either are refused before
    anything is launched (FP6 explainer, section 2.3: unsupported shapes get
    an explicit error)."""
    import torch
    assert _gemm(ldy=1 << 21) == 2                       # 256 rows x ldy x 4 B = 2^31
    assert _gemm(ldy=(1 << 21) + 12345) == 2
    # a row subset with 2^30 packed rows and 2^30 tokens: 2^46 blocks
    big = _weight(N=1 << 30, n_out=16, rmap=0x600000)
    assert _gemm(w=big, M=1 << 30, ldy=16) == 2
    # the SwiGLU output is 2 bytes per element: twice the columns fit
    L = mixq.lib()
    gw = _weight(N=64, gated=1)
    st = _state()
    rc = L.mixq_gemm_ex(ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
                        ctypes.byref(st), ctypes.byref(gw), 4, ctypes.c_void_p(0x50000), 1 << 22,
                        mixq.OUT_SWIGLU_F16, None, None, 0, None)
    assert rc == 2
    if not torch.cuda.is_available():
        assert _gemm(ldy=(1 << 21) - 1) == 4             # the largest row stride that fits
        rc = L.mixq_gemm_ex(ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000),
                            ctypes.c_void_p(0x40000), ctypes.byref(st), ctypes.byref(gw), 4,
                            ctypes.c_void_p(0x50000), (1 << 22) - 1, mixq.OUT_SWIGLU_F16, None,
                            None, 0, None)
        assert rc == 4


def test_status_strings():
    L = mixq.lib()
    for code, name in mixq.STATUS.items():
        text = L.mixq_status_string(code).decode()
        assert text and text != "unknown status", name
    assert L.mixq_status_string(99).decode() == "unknown status"


def test_gemm_workspace_bytes():
    """Split-K plan (256 compute units): only thin INT8 products with K a
    multiple of 256; 4 KiB of counters plus two 64 KiB partial tiles per
    128 x 128 output tile."""
    L = mixq.lib()
    slot = 128 * 128 * 4
    assert L.mixq_gemm_workspace_bytes(2048, 8192, 8192, 8) == 0      # 256x256 path
    assert L.mixq_gemm_workspace_bytes(256, 8192, 8192, 8) == 4096 + 128 * 2 * slot
    assert L.mixq_gemm_workspace_bytes(512, 11008, 4096, 8) == 0      # 344 tiles >= 256
    assert L.mixq_gemm_workspace_bytes(512, 28672, 8192, 8) == 0      # 256x256 path
    assert L.mixq_gemm_workspace_bytes(64, 1024, 4096, 8) == 4096 + 8 * 2 * slot
    assert L.mixq_gemm_workspace_bytes(256, 8192, 8192, 4) == 0       # INT4: no split
    assert L.mixq_gemm_workspace_bytes(256, 8192, 8192 - 128, 8) == 0  # K % 256 != 0
    assert L.mixq_gemm_workspace_bytes(0, 8192, 8192, 8) == 0
    # a 256 x 256 product one round plus a short tail: columns [8192, N) as
    # 128 x 128 tiles with K split four ways (16 x 8 tail tiles)
    assert L.mixq_gemm_workspace_bytes(2048, 9165, 8192, 4) == 4096 + 16 * 8 * 4 * slot
    assert L.mixq_gemm_workspace_bytes(2048, 8448, 1024, 8) == 4096 + 16 * 2 * 4 * slot
    assert L.mixq_gemm_workspace_bytes(2048, 8448, 128, 8) == 0       # K too short to split
    assert L.mixq_gemm_workspace_bytes(2048, 16384, 8192, 8) == 0     # two full rounds


def test_gemm_ws_validation():
    w = _weight()
    st = _state()
    f = mixq.lib().mixq_gemm_ws
    args = [ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
            ctypes.byref(st), ctypes.byref(w), 4, ctypes.c_void_p(0x50000), 16, None]
    assert f(*args, ctypes.c_void_p(0x60008), 1 << 20, None) == 2    # misaligned workspace
    bad = list(args)
    bad[6] = None
    assert f(*bad, ctypes.c_void_p(0x60000), 1 << 20, None) == 1     # Y null
    import torch
    if not torch.cuda.is_available():
        assert f(*args, ctypes.c_void_p(0x60000), 1 << 20, None) == 4
        assert f(*args, None, 0, None) == 4


@pytest.mark.parametrize("kw,code", [
    (dict(mode=5), 1),                                   # unknown output mode
    (dict(mode=1), 1),                                   # SwiGLU needs a gated weight
    (dict(mode=1, w=_weight(N=64, gated=1), ldy=31), 1),  # fp16 row shorter than N/2
    (dict(mode=0, w=_weight(N=64, gated=1), ldy=32), 1),  # fp32 row shorter than N
    (dict(mode=0, w=_weight(group=128, bits=8)), 1),       # groups need INT4
    (dict(mode=0, w=_weight(group=128, bits=4, gsz=0)), 1),
    (dict(mode=0, w=_weight(group=128, bits=4)), 2),       # K = 64 < 128
    (dict(mode=0, w=_rows(), ldy=2999), 1),                # Y row shorter than n_out
    (dict(mode=1, w=_rows(), ldy=3000), 1),                # no SwiGLU output
    (dict(mode=0, w=_rows(group=0), ldy=3000), 1),         # INT4 rows: groups
    (dict(mode=0, w=_rows(n_out=0), ldy=3000), 1),
    (dict(mode=0, w=_rows(bits=8, n_out=0), ldy=3000), 1),
])
def test_gemm_ex_validation(kw, code):
    w = kw.get("w", _weight())
    st = _state()
    rc = mixq.lib().mixq_gemm_ex(ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000),
                                 ctypes.c_void_p(0x40000), ctypes.byref(st), ctypes.byref(w), 4,
                                 ctypes.c_void_p(0x50000), kw.get("ldy", 16), kw["mode"], None,
                                 None, 0, None)
    assert rc == code


def test_gemm_ex_valid_arguments_need_a_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = _state()
    wg = _weight(N=64, gated=1)
    assert mixq.lib().mixq_pack_weight(ctypes.c_void_p(0x900000), 64, 64, 8, ctypes.byref(st), 0,
                                       ctypes.byref(wg), None) == 4
    w = _weight(N=64, gated=1)
    f = mixq.lib().mixq_gemm_ex
    for mode, ldy in ((1, 32), (0, 64)):
        assert f(ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
                 ctypes.byref(st), ctypes.byref(w), 4, ctypes.c_void_p(0x50000), ldy, mode, None,
                 None, 0, None) == 4
    # row subsets (INT4 progressive and INT8): W has n_out rows, Y n_out columns
    for wm, bits in ((_rows(), 4), (_rows(bits=8), 8)):
        assert mixq.lib().mixq_pack_weight(ctypes.c_void_p(0x900000), 512, 128, bits,
                                           ctypes.byref(st), 0, ctypes.byref(wm), None) == 4
        assert f(ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
                 ctypes.byref(st), ctypes.byref(wm), 4, ctypes.c_void_p(0x50000), 3000, 0, None,
                 None, 0, None) == 4


@pytest.mark.parametrize("args", [
    (0, 64, 0x2000, 64, 1, 1, 0x3000),            # null a
    (0x1000, 64, 0, 64, 1, 1, 0x3000),            # null b
    (0x1000, 64, 0x2000, 64, 1, 1, 0),            # null out
    (0x1000, 64, 0x2000, 64, 0, 1, 0x3000),       # no rounds
    (0x1000, 64, 0x2000, 64, 1, 0, 0x3000),       # no blocks
    (0x1000, 8, 0x2000, 64, 1, 1, 0x3000),        # fewer than 16 bytes
    (0x1000, 64, 0x2000, 72, 1, 1, 0x3000),       # not a multiple of 16
    (0x1008, 64, 0x2000, 64, 1, 1, 0x3000),       # unaligned operand
])
def test_mfma_probe_validation(args):
    a, na, b, nb, iters, blocks, out = args
    rc = mixq.lib().mixq_mfma_probe(ctypes.c_void_p(a), na, ctypes.c_void_p(b), nb, iters, blocks,
                                    ctypes.c_void_p(out), None, None)
    assert rc == 1  # MIXQ_ERR_INVALID_ARG
