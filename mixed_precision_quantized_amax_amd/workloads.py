"""Seeded synthetic inputs for the mixed-precision linear layer.

This module only draws random numbers: it holds none of the method's
arithmetic, and it is the one piece of code that both the CPU oracle's tests
and the GPU path's tests and benchmark use.  Shapes follow the LLaMA
projections the MixQ article benchmarks on (LLaMA-70B; section
"MixQ的解决方案", Fig. 14); the article's real activations and weights are not
available, so these generators stand in for them.

Recipe (NumPy PCG64, ``default_rng``):
  1. outlier channel ids: ``rng.choice(K, k, replace=False)``, sorted;
  2. X: standard normal float32 [M, K];
  3. outlier values on those channels, either a uniform magnitude in
     [lo, hi) with an independent random sign (replacing the normal draw) or
     the normal draw multiplied by a factor;
  4. W: normal float32 [N, K] with standard deviation ``w_std``;
  5. both cast to float16 (round to nearest even) at the end.
For an output-feature mixed-precision weight, the 8-bit rows are a seeded
choice of 10% of the output features (``make_salient``).
For the decode sequence, a separate stream per step is derived from
``SeedSequence([seed, 1 + step])``.  For the RMSNorm fused in front of the
layer, X serves as the hidden state and the norm's weight is drawn from its
own stream (``make_norm_gamma``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterator

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    bits: int
    n_outliers: int
    outlier_kind: str        # "uniform" (|x| ~ U(lo, hi), random sign) or "scale"
    lo: float = 20.0
    hi: float = 100.0
    factor: float = 1.0
    w_std: float = 0.02
    tau: float = 6.0
    seed: int = 0
    steps: int = 1           # > 1: a decode sequence
    transient_steps: int = 0
    transient_max: int = 4
    description: str = ""

    @property
    def ops(self) -> int:
        """Operations of one logical product, 2*M*N*K."""
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "tiny": Workload("tiny", 16, 512, 512, 8, 4, "scale", factor=50.0,
                     description="tiny W8A8+outlier GEMM: X [16,512], 4 channels x50, "
                                 "W [512,512] N(0,0.02) int8"),
    "llama7b_up": Workload("llama7b_up", 512, 4096, 11008, 8, 20, "uniform",
                           description="LLaMA-7B MLP-up, batch-512 decode: X [512,4096], "
                                       "20 channels U(20,100)*sign, W [11008,4096] int8"),
    "llama70b_up": Workload("llama70b_up", 512, 8192, 28672, 8, 82, "uniform", w_std=0.015,
                            description="LLaMA-70B MLP-up: X [512,8192], 1% (82) channels "
                                        "U(20,100)*sign, W [28672,8192] N(0,0.015) int8"),
    "prefill_w4": Workload("prefill_w4", 2048, 8192, 8192, 4, 41, "scale", factor=60.0,
                           description="INT4-weight prefill: X [2048,8192], 0.5% (41) "
                                       "channels x60, W [8192,8192] int4 packed 2/byte"),
    "decode_seq": Workload("decode_seq", 256, 8192, 8192, 8, 40, "uniform", steps=64,
                           transient_steps=3,
                           description="outlier-locality decode: 64 steps of X [256,8192], "
                                       "40 persistent channels U(20,100)*sign, on 3 steps "
                                       "1-4 transient ones, W [8192,8192] int8"),
    "prefill_w8": Workload("prefill_w8", 2048, 8192, 8192, 8, 82, "uniform",
                          description="M=2048, K=N=8192, 1% (82) outlier channels "
                                      "U(20,100)*sign, W [8192,8192] N(0,0.02) int8"),
}


def _fp16(a: np.ndarray) -> np.ndarray:
    return a.astype(np.float16)


def _plant(rng: np.random.Generator, X: np.ndarray, ch: np.ndarray, wl: Workload) -> None:
    if ch.size == 0:
        return
    M = X.shape[0]
    if wl.outlier_kind == "uniform":
        mag = rng.uniform(wl.lo, wl.hi, size=(M, ch.size)).astype(np.float32)
        sign = np.where(rng.random((M, ch.size)) < 0.5, -1.0, 1.0).astype(np.float32)
        X[:, ch] = mag * sign
    elif wl.outlier_kind == "scale":
        X[:, ch] = X[:, ch] * np.float32(wl.factor)
    else:
        raise ValueError(wl.outlier_kind)


def make_weight(wl: Workload, seed: int | None = None, chunk_rows: int = 4096) -> np.ndarray:
    """W fp16 [N, K] ~ N(0, w_std), drawn in row chunks from its own stream."""
    s = wl.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence([s, 0x57]))
    W = np.empty((wl.N, wl.K), np.float16)
    for r0 in range(0, wl.N, chunk_rows):
        r1 = min(wl.N, r0 + chunk_rows)
        W[r0:r1] = _fp16(rng.standard_normal((r1 - r0, wl.K), dtype=np.float32)
                         * np.float32(wl.w_std))
    return W


def outlier_channels(wl: Workload, seed: int | None = None) -> np.ndarray:
    s = wl.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence([s, 0x4F]))
    return np.sort(rng.choice(wl.K, wl.n_outliers, replace=False)).astype(np.int64)


def make_activation(wl: Workload, seed: int | None = None, M: int | None = None) -> np.ndarray:
    """X fp16 [M, K]: N(0,1) with the workload's planted outlier channels."""
    s = wl.seed if seed is None else seed
    ch = outlier_channels(wl, s)
    rng = np.random.default_rng(np.random.SeedSequence([s, 0x58]))
    m = wl.M if M is None else M
    X = rng.standard_normal((m, wl.K), dtype=np.float32)
    _plant(rng, X, ch, wl)
    return _fp16(X)


def make_salient(N: int, fraction: float = 0.1, seed: int = 0) -> np.ndarray:
    """Salient output features for an output-feature mixed-precision weight:
    round(fraction * N) rows drawn without replacement (the MixLLM page keeps
    10% of them at 8 bits; its global ranking by estimated loss needs a
    trained model, so a seeded choice stands in for it).  bool [N]."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, N, 0x5A]))
    sal = np.zeros(N, bool)
    sal[rng.choice(N, int(round(fraction * N)), replace=False)] = True
    return sal


def make_norm_gamma(wl: Workload, seed: int | None = None) -> np.ndarray:
    """RMSNorm weight fp16 [K] for feeding the workload's X as the hidden state
    before the norm: g0 * (1 + 0.1 * N(0,1)), with g0 the expected root mean
    square of one such token, so that the normalised tokens keep the spread
    of X (unit scale, the planted channels above the threshold)."""
    s = wl.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence([s, 0x47]))
    if wl.outlier_kind == "uniform":
        second = (wl.hi ** 3 - wl.lo ** 3) / (3.0 * (wl.hi - wl.lo))  # E[U^2], U ~ U(lo, hi)
    else:
        second = wl.factor ** 2
    g0 = np.sqrt(1.0 + wl.n_outliers / wl.K * (second - 1.0))
    return _fp16(np.float32(g0) * (1.0 + 0.1 * rng.standard_normal(wl.K, dtype=np.float32)))


@dataclass(frozen=True)
class DecodePlan:
    persistent: np.ndarray       # sorted channel ids present on every step
    events: dict                 # step -> sorted array of transient channel ids


def decode_plan(wl: Workload, seed: int | None = None) -> DecodePlan:
    s = wl.seed if seed is None else seed
    pers = outlier_channels(wl, s)
    rng = np.random.default_rng(np.random.SeedSequence([s, 0x45]))
    steps = np.sort(rng.choice(wl.steps, wl.transient_steps, replace=False))
    rest = np.setdiff1d(np.arange(wl.K), pers)
    events = {}
    for st in steps:
        n_new = int(rng.integers(1, wl.transient_max + 1))
        events[int(st)] = np.sort(rng.choice(rest, n_new, replace=False)).astype(np.int64)
    return DecodePlan(persistent=pers, events=events)


def decode_step(wl: Workload, step: int, plan: DecodePlan | None = None,
                seed: int | None = None) -> np.ndarray:
    """X fp16 [M, K] of one decode step."""
    s = wl.seed if seed is None else seed
    plan = plan or decode_plan(wl, s)
    rng = np.random.default_rng(np.random.SeedSequence([s, 1 + step]))
    X = rng.standard_normal((wl.M, wl.K), dtype=np.float32)
    _plant(rng, X, plan.persistent, wl)
    if step in plan.events:
        _plant(rng, X, plan.events[step], wl)
    return _fp16(X)


def decode_sequence(wl: Workload, seed: int | None = None) -> Iterator[np.ndarray]:
    plan = decode_plan(wl, seed)
    for st in range(wl.steps):
        yield decode_step(wl, st, plan, seed)


def random_case(seed: int, M: int, K: int, N: int, n_out: int, scale: float = 30.0,
                w_std: float = 0.05) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Small random case for parity sweeps: returns (X, W, planted channel ids)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, M, K, N, n_out]))
    ch = np.sort(rng.choice(K, n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    X = rng.standard_normal((M, K), dtype=np.float32)
    if n_out:
        X[:, ch] = X[:, ch] * np.float32(scale)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    return _fp16(X), _fp16(W), ch
