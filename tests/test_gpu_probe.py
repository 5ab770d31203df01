"""The matrix-core rate probe (mixq_mfma_probe) against a numpy evaluation of
what its header states it computes: every lane's sum of its 256 int32
accumulators after `iters` rounds of the 32 MFMAs on the stated operand
bytes, in 32-bit wrapping arithmetic.  The probe's figures are only worth
reporting if its MFMAs compute that product."""
import numpy as np
import pytest
import torch

from mixed_precision_quantized_amax_amd import mixq

pytestmark = pytest.mark.gpu


def probe_reference(a: np.ndarray, b: np.ndarray, iters: int, blocks: int) -> np.ndarray:
    """int32 [256 * blocks]: per lane, the sum of its accumulator values."""
    na, nb = a.size // 16 * 16, b.size // 16 * 16
    lanes = np.arange(64)
    # rows of the output fragment a lane holds: 8 (e / 4) + 4 (l / 32) + e % 4
    e = np.arange(16)
    rows = (8 * (e[None, :] // 4) + 4 * (lanes[:, None] // 32) + e[None, :] % 4)   # [64, 16]
    out = np.zeros(256 * blocks, np.int64)
    for g in range(4 * blocks):
        def operand(src, n, q):
            offs = ((8 * g + q) * 1024 + 16 * lanes) % n                          # [64]
            lane_bytes = src[offs[:, None] + np.arange(16)[None, :]].astype(np.int64)  # [64, 16]
            return np.concatenate([lane_bytes[:32], lane_bytes[32:]], axis=1)     # [32 rows, 32 k]
        acc = np.zeros((4, 4, 32, 32), np.int64)
        for ks in range(2):
            A = [operand(a, na, 4 * ks + i) for i in range(4)]
            B = [operand(b, nb, 4 * ks + j) for j in range(4)]
            for i in range(4):
                for j in range(4):
                    acc[i, j] += A[i] @ B[j].T
        acc *= iters
        tot = acc.sum(axis=(0, 1))                                                # [32 rows, 32 cols]
        for l in range(64):
            out[64 * g + l] = tot[rows[l], l % 32].sum()
    return ((out + 2**31) % 2**32 - 2**31).astype(np.int32)


@pytest.mark.parametrize("iters,blocks,na,nb", [(1, 1, 4096, 8192), (3, 2, 65536, 48),
                                                 (2, 3, 1040, 100000)])
def test_probe_computes_the_stated_product(iters, blocks, na, nb):
    rng = np.random.default_rng(np.random.SeedSequence([7, iters, blocks]))
    a = rng.integers(-128, 128, na, dtype=np.int8)
    b = rng.integers(-128, 128, nb, dtype=np.int8)
    dev = torch.device("cuda", 0)
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    out = torch.zeros(256 * blocks, dtype=torch.int32, device=dev)
    clk = torch.zeros(4 * blocks, dtype=torch.int64, device=dev)
    mixq.mfma_probe(ta, tb, iters, blocks, out, clk)
    torch.cuda.synchronize()
    ref = probe_reference(a, b, iters, blocks)
    assert np.array_equal(out.cpu().numpy(), ref)
    c = clk.cpu().numpy().reshape(blocks, 4)
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] >= c[:, 2]).all()
