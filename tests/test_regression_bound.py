"""The GPU tests' regression bound is tight enough to catch a precision loss (CPU only).

The matrix-core kernels split each softmax weight p into bf16 hi + lo parts before the
weighted sum of V rows. This emulates that sum in numpy on N(0, 1) inputs at a few lengths,
with the weights kept to hi + lo and with the lo part dropped, and measures both in the GPU
tests' measure (normwise relative per head against the fp64 oracle): the kept split stays
under REGRESSION["bf16"], the dropped one is far above it, so a kernel that lost the lo half
would fail every bf16 and fp8 matrix-core test while still passing the 2e-3 contract.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_case import REGRESSION, TOL


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


@pytest.mark.parametrize("n", [8, 300, 4000])
def test_dropping_the_low_half_of_the_weights_breaks_the_bound(n):
    rng = np.random.default_rng(n)
    d = 128
    q = _bf16(rng.standard_normal(d))
    K = _bf16(rng.standard_normal((n, d)))
    V = _bf16(rng.standard_normal((n, d)))
    scale = float(np.float32(1 / np.sqrt(d)))
    ref = oracle.head_f64(q, K, V, scale)["out"]
    s = (K.astype(np.float32) @ q.astype(np.float32)) * np.float32(scale)
    p = np.exp(s - s.max()).astype(np.float32)
    hi = _bf16(p)
    lo = _bf16(p - hi)

    def rel(weights):
        out = (weights.astype(np.float64) @ V.astype(np.float64)) / p.astype(np.float64).sum()
        return np.abs(out - ref).max() / np.abs(ref).max(), np.abs(out - ref).max()

    kept, _ = rel(hi + lo)
    dropped, dropped_abs = rel(hi)
    assert kept < REGRESSION["bf16"] / 4
    assert dropped > 4 * REGRESSION["bf16"]
    if n <= 300:  # short sequences: the loss would also hide under the absolute contract
        assert dropped_abs < TOL["bf16"][1]
