"""Host checks of the seeded input generator shared by the oracle and the HIP
path: its bf16 rounding agrees with torch's round-to-nearest-even conversion
bit for bit, and the draws are reproducible."""
import numpy as np
import torch

from partial_context_patch_amd import workloads as WL


def test_round_to_bf16_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    x = rng.standard_normal(200_000).astype(np.float32)
    x *= np.float32(10.0) ** rng.integers(-40, 38, x.size).astype(np.float32)
    ties = (np.arange(1, 20_000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, 1.1754942e-38],
                       np.float32)
    for a in (x, ties[np.isfinite(ties)], special):
        want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
        got = WL.round_to_bf16(a)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_round_to_bf16_keeps_nan_and_shape():
    a = np.array([[np.nan, 1.0], [2.5, -np.nan]], np.float32)
    r = WL.round_to_bf16(a)
    assert r.shape == a.shape and np.isnan(r[0, 0]) and np.isnan(r[1, 1]) and r[0, 1] == 1.0


def test_draws_are_reproducible():
    a = WL.attention_inputs(1, 2, 64, 4, 4, seed=3)
    b = WL.attention_inputs(1, 2, 64, 4, 4, seed=3)
    for n in a:
        assert np.array_equal(a[n], b[n])
