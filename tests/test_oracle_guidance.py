"""Pins for the fp64 structure-guidance oracle (CPU only)."""
import numpy as np
import pytest
import scipy.ndimage as ndi

from oracle import guidance as G


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def test_taps():
    w = G.gaussian_taps(4.0)
    assert len(w) == 25
    assert w.sum() == pytest.approx(1.0, abs=1e-15)
    np.testing.assert_array_equal(w, w[::-1])
    assert np.argmax(w) == 12


def test_reflect101_by_hand():
    # ... c b | a b c d | c b a ...   for n = 4
    got = G.reflect101(np.arange(-5, 10), 4).tolist()
    assert got == [1, 2, 3, 2, 1, 0, 1, 2, 3, 2, 1, 0, 1, 2, 3]
    assert G.reflect101(np.arange(-3, 4), 1).tolist() == [0] * 7


@pytest.mark.parametrize("shape", [(4, 40, 37), (2, 13, 64), (1, 3, 25, 26)])
def test_lowpass_matches_scipy_mirror(shape):
    x = _rand(shape, 1)
    axes = (len(shape) - 2, len(shape) - 1)
    ref = ndi.gaussian_filter(x, sigma=4.0, mode="mirror", truncate=3.0, axes=axes)
    np.testing.assert_allclose(G.lowpass(x, 4.0), ref, rtol=0, atol=1e-13)


def test_lowpass_other_sigma_matches_scipy():
    x = _rand((3, 30, 31), 2)
    ref = ndi.gaussian_filter(x, sigma=1.5, mode="mirror", truncate=3.0, axes=(1, 2))
    # scipy's radius is int(3*1.5 + 0.5) = 5 = ceil(4.5)
    np.testing.assert_allclose(G.lowpass(x, 1.5), ref, rtol=0, atol=1e-13)


def test_constant_field_passes_unchanged():
    x = np.full((2, 17, 19), 3.25)
    np.testing.assert_allclose(G.lowpass(x, 4.0), x, rtol=0, atol=1e-13)


def test_blend_identities_and_linearity():
    x, ref = _rand((4, 20, 24), 3), _rand((4, 20, 24), 4)
    np.testing.assert_array_equal(G.sg_blend(x, ref, 0.0, 4.0), x)
    np.testing.assert_allclose(G.sg_blend(x, x, 0.7, 4.0), x, rtol=0, atol=1e-13)
    lp = ndi.gaussian_filter(ref - x, sigma=4.0, mode="mirror", truncate=3.0, axes=(1, 2))
    np.testing.assert_allclose(G.sg_blend(x, ref, 0.5, 4.0), x + 0.5 * lp, rtol=0, atol=1e-13)
    # channels are independent
    y = G.sg_blend(x[:1], ref[:1], 0.5, 4.0)
    np.testing.assert_array_equal(y, G.sg_blend(x, ref, 0.5, 4.0)[:1])


def test_asg_blend():
    eps, ref, m = _rand((2, 8, 8), 5), _rand((2, 8, 8), 6), np.random.default_rng(7).random((2, 8, 8))
    np.testing.assert_array_equal(G.asg_blend(eps, ref, np.zeros_like(m), 0.9), eps)
    np.testing.assert_allclose(G.asg_blend(eps, ref, np.ones_like(m), 1.0), ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(G.asg_blend(eps, ref, m, 0.3), (1 - 0.3 * m) * eps + 0.3 * m * ref, rtol=0, atol=1e-14)
