"""fp64 reference for the structure-guidance blend.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"ScaleDiff ..." (atlas.scime.ai), "Approach": structure guidance acts on the
low-frequency content of the latent.  Written out here as

    out = x + w_t * (G_sigma * ref - G_sigma * x)

per channel, where G_sigma is a normalised 2-D Gaussian low-pass.  Readings
where the page is silent:

* the Gaussian is separable, taps at integer offsets |k| <= R = ceil(3*sigma),
  weights exp(-k^2 / (2 sigma^2)) normalised to sum 1;
* the border is reflect-101 (mirror about the edge sample, the edge itself not
  repeated): ... c b | a b c d | c b a ...;
* the latent is [C, H, W] (a leading batch dimension is allowed); w_t is a
  scalar supplied by the caller -- its schedule is not part of the blend.

The asynchronous-guidance blend of ASGDiffusion (the pith.science verdict page
on arXiv 2412.06163, sections "core_discovery" and "key_machinery") is the
element-wise form

    eps_corrected = eps + w_t * M * (eps_ref_prev - eps)

with a caller-supplied mask M.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def gaussian_taps(sigma: float, radius: Optional[int] = None) -> np.ndarray:
    if sigma <= 0:
        raise ValueError("sigma must be > 0")
    R = int(math.ceil(3.0 * sigma)) if radius is None else int(radius)
    offs = np.arange(-R, R + 1, dtype=np.float64)
    w = np.exp(-(offs**2) / (2.0 * sigma * sigma))
    return w / w.sum()


def reflect101(i: np.ndarray, n: int) -> np.ndarray:
    """Map any integer index onto [0, n) by mirroring about the edge samples."""
    i = np.asarray(i, dtype=np.int64)
    if n == 1:
        return np.zeros_like(i)
    period = 2 * (n - 1)
    i = np.mod(i, period)
    return np.where(i < n, i, period - i)


def _filter_axis(x: np.ndarray, taps: np.ndarray, axis: int) -> np.ndarray:
    n = x.shape[axis]
    R = (len(taps) - 1) // 2
    out = np.zeros_like(x)
    pos = np.arange(n)
    for t, wk in zip(range(-R, R + 1), taps):
        src = reflect101(pos + t, n)
        out += wk * np.take(x, src, axis=axis)
    return out


def lowpass(x, sigma: float, radius: Optional[int] = None) -> np.ndarray:
    """Separable Gaussian over the last two axes (rows then columns order-free)."""
    x = np.asarray(x, dtype=np.float64)
    taps = gaussian_taps(sigma, radius)
    return _filter_axis(_filter_axis(x, taps, x.ndim - 1), taps, x.ndim - 2)


def sg_blend(x, ref, w_t: float, sigma: float, radius: Optional[int] = None) -> np.ndarray:
    """x + w_t * (lowpass(ref) - lowpass(x)), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return x + w_t * (lowpass(ref, sigma, radius) - lowpass(x, sigma, radius))


def asg_blend(eps, eps_ref_prev, mask, w_t: float) -> np.ndarray:
    """eps + w_t * M * (eps_ref_prev - eps), element-wise in fp64."""
    eps = np.asarray(eps, dtype=np.float64)
    return eps + w_t * np.asarray(mask, dtype=np.float64) * (np.asarray(eps_ref_prev, dtype=np.float64) - eps)
