"""Seeded synthetic workloads shaped like the pages' diffusion attention layers.

This module is the only code that both the HIP path's tests/benchmark and the
CPU oracle consume.  It draws random tensors and rounds them to the storage
dtype; it holds none of the attention method's arithmetic (no halo sizes, no
membership, no softmax).

Value recipe (all seeded with numpy's PCG64):
* Q, K, V ~ N(0, 1), drawn in fp32 in that order;
* stale K/V (strip workloads only) = fresh + N(0, 0.05^2) noise, drawn next;
* FLUX-shaped workload: Q and K RMS-normalised per (token, head) over the
  head dimension, q / sqrt(mean(q^2) + 1e-6), with no learned weight;
* bf16 workloads: every tensor rounded to bf16 (round-to-nearest-even) on the
  host; the oracle receives exactly those values, upcast to fp64.
Layout: [batch, tokens, heads, head_dim] (BNHD), tokens row-major over the
map (t = r*W + c), head_dim contiguous.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

# Attention workloads.  Shapes follow the SDXL / FLUX layers the pages run
# (PCPP: SDXL on 4-8 devices with p = 0.3 / 0.8; ScaleDiff: SDXL and FLUX at
# 4096^2 with neighbourhood patch attention).
ATTENTION_WORKLOADS: Dict[str, dict] = {
    "pcpp_tiny_fp32": dict(
        mode="strips", batch=1, heads=2, head_dim=64, map_h=32, map_w=32,
        num_strips=4, p=0.3, dtype="f32", seed=1001,
        what="tiny PCPP strips, fp32: 32x32 tokens, 4 strips of 8 rows, p=0.3",
    ),
    "sdxl1024_strips": dict(
        mode="strips", batch=2, heads=10, head_dim=64, map_h=64, map_w=64,
        num_strips=4, p=0.3, dtype="bf16", seed=1002,
        what="SDXL 1024^2 mid-level self-attention: 64x64 tokens, 10x64 heads, 4 strips, p=0.3",
    ),
    "sdxl2048_strips": dict(
        mode="strips", batch=2, heads=10, head_dim=64, map_h=128, map_w=128,
        num_strips=8, p=0.8, dtype="bf16", seed=1003,
        what="SDXL 2048^2 mid-level self-attention: 128x128 tokens, 10x64 heads, 8 strips, p=0.8",
    ),
    "sdxl4096_npa": dict(
        mode="window", batch=2, heads=10, head_dim=64, map_h=256, map_w=256,
        tile_h=64, tile_w=64, halo_h=16, halo_w=16, dtype="bf16", seed=1004,
        what="SDXL 4096^2 first attention level, NPA: 256x256 tokens, 10x64 heads, 64x64 query tiles, 96x96 windows",
    ),
    # Halo settings at their limits (DistriFusion's full stale context, the
    # synchronous warm-up steps with full fresh attention): parity cases.
    "sdxl2048_fullstale": dict(
        mode="strips", batch=2, heads=10, head_dim=64, map_h=128, map_w=128,
        num_strips=8, p=None, halo_rows=128, dtype="bf16", seed=1007,
        what="SDXL 2048^2, 8 strips, full stale context: own strip fresh, every other row stale",
    ),
    "sdxl1024_warmup": dict(
        mode="strips", batch=2, heads=10, head_dim=64, map_h=64, map_w=64,
        num_strips=1, p=0.0, dtype="bf16", seed=1008,
        what="SDXL 1024^2 warm-up step: one strip, full fresh attention",
    ),
    "flux4096_npa": dict(
        mode="window", batch=1, heads=24, head_dim=128, map_h=256, map_w=256,
        tile_h=32, tile_w=32, halo_h=16, halo_w=16, dtype="bf16", seed=1005,
        rms_qk=True,
        what="FLUX 4096^2 DiT, NPA: 256x256 packed tokens, 24x128 heads, 32x32 query tiles, 64x64 windows",
    ),
    # Strips at head_dim 128 (a DiT run with PCPP): parity case.
    "flux2048_strips": dict(
        mode="strips", batch=1, heads=24, head_dim=128, map_h=64, map_w=64,
        num_strips=4, p=0.3, dtype="bf16", seed=1010, rms_qk=True,
        what="FLUX-shaped 2048^2 (64x64 packed tokens), 24x128 heads, 4 strips, p=0.3",
    ),
    # FLUX's joint attention with the prompt's text tokens stored before the
    # map's tokens (global: map queries also see every text token, text queries
    # see everything).
    "flux4096_joint": dict(
        mode="window", batch=1, heads=24, head_dim=128, map_h=256, map_w=256,
        tile_h=32, tile_w=32, halo_h=16, halo_w=16, text_tokens=512, dtype="bf16", seed=1009,
        rms_qk=True,
        what="FLUX 4096^2 joint attention: 512 text + 256x256 packed tokens, 24x128 heads, 32x32 query tiles, 64x64 windows",
    ),
}

# Structure-guidance blend on the SDXL 4096^2 latent (4 channels, 512x512).
SG_WORKLOAD = dict(channels=4, map_h=512, map_w=512, w_t=0.5, sigma=4.0, seed=1006,
                   what="structure-guidance blend: 4x512x512 fp32 latent, sigma=4, w_t=0.5")

STALE_NOISE_STD = 0.05


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32.

    On the bit pattern u: add 0x7FFF plus the lowest kept bit, clear the low
    16 bits.  For every finite or infinite value u + 0x8000 stays below 2^32,
    so 32-bit arithmetic is exact; NaNs are passed through unchanged."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = a[nan]
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of fp32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def attention_inputs(
    batch: int,
    heads: int,
    head_dim: int,
    map_h: int,
    map_w: int,
    *,
    seed: int,
    dtype: str = "bf16",
    stale: bool = True,
    rms_qk: bool = False,
    text_tokens: int = 0,
    **_ignored,
) -> Dict[str, Optional[np.ndarray]]:
    """Draw q, k, v (and k_stale, v_stale) as fp32 arrays of the storage values;
    with text tokens the sequence holds them first, then the map's tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (batch, text_tokens + map_h * map_w, heads, head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    k_stale = v_stale = None
    if stale:
        k_stale = k + np.float32(STALE_NOISE_STD) * rng.standard_normal(shape, dtype=np.float32)
        v_stale = v + np.float32(STALE_NOISE_STD) * rng.standard_normal(shape, dtype=np.float32)
    if rms_qk:
        for a in (q, k):
            a /= np.sqrt(np.mean(a.astype(np.float64) ** 2, axis=-1, keepdims=True) + 1e-6).astype(np.float32)
    out = dict(q=q, k=k, v=v, k_stale=k_stale, v_stale=v_stale)
    if dtype == "bf16":
        out = {n: (None if a is None else round_to_bf16(a)) for n, a in out.items()}
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    return out


def halo_kwargs(w: dict) -> dict:
    """The workload's strip or window settings as keyword arguments of
    npa.attn_fwd / npa.make_halo."""
    if w["mode"] == "strips":
        return dict(strips=w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
    return dict(tile=(w["tile_h"], w["tile_w"]), halo=(w["halo_h"], w["halo_w"]), text_tokens=w.get("text_tokens", 0))


def workload_inputs(name: str) -> Dict[str, Optional[np.ndarray]]:
    w = ATTENTION_WORKLOADS[name]
    return attention_inputs(**w, stale=(w["mode"] == "strips"))


def sg_inputs(channels: int, map_h: int, map_w: int, *, seed: int, batch: int = 1, **_ignored):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((batch, channels, map_h, map_w), dtype=np.float32)
    ref = rng.standard_normal((batch, channels, map_h, map_w), dtype=np.float32)
    return x, ref


def asg_inputs(shape, *, seed: int):
    """eps, eps_ref_prev ~ N(0,1); mask ~ U[0,1) (a normalised attention mask stand-in)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    eps = rng.standard_normal(shape, dtype=np.float32)
    ref = rng.standard_normal(shape, dtype=np.float32)
    mask = rng.random(shape, dtype=np.float32)
    return eps, ref, mask
