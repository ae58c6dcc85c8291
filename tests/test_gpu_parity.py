"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

* small ragged maps, every output compared (bf16 atol 2e-2, fp32 atol 1e-4);
* the attention workloads at full size, in the launch configuration the
  benchmark times: the whole output of two (batch, head) slices and one
  interior tile of every slice, which the oracle computes exactly;
* structural probes: Q = 0 set means, one-hot V exposing probability rows,
  NaN poisoning of everything the plan must not read;
* the structure-guidance and asynchronous-guidance blends.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import guidance as G
from partial_context_patch_amd import npa
from partial_context_patch_amd import workloads as WL

pytestmark = pytest.mark.gpu

ATOL = {"bf16": 2e-2, "f32": 1e-4}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _dev(a, dt):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(TDT[dt])


def _kw(spec):
    if isinstance(spec, A.Strips):
        return dict(strips=spec.num_strips, p=spec.p, halo_rows=spec.halo_rows)
    return dict(tile=(spec.tile_h, spec.tile_w), halo=(spec.halo_h, spec.halo_w), text_tokens=spec.text_tokens)


def _run(inp, H, W, spec, dt, scale=None):
    q, k, v = (_dev(inp[n], dt) for n in ("q", "k", "v"))
    ks, vs = _dev(inp.get("k_stale"), dt), _dev(inp.get("v_stale"), dt)
    out = npa.attn_fwd(q, k, v, ks, vs, map_hw=(H, W), scale=scale, **_kw(spec))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


SMALL = [
    # (H, W, B, Hh, d, spec, dtype)
    (24, 20, 1, 2, 64, A.Strips(3, halo_rows=3), "bf16"),
    (24, 20, 2, 3, 64, A.Strips(3, p=0.3), "bf16"),
    (30, 13, 1, 2, 64, A.Strips(5, halo_rows=9), "bf16"),
    (16, 24, 1, 2, 64, A.Strips(1, p=0.5), "bf16"),
    (16, 24, 1, 2, 128, A.Strips(4, p=0.5), "bf16"),
    (40, 36, 1, 2, 64, A.Windows(8, 12, 5, 3), "bf16"),
    (40, 36, 2, 2, 128, A.Windows(20, 12, 4, 7), "bf16"),
    (24, 24, 1, 1, 64, A.Windows(24, 24, 0, 0), "bf16"),
    (12, 10, 1, 2, 64, A.Windows(1, 2, 1, 3), "bf16"),
    (24, 20, 1, 2, 64, A.Strips(3, halo_rows=3), "f32"),
    (24, 20, 1, 2, 32, A.Strips(4, halo_rows=2), "f32"),
    (40, 36, 1, 2, 128, A.Windows(8, 12, 5, 3), "f32"),
    # joint attention: text tokens stored before the map (ragged counts, a whole-map window)
    (16, 16, 1, 2, 64, A.Windows(4, 4, 2, 2, 7), "bf16"),
    (16, 12, 1, 2, 128, A.Windows(8, 4, 3, 2, 64), "bf16"),
    (8, 8, 2, 2, 64, A.Windows(8, 8, 0, 0, 40), "bf16"),
    (32, 32, 1, 1, 128, A.Windows(16, 16, 8, 8, 200), "bf16"),
    (12, 8, 1, 2, 64, A.Windows(4, 4, 1, 1, 5), "f32"),
    (24, 16, 1, 2, 128, A.Windows(8, 8, 4, 4, 100), "f32"),
]


@pytest.mark.parametrize("H,W,B,Hh,d,spec,dt", SMALL)
def test_small_ragged_full_compare(H, W, B, Hh, d, spec, dt):
    stale = isinstance(spec, A.Strips)
    inp = WL.attention_inputs(B, Hh, d, H, W, seed=7 + H + W + d, dtype=dt, stale=stale,
                              text_tokens=A.text_tokens(spec))
    got = _run(inp, H, W, spec, dt)
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec)
    err = np.abs(got - ref).max()
    assert np.isfinite(got).all()
    assert err <= ATOL[dt], f"max abs err {err}"


def test_explicit_scale_and_halo_beyond_map():
    H, W = 16, 16
    inp = WL.attention_inputs(1, 2, 64, H, W, seed=5, dtype="bf16")
    spec = A.Strips(4, halo_rows=40)  # every other strip entirely stale
    got = _run(inp, H, W, spec, "bf16", scale=0.2)
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec, scale=0.2)
    assert np.abs(got - ref).max() <= 2e-2


# ------------------------------------------------------------- full sizes
def _workload_spec(w):
    if w["mode"] == "strips":
        return A.Strips(w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
    return A.Windows(w["tile_h"], w["tile_w"], w["halo_h"], w["halo_w"], w.get("text_tokens", 0))


def _interior_tile(w, spec):
    """Query tokens of an interior map tile (windows) or a middle strip."""
    tiles = list(A.iter_tiles(w["map_h"], w["map_w"], spec))
    if isinstance(spec, A.Strips):
        return tiles[spec.num_strips // 2][0]
    tx, ty = w["map_w"] // spec.tile_w, w["map_h"] // spec.tile_h
    return tiles[(ty // 2) * tx + tx // 2][0]


@pytest.mark.parametrize("name", list(WL.ATTENTION_WORKLOADS))
def test_workload_full_size(name):
    """The whole output of the first and the last (batch, head) slice (every
    tile, and the text tile with text tokens), and one interior tile of every
    slice (every workgroup-to-(batch, head) mapping), against the oracle."""
    w = WL.ATTENTION_WORKLOADS[name]
    print(f"[parity] workload {name}: {w['what']}", flush=True)
    inp = WL.workload_inputs(name)
    spec = _workload_spec(w)
    got = _run(inp, w["map_h"], w["map_w"], spec, w["dtype"])
    assert np.isfinite(got).all()
    heads = [(0, 0), (w["batch"] - 1, w["heads"] - 1)]
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], w["map_h"], w["map_w"],
                            spec, heads=heads)
    for b, j in heads:
        err = np.abs(got[b, :, j] - ref[b, :, j]).max()
        assert err <= ATOL[w["dtype"]], f"{name} (b={b}, head={j}): max abs err {err}"
    qt = _interior_tile(w, spec)
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], w["map_h"], w["map_w"],
                            spec, query_tokens=qt)
    err = np.abs(got[:, qt] - ref[:, qt]).max()
    assert err <= ATOL[w["dtype"]], f"{name}, one tile of every (batch, head): max abs err {err}"


@pytest.mark.parametrize("name", ["sdxl2048_strips", "flux4096_npa", "sdxl1024_strips", "pcpp_tiny_fp32"])
def test_repeated_calls_are_bitwise_identical(name):
    """The kernels use no atomics and no order-dependent reduction across
    workgroups, so the same call gives the same bits every time; a race on the
    double-buffered K/V tiles or on the copy cursor would show up here as
    run-to-run differences.  Five back-to-back calls at full size, with other
    work (a different call) interleaved between them."""
    w = WL.ATTENTION_WORKLOADS[name]
    print(f"[parity] repeatability {name}", flush=True)
    inp = WL.workload_inputs(name)
    dt = TDT[w["dtype"]]
    t = {n: (None if a is None else _dev(a, w["dtype"])) for n, a in inp.items()}
    kw = WL.halo_kwargs(w)
    hw = (w["map_h"], w["map_w"])
    first = npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], map_hw=hw, **kw)
    other = torch.empty_like(first)
    for rep in range(4):
        # a different call in between: the swapped roles of q and k
        npa.attn_fwd(t["k"], t["q"], t["v"], t["k_stale"], t["v_stale"], map_hw=hw, out=other, **kw)
        again = torch.full_like(first, float("nan"))
        npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], map_hw=hw, out=again, **kw)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           first.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), f"{name}: repeat {rep}"


def test_concurrent_calls_on_two_streams():
    """The library keeps no device state between calls: a strip layer, a
    d = 128 window layer and the blend issued on two streams at once (default
    priority) give the same bits as each call made alone."""
    print("[parity] two streams", flush=True)
    names = ["sdxl2048_strips", "flux2048_strips"]
    ts, kws, alone = [], [], []
    for name in names:
        w = WL.ATTENTION_WORKLOADS[name]
        t = {n: (None if a is None else _dev(a, w["dtype"])) for n, a in WL.workload_inputs(name).items()}
        kw = dict(WL.halo_kwargs(w), map_hw=(w["map_h"], w["map_w"]))
        ts.append(t)
        kws.append(kw)
        alone.append(npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], **kw))
    x, r = (torch.from_numpy(a).cuda() for a in WL.sg_inputs(4, 512, 512, seed=3))
    sg_alone = npa.sg_blend(x, r, 0.5, 4.0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                t = ts[i]
                outs.append((i, npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], **kws[i])))
                if i == rep % 2:
                    outs.append((2, npa.sg_blend(x, r, 0.5, 4.0)))
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for i, got in outs:
        want = sg_alone if i == 2 else alone[i]
        view = torch.int32 if want.dtype == torch.float32 else torch.int16
        assert torch.equal(got.view(view), want.view(view)), f"call {i} differs on a shared GPU"


# ----------------------------------------------------------- structural
@pytest.mark.parametrize("spec", [A.Strips(2, halo_rows=1), A.Strips(4, halo_rows=2), A.Strips(4, halo_rows=0),
                                  A.Windows(2, 2, 1, 1), A.Windows(1, 4, 2, 0)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_one_hot_values_expose_probability_rows(spec, dt):
    """4x4 map, d = 64: V_fresh = [I16|0|0], V_stale = [0|I16|0], so out[:, :32]
    is the probability row over the 32 candidate keys."""
    H = W = 4
    N = 16
    rng = np.random.Generator(np.random.PCG64(3))
    q = rng.standard_normal((1, N, 1, 64), dtype=np.float32)
    k = rng.standard_normal((1, N, 1, 64), dtype=np.float32)
    ks = rng.standard_normal((1, N, 1, 64), dtype=np.float32)
    if dt == "bf16":
        q, k, ks = (WL.round_to_bf16(a) for a in (q, k, ks))
    vf = np.zeros((1, N, 1, 64), np.float32)
    vs = np.zeros((1, N, 1, 64), np.float32)
    vf[0, :, 0, :N] = np.eye(N)
    vs[0, :, 0, N:2 * N] = np.eye(N)
    got = _run(dict(q=q, k=k, v=vf, k_stale=ks, v_stale=vs), H, W, spec, dt)[0, :, 0, :]
    P = got[:, :2 * N]
    ref = A.attention_tier1(q, k, vf, ks, vs, H, W, spec)[0, :, 0, :2 * N]
    sets = A.attended_sets(H, W, spec)
    for t in range(N):
        allowed = np.zeros(2 * N, dtype=bool)
        allowed[sets[t][0]] = True
        allowed[[N + u for u in sets[t][1]]] = True
        assert np.all(P[t, ~allowed] == 0.0), f"query {t} weighs keys outside its set"
        assert np.all(P[t, allowed] > 0.0), f"query {t} misses keys of its set"
    assert np.abs(got[:, 2 * N:]).max() == 0.0
    tol = 1e-2 if dt == "bf16" else 1e-5
    np.testing.assert_allclose(P.sum(1), 1.0, atol=tol)
    np.testing.assert_allclose(P, ref, atol=tol)


@pytest.mark.parametrize(
    "H,W,spec",
    [(16, 16, A.Strips(4, halo_rows=3)), (32, 8, A.Strips(8, halo_rows=5)), (16, 16, A.Strips(2, halo_rows=16)),
     (16, 16, A.Windows(4, 8, 3, 2)), (24, 24, A.Windows(8, 8, 5, 5))],
)
def test_zero_query_set_means(H, W, spec):
    """Q = 0 gives uniform weights: out = mean of V over the attended set, with
    V = (1, is_stale, row/H, col/W): set size ratio and mean row/col in closed form."""
    N = H * W
    rows, cols = np.arange(N) // W, np.arange(N) % W
    d = 64
    q = np.zeros((1, N, 1, d), np.float32)
    k = np.random.Generator(np.random.PCG64(4)).standard_normal((1, N, 1, d), dtype=np.float32)
    k = WL.round_to_bf16(k)
    vf = np.zeros((1, N, 1, d), np.float32)
    vs = np.zeros((1, N, 1, d), np.float32)
    vf[0, :, 0, 0] = 1.0
    vs[0, :, 0, 0] = 1.0
    vs[0, :, 0, 1] = 1.0
    for v in (vf, vs):
        v[0, :, 0, 2] = rows / 64.0  # exact in bf16
        v[0, :, 0, 3] = cols / 64.0
    got = _run(dict(q=q, k=k, v=vf, k_stale=k, v_stale=vs), H, W, spec, "bf16")[0, :, 0]
    sets = A.attended_sets(H, W, spec)
    for t in range(N):
        fr, st = sets[t]
        n = len(fr) + len(st)
        assert got[t, 0] == pytest.approx(1.0, abs=8e-3)
        assert got[t, 1] == pytest.approx(len(st) / n, abs=8e-3)
        assert got[t, 2] == pytest.approx((rows[fr].sum() + rows[st].sum()) / n / 64.0, abs=4e-3)
        assert got[t, 3] == pytest.approx((cols[fr].sum() + cols[st].sum()) / n / 64.0, abs=4e-3)


@pytest.mark.parametrize(
    "H,W,spec,d",
    [(32, 32, A.Strips(4, halo_rows=3), 64), (48, 16, A.Strips(3, halo_rows=5), 128),
     (40, 36, A.Windows(8, 12, 5, 3), 64), (32, 32, A.Windows(16, 16, 4, 4), 128)],
)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_nan_poisoned_unread_regions(H, W, spec, d, dt):
    """Fill everything the definition never reads with NaN; the result must be
    finite and equal to the clean run.  Stale copies of a strip's own rows and
    stale rows beyond the halo are poisoned; for one tile, every fresh key
    outside its set is poisoned and only that tile's outputs are checked."""
    inp = WL.attention_inputs(1, 2, d, H, W, seed=11, dtype=dt, stale=True)
    clean = _run(inp, H, W, spec, dt)
    tiles = list(A.iter_tiles(H, W, spec))
    used_stale = np.zeros(H * W, dtype=bool)
    for _, _, st in tiles:
        used_stale[st] = True
    pois = dict(inp)
    for n in ("k_stale", "v_stale"):
        a = pois[n].copy()
        a[:, ~used_stale] = np.nan
        pois[n] = a
    qt, ft, st = tiles[len(tiles) // 2]
    keep = np.zeros(H * W, dtype=bool)
    keep[ft] = True
    for n in ("k", "v"):
        a = pois[n].copy()
        a[:, ~keep & ~np.isin(np.arange(H * W), qt)] = np.nan
        pois[n] = a
    for n in ("k_stale", "v_stale"):
        a = pois[n].copy()
        other = np.ones(H * W, dtype=bool)
        other[st] = False
        a[:, other] = np.nan
        pois[n] = a
    got = _run(pois, H, W, spec, dt)
    assert np.isfinite(got[:, qt]).all()
    np.testing.assert_array_equal(got[:, qt], clean[:, qt])


# ------------------------------------------------------------- guidance
@pytest.mark.parametrize(
    "shape,sigma,w",
    [((1, 4, 512, 512), 4.0, 0.5), ((2, 3, 37, 70), 4.0, 0.8), ((1, 1, 5, 9), 4.0, 1.0),
     ((1, 2, 64, 33), 1.5, -0.3), ((1, 1, 100, 130), 8.0, 0.5)],
)
def test_sg_blend(shape, sigma, w):
    seed = sum(shape)
    x, ref = WL.sg_inputs(shape[1], shape[2], shape[3], seed=seed, batch=shape[0])
    out = npa.sg_blend(torch.from_numpy(x).cuda(), torch.from_numpy(ref).cuda(), w, sigma)
    torch.cuda.synchronize()
    exp = G.sg_blend(x, ref, w, sigma)
    err = np.abs(out.cpu().numpy().astype(np.float64) - exp).max()
    assert err <= 1e-5, f"max abs err {err}"


@pytest.mark.parametrize(
    "shape,sigma,w",
    [((1, 2, 37, 68), 4.0, 0.5),      # partial tiles on both axes
     ((1, 1, 100, 128), 1.5, 0.7),    # R = 5: staged radius 8, taps shifted by 3
     ((1, 3, 130, 132), 5.25, 0.5),   # R = 16, the largest matrix-core radius
     ((2, 1, 64, 64), 0.3, 1.0),      # R = 1
     ((1, 1, 17, 20), 4.0, -0.4),     # a 17 x 20 image inside one tile
     ((1, 2, 13, 16), 4.0, 0.5),      # H = R + 1, W = R + 4: the tightest one-reflection borders
     ((1, 1, 72, 96), 2.5, 0.3),      # R = 8: no tap shift
     ((2, 2, 40, 44), 0.5, 0.9)],     # R = 2: taps shifted by 2
)
def test_sg_blend_matrix_core_shapes(shape, sigma, w):
    """Shapes the matrix-core blend takes (W a multiple of 4, R <= 16): tile
    edges, shifted taps, one-tile images, against the fp64 oracle."""
    seed = sum(shape) + 11
    x, ref = WL.sg_inputs(shape[1], shape[2], shape[3], seed=seed, batch=shape[0])
    out = npa.sg_blend(torch.from_numpy(x).cuda(), torch.from_numpy(ref).cuda(), w, sigma)
    torch.cuda.synchronize()
    exp = G.sg_blend(x, ref, w, sigma)
    err = np.abs(out.cpu().numpy().astype(np.float64) - exp).max()
    assert err <= 1e-5, f"max abs err {err}"


@pytest.mark.parametrize("scale", [2.0**-60, 2.0**-20, 2.0**20, 2.0**60])
def test_sg_blend_magnitudes(scale):
    """The matrix-core blend scales each tile by a power of two before its f16
    split: inputs far from unit size keep fp32-like relative accuracy, and one
    plane 2^40 smaller than its neighbour plane is not swamped by it."""
    x, ref = (a[0] for a in WL.sg_inputs(2, 128, 128, seed=5))
    x = (x * scale).astype(np.float32)
    ref = (ref * scale).astype(np.float32)
    x[1] *= np.float32(2.0**-40)
    ref[1] *= np.float32(2.0**-40)
    out = npa.sg_blend(torch.from_numpy(x[None]).cuda(), torch.from_numpy(ref[None]).cuda(), 0.5, 4.0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0].astype(np.float64)
    exp = G.sg_blend(x, ref, 0.5, 4.0)
    for c in range(2):
        mag = np.abs(exp[c]).max()
        err = np.abs(got[c] - exp[c]).max()
        assert err <= 1e-5 * mag, f"plane {c}: rel err {err / mag}"


def test_sg_blend_non_finite_inputs():
    """A tile holding inf or NaN takes the fp32 path: infinities and NaNs reach
    exactly the outputs whose windows hold them, as in the fp64 oracle, and
    every other output stays within the tolerance."""
    x, ref = (a[0] for a in WL.sg_inputs(3, 192, 256, seed=9))
    ref[0, 70, 100] = np.inf          # one +inf
    x[1, 5, 250] = np.nan             # a NaN at the right border
    ref[2, 150, 3] = np.inf           # inf - inf in the difference
    x[2, 150, 3] = np.inf
    out = npa.sg_blend(torch.from_numpy(x[None]).cuda(), torch.from_numpy(ref[None]).cuda(), 0.5, 4.0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0].astype(np.float64)
    with np.errstate(invalid="ignore"):  # inf - inf in the oracle is the point
        exp = G.sg_blend(x, ref, 0.5, 4.0)
    assert np.array_equal(np.isnan(got), np.isnan(exp))
    assert np.array_equal(np.isposinf(got), np.isposinf(exp))
    assert np.array_equal(np.isneginf(got), np.isneginf(exp))
    fin = np.isfinite(exp)
    assert fin.sum() > 0.9 * fin.size
    assert np.abs(got[fin] - exp[fin]).max() <= 1e-5


def test_sg_blend_workload_is_lfm_at_w1():
    w = WL.SG_WORKLOAD
    x, ref = WL.sg_inputs(w["channels"], w["map_h"], w["map_w"], seed=w["seed"])
    out = npa.sg_blend(torch.from_numpy(x).cuda(), torch.from_numpy(ref).cuda(), 1.0, w["sigma"])
    torch.cuda.synchronize()
    # latent frequency mixing: low frequencies of ref plus high frequencies of x
    lfm = G.lowpass(ref, w["sigma"]) + (x - G.lowpass(x, w["sigma"]))
    assert np.abs(out.cpu().numpy() - lfm).max() <= 1e-5


@pytest.mark.parametrize("count", [1, 3, 4, 1000, 1 << 20, (1 << 20) + 3])
def test_asg_blend(count):
    eps, ref, mask = WL.asg_inputs((count,), seed=count)
    out = npa.asg_blend(*(torch.from_numpy(a).cuda() for a in (eps, ref, mask)), 0.7)
    torch.cuda.synchronize()
    exp = G.asg_blend(eps, ref, mask, 0.7)
    assert np.abs(out.cpu().numpy() - exp).max() <= 1e-6


@pytest.mark.parametrize("target", ["eps", "eps_ref_prev", "mask"])
def test_asg_blend_in_place(target):
    """out may be any one of the inputs (the sampler updates eps in place): the
    result equals the out-of-place call's, bit for bit."""
    eps, ref, mask = WL.asg_inputs(((1 << 20) + 3,), seed=21)
    dev = {n: torch.from_numpy(a).cuda() for n, a in (("eps", eps), ("eps_ref_prev", ref), ("mask", mask))}
    want = npa.asg_blend(dev["eps"], dev["eps_ref_prev"], dev["mask"], 0.7)
    got = npa.asg_blend(dev["eps"], dev["eps_ref_prev"], dev["mask"], 0.7, out=dev[target])
    torch.cuda.synchronize()
    assert got.data_ptr() == dev[target].data_ptr()
    assert torch.equal(got, want)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("spec,H,W,d", [(A.Windows(8, 8, 4, 4), 16, 16, 64), (A.Strips(2, halo_rows=3), 16, 16, 64),
                                        (A.Windows(8, 8, 4, 4), 16, 16, 128)])
def test_late_large_logits_take_the_robust_pass(spec, H, W, d, dt):
    """Keys far beyond the first 32 of a tile score ~100+ log2 units above them:
    the bf16 kernel's fixed-shift pass overflows and the workgroup must redo
    the tile with the tile's true row max; the fp32 kernel's per-block max and
    rescale must carry the same range.  Also rows whose logits are all hugely
    negative."""
    N = H * W
    rng = np.random.Generator(np.random.PCG64(21))
    q = 0.05 * rng.standard_normal((1, N, 2, d), dtype=np.float32)
    k = 0.05 * rng.standard_normal((1, N, 2, d), dtype=np.float32)
    v = rng.standard_normal((1, N, 2, d), dtype=np.float32)
    q[0, :, 0, 0] = 24.0           # head 0: a few late keys align with every query
    k[0, N - 5:, 0, 0] = 24.0
    q[0, :, 1, 0] = -40.0          # head 1: every logit very negative, spread by k
    k[0, :, 1, 0] = rng.uniform(20.0, 40.0, N).astype(np.float32)
    if dt == "bf16":
        q, k, v = (WL.round_to_bf16(a) for a in (q, k, v))
    inp = dict(q=q, k=k, v=v, k_stale=k.copy(), v_stale=v.copy())
    got = _run(inp, H, W, spec, dt)
    ref = A.attention_tier1(q, k, v, inp["k_stale"], inp["v_stale"], H, W, spec)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= ATOL[dt]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("spec", [A.Windows(2, 2, 1, 1, 3), A.Windows(4, 2, 0, 1, 9)])
def test_joint_one_hot_values_expose_probability_rows(spec, dt):
    """4x4 map after T text tokens, d = 64: V = one-hot over the T + 16 stored
    tokens, so out[:, :T+16] is each query's probability row; it must be zero
    off the query's key set (text + window for map queries, all for text)."""
    H = W = 4
    T = A.text_tokens(spec)
    N = T + H * W
    rng = np.random.Generator(np.random.PCG64(5))
    q = rng.standard_normal((1, N, 1, 64), dtype=np.float32)
    k = rng.standard_normal((1, N, 1, 64), dtype=np.float32)
    if dt == "bf16":
        q, k = WL.round_to_bf16(q), WL.round_to_bf16(k)
    v = np.zeros((1, N, 1, 64), np.float32)
    v[0, :, 0, :N] = np.eye(N)
    got = _run(dict(q=q, k=k, v=v), H, W, spec, dt)[0, :, 0, :]
    P = got[:, :N]
    ref = A.attention_tier1(q, k, v, None, None, H, W, spec)[0, :, 0, :N]
    sets = A.attended_sets(H, W, spec)
    for t in range(N):
        allowed = np.zeros(N, dtype=bool)
        allowed[sets[t][0]] = True
        assert np.all(P[t, ~allowed] == 0.0), f"query {t} weighs keys outside its set"
        assert np.all(P[t, allowed] > 0.0), f"query {t} misses keys of its set"
    tol = 1e-2 if dt == "bf16" else 1e-5
    np.testing.assert_allclose(P.sum(1), 1.0, atol=tol)
    np.testing.assert_allclose(P, ref, atol=tol)


@pytest.mark.parametrize("d", [64, 128])
def test_joint_text_logits_take_the_robust_pass(d):
    """Text keys (read after each map tile's window) score ~100 log2 units above
    the window's first keys: the fixed-shift pass overflows and the tile is redone
    with its true row max."""
    H = W = 16
    T = 40
    N = T + H * W
    spec = A.Windows(8, 8, 4, 4, T)
    rng = np.random.Generator(np.random.PCG64(22))
    q = 0.05 * rng.standard_normal((1, N, 2, d), dtype=np.float32)
    k = 0.05 * rng.standard_normal((1, N, 2, d), dtype=np.float32)
    v = rng.standard_normal((1, N, 2, d), dtype=np.float32)
    q[0, :, 0, 0] = 24.0
    k[0, T - 3:T, 0, 0] = 24.0   # the last text keys align with every query
    q, k, v = (WL.round_to_bf16(a) for a in (q, k, v))
    got = _run(dict(q=q, k=k, v=v), H, W, spec, "bf16")
    ref = A.attention_tier1(q, k, v, None, None, H, W, spec)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= 2e-2


def test_empty_batch_and_heads_touch_nothing():
    """batch = 0 or heads = 0 through the C ABI: NPA_OK, nothing is launched,
    and an `out` buffer handed in anyway keeps its contents; the Python
    binding and the SG blend accept empty tensors."""
    import ctypes

    lib = npa.load(build_if_missing=False)
    H, W, d = 16, 16, 64
    q = torch.randn(1, H * W, 2, d, device="cuda", dtype=torch.bfloat16)
    out = torch.full_like(q, 7.0)
    stream = torch.cuda.current_stream().cuda_stream
    for field in ("batch", "heads"):
        for h in (npa.make_halo(tile=(8, 8), halo=(4, 4)), npa.make_halo(strips=2, p=0.5)):
            L = npa.make_layout(1, 2, d, H, W)
            setattr(L, field, 0)
            st = lib.npa_attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                  ctypes.byref(L), ctypes.byref(h), out.data_ptr(), stream)
            assert st == npa.NPA_OK, lib.npa_last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    for shape in ((0, H * W, 2, d), (1, H * W, 0, d)):
        e = torch.empty(shape, device="cuda", dtype=torch.bfloat16)
        r = npa.attn_fwd(e, e.clone(), e.clone(), e.clone(), e.clone(), map_hw=(H, W), strips=2, p=0.5)
        assert tuple(r.shape) == shape
    x = torch.empty(0, 4, 8, 8, device="cuda")
    assert tuple(npa.sg_blend(x, x.clone(), 0.5, 4.0).shape) == (0, 4, 8, 8)
    torch.cuda.synchronize()


class _GpuRows:
    """Read-only view of a device tensor [B, N, Hh, d] for the oracle: indexing
    [b, token_indices, head] gathers those rows on the GPU and returns them as
    float32 numpy (exact for bf16)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        b, idx, j = key
        sel = torch.as_tensor(np.asarray(idx, dtype=np.int64), device=self.t.device)
        return self.t[b, sel, j].float().cpu().numpy()


@pytest.mark.parametrize("spec", [A.Windows(64, 64, 16, 16), A.Strips(8, p=0.3)])
def test_slice_at_the_32bit_offset_limit(spec):
    """One (batch, head) slice spanning 2^31 - 1920 bytes, just under the bf16
    kernel's 2^31 - 16 byte addressing limit: a 1024x1024 map whose tokens are
    2 KiB apart (head 0 of 16 used; the other 15 heads' rows are NaN padding
    that must never be read).  Sampled queries in the first, a middle and the
    last tile or strip (the largest offsets) against the oracle."""
    H = W = 1024
    N, d, pad_heads = H * W, 64, 16
    gen = torch.Generator(device="cuda").manual_seed(2024)

    def tensor(like=None):
        full = torch.full((1, N, pad_heads, d), float("nan"), device="cuda", dtype=torch.bfloat16)
        if like is None:
            full[:, :, 0] = torch.randn((1, N, d), generator=gen, device="cuda").to(torch.bfloat16)
        else:
            full[:, :, 0] = (like[:, :, 0].float()
                             + 0.05 * torch.randn((1, N, d), generator=gen, device="cuda")).to(torch.bfloat16)
        return full[:, :, :1]  # strides (N*1024, 1024, 64, 1)

    q, k, v = tensor(), tensor(), tensor()
    strips = isinstance(spec, A.Strips)
    ks, vs = (tensor(k), tensor(v)) if strips else (None, None)
    out = tensor()
    L = npa.make_layout(1, 1, d, H, W, strides=q.stride()[:3])
    assert npa.useful_flops(L, npa.make_halo(**_kw(spec))) > 0
    npa.attn_fwd(q, k, v, ks, vs, map_hw=(H, W), out=out, **_kw(spec))
    torch.cuda.synchronize()
    rows = [0, 1, H // 2, H - 2, H - 1]
    sample = np.array(sorted({r * W + c for r in rows for c in (0, 5, W // 2, W - 6, W - 1)}), dtype=np.int64)
    ref = A.attention_tier1(_GpuRows(q), _GpuRows(k), _GpuRows(v), None if ks is None else _GpuRows(ks),
                            None if vs is None else _GpuRows(vs), H, W, spec, query_tokens=sample,
                            heads=[(0, 0)])
    got = out[0, torch.as_tensor(sample, device="cuda"), 0].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref[0, sample, 0]).max()
    assert np.isfinite(got).all()
    assert err <= ATOL["bf16"], err


# Full compares on small ragged maps with enough (batch, head) pairs that the
# grid fills the GPU at least twice over, so the regular workgroup shape runs
# (the small cases above, and small calls generally, take the small-launch
# shape).  Queries per regular workgroup: 256 at d = 64 and d = 128.
REGULAR = [
    # (H, W, B, Hh, d, spec)
    (24, 20, 2, 172, 64, A.Strips(3, halo_rows=3)),
    (40, 36, 1, 90, 128, A.Windows(20, 12, 4, 7)),
    (16, 16, 2, 130, 64, A.Windows(8, 8, 2, 2, 7)),
]


@pytest.mark.parametrize("H,W,B,Hh,d,spec", REGULAR)
def test_regular_shape_full_compare(H, W, B, Hh, d, spec):
    T = A.text_tokens(spec)
    tiles = list(A.iter_tiles(H, W, spec))
    n_map = len(tiles) - (1 if T else 0)
    nq = len(tiles[0][0])
    grid = B * Hh * (n_map * -(-nq // 256) + (-(-T // 256) if T else 0))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_cu = 2 if d == 64 else 1
    assert grid >= 2 * cus * per_cu, "case too small to run the regular workgroup shape"
    inp = WL.attention_inputs(B, Hh, d, H, W, seed=77, dtype="bf16", text_tokens=T)
    got = _run(inp, H, W, spec, "bf16")
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec)
    assert np.abs(got - ref).max() <= ATOL["bf16"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_strided_views_match_contiguous_bit_for_bit(dt):
    """Inputs that are views into padded, heads-outer buffers, and out=None:
    the output is allocated with q's strides, and every row equals the
    contiguous call's bit for bit (a row's arithmetic does not depend on where
    its neighbours are stored)."""
    H = W = 24
    B, Hh, d = 2, 3, 64
    spec = A.Strips(4, p=0.3)
    inp = WL.attention_inputs(B, Hh, d, H, W, seed=5, dtype=dt)
    want = _run(inp, H, W, spec, dt)

    def view(a):
        t = _dev(a, dt)  # [B, N, Hh, d] contiguous
        buf = torch.full((B, Hh, H * W, d + 8), float("nan"), device="cuda", dtype=TDT[dt])
        buf[..., :d] = t.permute(0, 2, 1, 3)
        return buf[..., :d].permute(0, 2, 1, 3)  # strides (Hh*N*(d+8), d+8, N*(d+8), 1)

    q, k, v, ks, vs = (view(inp[n]) for n in ("q", "k", "v", "k_stale", "v_stale"))
    assert q.stride() == (Hh * H * W * (d + 8), d + 8, H * W * (d + 8), 1)
    out = npa.attn_fwd(q, k, v, ks, vs, map_hw=(H, W), **_kw(spec))
    torch.cuda.synchronize()
    assert out.stride() == q.stride()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)


# fp32: calls whose regular grid has fewer workgroups than the GPU has CUs
# run the key-split shape (every small f32 case above does, at d <= 64); these
# are sized so that the regular 64-query shape runs.
F32_REGULAR = [
    # (H, W, B, Hh, d, spec)
    (32, 32, 1, 80, 64, A.Strips(4, halo_rows=3)),
    (24, 20, 2, 60, 32, A.Windows(8, 10, 3, 2)),
    (16, 16, 1, 64, 64, A.Windows(8, 8, 2, 2, 7)),
]


@pytest.mark.parametrize("H,W,B,Hh,d,spec", F32_REGULAR)
def test_f32_regular_shape_full_compare(H, W, B, Hh, d, spec):
    T = A.text_tokens(spec)
    tiles = list(A.iter_tiles(H, W, spec))
    n_map = len(tiles) - (1 if T else 0)
    nq = len(tiles[0][0])
    grid = B * Hh * (n_map * -(-nq // 64) + (-(-T // 64) if T else 0))
    assert grid >= torch.cuda.get_device_properties(0).multi_processor_count, "case too small for the regular shape"
    inp = WL.attention_inputs(B, Hh, d, H, W, seed=78, dtype="f32", text_tokens=T)
    got = _run(inp, H, W, spec, "f32")
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec)
    assert np.abs(got - ref).max() <= ATOL["f32"]


def test_calls_replay_from_a_hip_graph():
    """npa_attn_fwd and npa_sg_blend captured into one HIP graph: every replay
    (with eager work and synchronisations between replays) reproduces the
    eager result bit for bit."""
    H = W = 32
    spec = A.Windows(8, 8, 4, 4)
    inp = WL.attention_inputs(1, 2, 64, H, W, seed=31, dtype="bf16")
    q, k, v = (_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    x, r = (torch.from_numpy(a).cuda() for a in WL.sg_inputs(4, 40, 56, seed=32))
    out, sg_out = torch.empty_like(q), torch.empty_like(x)

    def step():
        npa.attn_fwd(q, k, v, map_hw=(H, W), out=out, **_kw(spec))
        npa.sg_blend(x, r, 0.5, 4.0, out=sg_out)

    step()  # eager reference (also warms the library's per-device state)
    torch.cuda.synchronize()
    ref_attn, ref_sg = out.clone(), sg_out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        out.zero_()
        sg_out.zero_()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        sg_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_attn), f"replay {i}: attention differs"
        assert torch.equal(sg_out, ref_sg), f"replay {i}: SG blend differs"
        _ = (q.float() * 2).sum().item()  # eager work between replays
