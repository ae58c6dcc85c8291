"""GPU structural probes at the geometry the large layers run, through the C ABI.

The random-input compares pin the arithmetic; these pin which keys each query
reads, bit-exactly, at full size and in the launch configuration the benchmark
times (the kernels' copy cursor walks window rows of 64-128 keys there, a path
the small maps of the other parity cases reach only partly):

* marked keys: Q = 0 makes every weight 1/|S(q)|; V is zero except four keys
  per (batch, head, channel) holding 1, 2, 4 and 8, so out[q, channel] times
  |S(q)| is exactly the sum of the values of the marked keys inside the
  query's set -- which of the four keys each query reads, decoded exactly.
  The keys sit on window / strip edges (inside and just outside), on 64-key
  block boundaries, on the row wraps inside the blocks and on text tokens;
* NaN poisoning: everything outside one tile's key set (and every other
  tile's queries) is NaN; that tile's outputs must stay finite and equal the
  clean run bit for bit;
* window rows of 32, 33, 48, 63, 64 and 96 keys on small maps, in every
  workgroup shape of both kernels: full compares against the oracle and the
  marked-key probe;
* the fp32 path at the sizes of the bf16 layers (full compare of two (batch,
  head) slices, and of one tile for every slice).

Key sets and set sizes come from the oracle's tile enumeration (its
predicate over the whole map); nothing expected comes from the HIP path.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from partial_context_patch_amd import npa
from partial_context_patch_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
ATOL = {"bf16": 2e-2, "f32": 1e-4}
# queries per workgroup and workgroups per CU of the regular shapes
BF16_REGULAR_BM = 256
BF16_REGULAR_PER_CU = {64: 2, 128: 1}
F32_REGULAR_BM = 64


def _spec(w):
    if w["mode"] == "strips":
        return A.Strips(w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
    return A.Windows(w["tile_h"], w["tile_w"], w["halo_h"], w["halo_w"], w.get("text_tokens", 0))


def _kw(spec):
    if isinstance(spec, A.Strips):
        return dict(strips=spec.num_strips, p=spec.p, halo_rows=spec.halo_rows)
    return dict(tile=(spec.tile_h, spec.tile_w), halo=(spec.halo_h, spec.halo_w), text_tokens=spec.text_tokens)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _grid(H, W, spec, B, Hh, bm):
    """Workgroups of a launch with bm queries per workgroup (map tiles, plus the
    text tile's blocks)."""
    tiles = list(A.iter_tiles(H, W, spec))
    T = A.text_tokens(spec)
    n_map = len(tiles) - (1 if T else 0)
    nq = len(tiles[0][0])
    return B * Hh * (n_map * -(-nq // bm) + (-(-T // bm) if T else 0))


def _heads_for_regular(H, W, spec, B, d, dt):
    """Enough heads that the regular workgroup shape runs (the library picks
    the small-launch / key-split shape for grids that would not fill the GPU)."""
    if dt == "bf16":
        need, bm = 2 * _cus() * BF16_REGULAR_PER_CU[d], BF16_REGULAR_BM
    else:
        need, bm = _cus(), F32_REGULAR_BM
    per_head = _grid(H, W, spec, B, 1, bm)
    return -(-need // per_head) + 1


# ----------------------------------------------------------------- keys
def _edge_set(lo_hi, n):
    out = set()
    for lo, hi in lo_hi:
        out |= {lo - 1, lo, lo + 1, hi - 2, hi - 1, hi}
    return sorted(x for x in out if 0 <= x < n)


def _probe_keys(H, W, spec):
    """Candidate keys as stored-token indices, in classes (fresh classes, stale
    classes): keys on the edges of every key range (inside and just outside),
    on the 64-key block boundaries of every key run, on the row wraps of every
    window, and text tokens."""
    T = A.text_tokens(spec)
    tiles = list(A.iter_tiles(H, W, spec))
    if isinstance(spec, A.Strips):
        s = H // spec.num_strips
        h = A.halo_rows(H, spec)
        rows_f = _edge_set([(i * s, (i + 1) * s) for i in range(spec.num_strips)], H)
        rows_s = _edge_set([(max(0, i * s - h), i * s) for i in range(spec.num_strips)]
                           + [((i + 1) * s, min(H, (i + 1) * s + h)) for i in range(spec.num_strips)], H)
        cols = sorted({0, 1, W // 2, W - 2, W - 1})
        edge_f = [r * W + c for r in rows_f for c in cols]
        edge_s = [r * W + c for r in rows_s for c in cols]
        block_f, block_s = [], []
        for _, ft, st in tiles:
            for run, dst in ((ft, block_f), (st, block_s)):
                # runs are whole rows: the block boundaries of each contiguous piece
                pieces = np.split(run, np.flatnonzero(np.diff(run) != 1) + 1) if len(run) else []
                for p in pieces:
                    for j in range(0, len(p) + 1, 64):
                        dst += [int(p[x]) for x in (j - 1, j) if 0 <= x < len(p)]
        return [edge_f, block_f], [edge_s, block_s]
    th, tw, eh, ew = spec.tile_h, spec.tile_w, spec.halo_h, spec.halo_w
    rr = [(max(0, ti * th - eh), min(H, (ti + 1) * th + eh)) for ti in range(H // th)]
    cr = [(max(0, tj * tw - ew), min(W, (tj + 1) * tw + ew)) for tj in range(W // tw)]
    rows = _edge_set(rr + [(ti * th, (ti + 1) * th) for ti in range(H // th)], H)
    cols = _edge_set(cr + [(tj * tw, (tj + 1) * tw) for tj in range(W // tw)], W)
    edge = [T + r * W + c for r in rows for c in cols]
    block, wrap = [], []
    for (r0, r1) in rr:
        for (c0, c1) in cr:
            L = c1 - c0
            n = L * (r1 - r0)
            for j in range(0, n + 1, 64):  # block boundaries, in window order
                for x in (j - 1, j):
                    if 0 <= x < n:
                        block.append(T + (r0 + x // L) * W + c0 + x % L)
            for r in range(r0, r1):  # row wraps
                wrap += [T + r * W + c0, T + r * W + c1 - 1]
    classes = [edge, block, wrap]
    if T:
        classes.append(sorted({t for j in range(0, T + 1, 64) for t in (j - 1, j) if 0 <= t < T}
                              | {0, 1, T // 2, T - 2, T - 1}))
    return classes, []


def _dedupe(seq):
    seen, out = set(), []
    for x in seq:
        if x not in seen:
            seen.add(x)
            out.append(x)
    return out


def _assign(classes, slots, rng):
    """Distribute candidate keys over `slots` marks: each class in a seeded
    order, the classes interleaved (so every kind of key is marked even when
    there are more candidates than marks); recycled when there are fewer."""
    classes = [_dedupe(c) for c in classes if c]
    if not classes:
        return np.zeros(slots, dtype=np.int64)
    classes = [[c[i] for i in rng.permutation(len(c))] for c in classes]
    order, i = [], 0
    while any(i < len(c) for c in classes):
        order += [c[i] for c in classes if i < len(c)]
        i += 1
    order = _dedupe(order)
    return np.resize(np.array(order, dtype=np.int64), slots)


# Keys marked per (batch, head, channel), with values 1, 2, 4, 8: the output
# times |S(q)| is then the sum of the values of the marked keys in the set,
# an integer 0..15 that bf16 rounding (relative 2^-9) cannot blur.
MARKS = 4


def marked_key_probe(B, Hh, d, H, W, spec, dt="bf16", seed=0):
    """Run the probe; return the number of (query, channel) outputs checked."""
    T = A.text_tokens(spec)
    N = T + H * W
    strips = isinstance(spec, A.Strips)
    rng = np.random.Generator(np.random.PCG64(seed))
    cand_f, cand_s = _probe_keys(H, W, spec)
    nf = d // 2 if strips else d
    mf = _assign(cand_f, B * Hh * nf * MARKS, rng).reshape(B, Hh, nf, MARKS)
    ms = _assign(cand_s, B * Hh * (d - nf) * MARKS, rng).reshape(B, Hh, d - nf, MARKS) if strips else None
    weights = 2.0 ** np.arange(MARKS)
    dev, tdt = DEV, TDT[dt]
    gen = torch.Generator(device=dev).manual_seed(seed)

    def marked(m, ch0):
        x = torch.zeros((B, N, Hh, d), device=dev, dtype=torch.float32)
        idx = np.indices(m.shape)
        cols = [torch.as_tensor(a.ravel(), device=dev) for a in (idx[0], m, idx[1], idx[2] + ch0)]
        vals = torch.as_tensor(np.broadcast_to(weights, m.shape).ravel(), device=dev, dtype=torch.float32)
        x.index_put_(tuple(cols), vals, accumulate=True)  # a key marked twice in one channel sums
        return x.to(tdt)

    q = torch.zeros((B, N, Hh, d), device=dev, dtype=tdt)
    k = torch.randn((B, N, Hh, d), generator=gen, device=dev).to(tdt)
    v = marked(mf, 0)
    ks = vs = None
    if strips:
        ks = torch.randn((B, N, Hh, d), generator=gen, device=dev).to(tdt)
        vs = marked(ms, nf)
    n_keys = len(set(mf.ravel().tolist())) + (len(set(ms.ravel().tolist())) if strips else 0)
    print(f"[probe] marked keys B={B} heads={Hh} d={d} map={H}x{W} {spec} {dt}: {n_keys} distinct keys marked",
          flush=True)
    out = npa.attn_fwd(q, k, v, ks, vs, map_hw=(H, W), **_kw(spec))
    torch.cuda.synchronize()
    tiles = list(A.iter_tiles(H, W, spec))
    checked = 0
    for b in range(B):
        for j in range(Hh):
            code = np.zeros((N, d))   # expected sum of the values of the marked keys in S(q)
            size = np.zeros(N)        # |S(q)|
            for qt, ft, st in tiles:
                size[qt] = len(ft) + len(st)
                inf = np.zeros(N, dtype=bool)
                inf[ft] = True
                code[np.ix_(qt, np.arange(nf))] = (inf[mf[b, j]] @ weights)[None, :]
                if strips:
                    ins = np.zeros(N, dtype=bool)
                    ins[st] = True
                    code[np.ix_(qt, np.arange(nf, d))] = (ins[ms[b, j]] @ weights)[None, :]
            got = out[b, :, j, :].float().cpu().numpy().astype(np.float64) * size[:, None]
            bad = np.abs(got - code) > 0.05
            if bad.any():
                t, e = np.argwhere(bad)[0]
                keys = mf[b, j, e] if e < nf else ms[b, j, e - nf]
                raise AssertionError(
                    f"(b={b}, head={j}) query token {t}, channel {e} ({'fresh' if e < nf else 'stale'} keys "
                    f"{keys.tolist()} valued {weights.tolist()}): got {got[t, e]:.4f}, expected {code[t, e]:.0f} "
                    f"(|S| = {size[t]:.0f}); {int(bad.sum())} mismatches")
            checked += code.size
    return checked


# ----------------------------------------------------- full-size probes
FULL = ["sdxl4096_npa", "flux4096_npa", "flux4096_joint", "sdxl2048_strips", "sdxl2048_fullstale", "sdxl1024_strips"]


@pytest.mark.parametrize("name", FULL)
def test_marked_keys_at_full_size(name):
    w = WL.ATTENTION_WORKLOADS[name]
    print(f"[probe] workload {name}: {w['what']}", flush=True)
    n = marked_key_probe(w["batch"], w["heads"], w["head_dim"], w["map_h"], w["map_w"], _spec(w), w["dtype"],
                         seed=w["seed"])
    assert n == w["batch"] * w["heads"] * (A.text_tokens(_spec(w)) + w["map_h"] * w["map_w"]) * w["head_dim"]


def _pick_tiles(H, W, spec):
    """An interior, an edge and a corner map tile (strips: a middle, the first
    and the last strip)."""
    if isinstance(spec, A.Strips):
        n = spec.num_strips
        return sorted({n // 2, 0, n - 1})
    tx, ty = W // spec.tile_w, H // spec.tile_h
    return sorted({(ty // 2) * tx + tx // 2, tx // 2, 0, ty * tx - 1})


@pytest.mark.parametrize("name", FULL)
def test_nan_poisoning_at_full_size(name):
    """For each picked tile: every key outside its set (fresh and stale) and
    every query outside the tile is NaN; the tile's outputs equal the clean
    run bit for bit, for every batch item and head."""
    w = WL.ATTENTION_WORKLOADS[name]
    spec = _spec(w)
    H, W = w["map_h"], w["map_w"]
    T = A.text_tokens(spec)
    N = T + H * W
    B, Hh, d = w["batch"], w["heads"], w["head_dim"]
    tdt = TDT[w["dtype"]]
    gen = torch.Generator(device=DEV).manual_seed(w["seed"])
    t = {n: torch.randn((B, N, Hh, d), generator=gen, device=DEV).to(tdt) for n in ("q", "k", "v")}
    strips = isinstance(spec, A.Strips)
    if strips:
        for n in ("k", "v"):
            t[n + "s"] = (t[n].float() + 0.05 * torch.randn((B, N, Hh, d), generator=gen, device=DEV)).to(tdt)
    else:
        t["ks"] = t["vs"] = None
    hw = (H, W)
    clean = npa.attn_fwd(t["q"], t["k"], t["v"], t["ks"], t["vs"], map_hw=hw, **_kw(spec))
    tiles = list(A.iter_tiles(H, W, spec))
    nan = float("nan")
    for idx in _pick_tiles(H, W, spec):
        qt, ft, st = tiles[idx]
        print(f"[probe] {name}: NaN outside tile {idx} ({len(qt)} queries, {len(ft)} fresh, {len(st)} stale keys)",
              flush=True)

        def poisoned(x, keep):
            m = torch.ones(N, dtype=torch.bool, device=DEV)
            m[torch.as_tensor(keep, device=DEV)] = False
            y = x.clone()
            y[:, m] = nan
            return y

        q = poisoned(t["q"], qt)
        k, v = poisoned(t["k"], ft), poisoned(t["v"], ft)
        ks = vs = None
        if strips:
            ks, vs = poisoned(t["ks"], st), poisoned(t["vs"], st)
        got = npa.attn_fwd(q, k, v, ks, vs, map_hw=hw, **_kw(spec))
        torch.cuda.synchronize()
        qi = torch.as_tensor(qt, device=DEV)
        g, c = got[:, qi], clean[:, qi]
        assert bool(torch.isfinite(g.float()).all()), f"{name} tile {idx}: non-finite output"
        assert torch.equal(g.view(torch.int16), c.view(torch.int16)), f"{name} tile {idx}: differs from clean run"
        del q, k, v, ks, vs, got


# ------------------------------------- robust pass and NaN keys, full size
ROBUST = ["sdxl4096_npa", "flux4096_npa", "flux4096_joint", "sdxl2048_strips"]


def _planted(w, spec):
    """Stored-token indices of two map keys: the map's centre and a token one
    row above and one column left of the bottom-right corner."""
    T = A.text_tokens(spec)
    H, W = w["map_h"], w["map_w"]
    return [T + (H // 2) * W + W // 2, T + (H - 2) * W + (W - 2)]


def _tiles_holding(spec, H, W, key):
    """Query tokens of every tile whose fresh key set holds `key`."""
    return [qt for qt, ft, _ in A.iter_tiles(H, W, spec) if key in set(ft.tolist())]


@pytest.mark.parametrize("name", ROBUST)
def test_robust_pass_at_full_size(name):
    """Two keys per (batch, head) whose logits beat the rest by 180-280 log2
    units (q and k share a large first channel): past 2^128 the fixed-shift
    weights overflow fp32, so every workgroup whose key set holds one of them,
    after its first 32 keys, gives inf/inf unless it redoes its tile with the
    true row maxima -- a pass that walks the same copy cursor over the full
    layer's key runs.  The affected tiles and one unaffected tile, for two
    (batch, head) pairs, against the oracle."""
    w = WL.ATTENTION_WORKLOADS[name]
    print(f"[probe] robust pass {name}", flush=True)
    spec = _spec(w)
    H, W = w["map_h"], w["map_w"]
    inp = WL.workload_inputs(name)
    q, k = inp["q"].copy(), inp["k"].copy()
    q[:, :, :, 0] = 40.0
    keys = _planted(w, spec)
    for key in keys:
        k[:, key, :, 0] = 40.0
    t = {n: (None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(TDT[w["dtype"]]))
         for n, a in dict(inp, q=q, k=k).items()}
    out = npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], map_hw=(H, W), **_kw(spec))
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    sel = set()
    for key in keys:
        for qt in _tiles_holding(spec, H, W, key):
            sel |= set(qt.tolist())
    sel |= set(next(iter(A.iter_tiles(H, W, spec)))[0].tolist())  # the first map tile: no planted key
    qs = np.array(sorted(sel))
    heads = [(0, 0), (w["batch"] - 1, w["heads"] - 1)]
    ref = A.attention_tier1(q, k, inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec, query_tokens=qs, heads=heads)
    for b, j in heads:
        err = np.abs(got[b, qs, j] - ref[b, qs, j]).max()
        assert err <= ATOL[w["dtype"]], f"{name} (b={b}, head={j}): max abs err {err}"
    del t, out


@pytest.mark.parametrize("name", ["sdxl4096_npa", "flux4096_joint", "sdxl2048_strips"])
def test_nan_key_reaches_exactly_its_sets(name):
    """One NaN in a fresh key row of one (batch, head): the outputs that turn
    NaN are exactly those of the queries whose key set holds that key, in that
    (batch, head); every other output is finite and bit-identical to the clean
    run."""
    w = WL.ATTENTION_WORKLOADS[name]
    print(f"[probe] NaN key {name}", flush=True)
    spec = _spec(w)
    H, W = w["map_h"], w["map_w"]
    inp = WL.workload_inputs(name)
    dt = TDT[w["dtype"]]
    t = {n: (None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)) for n, a in inp.items()}
    kw = dict(_kw(spec), map_hw=(H, W))
    clean = npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], **kw)
    key = _planted(w, spec)[0]
    b, j = w["batch"] - 1, w["heads"] // 2
    t["k"][b, key, j, 5] = float("nan")
    got = npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], **kw)
    torch.cuda.synchronize()
    expect = torch.zeros(got.shape[:3], dtype=torch.bool)
    for qt in _tiles_holding(spec, H, W, key):
        expect[b, torch.from_numpy(qt), j] = True
    nan = torch.isnan(got.float()).any(dim=-1).cpu()
    assert torch.equal(nan, expect), f"{name}: {int(nan.sum())} NaN rows, {int(expect.sum())} expected"
    assert bool(torch.isnan(got.float()[expect.to(got.device)]).all())
    keep = ~expect.to(got.device)
    assert torch.equal(got[keep].view(torch.int16), clean[keep].view(torch.int16))
    del t, clean, got


# --------------------------------------------- window rows of 32..96 keys
# (H, W, spec): the widest window row of each case is 32, 33, 48, 63, 64 or 96
# keys; the border tiles' rows are narrower (24 .. 80), some windows end on a
# 64-key block boundary and some inside a block
WIDE = [
    (24, 64, A.Windows(8, 16, 4, 8)),     # rows of 24 / 32 keys
    (22, 44, A.Windows(11, 11, 5, 11)),   # 22 / 33: a 64-key block crosses two row ends
    (16, 96, A.Windows(8, 32, 3, 8)),     # 40 / 48
    (21, 63, A.Windows(7, 21, 7, 21)),    # 42 / 63 (the middle tile's window spans the map)
    (16, 96, A.Windows(8, 32, 4, 16)),    # 48 / 64
    (16, 192, A.Windows(8, 64, 4, 16)),   # 80 / 96
    (22, 44, A.Windows(11, 11, 5, 11, 70)),  # 22 / 33 with text tokens
]


def _widest_row(H, W, spec):
    return max(min(W, (tj + 1) * spec.tile_w + spec.halo_w) - max(0, tj * spec.tile_w - spec.halo_w)
               for tj in range(W // spec.tile_w))


def test_wide_cases_cover_the_row_widths():
    widths = {_widest_row(H, W, s) for H, W, s in WIDE}
    assert {32, 33, 48, 63, 64, 96} <= widths


@pytest.mark.parametrize("shape", ["small", "regular"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,W,spec", WIDE)
def test_wide_window_rows_full_compare(H, W, spec, d, shape):
    B = 1
    Hh = 2 if shape == "small" else _heads_for_regular(H, W, spec, B, d, "bf16")
    grid = _grid(H, W, spec, B, Hh, BF16_REGULAR_BM)
    regular = grid >= 2 * _cus() * BF16_REGULAR_PER_CU[d]
    assert regular == (shape == "regular"), "case does not select the intended workgroup shape"
    T = A.text_tokens(spec)
    print(f"[probe] wide rows {H}x{W} {spec} d={d} heads={Hh} ({shape} shape)", flush=True)
    inp = WL.attention_inputs(B, Hh, d, H, W, seed=H * W + d, dtype="bf16", stale=False, text_tokens=T)
    q, k, v = (torch.from_numpy(inp[n]).to(DEV).to(torch.bfloat16) for n in ("q", "k", "v"))
    out = npa.attn_fwd(q, k, v, map_hw=(H, W), **_kw(spec))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], None, None, H, W, spec)
    err = np.abs(got - ref).max()
    assert np.isfinite(got).all()
    assert err <= ATOL["bf16"], f"max abs err {err}"


@pytest.mark.parametrize("shape", ["small", "regular"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,W,spec", WIDE)
def test_wide_window_rows_marked_keys(H, W, spec, d, shape):
    B = 1
    Hh = 2 if shape == "small" else _heads_for_regular(H, W, spec, B, d, "bf16")
    assert (_grid(H, W, spec, B, Hh, BF16_REGULAR_BM) >= 2 * _cus() * BF16_REGULAR_PER_CU[d]) == (shape == "regular")
    marked_key_probe(B, Hh, d, H, W, spec, "bf16", seed=H + W + d)


@pytest.mark.parametrize("shape", ["split", "regular"])
@pytest.mark.parametrize("H,W,spec", WIDE)
def test_f32_wide_window_rows(H, W, spec, shape):
    """The fp32 kernel locates window rows by a float-reciprocal division:
    full compare (1e-4) and marked keys at the same widths, key-split and
    regular shapes (d = 64)."""
    B, d = 1, 64
    Hh = 2 if shape == "split" else _heads_for_regular(H, W, spec, B, d, "f32")
    regular = _grid(H, W, spec, B, Hh, F32_REGULAR_BM) >= _cus()
    assert regular == (shape == "regular")
    T = A.text_tokens(spec)
    inp = WL.attention_inputs(B, Hh, d, H, W, seed=H * W + 7, dtype="f32", stale=False, text_tokens=T)
    q, k, v = (torch.from_numpy(inp[n]).to(DEV) for n in ("q", "k", "v"))
    out = npa.attn_fwd(q, k, v, map_hw=(H, W), **_kw(spec))
    torch.cuda.synchronize()
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], None, None, H, W, spec)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max()
    assert err <= ATOL["f32"], f"max abs err {err}"
    marked_key_probe(B, Hh, d, H, W, spec, "f32", seed=H + W)


# ------------------------------------------------- fp32 at layer sizes
@pytest.mark.parametrize("name", ["sdxl4096_npa", "flux4096_npa", "sdxl2048_strips", "sdxl1024_strips"])
def test_f32_at_layer_size(name):
    """fp32 inputs of the bf16 layers' shapes (the sizes the fp32 throughput is
    quoted on): every query of the first and the last (batch, head) slice, and
    one interior tile of every slice, against the oracle at 1e-4."""
    w = dict(WL.ATTENTION_WORKLOADS[name], dtype="f32")
    spec = _spec(w)
    H, W = w["map_h"], w["map_w"]
    print(f"[probe] fp32 at the size of {name}", flush=True)
    inp = WL.attention_inputs(**w, stale=(w["mode"] == "strips"))
    t = {n: (None if a is None else torch.from_numpy(a).to(DEV)) for n, a in inp.items()}
    out = npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], map_hw=(H, W), **_kw(spec))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del t, out
    heads = [(0, 0), (w["batch"] - 1, w["heads"] - 1)]
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec, heads=heads)
    for b, j in heads:
        err = np.abs(got[b, :, j].astype(np.float64) - ref[b, :, j]).max()
        assert err <= ATOL["f32"], f"{name} fp32 (b={b}, head={j}): max abs err {err}"
    tiles = list(A.iter_tiles(H, W, spec))
    qt = tiles[_pick_tiles(H, W, spec)[len(_pick_tiles(H, W, spec)) // 2]][0]
    ref = A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec,
                            query_tokens=qt)
    err = np.abs(got[:, qt].astype(np.float64) - ref[:, qt]).max()
    assert err <= ATOL["f32"], f"{name} fp32, one tile of every slice: max abs err {err}"
