"""Pins for the fp64 attention oracle (CPU only).

Each pin checks the oracle against something other than itself: hand-written
key sets, closed forms, textbook attention computed by torch's fp64 SDPA, and
the brute-force tier.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from partial_context_patch_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _spec(case):
    if case["mode"] == "strips":
        return A.Strips(case["num_strips"], p=case.get("p"), halo_rows=case.get("halo_rows"))
    return A.Windows(case["tile_h"], case["tile_w"], case["halo_h"], case["halo_w"], case.get("text_tokens", 0))


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _sdpa(q, k, v, mask=None, scale=None):
    """Textbook attention by torch (fp64, CPU). q,k,v: [B, N, Hh, d] numpy."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# ---------------------------------------------------------------- halo rows
@pytest.mark.parametrize(
    "H,n,p,h",
    [(32, 4, 0.3, 3), (64, 4, 0.3, 5), (128, 8, 0.8, 13), (40, 4, 0.7, 7), (8, 1, 0.25, 2),
     (16, 2, 0.0, 0), (16, 2, 1.0, 8), (30, 3, 0.3, 3), (30, 3, 0.31, 4)],
)
def test_halo_rows(H, n, p, h):
    assert A.halo_rows(H, A.Strips(n, p=p)) == h
    # p handed over as float32 gives the same rows
    assert A.halo_rows(H, A.Strips(n, p=float(np.float32(p)))) == h


# ---------------------------------------------------------- hand-written sets
def test_golden_membership():
    gold = json.load(open(os.path.join(GOLDEN, "membership_tiny.json")))
    for case in gold["cases"]:
        spec, H, W = _spec(case), case["H"], case["W"]
        sets = A.attended_sets(H, W, spec)
        tiles = list(A.iter_tiles(H, W, spec))
        assert len(tiles) == len(case["tiles"]), case["name"]
        for exp, (qt, ft, st) in zip(case["tiles"], tiles):
            assert sorted(qt.tolist()) == exp["queries"], case["name"]
            assert sorted(ft.tolist()) == exp["fresh"], case["name"]
            assert sorted(st.tolist()) == sorted(exp["stale"]), case["name"]
            for t in exp["queries"]:
                assert sets[t][0] == exp["fresh"], case["name"]
                assert sets[t][1] == sorted(exp["stale"]), case["name"]


def test_workload_counts():
    gold = json.load(open(os.path.join(GOLDEN, "workload_counts.json")))["workloads"]
    for name, g in gold.items():
        w = WL.ATTENTION_WORKLOADS[name]
        H, W = w["map_h"], w["map_w"]
        if w["mode"] == "strips":
            spec = A.Strips(w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
            assert A.halo_rows(H, spec) == g["halo_rows"]
        else:
            spec = A.Windows(w["tile_h"], w["tile_w"], w["halo_h"], w["halo_w"], w.get("text_tokens", 0))
        sizes = [len(ft) + len(st) for _, ft, st in A.iter_tiles(H, W, spec)]
        assert max(sizes) == g["keys_interior"] and min(sizes) == g["keys_border"], name
        assert A.useful_pairs(H, W, spec) == g["pairs_per_bh"], name


# ------------------------------------------------------ textbook special cases
def test_one_strip_is_full_attention():
    H, W, B, Hh, d = 6, 5, 2, 3, 8
    q, k, v = (_rand((B, H * W, Hh, d), s) for s in (1, 2, 3))
    ks, vs = _rand(q.shape, 4), _rand(q.shape, 5)
    for spec in (A.Strips(1, p=0.7), A.Windows(H, W, 0, 0), A.Windows(2, 1, 9, 9)):
        got = A.attention_tier1(q, k, v, ks, vs, H, W, spec)
        np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_joint_whole_map_window_is_full_attention(T):
    """A window that covers the whole map makes every query, text or map, see
    every stored token: plain attention over all T + N tokens."""
    H, W, B, Hh, d = 4, 6, 2, 2, 8
    N = T + H * W
    q, k, v = (_rand((B, N, Hh, d), s) for s in (21 + T, 22 + T, 23 + T))
    for spec in (A.Windows(H, W, 0, 0, T), A.Windows(2, 3, 9, 9, T)):
        got = A.attention_tier1(q, k, v, None, None, H, W, spec)
        np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_joint_tiers_agree():
    """Loop tier (per-pair predicates) against the vectorised tier on a joint case."""
    H, W, B, Hh, d, T = 4, 4, 1, 2, 4, 3
    N = T + H * W
    q, k, v = (_rand((B, N, Hh, d), s) for s in (31, 32, 33))
    spec = A.Windows(2, 2, 1, 1, T)
    np.testing.assert_allclose(A.attention_tier1(q, k, v, None, None, H, W, spec),
                               A.attention_tier0(q, k, v, None, None, H, W, spec), rtol=0, atol=1e-12)


def test_joint_text_keys_are_reached():
    """Map queries put weight on the text keys: with every map key's value 0 and
    every text key's value 1, each map query's output is the softmax mass on the
    text keys, in (0, 1); text queries see the same keys plus the rest of the map."""
    H, W, B, Hh, d, T = 4, 4, 1, 1, 4, 2
    N = T + H * W
    q, k = _rand((B, N, Hh, d), 41), _rand((B, N, Hh, d), 42)
    v = np.zeros((B, N, Hh, 1))
    v[:, :T] = 1.0
    out = A.attention_tier1(q, k, v, None, None, H, W, A.Windows(2, 2, 0, 0, T))
    assert np.all(out > 0) and np.all(out < 1)


def test_p0_is_block_diagonal():
    H, W, B, Hh, d = 8, 3, 1, 2, 4
    q, k, v = (_rand((B, H * W, Hh, d), s) for s in (11, 12, 13))
    ks, vs = np.full_like(k, np.nan), np.full_like(v, np.nan)  # never read at p = 0
    got = A.attention_tier1(q, k, v, ks, vs, H, W, A.Strips(4, p=0.0))
    s = 2 * W
    for i in range(4):
        sl = slice(i * s, (i + 1) * s)
        np.testing.assert_allclose(got[:, sl], _sdpa(q[:, sl], k[:, sl], v[:, sl]), rtol=0, atol=1e-12)
    # windows with no halo: independent attention inside each tile
    got = A.attention_tier1(q, k, v, None, None, H, W, A.Windows(2, 3, 0, 0))
    for i in range(4):
        sl = slice(i * s, (i + 1) * s)
        np.testing.assert_allclose(got[:, sl], _sdpa(q[:, sl], k[:, sl], v[:, sl]), rtol=0, atol=1e-12)


def test_p1_two_strips_fresh_equals_stale_is_full():
    H, W, B, Hh, d = 6, 4, 1, 2, 8
    q, k, v = (_rand((B, H * W, Hh, d), s) for s in (21, 22, 23))
    got = A.attention_tier1(q, k, v, k, v, H, W, A.Strips(2, p=1.0))
    np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_p1_many_strips_is_block_tridiagonal():
    H, W, B, Hh, d, n = 12, 3, 1, 2, 8, 4
    q, k, v = (_rand((B, H * W, Hh, d), s) for s in (31, 32, 33))
    strip = (np.arange(H * W) // W) // (H // n)
    mask = np.abs(strip[:, None] - strip[None, :]) <= 1
    got = A.attention_tier1(q, k, v, k, v, H, W, A.Strips(n, p=1.0))
    np.testing.assert_allclose(got, _sdpa(q, k, v, mask=mask), rtol=0, atol=1e-12)


def test_distinct_stale_matches_masked_concatenation():
    """Library form: SDPA over [K_fresh; K_stale] with the membership mask."""
    H, W, B, Hh, d, n = 9, 4, 2, 2, 8, 3
    q, k, v, ks, vs = (_rand((B, H * W, Hh, d), s) for s in (41, 42, 43, 44, 45))
    N = H * W
    rows = np.arange(N) // W
    s = H // n
    h = 2
    mask = np.zeros((N, 2 * N), dtype=bool)
    for t in range(N):
        i = rows[t] // s
        mask[t, :N] = rows // s == i
        mask[t, N:] = ((rows >= i * s - h) & (rows < i * s)) | ((rows >= (i + 1) * s) & (rows < (i + 1) * s + h))
    got = A.attention_tier1(q, k, v, ks, vs, H, W, A.Strips(n, halo_rows=h), scale=0.37)
    ref = _sdpa(q, np.concatenate([k, ks], 1), np.concatenate([v, vs], 1), mask=mask, scale=0.37)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------- brute force
@pytest.mark.parametrize(
    "H,W,spec",
    [
        (4, 4, A.Strips(1, halo_rows=0)),
        (4, 4, A.Strips(2, halo_rows=1)),
        (4, 4, A.Strips(4, halo_rows=0)),
        (4, 4, A.Strips(4, halo_rows=3)),
        (4, 4, A.Strips(2, halo_rows=4)),
        (4, 4, A.Windows(1, 1, 1, 2)),
        (4, 4, A.Windows(2, 2, 1, 1)),
        (4, 4, A.Windows(4, 2, 0, 3)),
        (4, 4, A.Windows(2, 4, 4, 0)),
        (6, 5, A.Strips(3, p=0.5)),
        (6, 5, A.Windows(3, 5, 1, 2)),
    ],
)
def test_tier0_equals_tier1(H, W, spec):
    B, Hh, d = 1, 2, 5
    q, k, v, ks, vs = (_rand((B, H * W, Hh, d), 50 + s) for s in range(5))
    t0 = A.attention_tier0(q, k, v, ks, vs, H, W, spec, scale=0.6)
    t1 = A.attention_tier1(q, k, v, ks, vs, H, W, spec, scale=0.6)
    np.testing.assert_allclose(t0, t1, rtol=0, atol=1e-12)


def test_brute_force_sets_on_4x4():
    """Enumerate every (query, key) pair by the raw distance rule on a 4x4 map."""
    H = W = 4
    for n in (1, 2, 4):
        s = H // n
        for h in range(5):
            sets = A.attended_sets(H, W, A.Strips(n, halo_rows=h))
            for t in range(16):
                r = t // W
                lo, hi = (r // s) * s, (r // s) * s + s
                fresh = [u for u in range(16) if lo <= u // W < hi]
                stale = [u for u in range(16) if (lo - h <= u // W < lo) or (hi <= u // W < hi + h)]
                assert sets[t] == (fresh, stale)
    for th in (1, 2, 4):
        for tw in (1, 2, 4):
            for eh in range(5):
                for ew in range(5):
                    sets = A.attended_sets(H, W, A.Windows(th, tw, eh, ew))
                    for t in range(16):
                        r, c = divmod(t, W)
                        r0, c0 = (r // th) * th, (c // tw) * tw
                        fresh = [u for u in range(16)
                                 if r0 - eh <= u // W < r0 + th + eh and c0 - ew <= u % W < c0 + tw + ew]
                        assert sets[t] == (fresh, [])


# -------------------------------------------------------- probability rows
@pytest.mark.parametrize("spec", [A.Strips(2, halo_rows=1), A.Strips(4, halo_rows=2), A.Windows(2, 2, 1, 1)])
def test_one_hot_values_expose_rows_summing_to_one(spec):
    H = W = 4
    N = H * W
    q, k, ks = (_rand((1, N, 1, 6), s) for s in (61, 62, 63))
    vf = np.concatenate([np.eye(N), np.zeros((N, N))], 1)[None, :, None, :]
    vs = np.concatenate([np.zeros((N, N)), np.eye(N)], 1)[None, :, None, :]
    P = A.attention_tier1(q, k, vf, ks, vs, H, W, spec)[0, :, 0, :]
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-14)
    sets = A.attended_sets(H, W, spec)
    for t in range(N):
        allowed = np.zeros(2 * N, dtype=bool)
        allowed[sets[t][0]] = True
        allowed[[N + u for u in sets[t][1]]] = True
        assert np.all(P[t, ~allowed] == 0.0) and np.all(P[t, allowed] > 0.0)


def test_zero_query_gives_closed_form_set_means():
    """Q = 0 makes the weights uniform: O = mean of V over the attended set."""
    H, W, n, h = 12, 5, 3, 3
    N = H * W
    rows, cols = np.arange(N) // W, np.arange(N) % W
    q = np.zeros((1, N, 1, 4))
    k = _rand((1, N, 1, 4), 71)
    vf = np.stack([np.ones(N), np.zeros(N), rows, cols], 1)[None, :, None, :]
    vs = np.stack([np.ones(N), np.ones(N), rows, cols], 1)[None, :, None, :]
    O = A.attention_tier1(q, k, vf, k, vs, H, W, A.Strips(n, halo_rows=h))[0, :, 0]
    s = H // n
    for t in range(N):
        i = rows[t] // s
        above = min(h, i * s)
        below = min(h, H - (i + 1) * s)
        n_f, n_t = s * W, (above + below) * W
        row_sum = W * (sum(range(i * s, i * s + s)) + sum(range(i * s - above, i * s))
                       + sum(range((i + 1) * s, (i + 1) * s + below)))
        assert O[t, 0] == pytest.approx(1.0, abs=1e-14)
        assert O[t, 1] == pytest.approx(n_t / (n_f + n_t), abs=1e-14)
        assert O[t, 2] == pytest.approx(row_sum / (n_f + n_t), abs=1e-12)
        assert O[t, 3] == pytest.approx((W - 1) / 2, abs=1e-12)
    # windows: uniform mean over the clipped rectangle
    spec = A.Windows(4, 5, 2, 1)
    O = A.attention_tier1(q, k, vf, None, None, H, W, spec)[0, :, 0]
    for t in range(N):
        r, c = rows[t], cols[t]
        r0, r1 = max(0, (r // 4) * 4 - 2), min(H, (r // 4) * 4 + 6)
        c0, c1 = max(0, (c // 5) * 5 - 1), min(W, (c // 5) * 5 + 6)
        assert O[t, 2] == pytest.approx((r0 + r1 - 1) / 2, abs=1e-12)
        assert O[t, 3] == pytest.approx((c0 + c1 - 1) / 2, abs=1e-12)


def test_sampled_queries_match_full_run():
    H, W, B, Hh, d = 8, 8, 1, 2, 8
    q, k, v, ks, vs = (_rand((B, H * W, Hh, d), 80 + s) for s in range(5))
    spec = A.Strips(4, halo_rows=1)
    full = A.attention_tier1(q, k, v, ks, vs, H, W, spec)
    pick = [0, 7, 17, 40, 63]
    part = A.attention_tier1(q, k, v, ks, vs, H, W, spec, query_tokens=pick, heads=[(0, 1)])
    np.testing.assert_allclose(part[0, pick, 1], full[0, pick, 1], rtol=0, atol=1e-14)
    assert np.isnan(part[0, pick, 0]).all()


def test_useful_flops_definition():
    spec = A.Windows(2, 2, 1, 1)
    # 4 tiles of 4 queries, each with a 3x3 clipped window
    assert A.useful_pairs(4, 4, spec) == 4 * 4 * 9
    assert A.useful_flops(2, 3, 64, 4, 4, spec) == 4 * 64 * 144 * 2 * 3
