"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Each mutant replaces one oracle function with a wrong variant via monkeypatch;
the pin that should catch it is re-run and must fail.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import guidance as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_membership_holds() -> bool:
    gold = json.load(open(os.path.join(GOLDEN, "membership_tiny.json")))
    for case in gold["cases"]:
        spec = (A.Strips(case["num_strips"], p=case.get("p"), halo_rows=case.get("halo_rows"))
                if case["mode"] == "strips"
                else A.Windows(case["tile_h"], case["tile_w"], case["halo_h"], case["halo_w"], case.get("text_tokens", 0)))
        tiles = list(A.iter_tiles(case["H"], case["W"], spec))
        sets = A.attended_sets(case["H"], case["W"], spec)
        for exp, (qt, ft, st) in zip(case["tiles"], tiles):
            if sorted(ft.tolist()) != exp["fresh"] or sorted(st.tolist()) != sorted(exp["stale"]):
                return False
            for t in exp["queries"]:
                if sets[t] != (exp["fresh"], sorted(exp["stale"])):
                    return False
    return True


def test_unmutated_passes():
    assert _golden_membership_holds()


def test_floor_instead_of_ceil_is_caught(monkeypatch):
    def bad(H, spec):
        if spec.halo_rows is not None:
            return spec.halo_rows
        return int(math.floor(spec.p * (H // spec.num_strips)))
    monkeypatch.setattr(A, "halo_rows", bad)
    assert not _golden_membership_holds()


def test_far_side_halo_is_caught(monkeypatch):
    """Halo taken from the far end of each neighbour strip instead of the near end."""
    def bad(H, W, spec, q_rc, k_rc):
        if not isinstance(spec, A.Strips):
            return False
        s, h = A.strip_height(H, spec), A.halo_rows(H, spec)
        i, kr = q_rc[0] // s, k_rc[0]
        return ((i - 1) * s <= kr < (i - 1) * s + h and i > 0) or ((i + 2) * s - h <= kr < (i + 2) * s and i + 1 < spec.num_strips)
    monkeypatch.setattr(A, "pair_in_stale", bad)
    assert not _golden_membership_holds()


def test_window_shifted_not_clipped_is_caught(monkeypatch):
    orig = A.pair_in_fresh

    def bad(H, W, spec, q_rc, k_rc):
        if isinstance(spec, A.Strips):
            return orig(H, W, spec, q_rc, k_rc)
        th, tw, eh, ew = spec.tile_h, spec.tile_w, spec.halo_h, spec.halo_w
        ti, tj = q_rc[0] // th, q_rc[1] // tw
        r0 = min(max(0, ti * th - eh), H - (th + 2 * eh))
        c0 = min(max(0, tj * tw - ew), W - (tw + 2 * ew))
        return r0 <= k_rc[0] < r0 + th + 2 * eh and c0 <= k_rc[1] < c0 + tw + 2 * ew
    monkeypatch.setattr(A, "pair_in_fresh", bad)
    assert not _golden_membership_holds()


def test_stale_values_swapped_for_fresh_is_caught(monkeypatch):
    """Reading the fresh V for stale keys must break the one-hot probe."""
    orig = A.attention_tier1

    def bad(q, k, v, k_stale, v_stale, *a, **kw):
        return orig(q, k, v, k_stale, v, *a, **kw)
    monkeypatch.setattr(A, "attention_tier1", bad)
    H = W = 4
    N = 16
    rng = np.random.default_rng(0)
    q, kk = rng.standard_normal((1, N, 1, 6)), rng.standard_normal((1, N, 1, 6))
    vf = np.concatenate([np.eye(N), np.zeros((N, N))], 1)[None, :, None, :]
    vs = np.concatenate([np.zeros((N, N)), np.eye(N)], 1)[None, :, None, :]
    spec = A.Strips(2, halo_rows=1)
    P = A.attention_tier1(q, kk, vf, kk, vs, H, W, spec)[0, :, 0, :]
    sets = A.attended_sets(H, W, spec)
    ok = True
    for t in range(N):
        allowed = np.zeros(2 * N, dtype=bool)
        allowed[sets[t][0]] = True
        allowed[[N + u for u in sets[t][1]]] = True
        ok &= bool(np.all(P[t, ~allowed] == 0.0) and np.all(P[t, allowed] > 0.0))
    assert not ok


def test_wrong_scale_is_caught(monkeypatch):
    import torch
    monkeypatch.setattr(A, "default_scale", lambda d: 1.0 / d)
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 12, 2, 8)) for _ in range(3))
    got = A.attention_tier1(q, k, v, None, None, 3, 4, A.Windows(3, 4, 0, 0))
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).permute(0, 2, 1, 3).numpy()
    assert not np.allclose(got, ref, atol=1e-6)


def test_zero_padded_border_is_caught(monkeypatch):
    import scipy.ndimage as ndi

    def bad(i, n):
        return np.clip(i, 0, n - 1)  # edge-repeat instead of mirror
    monkeypatch.setattr(G, "reflect101", bad)
    x = np.random.default_rng(2).standard_normal((1, 30, 30))
    ref = ndi.gaussian_filter(x, sigma=4.0, mode="mirror", truncate=3.0, axes=(1, 2))
    assert not np.allclose(G.lowpass(x, 4.0), ref, atol=1e-6)


def test_text_keys_dropped_for_map_queries_is_caught(monkeypatch):
    """Map queries attend to their window only (text keys left out)."""
    orig = A.iter_tiles

    def bad(H, W, spec):
        T = A.text_tokens(spec)
        for qt, ft, st in orig(H, W, spec):
            if T and qt.min() >= T:
                ft = ft[ft >= T]
            yield qt, ft, st
    monkeypatch.setattr(A, "iter_tiles", bad)
    assert not _golden_membership_holds()


def test_text_queries_windowed_is_caught(monkeypatch):
    """Text queries attend to the text tokens only."""
    orig = A.iter_tiles

    def bad(H, W, spec):
        T = A.text_tokens(spec)
        for qt, ft, st in orig(H, W, spec):
            if T and qt.max() < T:
                ft = ft[ft < T]
            yield qt, ft, st
    monkeypatch.setattr(A, "iter_tiles", bad)
    assert not _golden_membership_holds()


def test_map_tokens_not_offset_is_caught(monkeypatch):
    """Map tokens indexed from 0 (as if no text tokens were stored before them)."""
    orig = A.iter_tiles

    def bad(H, W, spec):
        T = A.text_tokens(spec)
        for qt, ft, st in orig(H, W, spec):
            if T and qt.min() >= T:
                qt = qt - T
                ft = np.concatenate([ft[ft >= T] - T, ft[ft < T]])
            yield qt, ft, st
    monkeypatch.setattr(A, "iter_tiles", bad)
    assert not _golden_membership_holds()
