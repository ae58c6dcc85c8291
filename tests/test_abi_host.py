"""Host-side checks of the C-ABI library: symbols, struct layout, planner, validation.

No GPU needed: only host functions are called (the planner, useful-flop
accounting, and argument validation that fails before any launch).
"""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import attention as A
from partial_context_patch_amd import npa
from partial_context_patch_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "npa.h")


@pytest.fixture(scope="module")
def lib():
    return npa.load()


def test_every_declared_symbol_is_exported(lib):
    decl = set(re.findall(r"\b(npa_[a-z_0-9]+)\s*\(", open(HEADER).read()))
    assert decl == set(npa.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", npa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (npa_\w+)", out))
    assert decl <= exported
    for name in decl:
        assert hasattr(lib, name)


def test_struct_layout_matches_c():
    """Compile a probe against the header with gcc and compare sizes/offsets."""
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "npa.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\n", sizeof(npa_layout_t), offsetof(npa_layout_t, stride_b),
         offsetof(npa_layout_t, dtype), offsetof(npa_layout_t, scale), sizeof(npa_halo_t),
         sizeof(npa_segment_t), sizeof(npa_tile_desc_t));
  printf("%zu %zu %zu\n", offsetof(npa_halo_t, p), offsetof(npa_tile_desc_t, keys),
         offsetof(npa_halo_t, text_tokens));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I" + os.path.dirname(HEADER), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    L, H, S, T = npa.Layout, npa.Halo, npa.Segment, npa.TileDesc
    assert vals == [ctypes.sizeof(L), L.stride_b.offset, L.dtype.offset, L.scale.offset, ctypes.sizeof(H),
                    ctypes.sizeof(S), ctypes.sizeof(T), H.p.offset, T.keys.offset, H.text_tokens.offset]


def _oracle_spec(h: npa.Halo):
    if h.mode == npa.NPA_MODE_STRIPS:
        return A.Strips(h.num_strips, p=h.p if h.halo_rows < 0 else None,
                        halo_rows=h.halo_rows if h.halo_rows >= 0 else None)
    return A.Windows(h.tile_h, h.tile_w, h.halo_h, h.halo_w, h.text_tokens)


def _run_tokens(seg):
    return [seg["start"] + r * seg["pitch"] + c for r in range(seg["rows"]) for c in range(seg["row_len"])]


CASES = [
    (32, 32, dict(strips=4, p=0.3)),
    (64, 64, dict(strips=4, p=0.3)),
    (128, 128, dict(strips=8, p=0.8)),
    (24, 20, dict(strips=3, halo_rows=3)),
    (24, 20, dict(strips=3, halo_rows=20)),
    (24, 20, dict(strips=1, p=1.0)),
    (24, 20, dict(strips=6, p=0.0)),
    (30, 7, dict(strips=3, p=0.31)),
    (40, 36, dict(tile=(8, 12), halo=(5, 3))),
    (40, 36, dict(tile=(40, 36), halo=(0, 0))),
    (40, 36, dict(tile=(4, 4), halo=(50, 50))),
    (16, 16, dict(tile=(1, 1), halo=(1, 0))),
    (40, 36, dict(tile=(8, 12), halo=(5, 3), text_tokens=7)),
    (16, 16, dict(tile=(4, 4), halo=(2, 2), text_tokens=64)),
    (8, 8, dict(tile=(8, 8), halo=(0, 0), text_tokens=3)),
]


@pytest.mark.parametrize("H,W,kw", CASES)
def test_planner_matches_oracle(lib, H, W, kw):
    L = npa.make_layout(1, 1, 64, H, W)
    h = npa.make_halo(**kw)
    tiles, pairs = npa.plan(L, h)
    spec = _oracle_spec(h)
    ref = list(A.iter_tiles(H, W, spec))
    assert len(tiles) == len(ref)
    for t, (qt, ft, st) in zip(tiles, ref):
        assert sorted(_run_tokens(t["queries"])) == sorted(qt.tolist())
        fresh = [x for s in t["keys"] if s["src"] == 0 for x in _run_tokens(s)]
        stale = [x for s in t["keys"] if s["src"] == 1 for x in _run_tokens(s)]
        assert sorted(fresh) == sorted(ft.tolist())
        assert sorted(stale) == sorted(st.tolist())
    assert pairs == A.useful_pairs(H, W, spec)


@pytest.mark.parametrize("name", sorted(WL.ATTENTION_WORKLOADS))
def test_useful_flops_of_workloads(lib, name):
    w = WL.ATTENTION_WORKLOADS[name]
    L = npa.make_layout(w["batch"], w["heads"], w["head_dim"], w["map_h"], w["map_w"], dtype=w["dtype"])
    h = npa.make_halo(**WL.halo_kwargs(w))
    if w["mode"] == "strips":
        spec = A.Strips(w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
    else:
        spec = A.Windows(w["tile_h"], w["tile_w"], w["halo_h"], w["halo_w"], w.get("text_tokens", 0))
    assert npa.useful_flops(L, h) == A.useful_flops(w["batch"], w["heads"], w["head_dim"], w["map_h"], w["map_w"], spec)


@pytest.mark.parametrize("p", [0.3, 0.7, 0.31, 0.8, 0.25, 0.5, 1.0, 0.0, 0.123])
@pytest.mark.parametrize("H,n", [(32, 4), (40, 4), (128, 8), (30, 3), (100, 10)])
def test_halo_rows_from_p_matches_oracle(lib, p, H, n):
    L = npa.make_layout(1, 1, 64, H, 8)
    tiles, _ = npa.plan(L, npa.make_halo(strips=n, p=p))
    h_oracle = A.halo_rows(H, A.Strips(n, p=p))
    s = H // n
    # the middle strip (or the only one) shows the halo above it
    stale_rows = sum(seg["rows"] * seg["row_len"] for seg in tiles[n // 2]["keys"] if seg["src"] == 1) // 8
    expect = min(h_oracle, (n // 2) * s) + min(h_oracle, H - (n // 2 + 1) * s)
    assert stale_rows == expect


def _status(lib, L, h, q=1 << 20, k=2 << 20, v=3 << 20, ks=4 << 20, vs=5 << 20, out=6 << 20):
    return lib.npa_attn_fwd(q, k, v, ks, vs, ctypes.byref(L), ctypes.byref(h), out, None)


def test_validation_errors(lib):
    """Each bad argument is refused on the host, before any launch."""
    good_L = npa.make_layout(1, 2, 64, 32, 32)
    strips = npa.make_halo(strips=4, p=0.3)
    # shape errors
    bad = npa.make_halo(strips=5, p=0.3)
    assert _status(lib, good_L, bad) == npa.NPA_ERR_SHAPE
    assert b"divide" in lib.npa_last_error()
    assert _status(lib, good_L, npa.make_halo(strips=4, p=1.5)) == npa.NPA_ERR_SHAPE
    assert _status(lib, good_L, npa.make_halo(strips=4, p=-0.1)) == npa.NPA_ERR_SHAPE
    assert _status(lib, good_L, npa.make_halo(tile=(5, 8), halo=(1, 1))) == npa.NPA_ERR_SHAPE
    assert _status(lib, good_L, npa.make_halo(tile=(8, 8), halo=(-1, 1))) == npa.NPA_ERR_SHAPE
    neg = npa.make_layout(1, 2, 64, 32, 32)
    neg.batch = -1
    assert _status(lib, neg, strips) == npa.NPA_ERR_SHAPE
    neg = npa.make_layout(1, 2, 64, 32, 32)
    neg.heads = -2
    assert _status(lib, neg, strips) == npa.NPA_ERR_SHAPE
    huge = npa.make_layout(1, 1, 64, 8192, 4096)
    assert _status(lib, huge, npa.make_halo(tile=(64, 64), halo=(0, 0))) == npa.NPA_ERR_SHAPE
    # text tokens: window mode only, >= 0, within the token limit
    assert _status(lib, good_L, npa.make_halo(strips=4, p=0.3, text_tokens=8)) == npa.NPA_ERR_UNSUPPORTED
    assert _status(lib, good_L, npa.make_halo(tile=(8, 8), halo=(1, 1), text_tokens=-1)) == npa.NPA_ERR_SHAPE
    big = npa.make_layout(1, 1, 64, 4096, 4096)
    assert _status(lib, big, npa.make_halo(tile=(64, 64), halo=(0, 0), text_tokens=1)) == npa.NPA_ERR_SHAPE
    # unsupported head dim
    L96 = npa.make_layout(1, 2, 96, 32, 32)
    assert _status(lib, L96, strips) == npa.NPA_ERR_UNSUPPORTED
    # null / stale-missing / misaligned / aliasing / bad enum
    assert _status(lib, good_L, strips, q=0) == npa.NPA_ERR_INVALID_ARG
    assert _status(lib, good_L, strips, ks=0) == npa.NPA_ERR_INVALID_ARG
    assert b"stale" in lib.npa_last_error()
    assert _status(lib, good_L, strips, v=(3 << 20) + 8) == npa.NPA_ERR_INVALID_ARG
    assert _status(lib, good_L, strips, out=(1 << 20) + 4096) == npa.NPA_ERR_INVALID_ARG
    assert b"alias" in lib.npa_last_error()
    badmode = npa.make_halo(strips=4, p=0.3)
    badmode.mode = 7
    assert _status(lib, good_L, badmode) == npa.NPA_ERR_INVALID_ARG
    baddt = npa.make_layout(1, 2, 64, 32, 32)
    baddt.dtype = 9
    assert _status(lib, baddt, strips) == npa.NPA_ERR_INVALID_ARG
    odd = npa.make_layout(1, 2, 64, 32, 32, strides=(32 * 32 * 128, 128, 60))
    assert _status(lib, odd, strips) == npa.NPA_ERR_INVALID_ARG
    assert lib.npa_attn_fwd(None, None, None, None, None, None, None, None, None) == npa.NPA_ERR_INVALID_ARG
    # guidance kernels
    assert lib.npa_sg_blend(1 << 20, 2 << 20, 3 << 20, 1, 4, 8, 8, 0.5, 9.0, None) == npa.NPA_ERR_SHAPE
    assert lib.npa_sg_blend(1 << 20, 2 << 20, 1 << 20, 1, 4, 8, 8, 0.5, 4.0, None) == npa.NPA_ERR_INVALID_ARG
    assert lib.npa_sg_blend(0, 2 << 20, 3 << 20, 1, 4, 8, 8, 0.5, 4.0, None) == npa.NPA_ERR_INVALID_ARG
    assert lib.npa_asg_blend(1 << 20, 2 << 20, 3 << 20, 4 << 20, -1, 0.5, None) == npa.NPA_ERR_SHAPE
    assert lib.npa_asg_blend(1 << 20, 2 << 20, 3 << 20, 4 << 20, 0, 0.5, None) == npa.NPA_OK
    assert lib.npa_sg_blend(1 << 20, 2 << 20, 3 << 20, 1, 1, 1 << 30, 1 << 11, 0.5, 4.0, None) == npa.NPA_ERR_SHAPE


def test_layouts_that_map_rows_onto_each_other_are_refused(lib):
    """Q, K, V and out share one layout; one where two (batch, token, head)
    rows overlap would make the output race, so it is refused on the host."""
    strips = npa.make_halo(strips=4, p=0.3)
    N, Hh, d = 32 * 32, 2, 64
    fine = [
        (N * Hh * d, Hh * d, d),                  # [B, N, H, D]
        (N * Hh * d, d, N * d),                   # [B, H, N, D]
        (N * (Hh * d + 8) + 64, Hh * d + 8, d + 8),  # padded rows
        (d, 2 * Hh * d, 2 * d),                   # batch innermost, interleaved
    ]
    for st in fine:
        L = npa.make_layout(2, Hh, d, 32, 32, strides=st)
        # passes the layout check; stops later, at the aliasing check of
        # these fake pointers (the extents overlap)
        _status(lib, L, strips, q=1 << 30, k=2 << 30, v=3 << 30, ks=4 << 30, vs=5 << 30, out=6 << 30)
        assert b"overlapping memory" not in lib.npa_last_error(), st
    bad = [
        (0, Hh * d, d),                           # batches on top of each other
        (N * Hh * d, Hh * d, 0),                  # heads on top of each other
        (N * Hh * d, 8, d),                       # tokens overlap
        (N * Hh * d, Hh * d, 32),                 # heads half overlap
        (Hh * d, Hh * d, d),                      # batch stride equals the token stride
    ]
    for st in bad:
        L = npa.make_layout(2, Hh, d, 32, 32, strides=st)
        assert _status(lib, L, strips) == npa.NPA_ERR_INVALID_ARG, st
        assert b"overlapping memory" in lib.npa_last_error(), st
    # a dimension of one index may have any stride
    L = npa.make_layout(1, 1, d, 32, 32, strides=(0, d, 0))
    _status(lib, L, strips)
    assert b"overlapping memory" not in lib.npa_last_error()


def test_asg_out_is_an_input_or_apart(lib):
    """The element-wise ASG update may write over an input, but not over a
    shifted copy of one."""
    n = 1024
    base = 1 << 30
    eps, ref, mask, out = base, base + (1 << 20), base + (2 << 20), base + (3 << 20)
    for o in (eps, ref, mask):
        assert lib.npa_asg_blend(eps, ref, mask, o, 0, 0.5, None) == npa.NPA_OK
    for o in (eps + 16, ref - 16, mask + 4 * n - 16):
        assert lib.npa_asg_blend(eps, ref, mask, o, n, 0.5, None) == npa.NPA_ERR_INVALID_ARG
        assert b"overlap" in lib.npa_last_error()
    assert lib.npa_asg_blend(eps, ref, mask, out, 1 << 41, 0.5, None) == npa.NPA_ERR_SHAPE


def test_empty_calls_are_validated_no_ops(lib):
    """batch = 0 or heads = 0 (and an SG latent with n*c = 0) computes nothing:
    NPA_OK without touching any pointer (NULL allowed) and without a launch --
    but the rest of the arguments are still checked first."""
    strips = npa.make_halo(strips=4, p=0.3)
    for field in ("batch", "heads"):
        L = npa.make_layout(1, 2, 64, 32, 32)
        setattr(L, field, 0)
        assert lib.npa_attn_fwd(None, None, None, None, None, ctypes.byref(L), ctypes.byref(strips), None,
                                None) == npa.NPA_OK
        assert lib.npa_useful_flops(ctypes.byref(L), ctypes.byref(strips)) == 0
        # still validated: a strip count that does not divide the map, an unsupported head size
        assert _status(lib, L, npa.make_halo(strips=5, p=0.3)) == npa.NPA_ERR_SHAPE
        L96 = npa.make_layout(1, 2, 96, 32, 32)
        setattr(L96, field, 0)
        assert _status(lib, L96, strips) == npa.NPA_ERR_UNSUPPORTED
    for n, c in ((0, 4), (1, 0)):
        assert lib.npa_sg_blend(None, None, None, n, c, 8, 8, 0.5, 4.0, None) == npa.NPA_OK
    assert lib.npa_sg_blend(None, None, None, 0, 4, 8, 8, 0.5, 9.0, None) == npa.NPA_ERR_SHAPE
    assert lib.npa_sg_blend(None, None, None, -1, 4, 8, 8, 0.5, 4.0, None) == npa.NPA_ERR_SHAPE


def test_window_mode_needs_no_stale(lib):
    """A plan without stale rows must not demand stale pointers (checked via the planner)."""
    L = npa.make_layout(1, 2, 64, 32, 32)
    tiles, _ = npa.plan(L, npa.make_halo(tile=(8, 8), halo=(4, 4)))
    assert all(s["src"] == 0 for t in tiles for s in t["keys"])
    tiles, _ = npa.plan(L, npa.make_halo(strips=4, p=0.0))
    assert all(s["src"] == 0 for t in tiles for s in t["keys"])
    # text tokens are fresh keys: a joint plan needs no stale pointers either
    Lj = npa.make_layout(1, 2, 64, 32, 32)
    hj = npa.make_halo(tile=(8, 8), halo=(4, 4), text_tokens=16)
    tiles, _ = npa.plan(Lj, hj)
    assert all(s["src"] == 0 for t in tiles for s in t["keys"])


def test_last_error_is_per_thread(lib):
    """npa_last_error() keeps one message per host thread: two threads failing
    in different ways at the same time each read back their own message."""
    import threading

    L = npa.make_layout(1, 2, 64, 32, 32)
    kinds = {
        "shape": (npa.make_halo(strips=5, p=0.3), {}, npa.NPA_ERR_SHAPE, b"divide"),
        "alias": (npa.make_halo(strips=4, p=0.3), {"out": (1 << 20) + 4096}, npa.NPA_ERR_INVALID_ARG, b"alias"),
    }
    start = threading.Barrier(2)
    bad = []

    def run(kind):
        halo, kw, status, word = kinds[kind]
        start.wait()
        for _ in range(2000):
            if _status(lib, L, halo, **kw) != status or word not in lib.npa_last_error():
                bad.append(kind)
                return

    threads = [threading.Thread(target=run, args=(k,)) for k in kinds]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad

