"""fp64 reference for partially conditioned / neighbourhood patch attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed, for every batch item b, head j and query token q = (r, c)
of an H x W token map flattened row-major (t = r*W + c):

    S(q) = F(q) u T(q)   (F: keys read from the fresh K/V, T: from the stale K/V;
                          a token index present in both is two distinct keys)
    l_k  = scale * <Q[b,q,j,:], K_src(k)[b,k,j,:]>
    O[b,q,j,:] = sum_{k in S(q)} softmax_k(l) * V_src(k)[b,k,j,:]

Membership (the two methods):

* Strips -- "Partially Conditioned Patch Parallelism ..." (pith.science),
  "What carries the argument" / "Core claim": the map is cut into n horizontal
  strips of s = H/n rows.  A query in strip i attends to the fresh rows of its
  own strip and to the stale rows of its neighbours nearest to it: the last h
  rows above the strip and the first h rows below it, h = the p-fraction of the
  neighbour's height rounded up to whole rows.  Readings where the page is
  silent: no wrap-around at the image border (the first and last strip get one
  halo); a halo longer than one strip keeps extending into further strips, still
  stale; the strip's own stale rows are never read.
* Windows -- "ScaleDiff ..." (atlas.scime.ai), "Approach": the map is cut into
  non-overlapping th x tw query tiles; a query in tile (ti, tj) attends to the
  fresh keys of the rectangle grown by halo_h rows and halo_w columns on each
  side, clipped at the image border (the window shrinks; it is not shifted).
* Windows with text tokens (FLUX's joint attention; the ScaleDiff page applies
  NPA to FLUX but does not say how the prompt's tokens take part -- reading:
  they are global).  The tensors hold T text tokens first, then the map's
  tokens (map token t at index T + t).  A map query attends to its window and
  to all T text tokens; a text query attends to every token, text and map.

Two tiers that share no code with each other beyond the spec objects:
  tier 0 -- explicit Python loops over (q, k) with the per-pair predicate
            (tiny maps only);
  tier 1 -- per tile: select the attended tokens with a vectorised predicate
            over the whole map, then dense fp64 matmul / stable softmax /
            matmul.  Runs every workload in full; can restrict to sampled
            query tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, Iterator, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Specs
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Strips:
    """n horizontal strips; halo given as a fraction p or as whole rows."""

    num_strips: int
    p: Optional[float] = None
    halo_rows: Optional[int] = None


@dataclass(frozen=True)
class Windows:
    """Non-overlapping tile_h x tile_w query tiles with a (halo_h, halo_w) K/V halo;
    text_tokens global tokens stored before the map's tokens."""

    tile_h: int
    tile_w: int
    halo_h: int
    halo_w: int
    text_tokens: int = 0


def text_tokens(spec) -> int:
    """Global text tokens stored before the map's tokens (0 for strips)."""
    return spec.text_tokens if isinstance(spec, Windows) else 0


def strip_height(H: int, spec: Strips) -> int:
    if spec.num_strips <= 0 or H % spec.num_strips != 0:
        raise ValueError("the map height must split into equal strips")
    return H // spec.num_strips


def halo_rows(H: int, spec: Strips) -> int:
    """Stale rows taken from each neighbour.

    The PCPP page defines p as the fraction of the neighbour patch's height
    that joins the local key/value set.  Reading: round p*s up to whole rows.
    A product that is an integer up to floating-point rounding (0.7*10, or p
    handed over as float32) must not gain a row, so p*s is lowered by a
    tolerance of 1e-6*s before the ceiling.
    """
    if spec.halo_rows is not None:
        if spec.halo_rows < 0:
            raise ValueError("halo_rows must be >= 0")
        return int(spec.halo_rows)
    if spec.p is None or not (0.0 <= spec.p):
        raise ValueError("p must be given and >= 0")
    s = strip_height(H, spec)
    return max(0, math.ceil(spec.p * s - 1e-6 * s))


def default_scale(d: int) -> float:
    """Scaled dot-product attention: 1/sqrt(head_dim)."""
    return 1.0 / math.sqrt(d)


# --------------------------------------------------------------------------
# Per-pair predicates (tier 0).  Coordinates are (row, col) of the token map.
# --------------------------------------------------------------------------
def pair_in_fresh(H: int, W: int, spec, q_rc: Tuple[int, int], k_rc: Tuple[int, int]) -> bool:
    qr, qc = q_rc
    kr, kc = k_rc
    if isinstance(spec, Strips):
        s = strip_height(H, spec)
        return kr // s == qr // s
    ti, tj = qr // spec.tile_h, qc // spec.tile_w
    r_lo = max(0, ti * spec.tile_h - spec.halo_h)
    r_hi = min(H, (ti + 1) * spec.tile_h + spec.halo_h)
    c_lo = max(0, tj * spec.tile_w - spec.halo_w)
    c_hi = min(W, (tj + 1) * spec.tile_w + spec.halo_w)
    return r_lo <= kr < r_hi and c_lo <= kc < c_hi


def pair_in_stale(H: int, W: int, spec, q_rc: Tuple[int, int], k_rc: Tuple[int, int]) -> bool:
    if not isinstance(spec, Strips):
        return False
    qr, _ = q_rc
    kr, _ = k_rc
    s = strip_height(H, spec)
    h = halo_rows(H, spec)
    i = qr // s
    above = max(0, i * s - h) <= kr < i * s
    below = (i + 1) * s <= kr < min(H, (i + 1) * s + h)
    return above or below


def attended_sets(H: int, W: int, spec) -> list:
    """For every stored token (text tokens first, then the map row-major):
    (sorted fresh key indices, sorted stale key indices)."""
    T = text_tokens(spec)
    out = []
    for t in range(T):  # a text query sees everything
        out.append((list(range(T + H * W)), []))
    for t in range(H * W):
        q_rc = divmod(t, W)
        fr = [T + k for k in range(H * W) if pair_in_fresh(H, W, spec, q_rc, divmod(k, W))]
        st = [T + k for k in range(H * W) if pair_in_stale(H, W, spec, q_rc, divmod(k, W))]
        out.append((list(range(T)) + fr, st))
    return out


def attention_tier0(q, k, v, k_stale, v_stale, H: int, W: int, spec, scale: Optional[float] = None,
                    query_tokens: Optional[Sequence[int]] = None, heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Brute force: Python loops over every (query, key, channel).

    query_tokens / heads -- if given, only those queries / (batch, head) pairs
    are computed; the other outputs stay NaN (a bounded sample for timing)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, Hh, d = q.shape
    assert N == text_tokens(spec) + H * W
    scale = default_scale(d) if scale is None else scale
    if k_stale is not None:
        k_stale = np.asarray(k_stale, dtype=np.float64)
        v_stale = np.asarray(v_stale, dtype=np.float64)
    sample = query_tokens is not None or heads is not None
    out = np.full((B, N, Hh, v.shape[-1]), np.nan) if sample else np.zeros((B, N, Hh, v.shape[-1]))
    sets = attended_sets(H, W, spec)
    bh = list(heads) if heads is not None else [(b, j) for b in range(B) for j in range(Hh)]
    qs = list(query_tokens) if query_tokens is not None else range(N)
    for b, j in bh:
        for t in qs:
            fresh, stale = sets[t]
            keys = [(k[b, kk, j], v[b, kk, j]) for kk in fresh]
            keys += [(k_stale[b, kk, j], v_stale[b, kk, j]) for kk in stale]
            logits = []
            for kvec, _ in keys:
                acc = 0.0
                for e in range(d):
                    acc += q[b, t, j, e] * kvec[e]
                logits.append(scale * acc)
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            z = sum(w)
            for e in range(v.shape[-1]):
                acc = 0.0
                for wk, (_, vvec) in zip(w, keys):
                    acc += wk * vvec[e]
                out[b, t, j, e] = acc / z
    return out


# --------------------------------------------------------------------------
# Tiles and vectorised membership (tier 1)
# --------------------------------------------------------------------------
def iter_tiles(H: int, W: int, spec) -> Iterator[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Yield (query tokens, fresh key tokens, stale key tokens) per query tile.

    Every token of the map belongs to exactly one tile; all queries of a tile
    share one key set.  Selection is by predicate over all H*W tokens.  With
    text tokens, indices are into the stored sequence (text first) and the
    text queries form one more tile, last.
    """
    tok = np.arange(H * W)
    rows, cols = tok // W, tok % W
    if isinstance(spec, Strips):
        s = strip_height(H, spec)
        h = halo_rows(H, spec)
        for i in range(spec.num_strips):
            qsel = rows // s == i
            fsel = rows // s == i
            ssel = ((rows >= max(0, i * s - h)) & (rows < i * s)) | (
                (rows >= (i + 1) * s) & (rows < min(H, (i + 1) * s + h))
            )
            yield tok[qsel], tok[fsel], tok[ssel]
        return
    th, tw, eh, ew = spec.tile_h, spec.tile_w, spec.halo_h, spec.halo_w
    T = spec.text_tokens
    if H % th or W % tw:
        raise ValueError("query tiles must divide the map")
    text = np.arange(T)
    empty = np.zeros(0, dtype=tok.dtype)
    for ti in range(H // th):
        for tj in range(W // tw):
            qsel = (rows // th == ti) & (cols // tw == tj)
            r_lo, r_hi = max(0, ti * th - eh), min(H, (ti + 1) * th + eh)
            c_lo, c_hi = max(0, tj * tw - ew), min(W, (tj + 1) * tw + ew)
            fsel = (rows >= r_lo) & (rows < r_hi) & (cols >= c_lo) & (cols < c_hi)
            yield T + tok[qsel], np.concatenate([T + tok[fsel], text]), empty
    if T:
        yield text, np.arange(T + H * W), empty


def useful_pairs(H: int, W: int, spec) -> int:
    """Number of attended (query, key) pairs per (batch, head): sum_q |S(q)|."""
    return int(sum(len(qt) * (len(ft) + len(st)) for qt, ft, st in iter_tiles(H, W, spec)))


def useful_flops(B: int, Hh: int, d: int, H: int, W: int, spec) -> int:
    """4*d flops per attended pair (QK^T and PV multiply-adds), all batches and heads."""
    return 4 * d * useful_pairs(H, W, spec) * B * Hh


def _softmax_attend(qt: np.ndarray, kt: np.ndarray, vt: np.ndarray, scale: float) -> np.ndarray:
    logits = scale * (qt @ kt.T)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ vt


def attention_tier1(
    q,
    k,
    v,
    k_stale,
    v_stale,
    H: int,
    W: int,
    spec,
    scale: Optional[float] = None,
    query_tokens: Optional[Sequence[int]] = None,
    heads: Optional[Iterable[Tuple[int, int]]] = None,
    chunk: int = 2048,
):
    """Per-tile gather + dense fp64 attention.

    query_tokens -- if given, only these query tokens are computed (others
                    stay NaN in the result); the sampled form for full sizes.
    heads        -- if given, only these (batch, head) pairs are computed.
    Returns an fp64 array of shape [B, N, Hh, dv].
    """
    B, N, Hh, d = q.shape
    assert N == text_tokens(spec) + H * W
    scale = default_scale(d) if scale is None else scale
    out = np.full((B, N, Hh, v.shape[-1]), np.nan)
    want = None
    if query_tokens is not None:
        want = np.zeros(N, dtype=bool)
        want[np.asarray(query_tokens, dtype=np.int64)] = True
    bh = list(heads) if heads is not None else [(b, j) for b in range(B) for j in range(Hh)]
    for qt, ft, st in iter_tiles(H, W, spec):
        if want is not None:
            qt = qt[want[qt]]
        if len(qt) == 0:
            continue
        for b, j in bh:
            kt = np.asarray(k[b, ft, j], dtype=np.float64)
            vt = np.asarray(v[b, ft, j], dtype=np.float64)
            if len(st):
                kt = np.concatenate([kt, np.asarray(k_stale[b, st, j], dtype=np.float64)])
                vt = np.concatenate([vt, np.asarray(v_stale[b, st, j], dtype=np.float64)])
            for c0 in range(0, len(qt), chunk):
                qs = qt[c0 : c0 + chunk]
                out[b, qs, j] = _softmax_attend(np.asarray(q[b, qs, j], dtype=np.float64), kt, vt, scale)
    return out
