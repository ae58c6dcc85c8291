// Internal declarations shared by the host API and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "npa.h"

#define NPA_HD __host__ __device__ __forceinline__

namespace npa {

// Division by a divisor that is fixed for a whole launch, as a multiply-high,
// an add and a shift (division by invariant integers, Granlund and Montgomery,
// PLDI 1994): for 1 <= d < 2^31 let s = ceil(log2 d) and m = ceil(2^(32+s) / d),
// which lies in [2^32, 2^33); then n / d = floor(n * m / 2^(32+s)) for every
// 0 <= n < 2^31, because m * d - 2^(32+s) < d <= 2^s.  m - 2^32 is stored, so
// floor(n * m / 2^32) = mulhi(n, m - 2^32) + n, which stays below 2^32.  In the
// kernels the divisors are uniform: three scalar instructions instead of the
// ~30 of a general 32-bit division (with a round trip through the vector unit).
struct DivBy {
  uint32_t d, m, s;
  static DivBy of(int32_t divisor) {  // host: 1 <= divisor < 2^31
    DivBy r{(uint32_t)divisor, 0, 0};
    while ((1u << r.s) < r.d) ++r.s;
    r.m = (uint32_t)((((uint64_t)1 << (32 + r.s)) + r.d - 1) / r.d - ((uint64_t)1 << 32));
    return r;
  }
  NPA_HD int32_t div(int32_t n) const {  // 0 <= n < 2^31
    const uint32_t u = (uint32_t)n;
    return (int32_t)(((uint32_t)(((uint64_t)u * m) >> 32) + u) >> s);
  }
  NPA_HD int32_t mod(int32_t n) const { return n - div(n) * (int32_t)d; }
};

// Validated plan parameters.  Tiles are enumerated in closed form from these,
// on the host by the planner and on the device by each workgroup, so no tile
// table ever lives in device memory.
struct Geo {
  int32_t mode;      // npa_mode_t
  int32_t H, W;      // token map
  int32_t s, h;      // strips: strip height, halo rows
  int32_t th, tw;    // window: query tile
  int32_t eh, ew;    // window: halo
  int32_t tiles_x;   // window: tiles per map row
  int32_t T;         // window: text tokens stored before the map's tokens
  int32_t n_img;     // map tiles; the text tile (T > 0) is tile n_img
  int32_t n_tiles;   // n_img, plus one when T > 0
  DivBy by_tiles_x;  // window: division by tiles_x (set by set_divisors)
};

// A run of tokens: `rows` runs of `row_len` tokens, first at `start`, `pitch` apart.
struct Run {
  int32_t start, row_len, rows, pitch;
  NPA_HD int32_t count() const { return row_len * rows; }
};

// The query run of a tile and its key runs (fresh first, then up to two stale).
struct TileRuns {
  Run q;
  Run k[3];
  int32_t src[3];
  int32_t nk[3];  // key count per run (0 for an absent run)
};

NPA_HD int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }
NPA_HD int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }

// Partially conditioned attention (strips): strip i attends to its own rows
// fresh, plus the h rows nearest to it above and below, stale.
// Neighbourhood patch attention (window): tile (ti, tj) attends to its window
// grown by (eh, ew) and clipped at the map border, fresh.  With T text tokens
// (stored first; map token t at T + t) every map tile also attends to the text
// tokens (run 1), and the text tile's T queries attend to every stored token.
NPA_HD TileRuns tile_runs(const Geo& g, int32_t tile) {
  TileRuns t;
  if (g.mode == NPA_MODE_STRIPS) {
    const int32_t r0 = tile * g.s, r1 = r0 + g.s;
    const int32_t a0 = imax(0, r0 - g.h), b1 = imin(g.H, r1 + g.h);
    t.q = Run{r0 * g.W, g.s * g.W, 1, g.s * g.W};
    t.k[0] = t.q;
    t.src[0] = 0;
    t.k[1] = Run{a0 * g.W, (r0 - a0) * g.W, 1, (r0 - a0) * g.W};
    t.src[1] = 1;
    t.k[2] = Run{r1 * g.W, (b1 - r1) * g.W, 1, (b1 - r1) * g.W};
    t.src[2] = 1;
  } else if (tile >= g.n_img) {
    const int32_t all = g.T + g.H * g.W;
    t.q = Run{0, g.T, 1, g.T};
    t.k[0] = Run{0, all, 1, all};
    t.src[0] = 0;
    t.k[1] = Run{0, 0, 0, 0};
    t.src[1] = 0;
    t.k[2] = Run{0, 0, 0, 0};
    t.src[2] = 0;
  } else {
    const int32_t ti = g.by_tiles_x.div(tile), tj = tile - ti * g.tiles_x;
    const int32_t r0 = imax(0, ti * g.th - g.eh), r1 = imin(g.H, (ti + 1) * g.th + g.eh);
    const int32_t c0 = imax(0, tj * g.tw - g.ew), c1 = imin(g.W, (tj + 1) * g.tw + g.ew);
    t.q = Run{g.T + ti * g.th * g.W + tj * g.tw, g.tw, g.th, g.W};
    t.k[0] = Run{g.T + r0 * g.W + c0, c1 - c0, r1 - r0, g.W};
    t.src[0] = 0;
    t.k[1] = Run{0, g.T, 1, g.T};
    t.src[1] = 0;
    t.k[2] = Run{0, 0, 0, 0};
    t.src[2] = 0;
  }
  for (int i = 0; i < 3; ++i) t.nk[i] = t.k[i].count();
  return t;
}

// Queries of each map tile (strips or windows; the text tile has g.T).
NPA_HD int32_t tile_queries(const Geo& g) {
  return g.mode == NPA_MODE_STRIPS ? g.s * g.W : g.th * g.tw;
}

// Arguments of the attention kernels (passed by value).
struct AttnArgs {
  const void* q;
  const void* kf;
  const void* vf;
  const void* ks;
  const void* vs;
  void* o;
  int64_t sb, sn, sh;  // strides in elements
  int32_t B, Hh;
  Geo g;
  int32_t qblocks;  // query blocks per map tile
  int32_t nblocks;  // grid size
  int32_t text_qblocks;  // query blocks of the text tile (0 without text tokens)
  int32_t text_blocks;   // B * Hh * text_qblocks: the grid's first blocks
  float scale;      // softmax scale
  float c;          // scale * log2(e)
  uint32_t range_bytes;  // bytes spanned by one (batch, head) slice: ((N-1)*sn + d) * esize
  int32_t partial;       // some key run is not a multiple of 64 keys
  // division by qblocks, text_qblocks (1 when 0), n_img, Hh and B * Hh (set by set_divisors)
  DivBy by_qblocks, by_text_qblocks, by_n_img, by_hh, by_bh;
  int32_t largest_first;  // window tiles listed interior, edge, corner (see decode_block)
  DivBy by_inner_x;       // division by tiles_x - 2
};

// The division constants of a and a.g, from their plain fields (host side).
inline void set_divisors(AttnArgs& a) {
  auto pos = [](int32_t v) { return v > 0 ? v : 1; };
  a.g.by_tiles_x = DivBy::of(pos(a.g.tiles_x));
  a.by_qblocks = DivBy::of(pos(a.qblocks));
  a.by_text_qblocks = DivBy::of(pos(a.text_qblocks));
  a.by_n_img = DivBy::of(pos(a.g.n_img));
  a.by_hh = DivBy::of(pos(a.Hh));
  a.by_bh = DivBy::of(pos(a.B * a.Hh));
  a.by_inner_x = DivBy::of(pos(a.g.tiles_x - 2));
}

// Window tile of rank r when the tiles of a head are listed interior first, then
// edge tiles, then the four corners (tiles_x, tiles_y >= 3): the windows clipped
// by the border (fewer keys) come last.
template <class A>
NPA_HD int32_t tile_by_class(const A& a, int32_t r) {
  const int32_t tx = a.g.tiles_x, ty = a.g.n_img / tx, ix = tx - 2, iy = ty - 2;
  const int32_t n0 = ix * iy, n1 = 2 * ix + 2 * iy;
  int32_t ti, tj;
  if (r < n0) {
    ti = a.by_inner_x.div(r);
    tj = 1 + (r - ti * ix);
    ti += 1;
  } else if (r < n0 + n1) {
    // edge tiles in raster order: top row, then the left and right ends of
    // each interior row, then the bottom row (neighbours stay together)
    const int32_t e = r - n0;
    if (e < ix) {
      ti = 0, tj = 1 + e;
    } else if (e < ix + 2 * iy) {
      const int32_t k = e - ix;
      ti = 1 + (k >> 1), tj = (k & 1) ? tx - 1 : 0;
    } else {
      ti = ty - 1, tj = 1 + (e - ix - 2 * iy);
    }
  } else {
    const int32_t k = r - n0 - n1;
    ti = (k >> 1) ? ty - 1 : 0;
    tj = (k & 1) ? tx - 1 : 0;
  }
  return ti * tx + tj;
}

// Which (query block, tile, head, batch) workgroup i of the grid computes.
// The text tile's workgroups come first: each one walks every stored token,
// many times the keys of a map tile, so they are started first (spread over
// the XCDs by the hardware's round-robin) rather than left as a tail.  The map
// tiles follow as units of (tile, batch, head), each unit's query blocks
// consecutive.  Workgroups are dealt to the 8 XCDs round-robin by id; with
// `remap` the ids are regrouped so that all query blocks of a unit run on one
// XCD (they share the unit's K/V through that XCD's L2):
//   windows: each XCD runs one contiguous range of units, so neighbouring
//            tiles of a head (whose windows overlap) share that L2 too; with
//            `largest_first` (set by the host for windows at most 2.25x their
//            tile's area, where neighbours share little) a head's tiles are
//            listed interior, edge, corner, so each XCD ends on short units;
//   strips:  units are listed interior strips first, border strips (one
//            stale halo, fewer keys) last, and dealt round-robin over the
//            XCDs; each XCD then runs its longest units first, which keeps the
//            end of the launch even.
struct BlockCoord {
  int32_t qb, tile, head, b;
};

NPA_HD int32_t xcd_remap(int32_t i, int32_t n) {
  const int32_t per = n >> 3, rem = n & 7;
  const int32_t x = i & 7, k = i >> 3;
  return (x < rem) ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// Strip of rank r with the border strips (0 and n-1) listed last; a
// bijection on 0 .. n-1.
NPA_HD int32_t border_last(int32_t r, int32_t n) {
  return n < 3 ? r : (r < n - 2 ? r + 1 : (r == n - 2 ? 0 : n - 1));
}

NPA_HD BlockCoord decode_block(const AttnArgs& a, int32_t i, bool remap) {
  BlockCoord c;
  int32_t rest;
  const int32_t j = i - a.text_blocks;
  if (i < a.text_blocks) {
    rest = a.by_text_qblocks.div(i);
    c.qb = i - rest * a.text_qblocks;
    c.tile = a.g.n_img;
  } else if (!remap || a.g.mode != NPA_MODE_STRIPS) {
    const int32_t jj = remap ? xcd_remap(j, a.nblocks - a.text_blocks) : j;
    rest = a.by_qblocks.div(jj);
    c.qb = jj - rest * a.qblocks;
    const int32_t r2 = a.by_n_img.div(rest);
    c.tile = rest - r2 * a.g.n_img;
    if (remap && a.largest_first) c.tile = tile_by_class(a, c.tile);
    rest = r2;
  } else {
    // units (rank, batch * heads + head), rank slowest; the first 8*floor(U/8)
    // units are dealt round-robin over the XCDs, the rest (the smallest) in order
    const int32_t units = a.by_qblocks.div(a.nblocks - a.text_blocks);
    const int32_t dealt = (units & ~7) * a.qblocks;
    int32_t unit;
    if (j < dealt) {
      const int32_t k = j >> 3;
      const int32_t kq = a.by_qblocks.div(k);
      unit = kq * 8 + (j & 7);
      c.qb = k - kq * a.qblocks;
    } else {
      const int32_t jq = a.by_qblocks.div(j - dealt);
      unit = (units & ~7) + jq;
      c.qb = (j - dealt) - jq * a.qblocks;
    }
    const int32_t rank = a.by_bh.div(unit);
    c.tile = border_last(rank, a.g.n_img);
    rest = unit - rank * (a.B * a.Hh);
  }
  c.b = a.by_hh.div(rest);
  c.head = rest - c.b * a.Hh;
  return c;
}

// Arguments of the structure-guidance kernel.
constexpr int kSgMaxRadius = 24;  // sigma <= 8; keeps the LDS tile under 64 KiB
struct SgArgs {
  const float* x;
  const float* ref;
  float* out;
  int32_t planes, H, W, R;
  float w;
  float taps[2 * kSgMaxRadius + 1];
};

// Launchers (return the HIP error of the launch).
// bf16: `small` selects the small-launch workgroup shape (see attn_bf16.hip);
// f32: `split` selects the key-split shape (see attn_f32.hip).
hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool small, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, bool split, hipStream_t st);
int attn_bf16_block_m(int head_dim, bool small);  // queries per workgroup, 0 if unsupported
int attn_bf16_per_cu(int head_dim, bool small);   // workgroups resident per CU
int attn_f32_block_m(int head_dim, bool split);   // queries per workgroup, 0 if unsupported
hipError_t launch_sg_blend(const SgArgs& a, hipStream_t st);
hipError_t launch_asg_blend(const float* eps, const float* ref, const float* mask, float* out,
                            int64_t count, float w, hipStream_t st);

}  // namespace npa
