// Host side of the C ABI: argument validation, the closed-form tile planner,
// useful-flop accounting, kernel selection and launch, error reporting.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "npa.h"
#include "npa_internal.hpp"

namespace {

thread_local std::string g_last_error;

npa_status_t fail(npa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
npa_status_t fail(npa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

npa_status_t ok() {
  g_last_error.clear();
  return NPA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Halo rows from the fraction p of a neighbour strip of s rows: ceil(p*s),
// with p*s lowered by 1e-6*s first so that a product that is an integer up
// to float rounding (p given as float) does not gain a row.
int32_t halo_from_p(float p, int32_t s) {
  const double v = std::ceil((double)p * (double)s - 1e-6 * (double)s);
  return v < 0.0 ? 0 : (int32_t)v;
}

// Compute units of the current device (queried once per device), 0 if unknown.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Validate the layout and halo; build the plan parameters.
npa_status_t make_geo(const npa_layout_t* L, const npa_halo_t* h, npa::Geo* g) {
  if (!L || !h) return fail(NPA_ERR_INVALID_ARG, "layout and halo must not be NULL");
  if (L->batch < 0 || L->heads < 0 || L->head_dim < 1 || L->map_h < 1 || L->map_w < 1)
    return fail(NPA_ERR_SHAPE, "batch and heads must be >= 0, head_dim, map_h and map_w >= 1");
  if (h->text_tokens < 0) return fail(NPA_ERR_SHAPE, "text_tokens=%d must be >= 0", h->text_tokens);
  if ((int64_t)h->text_tokens + (int64_t)L->map_h * L->map_w > (int64_t(1) << 24))
    return fail(NPA_ERR_SHAPE, "text_tokens + map_h*map_w = %lld exceeds 2^24 tokens",
                (long long)h->text_tokens + (long long)L->map_h * L->map_w);
  std::memset(g, 0, sizeof *g);
  g->mode = h->mode;
  g->H = L->map_h;
  g->W = L->map_w;
  if (h->mode == NPA_MODE_STRIPS) {
    if (h->num_strips < 1 || L->map_h % h->num_strips != 0)
      return fail(NPA_ERR_SHAPE, "num_strips=%d must be >= 1 and divide map_h=%d", h->num_strips,
                  L->map_h);
    g->s = L->map_h / h->num_strips;
    if (h->halo_rows >= 0) {
      g->h = h->halo_rows;
    } else {
      if (!(h->p >= 0.0f && h->p <= 1.0f))
        return fail(NPA_ERR_SHAPE, "p=%g must lie in [0, 1] (or give halo_rows >= 0)", (double)h->p);
      g->h = halo_from_p(h->p, g->s);
    }
    if (g->h > L->map_h) g->h = L->map_h;  // a longer halo reads nothing more
    if (h->text_tokens != 0)
      return fail(NPA_ERR_UNSUPPORTED, "text tokens are supported in window mode only");
    g->n_img = h->num_strips;
    g->n_tiles = g->n_img;
  } else if (h->mode == NPA_MODE_WINDOW) {
    if (h->tile_h < 1 || h->tile_w < 1 || L->map_h % h->tile_h || L->map_w % h->tile_w)
      return fail(NPA_ERR_SHAPE, "tile %dx%d must be >= 1 and divide the %dx%d map", h->tile_h,
                  h->tile_w, L->map_h, L->map_w);
    if (h->halo_h < 0 || h->halo_w < 0)
      return fail(NPA_ERR_SHAPE, "window halo must be >= 0");
    g->th = h->tile_h;
    g->tw = h->tile_w;
    g->eh = h->halo_h < L->map_h ? h->halo_h : L->map_h;
    g->ew = h->halo_w < L->map_w ? h->halo_w : L->map_w;
    g->tiles_x = L->map_w / h->tile_w;
    g->by_tiles_x = npa::DivBy::of(g->tiles_x);
    g->T = h->text_tokens;
    g->n_img = (L->map_h / h->tile_h) * g->tiles_x;
    g->n_tiles = g->n_img + (g->T > 0 ? 1 : 0);
  } else {
    return fail(NPA_ERR_INVALID_ARG, "unknown mode %d", h->mode);
  }
  return NPA_OK;
}

int64_t pairs_per_bh(const npa::Geo& g) {
  int64_t total = 0;
  for (int32_t t = 0; t < g.n_tiles; ++t) {
    const npa::TileRuns r = npa::tile_runs(g, t);
    total += (int64_t)r.q.count() * (r.nk[0] + r.nk[1] + r.nk[2]);
  }
  return total;
}

// Does any tile have a key run that is not a whole number of 64-key blocks?
bool has_partial_blocks(const npa::Geo& g) {
  for (int32_t t = 0; t < g.n_tiles; ++t) {
    const npa::TileRuns r = npa::tile_runs(g, t);
    if (r.nk[0] % 64 || r.nk[1] % 64 || r.nk[2] % 64) return true;
  }
  return false;
}

bool reads_stale(const npa::Geo& g) {
  for (int32_t t = 0; t < g.n_tiles; ++t) {
    const npa::TileRuns r = npa::tile_runs(g, t);
    for (int i = 0; i < 3; ++i)
      if (r.src[i] == 1 && r.nk[i] > 0) return true;
  }
  return false;
}

// [lo, hi) byte extent of one tensor of N stored tokens under the layout.
void extent(const void* p, const npa_layout_t* L, int64_t N, int64_t esize, uintptr_t* lo, uintptr_t* hi) {
  const int64_t last = (int64_t)(L->batch - 1) * L->stride_b + (N - 1) * L->stride_n +
                       (int64_t)(L->heads - 1) * L->stride_h + L->head_dim;
  *lo = reinterpret_cast<uintptr_t>(p);
  *hi = *lo + (uintptr_t)(last * esize);
}

// Do distinct (batch, token, head, channel) indices address distinct elements?
// Tested the sufficient way: taken in order of increasing stride, every
// dimension with more than one index steps past the whole span of the
// dimensions inside it (the channels are the contiguous innermost run).
// Returns false also when the span does not fit in 2^62 elements.
bool one_to_one(const npa_layout_t* L, int64_t tokens) {
  struct Dim {
    int64_t stride, n;
  } d[3] = {{L->stride_b, L->batch}, {L->stride_n, tokens}, {L->stride_h, L->heads}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (d[j].stride < d[i].stride) {
        const Dim t = d[i];
        d[i] = d[j];
        d[j] = t;
      }
  const int64_t limit = int64_t(1) << 62;
  int64_t span = L->head_dim;
  for (const Dim& x : d) {
    if (x.n <= 1) continue;
    if (x.stride < span) return false;
    if (x.stride > (limit - span) / (x.n - 1)) return false;
    span += x.stride * (x.n - 1);
  }
  return true;
}

bool overlaps(const void* a, const void* b, const npa_layout_t* L, int64_t N, int64_t esize) {
  if (!a || !b) return false;
  uintptr_t a0, a1, b0, b1;
  extent(a, L, N, esize, &a0, &a1);
  extent(b, L, N, esize, &b0, &b1);
  return a0 < b1 && b0 < a1;
}

}  // namespace

extern "C" {

const char* npa_last_error(void) { return g_last_error.c_str(); }

npa_status_t npa_plan(const npa_layout_t* layout, const npa_halo_t* halo, npa_tile_desc_t* tiles,
                      int32_t capacity, int32_t* n_tiles, int64_t* useful_pairs_per_bh) {
  npa::Geo g;
  npa_status_t st = make_geo(layout, halo, &g);
  if (st != NPA_OK) return st;
  if (capacity < 0 || (capacity > 0 && !tiles))
    return fail(NPA_ERR_INVALID_ARG, "tiles must be non-NULL when capacity > 0");
  for (int32_t t = 0; t < g.n_tiles && t < capacity; ++t) {
    const npa::TileRuns r = npa::tile_runs(g, t);
    npa_tile_desc_t& d = tiles[t];
    d.queries = npa_segment_t{0, r.q.start, r.q.row_len, r.q.rows, r.q.pitch};
    d.n_segments = 0;
    for (int i = 0; i < 3; ++i) {
      if (r.nk[i] == 0) continue;
      d.keys[d.n_segments++] = npa_segment_t{r.src[i], r.k[i].start, r.k[i].row_len, r.k[i].rows,
                                             r.k[i].pitch};
    }
    for (int i = d.n_segments; i < 3; ++i) d.keys[i] = npa_segment_t{0, 0, 0, 0, 0};
  }
  if (n_tiles) *n_tiles = g.n_tiles;
  if (useful_pairs_per_bh) *useful_pairs_per_bh = pairs_per_bh(g);
  return ok();
}

int64_t npa_useful_flops(const npa_layout_t* layout, const npa_halo_t* halo) {
  npa::Geo g;
  if (make_geo(layout, halo, &g) != NPA_OK) return -1;
  g_last_error.clear();
  return 4 * (int64_t)layout->head_dim * pairs_per_bh(g) * layout->batch * layout->heads;
}

npa_status_t npa_attn_fwd(const void* Q, const void* K_fresh, const void* V_fresh,
                          const void* K_stale, const void* V_stale, const npa_layout_t* layout,
                          const npa_halo_t* halo, void* out, void* hip_stream) {
  npa::Geo g;
  npa_status_t st = make_geo(layout, halo, &g);
  if (st != NPA_OK) return st;
  const npa_layout_t* L = layout;
  int64_t esize;
  int block_m;
  if (L->dtype == NPA_BF16) {
    esize = 2;
    block_m = npa::attn_bf16_block_m(L->head_dim, false);
  } else if (L->dtype == NPA_F32) {
    esize = 4;
    block_m = npa::attn_f32_block_m(L->head_dim, false);
  } else {
    return fail(NPA_ERR_INVALID_ARG, "unknown dtype %d", L->dtype);
  }
  if (block_m == 0)
    return fail(NPA_ERR_UNSUPPORTED, "head_dim=%d is not supported for %s", L->head_dim,
                L->dtype == NPA_BF16 ? "bf16 (64 or 128)" : "f32 (32, 64 or 128)");
  // no (batch, head) slice: a valid call with nothing to compute or touch
  if (L->batch == 0 || L->heads == 0) return ok();
  if (!Q || !K_fresh || !V_fresh || !out)
    return fail(NPA_ERR_INVALID_ARG, "Q, K_fresh, V_fresh and out must not be NULL");
  const bool stale = reads_stale(g);
  if (stale && (!K_stale || !V_stale))
    return fail(NPA_ERR_INVALID_ARG, "the plan reads %d stale halo rows: K_stale and V_stale are required", g.h);
  const void* ins[5] = {Q, K_fresh, V_fresh, stale ? K_stale : nullptr, stale ? V_stale : nullptr};
  for (const void* p : ins)
    if (p && !aligned16(p)) return fail(NPA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (!aligned16(out)) return fail(NPA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const int64_t vec = 16 / esize;
  if (L->stride_b < 0 || L->stride_n < 0 || L->stride_h < 0 || L->stride_b % vec || L->stride_n % vec ||
      L->stride_h % vec)
    return fail(NPA_ERR_INVALID_ARG, "strides must be >= 0 and multiples of %lld elements",
                (long long)vec);
  const int64_t tokens = (int64_t)g.T + (int64_t)L->map_h * L->map_w;  // stored per (batch, head)
  if (!one_to_one(L, tokens))
    return fail(NPA_ERR_INVALID_ARG,
                "the strides map two (batch, token, head) rows onto overlapping memory (the output would race)");
  for (const void* p : ins)
    if (overlaps(out, p, L, tokens, esize)) return fail(NPA_ERR_INVALID_ARG, "out must not alias an input");

  const int64_t range = (tokens - 1) * L->stride_n * esize + (int64_t)L->head_dim * esize;
  if (L->dtype == NPA_BF16 && range > 0x7FFFFFF0ll)
    return fail(NPA_ERR_UNSUPPORTED,
                "one (batch, head) slice spans %lld bytes; the bf16 kernel addresses at most 2^31-16",
                (long long)range);
  npa::AttnArgs a;
  a.range_bytes = (uint32_t)(range > 0xFFFFFFFFll ? 0xFFFFFFFFll : range);
  a.partial = has_partial_blocks(g) ? 1 : 0;
  a.q = Q;
  a.kf = K_fresh;
  a.vf = V_fresh;
  a.ks = stale ? K_stale : K_fresh;  // never dereferenced when the plan has no stale rows
  a.vs = stale ? V_stale : V_fresh;
  a.o = out;
  a.sb = L->stride_b;
  a.sn = L->stride_n;
  a.sh = L->stride_h;
  a.B = L->batch;
  a.Hh = L->heads;
  a.g = g;
  const int32_t nq = npa::tile_queries(g);
  int64_t text_blocks = 0, nblocks = 0;
  auto grid = [&](int bm) {
    a.qblocks = (nq + bm - 1) / bm;
    a.text_qblocks = (g.T + bm - 1) / bm;
    text_blocks = (int64_t)L->batch * L->heads * a.text_qblocks;
    nblocks = text_blocks + (int64_t)L->batch * L->heads * g.n_img * a.qblocks;
  };
  grid(block_m);
  // bf16: a grid that would not fill the GPU's workgroup slots twice runs in
  // the small-launch shape (twice the workgroups, each half as long)
  bool small = false;
  if (L->dtype == NPA_BF16) {
    const int cus = cu_count();
    if (cus > 0 && nblocks < 2ll * cus * npa::attn_bf16_per_cu(L->head_dim, false)) {
      small = true;
      grid(npa::attn_bf16_block_m(L->head_dim, true));
    }
  }
  // f32: a grid with fewer workgroups than the GPU has CUs runs in the
  // key-split shape where there is one (four times the workgroups, each
  // walking a quarter of the keys)
  bool split = false;
  if (L->dtype == NPA_F32) {
    const int cus = cu_count();
    const int bm = npa::attn_f32_block_m(L->head_dim, true);
    if (cus > 0 && bm > 0 && nblocks < cus) {
      split = true;
      grid(bm);
    }
  }
  if (nblocks >= (int64_t(1) << 31))
    return fail(NPA_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)nblocks);
  a.nblocks = (int32_t)nblocks;
  a.text_blocks = (int32_t)text_blocks;
  // windows whose halo is small against the tile (window area <= 2.25x the
  // tile's) share little between neighbouring tiles: list the longest tiles first
  a.largest_first = 0;
  if (g.mode == NPA_MODE_WINDOW && g.tiles_x >= 3 && g.n_img / g.tiles_x >= 3) {
    const int64_t win = (int64_t)(g.th + 2 * g.eh) * (g.tw + 2 * g.ew), tile = (int64_t)g.th * g.tw;
    a.largest_first = (4 * win <= 9 * tile) ? 1 : 0;
  }
  npa::set_divisors(a);
  float scale = L->scale;
  if (!(scale > 0.0f)) scale = (float)(1.0 / std::sqrt((double)L->head_dim));
  if (!std::isfinite(scale)) return fail(NPA_ERR_INVALID_ARG, "scale must be finite");
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)

  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const hipError_t e = (L->dtype == NPA_BF16) ? npa::launch_attn_bf16(a, L->head_dim, small, s)
                                              : npa::launch_attn_f32(a, L->head_dim, split, s);
  if (e != hipSuccess) return fail(NPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

npa_status_t npa_sg_blend(const float* x, const float* ref, float* out, int32_t n, int32_t c,
                          int32_t h, int32_t w, float w_t, float sigma, void* hip_stream) {
  if (n < 0 || c < 0 || h < 1 || w < 1) return fail(NPA_ERR_SHAPE, "n, c must be >= 0 and h, w >= 1");
  if (!(sigma > 0.0f && sigma <= 8.0f)) return fail(NPA_ERR_SHAPE, "sigma=%g must lie in (0, 8]", (double)sigma);
  if (!std::isfinite(w_t)) return fail(NPA_ERR_INVALID_ARG, "w_t must be finite");
  if (n == 0 || c == 0) return ok();  // no plane: nothing to compute or touch
  if (!x || !ref || !out) return fail(NPA_ERR_INVALID_ARG, "x, ref and out must not be NULL");
  if (!aligned16(x) || !aligned16(ref) || !aligned16(out))
    return fail(NPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const int64_t planes = (int64_t)n * c;
  if (planes > 65535) return fail(NPA_ERR_SHAPE, "n*c=%lld exceeds 65535 planes", (long long)planes);
  if ((int64_t)h * w > (int64_t(1) << 40) / planes)
    return fail(NPA_ERR_SHAPE, "n*c*h*w exceeds 2^40 elements");
  const uintptr_t bytes = (uintptr_t)planes * h * w * sizeof(float);
  const uintptr_t o0 = (uintptr_t)out, x0 = (uintptr_t)x, r0 = (uintptr_t)ref;
  if ((o0 < x0 + bytes && x0 < o0 + bytes) || (o0 < r0 + bytes && r0 < o0 + bytes))
    return fail(NPA_ERR_INVALID_ARG, "out must not alias x or ref");
  npa::SgArgs a;
  a.x = x;
  a.ref = ref;
  a.out = out;
  a.planes = (int32_t)planes;
  a.H = h;
  a.W = w;
  a.R = (int32_t)std::ceil(3.0 * (double)sigma);
  a.w = w_t;
  double taps[2 * npa::kSgMaxRadius + 1];
  double sum = 0.0;
  for (int k = -a.R; k <= a.R; ++k) {
    taps[k + a.R] = std::exp(-(double)k * k / (2.0 * (double)sigma * sigma));
    sum += taps[k + a.R];
  }
  for (int k = 0; k <= 2 * a.R; ++k) a.taps[k] = (float)(taps[k] / sum);
  const hipError_t e = npa::launch_sg_blend(a, reinterpret_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(NPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

npa_status_t npa_asg_blend(const float* eps, const float* eps_ref_prev, const float* mask, float* out,
                           int64_t count, float w_t, void* hip_stream) {
  if (!eps || !eps_ref_prev || !mask || !out)
    return fail(NPA_ERR_INVALID_ARG, "eps, eps_ref_prev, mask and out must not be NULL");
  if (!aligned16(eps) || !aligned16(eps_ref_prev) || !aligned16(mask) || !aligned16(out))
    return fail(NPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (count < 0) return fail(NPA_ERR_SHAPE, "count must be >= 0");
  if (count > (int64_t(1) << 40)) return fail(NPA_ERR_SHAPE, "count exceeds 2^40 elements");
  if (!std::isfinite(w_t)) return fail(NPA_ERR_INVALID_ARG, "w_t must be finite");
  // element-wise: out may be any input itself, but a shifted overlap would
  // let one element's result feed another element's inputs
  const uintptr_t bytes = (uintptr_t)count * sizeof(float), o0 = (uintptr_t)out;
  for (const float* p : {eps, eps_ref_prev, mask}) {
    const uintptr_t p0 = (uintptr_t)p;
    if (p0 != o0 && o0 < p0 + bytes && p0 < o0 + bytes)
      return fail(NPA_ERR_INVALID_ARG, "out must be an input itself or not overlap it");
  }
  if (count == 0) return ok();
  const hipError_t e = npa::launch_asg_blend(eps, eps_ref_prev, mask, out, count, w_t,
                                             reinterpret_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(NPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
