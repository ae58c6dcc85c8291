/*
 * npa.h -- partial-context patch attention on gfx950 (MI355X): C ABI.
 *
 * One launch computes, for every query token of an H x W latent token map,
 * multi-head scaled dot-product attention over a partial key/value set:
 *
 *   - NPA_MODE_STRIPS (partially conditioned attention): "Partially
 *     Conditioned Patch Parallelism for Accelerated Diffusion Model
 *     Inference" (pith.science review page), sections "What carries the
 *     argument" and "Core claim".  The map is cut into num_strips horizontal
 *     strips of s = map_h / num_strips rows.  A query of strip i attends to
 *     the fresh keys/values of its own strip plus the stale (previous-step)
 *     keys/values of the h rows nearest to it in each neighbouring strip:
 *     rows [max(0, i*s - h), i*s) and [(i+1)*s, min(map_h, (i+1)*s + h)).
 *     h = ceil(p * s) (p is a fraction of the neighbour's height; p*s is
 *     lowered by 1e-6*s before the ceiling so that an integer product that
 *     carries float rounding does not gain a row), or given directly as
 *     halo_rows.  No wrap-around at the image border.
 *   - NPA_MODE_WINDOW (Neighborhood Patch Attention): "ScaleDiff:
 *     Higher-Resolution Image Synthesis via Efficient and Model-Agnostic
 *     Diffusion" (atlas.scime.ai), section "Approach".  The map is cut into
 *     non-overlapping tile_h x tile_w query tiles; a query of tile (ti, tj)
 *     attends to the fresh keys/values of rows
 *     [max(0, ti*tile_h - halo_h), min(map_h, (ti+1)*tile_h + halo_h)) x cols
 *     [max(0, tj*tile_w - halo_w), min(map_w, (tj+1)*tile_w + halo_w)),
 *     i.e. the window is clipped (not shifted) at the border.
 *     Joint attention (FLUX): with text_tokens = T > 0 the tensors hold T
 *     text tokens first, then the map's tokens (map token t at index T + t).
 *     The same page applies NPA to FLUX without saying how the prompt's tokens
 *     take part; reading: they are global -- a map query also attends to all
 *     T text tokens, and a text query attends to every token, text and map.
 *
 * Attention itself (the multi-head scaled dot-product attention named in the
 * PCPP review's minor comment on Sec. 3.3):
 *   O[b,q,j,:] = sum_{k in S(q)} softmax_k(scale * <Q[b,q,j,:], K(k)[b,k,j,:]>) V(k)[b,k,j,:]
 * with K(k), V(k) read from the fresh or the stale buffers in place; the
 * concatenated key set is never materialised.
 *
 * Conventions for every entry point:
 *   - All device pointers are caller-owned device memory; the library
 *     allocates no device memory, never synchronises, and enqueues its work
 *     on `hip_stream` (a hipStream_t, NULL = the default stream).
 *   - Arguments are validated on the host before anything is launched; on a
 *     non-OK status nothing was enqueued and npa_last_error() returns a
 *     thread-local message.  No C++ exception crosses this interface.
 *   - Launch failures reported by the HIP runtime return NPA_ERR_HIP.
 */
#ifndef NPA_H
#define NPA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NPA_OK = 0,
  NPA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, aliasing, bad enum */
  NPA_ERR_SHAPE = -2,       /* sizes that do not tile, p out of range, ... */
  NPA_ERR_UNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim)   */
  NPA_ERR_HIP = -4          /* the HIP runtime reported an error           */
} npa_status_t;

typedef enum { NPA_F32 = 0, NPA_BF16 = 1 } npa_dtype_t;
typedef enum { NPA_MODE_STRIPS = 0, NPA_MODE_WINDOW = 1 } npa_mode_t;

/* Shape and layout shared by Q, K_fresh, V_fresh, K_stale, V_stale and out.
 * Element (b, token t, head j, channel e) lives at
 *   base + b*stride_b + t*stride_n + j*stride_h + e        (elements)
 * with tokens row-major over the map, t = r*map_w + c (after the halo's
 * text_tokens, when there are any: t = text_tokens + r*map_w + c).  Every
 * pointer must be 16-byte aligned and stride_b/stride_n/stride_h must keep
 * each head's row 16-byte aligned.  Distinct (b, t, j, e) must address
 * distinct elements (checked: ordered by stride, each dimension with more than
 * one index must step past the span of the ones inside it; otherwise
 * NPA_ERR_INVALID_ARG -- out would race).  Limits: text_tokens + map_h*map_w
 * <= 2^24, batch*heads*tiles*blocks < 2^31.  batch and heads may be 0: such a call is
 * validated, computes nothing, touches no memory and returns NPA_OK (its
 * pointers may then be NULL); head_dim, map_h, map_w are >= 1. */
typedef struct {
  int32_t batch, heads, head_dim; /* head_dim: 64 or 128 for bf16; 32/64/128 for f32 */
  int32_t map_h, map_w;
  int64_t stride_b, stride_n, stride_h;
  int32_t dtype;                  /* npa_dtype_t; one dtype for every tensor */
  float scale;                    /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
} npa_layout_t;

/* Which keys each query tile attends to. */
typedef struct {
  int32_t mode;       /* npa_mode_t */
  /* strips */
  int32_t num_strips; /* must divide map_h */
  float p;            /* used when halo_rows < 0; must be in [0, 1] then */
  int32_t halo_rows;  /* >= 0: explicit halo height in rows (may exceed s) */
  /* window */
  int32_t tile_h, tile_w; /* must divide map_h, map_w */
  int32_t halo_h, halo_w; /* >= 0 */
  int32_t text_tokens;    /* window mode: global text tokens stored before the
                             map's tokens (>= 0; strips mode requires 0) */
} npa_halo_t;

/* One contiguous-by-rows run of tokens: `rows` runs of `row_len` tokens, the
 * first starting at token `start`, successive runs `pitch` tokens apart. */
typedef struct {
  int32_t src; /* 0: fresh K/V buffers, 1: stale K/V buffers */
  int32_t start, row_len, rows, pitch;
} npa_segment_t;

/* The plan of one query tile: its query tokens and up to three key runs.
 * With text tokens the last tile holds the text queries (one run of T
 * tokens, keys: every stored token) and each map tile has the text tokens as
 * an extra key run. */
typedef struct {
  npa_segment_t queries;   /* src is 0 */
  int32_t n_segments;      /* 1..3 */
  npa_segment_t keys[3];
} npa_tile_desc_t;

/* Partial attention forward.
 *   Q, K_fresh, V_fresh, out: required device pointers (layout above).
 *   K_stale, V_stale: device pointers to the previous step's keys/values;
 *     may be NULL only when the plan reads no stale row (window mode, or a
 *     halo of zero rows); otherwise NPA_ERR_INVALID_ARG.
 *   out must not alias any input (NPA_ERR_INVALID_ARG).
 *   Computation: scores and softmax in fp32; for bf16 the two products run on
 *   bf16 MFMA with fp32 accumulation and the result is rounded to bf16
 *   (nearest-even); for f32 every step is fp32. */
npa_status_t npa_attn_fwd(const void* Q, const void* K_fresh, const void* V_fresh,
                          const void* K_stale, const void* V_stale,
                          const npa_layout_t* layout, const npa_halo_t* halo,
                          void* out, void* hip_stream);

/* Host-only planner (no GPU needed): the key sets defined at the top of this
 * file (PCPP review page, "What carries the argument"; ScaleDiff page,
 * "Approach"), written out per query tile as runs of tokens -- the same
 * closed form every workgroup of npa_attn_fwd evaluates.  Writes up to `capacity` tile
 * descriptors into `tiles` (may be NULL with capacity 0), the total tile
 * count into *n_tiles and the number of attended (query, key) pairs per
 * (batch, head) into *useful_pairs_per_bh (either output may be NULL). */
npa_status_t npa_plan(const npa_layout_t* layout, const npa_halo_t* halo,
                      npa_tile_desc_t* tiles, int32_t capacity, int32_t* n_tiles,
                      int64_t* useful_pairs_per_bh);

/* Useful attention flops of one npa_attn_fwd call:
 * 4 * head_dim * attended pairs * batch * heads; -1 on invalid arguments.
 * Only (query, key) pairs inside the key sets defined above count -- 2*d
 * flops for the score and 2*d for the weighted value sum of each pair --
 * so padding, masked keys and the softmax itself add nothing.  This is the
 * work measure behind the useful partial-attention throughput (the pages
 * report only end-to-end times; the partial key set is the compute saving
 * the PCPP review page's "Core claim" and the ScaleDiff page's "Approach"
 * attribute to the method). */
int64_t npa_useful_flops(const npa_layout_t* layout, const npa_halo_t* halo);

/* Structure-guidance blend: "ScaleDiff ..." (atlas.scime.ai), "Approach"
 * (the latent's low frequencies are pulled towards those of a reference):
 *   out = x + w_t * (G_sigma * ref - G_sigma * x)     per channel,
 * G_sigma a separable Gaussian with taps |k| <= ceil(3*sigma), weights
 * exp(-k^2/(2 sigma^2)) normalised to 1, reflect-101 borders.
 * x, ref, out: fp32 device tensors [n, c, h, w] contiguous, 16-byte aligned;
 * out must not alias x or ref (the stencil reads neighbours).  sigma in
 * (0, 8]; h, w >= 1; n, c >= 0 (n*c = 0: nothing to do, NPA_OK, pointers
 * unchecked); n*c <= 65535 and n*c*h*w <= 2^40 (else NPA_ERR_SHAPE).
 * With w_t = 1 this is also latent frequency mixing: low frequencies of ref,
 * high frequencies of x. */
npa_status_t npa_sg_blend(const float* x, const float* ref, float* out, int32_t n,
                          int32_t c, int32_t h, int32_t w, float w_t, float sigma,
                          void* hip_stream);

/* Asynchronous structure-guidance correction: the pith.science verdict page
 * on ASGDiffusion (arXiv 2412.06163), section "core_discovery":
 *   out = eps + w_t * mask * (eps_ref_prev - eps)        element-wise,
 * where eps_ref_prev is the reference patch's prediction from the previous
 * step and mask the normalised cross-attention mask (caller-supplied).
 * fp32 device arrays of `count` elements (0 <= count <= 2^40), 16-byte
 * aligned; out may be any of the inputs itself (the update is element-wise),
 * while a shifted overlap with an input is NPA_ERR_INVALID_ARG. */
npa_status_t npa_asg_blend(const float* eps, const float* eps_ref_prev, const float* mask,
                           float* out, int64_t count, float w_t, void* hip_stream);

/* Thread-local message for the last non-OK status of this thread ("" if none). */
const char* npa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NPA_H */
