// Structure-guidance kernels.
//
// sg_blend: out = x + w * G_sigma * (ref - x), the low-frequency structure
// guidance of "ScaleDiff ..." (atlas.scime.ai), "Approach", written as one
// filter of the difference (the filter is linear, so this equals
// G*ref - G*x).  Separable Gaussian, reflect-101 borders.  Each workgroup
// produces one output tile from the tile plus an R-pixel apron of (ref - x).
// x and ref are read once from HBM (the apron re-reads hit the caches), out is
// written once: 12 bytes of HBM traffic per element.  sg_blend_mfma (radius
// <= 16, W a multiple of 4) runs both filter passes on the matrix cores;
// sg_blend_kernel, plain fp32 through LDS, serves every other shape.
//
// asg_blend: out = eps + w * mask * (eps_ref_prev - eps), element-wise
// (asynchronous structure guidance, pith.science verdict on ASGDiffusion,
// "core_discovery").
#include <hip/hip_runtime.h>

#include "npa_internal.hpp"

namespace npa {
namespace {

constexpr int kTW = 64, kTH = 32, kThreads = 256;

__device__ __forceinline__ int reflect101(int i, int n) {
  if (n == 1) return 0;
  const int period = 2 * (n - 1);
  i %= period;
  if (i < 0) i += period;
  return i < n ? i : period - i;
}

__global__ __launch_bounds__(kThreads) void sg_blend_kernel(const SgArgs a) {
  extern __shared__ float smem[];
  const int R = a.R;
  const int LW = kTW + 2 * R, LH = kTH + 2 * R;
  float* diff = smem;           // LH x LW
  float* tmp = smem + LH * LW;  // LH x kTW
  const int r0 = blockIdx.y * kTH, c0 = blockIdx.x * kTW;
  const size_t pb = (size_t)blockIdx.z * a.H * a.W;
  const float* x = a.x + pb;
  const float* ref = a.ref + pb;

  for (int i = threadIdx.x; i < LH * LW; i += kThreads) {
    const int rr = i / LW, cc = i - rr * LW;
    const int gr = reflect101(r0 - R + rr, a.H), gc = reflect101(c0 - R + cc, a.W);
    const size_t at = (size_t)gr * a.W + gc;
    diff[i] = ref[at] - x[at];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < LH * kTW; i += kThreads) {
    const int rr = i / kTW, cc = i - rr * kTW;
    const float* src = diff + rr * LW + cc;
    float acc = 0.0f;
    for (int t = 0; t <= 2 * R; ++t) acc = __builtin_fmaf(a.taps[t], src[t], acc);
    tmp[i] = acc;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kTH * kTW; i += kThreads) {
    const int rr = i / kTW, cc = i - rr * kTW;
    const int gr = r0 + rr, gc = c0 + cc;
    if (gr >= a.H || gc >= a.W) continue;
    const float* src = tmp + rr * kTW + cc;
    float acc = 0.0f;
    for (int t = 0; t <= 2 * R; ++t) acc = __builtin_fmaf(a.taps[t], src[t * kTW], acc);
    const size_t at = (size_t)gr * a.W + gc;
    a.out[pb + at] = __builtin_fmaf(a.w, acc, x[at]);
  }
}


// ---- Matrix-core form (R <= 16, W a multiple of 4, the border one reflection
// deep).  Each row pass and column pass is a product with a banded Toeplitz
// matrix of taps, run as v_mfma_f32_16x16x32_f16 with every fp32 operand split
// into an f16 high part and an f16 remainder (a = hi + lo; the products
// hi*hi', hi*lo', lo*hi' are summed in fp32; the dropped lo*lo' term and the
// two roundings leave ~2^-22 relative error per operand).  To keep both parts
// in f16's normal range, the tile's differences are scaled by a power of two
// that puts their max |.| in [2^13, 2^14) and the taps by 2^10; both scalings
// are exact and undone at the end.  A tile holding a non-finite difference
// takes the plain fp32 path instead, so infinities and NaNs propagate exactly
// as in the VALU form.
//
// One workgroup of four waves per 64 x 64 output tile; wave s owns the tile's
// 16-column strip s.  The apron (64 + 2RS rows and columns, RS = R rounded up
// to a multiple of 4 so that its quads are 16-byte aligned; the taps are
// shifted by RS - R) is staged as hi/lo f16 rows in LDS.  Row pass: for each
// 32-row chunk c of the apron and half h, rows 32c + 8u + 4h + i (u, i < 4)
// form one 16-row A operand, so that the two halves' accumulators hold, lane
// by lane, the 8 consecutive rows 32c + 8g .. +8 of the strip's column l16 --
// exactly the operand layout of the column pass, which then needs no LDS
// round trip.  Column pass, transposed (O^T = TMP^T T^T): output tile i
// (rows 16i .. +16) reads chunks i/2 and i/2 + 1, with the taps shifted by 16
// for odd i; each lane ends with 4 adjacent columns of one output row (one
// 16-byte store).  All 22 global loads of a lane are issued before any is
// used; quads left or right of the image are the mirrored quads, loaded
// ascending and reversed in registers.
namespace sgm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 64;         // output tile edge
constexpr int kRows = 96;      // staged apron rows: three 32-row chunks
constexpr int kQ = 24;         // staged quads per row (columns 0..95)
constexpr int kPitch = 128;    // f16 per staged row: 16 chunks of 8
constexpr int kReadQuads = 28; // the row pass reads columns 0..111
constexpr int kMaxR = 16;
constexpr float kTapScale = 1024.0f;
constexpr int kPoolBytes = (kRows * kRows + kRows * kT) * 4;  // the fp32 form's diff + rows
static_assert(kPoolBytes >= 2 * kRows * kPitch * 2, "hi/lo rows fit the pool");
static_assert(kMaxR <= kSgMaxRadius, "every tap index the kernel reads lies in SgArgs::taps");

// 8-element chunk q of staged row r sits at chunk q ^ swz(r): the 16 rows
// 8u + 4h + i (u, i < 4) of one A operand get 16 distinct masks, so its 16
// lanes of one column chunk hit 16 distinct bank groups
__device__ __forceinline__ int swz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
__device__ __forceinline__ int at(int r, int col) { return r * kPitch + ((((col >> 3) ^ swz(r)) << 3) | (col & 7)); }
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// plain fp32 separable blur of one tile through LDS (tiles with a non-finite value)
__device__ void tile_fp32(const SgArgs& a, float* pool, int r0, int c0, size_t pb) {
  const int R = a.R, AW = kT + 2 * R;
  float* diff = pool;           // AW x AW
  float* tmp = pool + AW * AW;  // AW x kT
  const float* x = a.x + pb;
  const float* ref = a.ref + pb;
  for (int i = threadIdx.x; i < AW * AW; i += 256) {
    const int rr = i / AW, cc = i - rr * AW;
    const size_t p = (size_t)reflect101(r0 - R + rr, a.H) * a.W + reflect101(c0 - R + cc, a.W);
    diff[i] = ref[p] - x[p];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < AW * kT; i += 256) {
    const int rr = i / kT, cc = i - rr * kT;
    float acc = 0.0f;
    for (int t = 0; t <= 2 * R; ++t) acc = __builtin_fmaf(a.taps[t], diff[rr * AW + cc + t], acc);
    tmp[i] = acc;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kT * kT; i += 256) {
    const int rr = i / kT, cc = i - rr * kT;
    const int gr = r0 + rr, gc = c0 + cc;
    if (gr >= a.H || gc >= a.W) continue;
    float acc = 0.0f;
    for (int t = 0; t <= 2 * R; ++t) acc = __builtin_fmaf(a.taps[t], tmp[(rr + t) * kT + cc], acc);
    const size_t p = (size_t)gr * a.W + gc;
    a.out[pb + p] = __builtin_fmaf(a.w, acc, x[p]);
  }
}

__global__ __launch_bounds__(256) void sg_blend_mfma(const SgArgs a) {
  __shared__ __attribute__((aligned(16))) float pool[kPoolBytes / 4];
  __shared__ float staps[96];  // taps * 2^10 at [32 + index + shift], zero elsewhere
  __shared__ float wmax[4];
  __shared__ int wbad[4];
  _Float16* shi = (_Float16*)pool;
  _Float16* slo = shi + kRows * kPitch;
  const int R = a.R, RS = (R + 3) & ~3, AW = kT + 2 * RS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int r0 = blockIdx.y * kT, c0 = blockIdx.x * kT;
  const size_t pb = (size_t)blockIdx.z * a.H * a.W;
  const float* x = a.x + pb;
  const float* ref = a.ref + pb;

  // taps through scalar loads (uniform index): no vector-memory wait ahead of
  // the staging loads
  if (tid < 96) {
    float v = 0.0f;
#pragma unroll
    for (int t = 0; t <= 2 * kMaxR; ++t)
      if (tid - 32 - (RS - R) == t && t <= 2 * R) v = a.taps[t] * kTapScale;
    staps[tid] = v;
  }

  // x at this lane's outputs: 4 adjacent columns of rows 16i + l16
  const int s = wave;
  const int oc = c0 + 16 * s + 4 * g;
  const bool vout = oc + 4 <= a.W;  // W is a multiple of 4: a quad is all in or all out
  f32x4 xo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int orow = min(r0 + 16 * i + l16, a.H - 1);
    xo[i] = *(const f32x4*)(x + (size_t)orow * a.W + min(oc, a.W - 4));
  }

  // the apron: quad q of the 96 x 24-quad grid (rows/columns past AW give zeros)
  constexpr int kStage = kRows * kQ / 256;
  f32x4 rv[kStage], xv[kStage];
  uint32_t flip = 0;
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int q = tid + 256 * k;
    const int rr = q / kQ, cc = 4 * (q - rr * kQ);
    rv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    xv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (rr < AW && cc < AW) {
      // one reflection (RS < H, W); rows and columns that only feed outputs
      // past the image's end are clamped into it
      int gr = r0 - RS + rr;
      gr = gr < 0 ? -gr : (gr >= a.H ? 2 * a.H - 2 - gr : gr);
      gr = min(max(gr, 0), a.H - 1);
      int gc = c0 - RS + cc;
      const bool mirror = gc < 0 || gc >= a.W;
      gc = gc < 0 ? -gc - 3 : (gc >= a.W ? 2 * a.W - 5 - gc : gc);
      gc = min(max(gc, 0), a.W - 4);
      const size_t p = (size_t)gr * a.W + gc;
      rv[k] = *(const f32x4*)(ref + p);
      xv[k] = *(const f32x4*)(x + p);
      flip |= (uint32_t)mirror << k;
    }
  }
  float m = 0.0f;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    rv[k] -= xv[k];
    if ((flip >> k) & 1) rv[k] = rv[k].wzyx;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = __builtin_fabsf(rv[k][e]);
      bad |= !(v <= 3.4028234663852886e38f);  // inf or NaN
      m = fmaxf(m, v);
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh));
  const bool wb = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (lane == 0) {
    wmax[wave] = m;
    wbad[wave] = wb;
  }
  __syncthreads();
  if (wbad[0] | wbad[1] | wbad[2] | wbad[3]) {
    tile_fp32(a, pool, r0, c0, pb);
    return;
  }
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int ex = 0;
  if (M > 0.0f) (void)frexpf(M, &ex);
  const int sc = min(max(14 - ex, -114), 100);  // M * 2^sc in [2^13, 2^14)
  const float up = ldexpf(1.0f, sc);
  const float down = ldexpf(1.0f, -sc - 10);  // undoes the data scale and the column taps' 2^10

  // tap operands: lane (n = l16, g) element i holds shifted tap 32j + 8g + i - n - off
  // (off = 0: row pass and even output tiles; off = 16: odd output tiles)
  f16x8 th[2][2], tl[2][2];  // [off][j]
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = staps[32 + 32 * j + 8 * g + i - l16 - 16 * o];
        th[o][j][i] = (_Float16)v;
        tl[o][j][i] = (_Float16)(v - (float)th[o][j][i]);
      }

  // hi/lo split into LDS; columns 96..111, which the row pass also reads, are zeros
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int q = tid + 256 * k;
    const int rr = q / kQ, cc = 4 * (q - rr * kQ);
    const f32x4 v = rv[k] * up;
    f16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (_Float16)v[e];
      l[e] = (_Float16)(v[e] - (float)h[e]);
    }
    *(f16x4*)&shi[at(rr, cc)] = h;
    *(f16x4*)&slo[at(rr, cc)] = l;
  }
  for (int q = tid; q < kRows * (kReadQuads - kQ); q += 256) {
    const int rr = q / (kReadQuads - kQ), cc = 4 * (kQ + q - rr * (kReadQuads - kQ));
    *(f16x4*)&shi[at(rr, cc)] = f16x4{};
    *(f16x4*)&slo[at(rr, cc)] = f16x4{};
  }
  __syncthreads();

  // row pass for the strip's 16 columns
  f16x8 bh[3], bl[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    f32x4 acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 32 * c + 8 * (l16 >> 2) + 4 * h + (l16 & 3);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = 16 * s + 32 * j + 8 * g;
        const f16x8 ah = *(const f16x8*)&shi[at(row, col)];
        const f16x8 al = *(const f16x8*)&slo[at(row, col)];
        acc[h] = mfma(ah, th[0][j], acc[h]);
        acc[h] = mfma(ah, tl[0][j], acc[h]);
        acc[h] = mfma(al, th[0][j], acc[h]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = acc[i >> 2][i & 3] * (1.0f / kTapScale);
      bh[c][i] = (_Float16)v;
      bl[c][i] = (_Float16)(v - (float)bh[c][i]);
    }
  }

  // column pass and blend
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = i & 1, cb = i >> 1;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc = mfma(bh[cb + j], th[o][j], acc);
      acc = mfma(bh[cb + j], tl[o][j], acc);
      acc = mfma(bl[cb + j], th[o][j], acc);
    }
    const int orow = r0 + 16 * i + l16;
    if (orow < a.H && vout) {
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(a.w, acc[e] * down, xo[i][e]);
      *(f32x4*)(a.out + pb + (size_t)orow * a.W + oc) = y;
    }
  }
}

}  // namespace sgm

// out may be one of the inputs itself (an in-place update): no pointer is
// marked __restrict__, since out is written while the same memory is read
// through the input pointers.  Each element is read before its own store and
// never again, so the in-place form is well defined.
__global__ __launch_bounds__(kThreads) void asg_blend_kernel(const float* eps, const float* ref,
                                                             const float* mask, float* out, int64_t n4,
                                                             int64_t count, float w) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    const f32x4 e = ((const f32x4*)eps)[i];
    const f32x4 r = ((const f32x4*)ref)[i];
    const f32x4 m = ((const f32x4*)mask)[i];
    f32x4 y;
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = __builtin_fmaf(w * m[k], r[k] - e[k], e[k]);
    ((f32x4*)out)[i] = y;
  }
  // tail (count % 4 elements) by the first threads of block 0
  if (blockIdx.x == 0) {
    const int64_t t = n4 * 4 + threadIdx.x;
    if (t < count) out[t] = __builtin_fmaf(w * mask[t], ref[t] - eps[t], eps[t]);
  }
}

}  // namespace

hipError_t launch_sg_blend(const SgArgs& a, hipStream_t st) {
  const int rs = (a.R + 3) & ~3;
  if (a.R <= sgm::kMaxR && (a.W & 3) == 0 && rs < a.H && rs < a.W) {
    const dim3 grid((a.W + sgm::kT - 1) / sgm::kT, (a.H + sgm::kT - 1) / sgm::kT, a.planes);
    hipLaunchKernelGGL(sgm::sg_blend_mfma, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((a.W + kTW - 1) / kTW, (a.H + kTH - 1) / kTH, a.planes), block(kThreads);
  const size_t lds = sizeof(float) * ((size_t)(kTH + 2 * a.R) * (kTW + 2 * a.R) + (size_t)(kTH + 2 * a.R) * kTW);
  hipLaunchKernelGGL(sg_blend_kernel, grid, block, lds, st, a);
  return hipGetLastError();
}

hipError_t launch_asg_blend(const float* eps, const float* ref, const float* mask, float* out,
                            int64_t count, float w, hipStream_t st) {
  const int64_t n4 = count / 4;
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(asg_blend_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, eps, ref,
                     mask, out, n4, count, w);
  return hipGetLastError();
}

}  // namespace npa
