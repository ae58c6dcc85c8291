// Structure-guidance kernels.
//
// sg_blend: out = x + w * G_sigma * (ref - x), the low-frequency structure
// guidance of "ScaleDiff ..." (atlas.scime.ai), "Approach", written as one
// filter of the difference (the filter is linear, so this equals
// G*ref - G*x).  Separable Gaussian, reflect-101 borders.  Each workgroup
// produces one output tile: the tile plus an R-pixel apron of (ref - x) is
// staged in LDS, filtered along rows into a second LDS buffer, then along
// columns straight into the output.  Bandwidth-bound: x and ref are read once
// from HBM (the apron re-reads hit L2), out is written once: 12 bytes of HBM
// traffic per element.  sg_blend_tile<12, ...> is the radius-12 (sigma = 4)
// form; sg_blend_kernel serves any other radius.
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


// Radius known at compile time (sigma = 4 -> R = 12): a TW x TH output tile per
// workgroup of NTH threads.  The row pass gives each thread RO outputs from a
// register window of RO + 2R inputs, the column pass CO outputs from CO + 2R,
// so each staged value is read from LDS about (RO + 2R) / RO times instead of
// 2R + 1 times, and no index needs a run-time division by the tile width.
// Tiles whose apron lies inside the image stage 16-byte vectors; the others
// reflect (101) index by index.  The launch is one round of large workgroups
// (64 x 64 tiles, 1024 threads: one per CU at 4 x 512 x 512): bigger tiles
// re-read less apron, and sixteen waves per CU hide the load latency.
template <int R, int TW, int TH, int RO, int CO, int NTH>
__global__ __launch_bounds__(NTH) void sg_blend_tile(const SgArgs a) {
  constexpr int kThreads = NTH;
  constexpr int LW = TW + 2 * R, LH = TH + 2 * R;
  __shared__ __attribute__((aligned(16))) float diff[LH * LW];
  __shared__ float tmp[LH * TW];
  __shared__ __attribute__((aligned(16))) float xs[TH * TW];
  const int r0 = blockIdx.y * TH, c0 = blockIdx.x * TW;
  const size_t pb = (size_t)blockIdx.z * a.H * a.W;
  const float* x = a.x + pb;
  const float* ref = a.ref + pb;
  float taps[2 * R + 1];
#pragma unroll
  for (int t = 0; t <= 2 * R; ++t) taps[t] = a.taps[t];
  static_assert(LW % 4 == 0 && R % 4 == 0 && TW % 4 == 0, "vector staging");
  const bool inside = r0 - R >= 0 && c0 - R >= 0 && r0 + TH + R <= a.H && c0 + TW + R <= a.W && (a.W & 3) == 0;
  if (inside) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int LW4 = LW / 4;
    constexpr int kStage4 = (LH * LW4 + kThreads - 1) / kThreads;
    f32x4 rv[kStage4], xv[kStage4];
#pragma unroll
    for (int k = 0; k < kStage4; ++k) {
      const int i = threadIdx.x + k * kThreads;
      const int rr = i / LW4, c4 = i - rr * LW4;
      const size_t at = (size_t)(r0 - R + rr) * a.W + (c0 - R + 4 * c4);
      rv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      xv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < LH * LW4) {
        rv[k] = *(const f32x4*)(ref + at);
        xv[k] = *(const f32x4*)(x + at);
      }
    }
#pragma unroll
    for (int k = 0; k < kStage4; ++k) {
      const int i = threadIdx.x + k * kThreads;
      if (i < LH * LW4) {
        *(f32x4*)&diff[4 * i] = rv[k] - xv[k];
        const int rr = i / LW4 - R, cc = 4 * (i % LW4) - R;
        if (rr >= 0 && rr < TH && cc >= 0 && cc < TW) *(f32x4*)&xs[rr * TW + cc] = xv[k];
      }
    }
  } else {
    constexpr int kStage = (LH * LW + kThreads - 1) / kThreads;
    float rv[kStage], xv[kStage];
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int i = threadIdx.x + k * kThreads;
      const int rr = i / LW, cc = i - rr * LW;
      int gr = r0 - R + rr, gc = c0 - R + cc;
      if ((unsigned)gr >= (unsigned)a.H) gr = reflect101(gr, a.H);
      if ((unsigned)gc >= (unsigned)a.W) gc = reflect101(gc, a.W);
      const size_t at = (size_t)gr * a.W + gc;
      rv[k] = 0.0f;
      xv[k] = 0.0f;
      if (i < LH * LW) {
        rv[k] = ref[at];
        xv[k] = x[at];
      }
    }
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int i = threadIdx.x + k * kThreads;
      if (i < LH * LW) {
        diff[i] = rv[k] - xv[k];
        const int rr = i / LW - R, cc = i % LW - R;
        if (rr >= 0 && rr < TH && cc >= 0 && cc < TW) xs[rr * TW + cc] = xv[k];
      }
    }
  }
  __syncthreads();
  constexpr int RSEG = TW / RO, RWIN = RO + 2 * R;
  for (int job = threadIdx.x; job < LH * RSEG; job += kThreads) {
    const int rr = job / RSEG, cs = (job % RSEG) * RO;
    float w[RWIN];
#pragma unroll
    for (int k = 0; k < RWIN; ++k) w[k] = diff[rr * LW + cs + k];
#pragma unroll
    for (int o = 0; o < RO; ++o) {
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t <= 2 * R; ++t) acc = __builtin_fmaf(taps[t], w[o + t], acc);
      tmp[rr * TW + cs + o] = acc;
    }
  }
  __syncthreads();
  constexpr int CSEG = TH / CO, CWIN = CO + 2 * R;
  for (int job = threadIdx.x; job < TW * CSEG; job += kThreads) {
    const int cc = job % TW, rs = (job / TW) * CO;
    float w[CWIN];
#pragma unroll
    for (int k = 0; k < CWIN; ++k) w[k] = tmp[(rs + k) * TW + cc];
    const int gc = c0 + cc;
#pragma unroll
    for (int o = 0; o < CO; ++o) {
      const int gr = r0 + rs + o;
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t <= 2 * R; ++t) acc = __builtin_fmaf(taps[t], w[o + t], acc);
      if (gr < a.H && gc < a.W) a.out[pb + (size_t)gr * a.W + gc] = __builtin_fmaf(a.w, acc, xs[(rs + o) * TW + cc]);
    }
  }
}

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
  if (a.R == 12) {
    constexpr int TW = 64, TH = 64, NTH = 1024;
    const dim3 grid((a.W + TW - 1) / TW, (a.H + TH - 1) / TH, a.planes);
    hipLaunchKernelGGL((sg_blend_tile<12, TW, TH, 8, 4, NTH>), grid, dim3(NTH), 0, st, a);
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
