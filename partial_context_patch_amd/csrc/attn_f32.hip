// Partial-context patch attention, fp32 throughout (no bf16 rounding anywhere).
//
// Same partial key sets as the bf16 kernel (own strip fresh plus stale halo
// rows, "Partially Conditioned Patch Parallelism ...", "What carries the
// argument"; or a clipped window, "ScaleDiff ...", "Approach").  One thread
// per query, K/V blocks staged in LDS and broadcast to every thread; blockwise
// online softmax with expf.  This is the accuracy path (tiny fp32 workloads),
// not the throughput path.
#include <hip/hip_runtime.h>

#include "npa_internal.hpp"

namespace npa {
namespace {

constexpr int kThreads = 128;  // queries per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__device__ __forceinline__ int token_of(const Run& r, int j) {
  if (MODE == NPA_MODE_STRIPS) return r.start + j;
  const int row = j / r.row_len;
  return r.start + row * r.pitch + (j - row * r.row_len);
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(const AttnArgs a) {
  constexpr int BN = (D >= 128) ? 16 : 32;  // keys per LDS block
  constexpr int C4 = D / 4;                 // float4 chunks per key row
  __shared__ __attribute__((aligned(16))) float sk[BN * D];
  __shared__ __attribute__((aligned(16))) float sv[BN * D];

  const int tid = threadIdx.x;
  const BlockCoord bc = decode_block(a, blockIdx.x, false);
  const int qb = bc.qb, tile = bc.tile, head = bc.head, b = bc.b;

  const TileRuns tr = tile_runs(a.g, tile);
  const int nq = tr.q.count();
  const int nk = tr.nk[0] + tr.nk[1] + tr.nk[2];
  const int64_t bh = (int64_t)b * a.sb + (int64_t)head * a.sh;
  const float* qp = (const float*)a.q;

  const int qi = qb * kThreads + tid;
  const bool ok = qi < nq;
  const int64_t qoff = bh + (int64_t)(ok ? token_of<MODE>(tr.q, qi) : 0) * a.sn;

  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = ok ? qp[qoff + e] : 0.0f;
    o[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  for (int k0 = 0; k0 < nk; k0 += BN) {
    __syncthreads();
    for (int c = tid; c < BN * C4; c += kThreads) {
      const int key = c / C4, dc = c % C4;
      int j = k0 + key;
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (j < nk) {
        int run = 0;
        if (j >= tr.nk[0]) {
          j -= tr.nk[0];
          run = 1;
          if (j >= tr.nk[1]) {
            j -= tr.nk[1];
            run = 2;
          }
        }
        const int64_t off = bh + (int64_t)token_of<MODE>(tr.k[run], j) * a.sn + dc * 4;
        const float* kp = (const float*)(tr.src[run] ? a.ks : a.kf);
        const float* vp = (const float*)(tr.src[run] ? a.vs : a.vf);
        kk = *(const f32x4*)(kp + off);
        vv = *(const f32x4*)(vp + off);
      }
      *(f32x4*)&sk[key * D + dc * 4] = kk;
      *(f32x4*)&sv[key * D + dc * 4] = vv;
    }
    __syncthreads();
    const int nvalid = nk - k0 < BN ? nk - k0 : BN;
    float sc[BN];
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < BN; ++k) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = __builtin_fmaf(q[e], sk[k * D + e], acc);
      sc[k] = (k < nvalid) ? acc * a.scale : -INFINITY;
      mb = fmaxf(mb, sc[k]);
    }
    const float mn = fmaxf(m, mb);
    const float alpha = expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
    for (int k = 0; k < BN; ++k) {
      const float p = (k < nvalid) ? expf(sc[k] - mn) : 0.0f;
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = __builtin_fmaf(p, sv[k * D + e], o[e]);
    }
    m = mn;
  }
  if (!ok) return;
  float* op = (float*)a.o;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    f32x4 v = {o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    *(f32x4*)(op + qoff + e) = v;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.nblocks), block(kThreads);
  if (a.g.mode == NPA_MODE_STRIPS)
    hipLaunchKernelGGL((attn_f32_kernel<D, NPA_MODE_STRIPS>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, NPA_MODE_WINDOW>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

int attn_f32_block_m(int head_dim) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) ? kThreads : 0;
}

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int /*block_m*/, hipStream_t st) {
  if (head_dim == 32) return launch_d<32>(a, st);
  if (head_dim == 64) return launch_d<64>(a, st);
  return launch_d<128>(a, st);
}

}  // namespace npa
