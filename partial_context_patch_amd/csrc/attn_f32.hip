// Partial-context patch attention, fp32 throughout (no bf16 rounding anywhere).
//
// Same partial key sets as the bf16 kernel (own strip fresh plus stale halo
// rows, "Partially Conditioned Patch Parallelism ...", "What carries the
// argument"; or a clipped window, "ScaleDiff ...", "Approach").  Each query is
// served by kSplit consecutive lanes: K/V blocks are staged in LDS, lane s of a
// query takes the block's keys s, s + kSplit, ..., keeps its own running max,
// sum and output (blockwise online softmax with expf), and the lanes' partial
// results are merged once at the end by cross-lane exchange.  This is the
// accuracy path (fp32 inputs), not the throughput path; the key split keeps
// small fp32 calls from running on a handful of serial threads.
#include <hip/hip_runtime.h>

#include "npa_internal.hpp"

namespace npa {
namespace {

constexpr int kThreads = 256;                // threads per workgroup
constexpr int kSplit = 16;                   // lanes per query
constexpr int kQueries = kThreads / kSplit;  // queries per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__device__ __forceinline__ int token_of(const Run& r, int j) {
  if (MODE == NPA_MODE_STRIPS) return r.start + j;
  const int row = j / r.row_len;
  return r.start + row * r.pitch + (j - row * r.row_len);
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(const AttnArgs a) {
  constexpr int BN = D <= 64 ? 64 : 32;  // keys per LDS block: BN / kSplit per lane
  constexpr int C4 = D / 4;   // float4 chunks per key row
  constexpr int LD = D + 4;   // LDS row pitch: the kSplit lanes of a query read
                              // kSplit consecutive rows, 16 bytes apart in bank order
  __shared__ __attribute__((aligned(16))) float sk[BN * LD];
  __shared__ __attribute__((aligned(16))) float sv[BN * LD];

  const int tid = threadIdx.x, sub = tid % kSplit;
  const BlockCoord bc = decode_block(a, blockIdx.x, false);
  const int qb = bc.qb, tile = bc.tile, head = bc.head, b = bc.b;

  const TileRuns tr = tile_runs(a.g, tile);
  const int nq = tr.q.count();
  const int nk = tr.nk[0] + tr.nk[1] + tr.nk[2];
  const int64_t bh = (int64_t)b * a.sb + (int64_t)head * a.sh;
  const float* qp = (const float*)a.q;

  const int qi = qb * kQueries + tid / kSplit;
  const bool ok = qi < nq;
  const int64_t qoff = bh + (int64_t)(ok ? token_of<MODE>(tr.q, qi) : 0) * a.sn;

  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = ok ? qp[qoff + e] * a.scale : 0.0f;
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
      *(f32x4*)&sk[key * LD + dc * 4] = kk;
      *(f32x4*)&sv[key * LD + dc * 4] = vv;
    }
    __syncthreads();
    const int nvalid = nk - k0 < BN ? nk - k0 : BN;
    constexpr int KL = BN / kSplit;  // keys of the block this lane takes
    float sc[KL];
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int k = i * kSplit + sub;
      // four independent partial sums shorten the dependent chain
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e & 3] = __builtin_fmaf(q[e], sk[k * LD + e], acc[e & 3]);
      sc[i] = (k < nvalid) ? (acc[0] + acc[1]) + (acc[2] + acc[3]) : -INFINITY;
      mb = fmaxf(mb, sc[i]);
    }
    const float mn = fmaxf(m, mb);
    if (mn == -INFINITY) continue;  // this lane has seen no key yet
    if (mn > m) {  // rescale only when the running max rises
      const float alpha = expf(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int k = i * kSplit + sub;
      const float p = (k < nvalid) ? expf(sc[i] - mn) : 0.0f;
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = __builtin_fmaf(p, sv[k * LD + e], o[e]);
    }
    m = mn;
  }
  // merge the kSplit lanes of each query: common max, then weighted sums
  float mq = m;
#pragma unroll
  for (int w = 1; w < kSplit; w <<= 1) mq = fmaxf(mq, __shfl_xor(mq, w));
  const float f = (m == -INFINITY) ? 0.0f : expf(m - mq);
  float lq = l * f;
#pragma unroll
  for (int w = 1; w < kSplit; w <<= 1) lq += __shfl_xor(lq, w);
#pragma unroll
  for (int e = 0; e < D; ++e) {
    float v = o[e] * f;
#pragma unroll
    for (int w = 1; w < kSplit; w <<= 1) v += __shfl_xor(v, w);
    o[e] = v;
  }
  if (!ok) return;
  // every lane of the query holds the merged row; lane s stores its D/kSplit slice
  float* op = (float*)a.o;
  const float inv = 1.0f / lq;
  constexpr int PER = D / kSplit;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    if (e / PER == sub) {
      f32x4 v = {o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
      *(f32x4*)(op + qoff + e) = v;
    }
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
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) ? kQueries : 0;
}

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int /*block_m*/, hipStream_t st) {
  if (head_dim == 32) return launch_d<32>(a, st);
  if (head_dim == 64) return launch_d<64>(a, st);
  return launch_d<128>(a, st);
}

}  // namespace npa
