// Partial-context patch attention, fp32 throughout (no bf16 rounding anywhere),
// on the fp32 matrix cores (v_mfma_f32_16x16x4_f32).
//
// Same partial key sets as the bf16 kernel (own strip fresh plus stale halo
// rows, "Partially Conditioned Patch Parallelism ...", "What carries the
// argument"; or a clipped window, "ScaleDiff ...", "Approach").
//
// Workgroup = 4 waves, one 16-query tile per wave (64 queries), sharing each
// 32-key K/V block staged in LDS; the next block's global loads are in flight
// in registers while the current one is computed.  Three workgroups per CU at
// d <= 64 (two at d = 128, where a third would spill registers).  Per block
// and wave:
//
//   S^T = K Q^T   one 16-key x 16-query tile per 16 keys.  The instruction
//                 takes A[m][k] from lane (m + 16k), B[k][n] from lane
//                 (n + 16k) and leaves D[4g + i][n] in entry i of lane
//                 (n + 16g).  Lane group g supplies the contiguous quarter
//                 d in [g*D/4, (g+1)*D/4) of the dot product, so its K reads
//                 are 16-byte row reads and its Q quarter stays in registers.
//                 Lane (n + 16g) ends with the scores of keys 4g..4g+3 of each
//                 tile for query n.
//   softmax       exact block max (in-lane, then across the four lane groups),
//                 running max / sum with one rescale of O per block, exp2 of
//                 scores pre-scaled by scale*log2(e) (folded into Q).
//   O^T += V^T P^T  MFMA (tile t, j) contracts keys 16t + 4g + j (g = the lane
//                 group), so the B operand is the lane's own weight of entry j
//                 -- the score layout feeds PV with no data movement.  Output
//                 row m of 16-dim step dt is channel m*DT + dt: a lane's V
//                 operands for all steps are DT consecutive floats of one key
//                 row, and at the end a lane holds 4*DT consecutive channels
//                 of its query's output row.
//
// Key-split shape, for calls whose grid would leave most CUs idle (d <= 64):
// the four waves share one 16-query tile and wave w takes the 32-key blocks
// w, w + 4, w + 8, ... of its keys, staged by itself in its own LDS region
// (wave-level synchronisation only); at the end the waves' running max, sum
// and output are merged through LDS (out = sum_w 2^(m_w - M) O_w / sum_w
// 2^(m_w - M) l_w with M = max_w m_w).  Four times the workgroups, each a
// quarter as long.
//
// This is the accuracy path for fp32 inputs; products and sums stay in fp32.
#include <hip/hip_runtime.h>

#include "npa_internal.hpp"

namespace npa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;  // threads per workgroup
constexpr int kQueries = 16 * kWaves;  // queries per workgroup (one 16-query tile per wave)
constexpr int kSplitQueries = 16;      // key-split shape: one tile for the whole workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// j / d for 0 <= j < 2^24 via a float reciprocal and one correction step.
__device__ __forceinline__ int fast_div(int j, int d, float inv) {
  int q = (int)((float)j * inv);
  const int r = j - q * d;
  q += (r < 0) ? -1 : ((r >= d) ? 1 : 0);
  return q;
}

// Token index of entry j of run r (windows: rows of row_len tokens, pitch apart).
template <int MODE>
__device__ __forceinline__ int token_of(const Run& r, int j, float inv_row_len) {
  if (MODE == NPA_MODE_STRIPS) return r.start + j;
  const int row = fast_div(j, r.row_len, inv_row_len);
  return r.start + row * r.pitch + (j - row * r.row_len);
}

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Token index and source buffer of key j (0 <= j < nk) of the tile's key runs.
template <int MODE>
__device__ __forceinline__ int key_token(const TileRuns& tr, const float (&inv)[3], int j, bool& stale) {
  if (j < tr.nk[0]) {
    stale = tr.src[0] != 0;
    return token_of<MODE>(tr.k[0], j, inv[0]);
  }
  j -= tr.nk[0];
  if (j < tr.nk[1]) {
    stale = tr.src[1] != 0;
    return token_of<MODE>(tr.k[1], j, inv[1]);
  }
  stale = tr.src[2] != 0;
  return token_of<MODE>(tr.k[2], j - tr.nk[1], inv[2]);
}

// Wave-level barrier: the wave's LDS writes before it are visible to its reads after it.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(kThreads, (SPLIT ? 1 : (D == 128 ? 2 : 3))) void attn_f32_kernel(const AttnArgs a) {
  constexpr int kBN = 32;                   // keys per LDS block
  constexpr int NTL = kBN / 16;             // 16-key tiles per block
  constexpr int LD = D + 4;                 // LDS row pitch (floats)
  constexpr int C4 = D / 4;                 // 16-byte chunks per key row
  constexpr int NTHR = SPLIT ? 64 : kThreads;  // threads staging one block
  constexpr int CH = kBN * C4 / NTHR;       // chunks per thread per K (and V) block
  constexpr int DQ = D / 4;                 // channels per lane group in S^T
  constexpr int DT = D / 16;                // 16-dim steps of O^T
  constexpr int NBUF = SPLIT ? kWaves : 1;  // LDS block buffers (one per wave when split)
  static_assert(CH * NTHR == kBN * C4 && DT >= 2 && DT % 2 == 0, "shape");
  static_assert(!SPLIT || kWaves * 16 * (D + 2) <= NBUF * kBN * LD, "merge buffer");
  __shared__ __attribute__((aligned(16))) float sk[NBUF * kBN * LD];
  __shared__ __attribute__((aligned(16))) float sv[NBUF * kBN * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int stid = SPLIT ? lane : tid;  // index among the threads staging a block
  float* const skw = sk + (SPLIT ? wave * kBN * LD : 0);
  float* const svw = sv + (SPLIT ? wave * kBN * LD : 0);
  const int g4 = lane >> 4, l16 = lane & 15;
  // regular shape: the query blocks of a unit on one XCD (they share its K/V in
  // that XCD's L2: +0.7% sdxl4096_npa, +5.6% sdxl2048_strips, 26-34 W less);
  // the key-split shape's few workgroups stay spread over all XCDs
  const BlockCoord bc = decode_block(a, blockIdx.x, !SPLIT);
  const TileRuns tr = tile_runs(a.g, bc.tile);
  const int nq = tr.q.count();
  const int nk = tr.nk[0] + tr.nk[1] + tr.nk[2];
  const int64_t bh = (int64_t)bc.b * a.sb + (int64_t)bc.head * a.sh;
  float inv_len[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) inv_len[r] = tr.k[r].row_len > 0 ? 1.0f / (float)tr.k[r].row_len : 0.0f;

  // this lane's query (column l16 of the wave's tile) and its quarter of Q,
  // pre-scaled by scale * log2(e)
  const int qi = SPLIT ? bc.qb * kSplitQueries + l16 : bc.qb * kQueries + wave * 16 + l16;
  const bool ok = qi < nq;
  const int64_t qoff = bh + (int64_t)(ok ? token_of<MODE>(tr.q, qi, 1.0f / (float)tr.q.row_len) : 0) * a.sn;
  float qf[DQ];
#pragma unroll
  for (int e = 0; e < DQ; e += 4) {
    const f32x4 v = ok ? *(const f32x4*)((const float*)a.q + qoff + g4 * DQ + e) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[e + i] = v[i] * a.c;
  }

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max of the query's scores (log2 domain)
  float l = 0.0f;       // sum of this lane's weights (its keys 4g4..4g4+3 of every tile)

  // K/V block staging: chunk c of this thread is key (stid + c*NTHR) / C4
  f32x4 rk[CH], rv[CH];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = stid + c * NTHR, key = idx / C4, dc = idx % C4;
      const int j = k0 + key;
      rk[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      rv[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < nk) {
        bool stale;
        const int64_t off = bh + (int64_t)key_token<MODE>(tr, inv_len, j, stale) * a.sn + dc * 4;
        rk[c] = *(const f32x4*)((const float*)(stale ? a.ks : a.kf) + off);
        rv[c] = *(const f32x4*)((const float*)(stale ? a.vs : a.vf) + off);
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = stid + c * NTHR, key = idx / C4, dc = idx % C4;
      *(f32x4*)&skw[key * LD + dc * 4] = rk[c];
      *(f32x4*)&svw[key * LD + dc * 4] = rv[c];
    }
  };
  // the threads that stage a block agree it is complete (or consumed)
  auto sync = [&]() __attribute__((always_inline)) {
    if (SPLIT)
      wave_sync();
    else
      __syncthreads();
  };

  const int kfirst = SPLIT ? wave * kBN : 0, kstep = SPLIT ? kWaves * kBN : kBN;
  if (kfirst < nk) load(kfirst);
  for (int k0 = kfirst; k0 < nk; k0 += kstep) {
    sync();  // done with the previous block
    store();
    sync();
    if (k0 + kstep < nk) load(k0 + kstep);
    const int nvalid = nk - k0 < kBN ? nk - k0 : kBN;

    // S^T, the block's 16-key tiles interleaved (independent accumulation chains)
    f32x4 s[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < DQ; e += 4) {
      f32x4 kv[NTL];
#pragma unroll
      for (int t = 0; t < NTL; ++t) kv[t] = *(const f32x4*)&skw[(16 * t + l16) * LD + g4 * DQ + e];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < NTL; ++t) s[t] = mfma(kv[t][i], qf[e + i], s[t]);
    }
    // keys past the block's end (entry i of tile t is key 16t + 4*g4 + i)
    if (nvalid < kBN) {
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * t + 4 * g4 + i >= nvalid) s[t][i] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < NTL; ++t) mt = fmaxf(mt, fmaxf(fmaxf(s[t][0], s[t][1]), fmaxf(s[t][2], s[t][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    // no finite score yet (only for non-finite inputs): keep the zero state
    const float sh = (mn == -INFINITY) ? 0.0f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m - sh);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    m = mn;
    float p[NTL][4];
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = __builtin_amdgcn_exp2f(s[t][i] - sh);
        l += p[t][i];
      }

    // O^T += V^T P^T: MFMA (t, j) contracts keys 16t + 4*g4 + j
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* vr = &svw[(16 * t + 4 * g4 + j) * LD + l16 * DT];
        float vv[DT];
#pragma unroll
        for (int dt = 0; dt < DT; dt += 2) {
          const f32x2 w = *(const f32x2*)(vr + dt);
          vv[dt] = w[0];
          vv[dt + 1] = w[1];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = mfma(vv[dt], p[t][j], o[dt]);
      }
  }

  // the query's keys are spread over the four lane groups
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  if (SPLIT) {
    // merge the four waves' partial results for the shared 16 queries, through
    // LDS: per wave 16 maxima, 16 sums and 16 output rows (channel order as in o)
    __syncthreads();  // every wave is done with its blocks
    float* rm = sk;                    // [kWaves][16]
    float* rl = sk + kWaves * 16;      // [kWaves][16]
    float* ro = sk + 2 * kWaves * 16;  // [kWaves][16][D]
    if (g4 == 0) {
      rm[wave * 16 + l16] = m;
      rl[wave * 16 + l16] = lt;
    }
    float* my = ro + (wave * 16 + l16) * D + 4 * g4 * DT;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) my[i * DT + dt] = o[dt][i];
    __syncthreads();
    if (wave != 0) return;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, rm[w * 16 + l16]);
    const float msh = (mx == -INFINITY) ? 0.0f : mx;
    lt = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(rm[w * 16 + l16] - msh);
      lt += f * rl[w * 16 + l16];
      const float* src = ro + (w * 16 + l16) * D + 4 * g4 * DT;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][i] += f * src[i * DT + dt];
    }
  }
  if (!ok) return;
  const float inv = 1.0f / lt;
  // entry i of o[dt] is channel (4*g4 + i)*DT + dt
  float* op = (float*)a.o + qoff + 4 * g4 * DT;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int dt = 0; dt < DT; dt += 2) {
      const f32x2 w = {o[dt][i] * inv, o[dt + 1][i] * inv};
      *(f32x2*)(op + i * DT + dt) = w;
    }
}

template <int D, bool SPLIT>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.nblocks), block(kThreads);
  if (a.g.mode == NPA_MODE_STRIPS)
    hipLaunchKernelGGL((attn_f32_kernel<D, NPA_MODE_STRIPS, SPLIT>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, NPA_MODE_WINDOW, SPLIT>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

int attn_f32_block_m(int head_dim, bool split) {
  if (split) return (head_dim == 32 || head_dim == 64) ? kSplitQueries : 0;
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) ? kQueries : 0;
}

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, bool split, hipStream_t st) {
  if (split) return head_dim == 32 ? launch_d<32, true>(a, st) : launch_d<64, true>(a, st);
  if (head_dim == 32) return launch_d<32, false>(a, st);
  if (head_dim == 64) return launch_d<64, false>(a, st);
  return launch_d<128, false>(a, st);
}

}  // namespace npa
