// Partial-context patch attention, bf16 inputs, MFMA on gfx950.
//
// Method: multi-head scaled dot-product attention over the partial key set of
// each query tile -- own strip fresh plus a stale halo of neighbour rows
// ("Partially Conditioned Patch Parallelism ...", "What carries the
// argument"), or a clipped overlapping window ("ScaleDiff ...", "Approach").
// Flash-style: one pass over the tile's keys with an online softmax, so the
// score matrix never leaves registers and K/V are read in place from the
// fresh and stale buffers (never concatenated).
//
// Workgroup = 4 waves; each wave owns ROWS = 32*NT queries of one tile, and
// the workgroup walks the tile's keys in blocks of 64, staged through a
// double-buffered LDS tile (one barrier per block).
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16, lane l: column l%32, half g=l/32):
//   S^T = K * Q^T   A = K rows (keys),  B = Q^T (queries in columns)
//   O^T = V^T * P^T A = V^T (head dims), B = P^T
// With scores transposed, each lane holds 32 keys of ONE query, so the row max
// and row sum are in-lane reductions plus one exchange with lane l^32
// (v_permlane32_swap), and rescaling O^T by a per-query factor is in-lane.
// K rows are loaded in the order pi(r) = r with bits 2 and 3 swapped, which
// makes the accumulator entries j=0..7 of lane half g hold keys 8g..8g+7 --
// exactly the B-operand layout the PV product needs, so P goes from the score
// accumulator to the MFMA operand without any lane movement.  V^T fragments
// come from the row-major V tile through ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>

#include "npa_internal.hpp"

namespace npa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;  // keys per block

template <int D>
struct Cfg;
template <>
struct Cfg<64> {
  static constexpr int NT = 2;  // 64 queries per wave
};
template <>
struct Cfg<128> {
  static constexpr int NT = 1;  // 32 queries per wave
};

// Blocks are dealt to the 8 XCDs round-robin; remap so that each XCD runs one
// contiguous range of logical blocks (all query blocks of a tile share the
// tile's K/V through that XCD's L2).
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = i & 7, k = i >> 3;
  return (x < rem) ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// j / d for 0 <= j < 2^24 via a float reciprocal and one correction step.
__device__ __forceinline__ int fast_div(int j, int d, float inv) {
  int q = (int)((float)j * inv);
  const int r = j - q * d;
  q += (r < 0) ? -1 : ((r >= d) ? 1 : 0);
  return q;
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Token of the j-th key of the tile and which buffer (0 fresh, 1 stale) holds it.
template <int MODE>
__device__ __forceinline__ int key_token(const TileRuns& t, int j, float inv_len, int& src) {
  if (MODE == NPA_MODE_STRIPS) {
    if (j < t.nk[0]) {
      src = 0;
      return t.k[0].start + j;
    }
    j -= t.nk[0];
    src = 1;
    if (j < t.nk[1]) return t.k[1].start + j;
    return t.k[2].start + (j - t.nk[1]);
  } else {
    src = 0;
    const int r = fast_div(j, t.k[0].row_len, inv_len);
    return t.k[0].start + r * t.k[0].pitch + (j - r * t.k[0].row_len);
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(const AttnArgs a) {
  constexpr int NT = Cfg<D>::NT;
  constexpr int ROWS = 32 * NT;
  constexpr int BM = kWaves * ROWS;
  constexpr int MT = kBN / 32;  // 32-key tiles per block
  constexpr int KS = D / 16;    // k-steps of S^T
  constexpr int DT = D / 32;    // 32-wide head-dim tiles of O^T
  constexpr int PK = kBN / 16;  // k-steps of O^T
  constexpr int LDR = D + 8;    // LDS row pitch in elements (16-byte pad)
  constexpr int CPR = D / 8;    // 16-byte chunks per key row
  constexpr int CH = kBN * CPR / kThreads;
  static_assert(CH * kThreads == kBN * CPR, "chunking");

  __shared__ __attribute__((aligned(16))) __bf16 sk[2][kBN * LDR];
  __shared__ __attribute__((aligned(16))) __bf16 sv[2][kBN * LDR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  const int bid = xcd_remap(blockIdx.x, a.nblocks);
  const int qb = bid % a.qblocks;
  int rest = bid / a.qblocks;
  const int tile = rest % a.g.n_tiles;
  rest /= a.g.n_tiles;
  const int head = rest % a.Hh;
  const int b = rest / a.Hh;

  const TileRuns tr = tile_runs(a.g, tile);
  const int nq = tr.q.count();
  const int nk = tr.nk[0] + tr.nk[1] + tr.nk[2];
  const int64_t bh = (int64_t)b * a.sb + (int64_t)head * a.sh;
  const float inv_qlen = 1.0f / (float)tr.q.row_len;
  const float inv_klen = 1.0f / (float)tr.k[0].row_len;

  const __bf16* qp = (const __bf16*)a.q;
  const __bf16* kfp = (const __bf16*)a.kf;
  const __bf16* vfp = (const __bf16*)a.vf;
  const __bf16* ksp = (const __bf16*)a.ks;
  const __bf16* vsp = (const __bf16*)a.vs;

  // ---- Q^T fragments: lane (query l32, half g) holds dims 16*ks + 8g .. +8
  bf16x8 qf[NT][KS];
  int64_t qoff[NT];
  bool qok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int qi = qb * BM + wave * ROWS + nt * 32 + l32;
    qok[nt] = qi < nq;
    int tok = 0;
    if (qok[nt]) {
      if (MODE == NPA_MODE_STRIPS) {
        tok = tr.q.start + qi;
      } else {
        const int r = fast_div(qi, tr.q.row_len, inv_qlen);
        tok = tr.q.start + r * tr.q.pitch + (qi - r * tr.q.row_len);
      }
    }
    qoff[nt] = bh + (int64_t)tok * a.sn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qok[nt]) v = *(const u32x4*)(qp + qoff[nt] + ks * 16 + g * 8);
      qf[nt][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- K/V staging registers
  u32x4 kr[CH], vr[CH];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int c = tid + r * kThreads;
      const int key = c / CPR, dc = c % CPR;
      const int kidx = kb * kBN + key;
      u32x4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (kidx < nk) {
        int src;
        const int tok = key_token<MODE>(tr, kidx, inv_klen, src);
        const int64_t off = bh + (int64_t)tok * a.sn + dc * 8;
        kk = *(const u32x4*)((src ? ksp : kfp) + off);
        vv = *(const u32x4*)((src ? vsp : vfp) + off);
      }
      kr[r] = kk;
      vr[r] = vv;
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int c = tid + r * kThreads;
      const int key = c / CPR, dc = c % CPR;
      *(u32x4*)&sk[buf][key * LDR + dc * 8] = kr[r];
      *(u32x4*)&sv[buf][key * LDR + dc * 8] = vr[r];
    }
  };

  f32x16 o[DT][NT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[dt][nt] = f32x16{};
  float m[NT], l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.0f;
  }

  // row of the K tile this lane feeds into the S^T product: bits 2,3 of l32 swapped
  const int krow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  // ds_read_b64_tr_b16 source address pattern for the V^T fragments
  const int vkey = 8 * g + ((lane & 15) >> 2);
  const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const float c = a.c;

  const int nkb = (nk + kBN - 1) / kBN;
  fetch(0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    stage(buf);
    __syncthreads();
    if (kb + 1 < nkb) fetch(kb + 1);

    // ---- S^T = K Q^T
    f32x16 s[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[mt][nt] = f32x16{};
    const __bf16* skb = sk[buf];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *(const bf16x8*)&skb[(mt * 32 + krow) * LDR + ks * 16 + g * 8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[mt][nt] = mfma(kf, qf[nt][ks], s[mt][nt]);
      }
    }

    // ---- mask keys past the end of the tile's key set (last block only)
    if (kb * kBN + kBN > nk) {
      const int base = nk - kb * kBN;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kl = 32 * mt + (j < 8 ? 8 * g + j : 16 + 8 * g + (j - 8));
          if (kl >= base)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) s[mt][nt][j] = -INFINITY;
        }
    }

    // ---- online softmax (exp2 domain); P packed straight into PV operands
    bf16x8 pf[NT][PK];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = s[0][nt][0];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mt][nt][j]);
      mx = pair_max(mx);
      const float mn = fmaxf(m[nt], mx);
      const float alpha = __builtin_amdgcn_exp2f((m[nt] - mn) * c);
      const float mc = mn * c;
      float rs = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 pv;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][8 * h2 + i], c, -mc));
            rs += p;
            pv[i] = p;
          }
          pf[nt][2 * mt + h2] = __builtin_convertvector(pv, bf16x8);
        }
      }
      l[nt] = l[nt] * alpha + rs;
      m[nt] = mn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][nt] *= alpha;
    }

    // ---- O^T += V^T P^T
    const __bf16* svb = sv[buf];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) {
        const __bf16* p0 = &svb[(16 * kk + vkey) * LDR + 32 * dt + vdim];
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * LDR));
        const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[dt][nt] = mfma(vf, pf[nt][kk], o[dt][nt]);
      }
    }
  }

  // ---- normalise and store: lane (query, g) holds dims 32dt + 8*j4 + 4g .. +4
  __bf16* op = (__bf16*)a.o;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float inv = 1.0f / pair_sum(l[nt]);
    if (!qok[nt]) continue;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = o[dt][nt][4 * j4 + i] * inv;
        *(bf16x4*)(op + qoff[nt] + 32 * dt + 8 * j4 + 4 * g) = __builtin_convertvector(v, bf16x4);
      }
  }
}

}  // namespace

int attn_bf16_block_m(int head_dim) {
  if (head_dim == 64) return kWaves * 32 * Cfg<64>::NT;
  if (head_dim == 128) return kWaves * 32 * Cfg<128>::NT;
  return 0;
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int /*block_m*/, hipStream_t st) {
  const dim3 grid(a.nblocks), block(kThreads);
  if (head_dim == 64) {
    if (a.g.mode == NPA_MODE_STRIPS)
      hipLaunchKernelGGL((attn_bf16_kernel<64, NPA_MODE_STRIPS>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64, NPA_MODE_WINDOW>), grid, block, 0, st, a);
  } else {
    if (a.g.mode == NPA_MODE_STRIPS)
      hipLaunchKernelGGL((attn_bf16_kernel<128, NPA_MODE_STRIPS>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<128, NPA_MODE_WINDOW>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace npa
