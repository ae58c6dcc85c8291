// Partial-context patch attention, bf16 inputs, MFMA on gfx950.
//
// Method: multi-head scaled dot-product attention over the partial key set of
// each query tile -- own strip fresh plus a stale halo of neighbour rows
// ("Partially Conditioned Patch Parallelism ...", "What carries the
// argument"), or a clipped overlapping window ("ScaleDiff ...", "Approach").
// Flash-style: one pass over the tile's keys with a fixed softmax shift, so
// the score matrix never leaves registers and K/V are read in place from the
// fresh and stale buffers (never concatenated).
//
// Workgroup = WAVES waves (regular shape: 4 at d = 64, 8 at d = 128, 256
// queries; small-launch shape: 4 waves, 128 queries); each wave owns ROWS =
// 16*NT queries of one tile.  The workgroup walks the tile's keys in blocks
// of 64 staged through a double-buffered LDS tile (one barrier per block);
// each wave consumes a block as two 32-key steps.
//
// MFMA orientation (v_mfma_f32_16x16x32_bf16; lane l: column l%16, group
// g4 = l/16; A and B hold k = 8*g4 .. +8, D holds rows 4*g4 .. +4):
//   S^T = K * Q^T   A = K rows (16 keys),  B = Q^T (16 queries in columns)
//   O^T = V^T * P^T A = V^T (16 head dims), B = P^T (32 keys)
// With scores transposed, each lane holds keys of ONE query: row reductions
// are in-lane plus two lane swaps (v_permlane16_swap, v_permlane32_swap), and
// rescaling O^T by a per-query factor is in-lane.  Of the 16x16x32 and
// 32x32x16 bf16 MFMAs the smaller one touches half the accumulator registers
// per flop; on random bf16 data it sustains ~14% more under the board's power
// limit.  Within each 32-key step the K rows of the two 16-key score tiles
// are permuted (tile h, row r <- key 8*(r/4) + 4h + r%4), which puts the two
// tiles' accumulator entries of lane group g4 on keys 8*g4 .. 8*g4+7 -- the
// B-operand layout of the PV product -- so P goes from the score accumulators
// to the MFMA operand with no lane movement.  V^T fragments come from the
// row-major V tile through two ds_read_b64_tr_b16 of four key rows each.
//
// Softmax arithmetic is kept off the VALU wherever the MFMA can carry it:
//   * Q is multiplied by scale*log2(e) once at load (re-rounded to bf16), so
//     the product is already in the exp2 domain;
//   * the running shift -m enters as the C operand of the first S^T MFMA
//     (a persistent register tile), so p = exp2(acc) with no subtraction;
//   * the shift is the exact row max of the first 32 keys and never moves, so
//     the common path has no max, no rescale of O and no branch per query; if
//     a row sum ends outside [1, 2^60] (checked from the sums themselves) the
//     workgroup computes the true row maxima and runs the tile again with them;
//   * row sums run on the matrix core too: one more 16x16x32 MFMA per 32-key
//     step and 16-query tile, with an all-ones A operand and the packed bf16
//     P as B, leaves the query's sum in every accumulator entry -- the
//     denominator sums exactly the weights the numerator uses, with the same
//     fp32 accumulation.  At d = 64 that is one MFMA more per eight; the VALU
//     alternatives cost more (v_dot2c_f32_bf16 does not co-issue with MFMAs:
//     measured ~12 cycles per dot2c beside a dense MFMA stream, and the fp32
//     adds of the weights do not fit beside the exps).
// Loads and stores go through buffer descriptors: out-of-range keys and
// queries read zeros / drop their stores without branches.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "npa_internal.hpp"

namespace npa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kBN = 64;                  // keys per LDS block
constexpr uint32_t kOOB = 0x7FFFFFF0u;   // byte offset past every buffer's range
constexpr float kOverflow = 1.152921504606846976e18f;  // 2^60

// Workgroup shape per head size: NT = 16-query column tiles per wave, WAVES =
// waves per workgroup (all sharing the workgroup's K/V tiles), MINB =
// workgroups per CU the register budget is sized for.
//   regular (SMALL = false), two waves per SIMD: d = 64 takes 4 waves of 64
//     queries; d = 128 takes 8 waves of 32 -- its K/V tiles are twice as large
//     per query, and sharing them among more queries halves the copies per
//     MFMA.  256 queries per workgroup either way.
//   small-launch (SMALL = true): 128 queries per workgroup (4 waves of 32),
//     for calls whose regular grid would not fill the GPU twice: twice the
//     workgroups, each half as long, so the launch ends evenly; at d = 64 the
//     smaller register set fits three waves per SIMD.  On large grids it is
//     ~7% slower (each K/V tile serves half the queries).
template <int D, bool SMALL>
struct Cfg;
template <>
struct Cfg<64, false> {
  static constexpr int NT = 4, WAVES = 4, MINB = 2;
};
template <>
struct Cfg<128, false> {
  static constexpr int NT = 2, WAVES = 8, MINB = 1;
};
template <>
struct Cfg<64, true> {
  static constexpr int NT = 2, WAVES = 4, MINB = 3;
};
template <>
struct Cfg<128, true> {
  static constexpr int NT = 2, WAVES = 4, MINB = 2;
};

// j / d for 0 <= j < 2^24 via a float reciprocal and one correction step.
__device__ __forceinline__ int fast_div(int j, int d, float inv) {
  int q = (int)((float)j * inv);
  const int r = j - q * d;
  q += (r < 0) ? -1 : ((r >= d) ? 1 : 0);
  return q;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float max4(const f32x4& a) { return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// 16-byte chunk permutation of LDS row r (16 slots of 16 bytes span the 64
// banks).  The reads it serves:
//   K fragments, ds_read_b128: each 8 lanes read one chunk of rows
//     {0..3, 8..11} (+ 4h + 16j);
//   V^T fragments, ds_read_b64_tr_b16: each 32 lanes read two adjacent
//     chunks of rows {0..3, 8..11} (+ 32s + 16j), the fragment's second half
//     the same rows + 4.
// The masks depend on bits 0, 1 and 3 of the row only: rows r and r + 4 (the
// second score tile, the second half of a V^T fragment) share their mask, so
// those reads are the first ones' addresses plus an immediate offset and need
// no address registers of their own.
// d = 64 (two rows per 256 bytes): within each row parity the rows 0..3,
// 8..11 get XOR masks {0, 4, 2, 6}, all differing above bit 0, so both
// patterns hit distinct slots.  d = 128 (one row per 256 bytes): the eight
// rows get the eight even masks {0, 4, 8, 12, 2, 6, 10, 14}, distinct above
// bit 0 (a pair of adjacent chunks stays a pair).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 64) return ((r & 3) << 1) ^ (((r >> 3) & 1) << 1);
  return ((r & 3) << 2) | (((r >> 3) & 1) << 1);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Key blocks never straddle two key runs: every run starts on a 64-key block
// boundary (the padding keys are masked), so which buffer a block comes from
// is a per-block scalar.
__device__ __forceinline__ int pad_blocks(int n) { return (n + kBN - 1) / kBN; }

// Token of key j of run r (strips: runs are contiguous; windows: one run of rows).
template <int MODE>
__device__ __forceinline__ int run_token(const Run& r, int j, float inv_len) {
  if (MODE == NPA_MODE_STRIPS) return r.start + j;
  const int row = fast_div(j, r.row_len, inv_len);
  return r.start + row * r.pitch + (j - row * r.row_len);
}

// exp2 of the 8 accumulator entries of one lane for a 32-key step (tiles 0
// and 1), packed to bf16 in key order as the PV B operand.
__device__ __forceinline__ void exp_pack(const f32x4& a0, const f32x4& a1, float shift, bf16x8& p) {
  f32x8 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = __builtin_amdgcn_exp2f(a0[i] - shift);
    e[4 + i] = __builtin_amdgcn_exp2f(a1[i] - shift);
  }
  p = __builtin_convertvector(e, bf16x8);
}

// Same without a shift argument (the common path: the shift is inside acc).
__device__ __forceinline__ void exp_pack0(const f32x4& a0, const f32x4& a1, bf16x8& p) {
  f32x8 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = __builtin_amdgcn_exp2f(a0[i]);
    e[4 + i] = __builtin_amdgcn_exp2f(a1[i]);
  }
  p = __builtin_convertvector(e, bf16x8);
}


// PARTIAL: some key run of the plan is not a multiple of 64 keys, so some
// blocks end inside the padding and need masking (instantiated only then).
// Kernel modes: strips, windows, and windows with text tokens (joint
// attention; a separate instantiation so that plain windows keep the
// single-run cursor).
constexpr int kModeJoint = 2;

// Every 32-bit word of the kernel arguments into scalar registers at once: one
// batch of scalar loads at the start instead of a chain of dependent ones
// spread over the prologue's branches.
template <typename T>
__device__ __forceinline__ void load_args_now(const T& a) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&a);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"s"(w[i]));
}

template <int D, int MODE, bool PARTIAL, bool SMALL>
__global__ __launch_bounds__((64 * Cfg<D, SMALL>::WAVES), (Cfg<D, SMALL>::MINB)) void attn_bf16_kernel(
    const AttnArgs a) {
  load_args_now(a);
  constexpr bool kWin = MODE != NPA_MODE_STRIPS;  // map tiles are 2-D windows
  constexpr bool kRuns = MODE != NPA_MODE_WINDOW;  // more than one key run per tile
  constexpr int kWaves = Cfg<D, SMALL>::WAVES;
  constexpr int kThreads = 64 * kWaves;
  constexpr int NT = Cfg<D, SMALL>::NT;
  constexpr int ROWS = 16 * NT;
  constexpr int BM = kWaves * ROWS;
  constexpr int KS = D / 32;    // k-steps of S^T (32 head dims each)
  constexpr int DT = D / 16;    // 16-wide head-dim tiles of O^T
  constexpr int LDR = D;        // LDS row pitch in elements (unpadded; chunks XOR-swizzled)
  constexpr int CPR = D / 8;    // 16-byte chunks per key row
  constexpr int CH = kBN * CPR / kThreads;  // DMA instructions per thread per tile
  static_assert(CH * kThreads == kBN * CPR, "chunking");

  // Two K and two V tiles as four separate objects: the copy into one tile is
  // then provably disjoint from the reads of the other, so waiting for it is
  // left to the explicit wait before each barrier.
  __shared__ __attribute__((aligned(16))) __bf16 sk0[kBN * LDR];
  __shared__ __attribute__((aligned(16))) __bf16 sk1[kBN * LDR];
  __shared__ __attribute__((aligned(16))) __bf16 sv0[kBN * LDR];
  __shared__ __attribute__((aligned(16))) __bf16 sv1[kBN * LDR];

  // wave index as a uniform value: everything derived from it (LDS tile slots,
  // the DMA destinations) stays in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;

  const BlockCoord bc = decode_block(a, blockIdx.x, true);
  const int qb = bc.qb, tile = bc.tile, head = bc.head, b = bc.b;

  const TileRuns tr = tile_runs(a.g, tile);
  const int nq = tr.q.count();
  const int64_t bh = (int64_t)b * a.sb + (int64_t)head * a.sh;
  const float inv_qlen = 1.0f / (float)tr.q.row_len;
  const float inv_klen = 1.0f / (float)tr.k[0].row_len;
  const uint32_t sn2 = (uint32_t)a.sn * 2u;  // token stride in bytes

  const rsrc_t rq = make_rsrc((const __bf16*)a.q + bh, a.range_bytes);
  const __bf16* kf_base = (const __bf16*)a.kf + bh;
  const __bf16* vf_base = (const __bf16*)a.vf + bh;
  const __bf16* ks_base = (const __bf16*)a.ks + bh;
  const __bf16* vs_base = (const __bf16*)a.vs + bh;
  const rsrc_t ro = make_rsrc((__bf16*)a.o + bh, a.range_bytes);

  // ---- Q^T fragments, pre-multiplied by scale*log2(e):
  //      lane (query l16, group g4) holds dims 32*ks + 8*g4 .. +8
  bf16x8 qf[NT][KS];
  uint32_t qoff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int qi = qb * BM + wave * ROWS + nt * 16 + l16;
    uint32_t off = kOOB;
    if (qi < nq) {
      int tok;
      if (MODE == NPA_MODE_STRIPS) {
        tok = tr.q.start + qi;
      } else {
        const int r = fast_div(qi, tr.q.row_len, inv_qlen);
        tok = tr.q.start + r * tr.q.pitch + (qi - r * tr.q.row_len);
      }
      off = (uint32_t)tok * sn2;
    }
    qoff[nt] = off;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, off + ks * 64 + g4 * 16, 0, 0);
      f32x8 f = __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] *= a.c;
      qf[nt][ks] = __builtin_convertvector(f, bf16x8);
    }
  }

  // ---- K/V tiles go from HBM straight into LDS (buffer_load ... lds): one
  // instruction fills 1 KiB, lane L's 16 bytes landing at byte 16*L.  Each lane
  // picks the global chunk that belongs at its slot, so the tile is stored
  // row-major with the 16-byte chunks of row r XOR-permuted by swz(r); keys past
  // the end of the set read zeros (out-of-range offset).
  //
  // The slot a lane fills is the same in every block: key row krow_c[r] of the
  // block, at byte lane_off[r] from the block's first key when the block's keys
  // are consecutive tokens.  Per block only uniform values change, and they are
  // kept in a cursor that advances one block per fetch (blocks are always
  // fetched in order 0, 1, ..., nkb-1): the key run, the keys of the run left
  // from the block's first key (the block's valid count when below 64), that
  // key's byte offset and, in a window, its column; keys of the block at or
  // past lim1 (lim2) lie one (two) window rows further down.
  int krow_c[CH];
  uint32_t lane_off[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int pos = (wave * CH + r) * 64 + lane;  // chunk slot in the tile
    const int row = pos / CPR, slot = pos % CPR;
    krow_c[r] = row;
    lane_off[r] = (uint32_t)row * sn2 + (uint32_t)((slot ^ swz<D>(row)) * 16);
  }
  // Window mode: run 0 is the window (rows of cur_len keys, pitch apart) or,
  // in the text tile, every stored token; run 1 is the text tokens.  A run
  // of one row, and every run after the first, is contiguous: cur_len is then
  // kContig and the block never crosses a row.
  constexpr int kContig = 1 << 29;
  const uint32_t wrap_add = (uint32_t)(tr.k[0].pitch - tr.k[0].row_len) * sn2;
  const uint32_t step_bytes = (uint32_t)kBN * sn2;
  int cur_run = 0, cur_left = 0, cur_off = 0, cur_c0 = 0, cur_len = kContig;
  uint32_t cur_base = 0;
  auto cursor_reset = [&]() __attribute__((always_inline)) {
    cur_run = 0;
    cur_left = tr.nk[0];
    cur_off = 0;
    cur_c0 = 0;
    cur_len = (kWin && tr.k[0].rows > 1) ? tr.k[0].row_len : kContig;
    cur_base = (uint32_t)tr.k[0].start * sn2;
  };
  auto cursor_next = [&]() __attribute__((always_inline)) {
    cur_left -= kBN;
    cur_off += kBN;
    if (kRuns && cur_left <= 0) {
      // next non-empty key run (strips: the stale halos; joint: the text tokens)
      cur_run = (cur_run == 0 && tr.nk[1] > 0) ? 1 : 2;
      cur_left = cur_run == 1 ? tr.nk[1] : tr.nk[2];
      cur_off = 0;
      cur_c0 = 0;
      cur_len = kContig;
      cur_base = (uint32_t)(cur_run == 1 ? tr.k[1].start : tr.k[2].start) * sn2;
    } else {
      cur_base += step_bytes;
      if (kWin) {
        cur_c0 += kBN;
        while (cur_c0 >= cur_len) {
          cur_c0 -= cur_len;
          cur_base += wrap_add;
        }
      }
    }
  };
  // Copies of the block the cursor is on: 2*CH buffer_load ... lds per wave
  // (the K and the V chunk of each of its CH chunk slots); fetch_offsets
  // computes the lanes' source offsets once per block.
  auto fetch_offsets = [&](uint32_t (&off)[CH]) __attribute__((always_inline)) {
    const bool general = kWin && cur_len < 32;
    const int lim1 = kWin ? cur_len - cur_c0 : kBN;
    const int lim2 = kWin ? lim1 + cur_len : kBN;
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int row = krow_c[r];
      if (general) {
        // narrow windows (run 0 only): a block may cross more than two window rows
        off[r] = kOOB;
        if (row < cur_left)
          off[r] = (uint32_t)run_token<MODE>(tr.k[0], cur_off + row, inv_klen) * sn2 + (lane_off[r] - (uint32_t)row * sn2);
      } else {
        off[r] = cur_base + lane_off[r];
        if (kWin) off[r] += (row >= lim1 ? wrap_add : 0u) + (row >= lim2 ? wrap_add : 0u);
        if (PARTIAL && row >= cur_left) off[r] = kOOB;
      }
    }
  };
  auto fetch_part = [&](int r, bool is_v, uint32_t voff, __bf16* skd, __bf16* svd) __attribute__((always_inline)) {
    // runs 1 and 2 are the stale halos; the descriptor is built from the chosen
    // base pointer (a select between two descriptors would be lowered through memory)
    const bool stale = MODE == NPA_MODE_STRIPS && cur_run != 0;
    const __bf16* src = is_v ? (stale ? vs_base : vf_base) : (stale ? ks_base : kf_base);
    const rsrc_t rs = make_rsrc(src, a.range_bytes);
    lds_ptr dst = (lds_ptr)&(is_v ? svd : skd)[(wave * CH + r) * 512];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
  };
  auto fetch = [&](__bf16* skd, __bf16* svd) __attribute__((always_inline)) {
    uint32_t off[CH];
    fetch_offsets(off);
#pragma unroll
    for (int j = 0; j < 2 * CH; ++j) fetch_part(j >> 1, j & 1, off[j >> 1], skd, svd);
  };

  f32x4 o[DT][NT];
  f32x4 shift[NT];  // -m in every entry: C operand of the first S^T MFMA
  f32x4 l[NT];      // row sums, from the ones MFMA: every entry holds the query's sum
  const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};

  // K row this lane feeds into the S^T tile h (0, 1) of a 32-key step: rows
  // are permuted so that the tiles' accumulator entries of lane group g4 are
  // the step's keys 8*g4 + 4h .. +4 -- together the B-operand layout of the
  // PV product (keys 8*g4 .. +8).
  const int krow0 = 8 * (l16 >> 2) + (l16 & 3);
  // ds_read_b64_tr_b16 source pattern for the V^T fragments: within each
  // 16-lane group, lanes 4r..4r+3 address 16 consecutive dims of key row r
  const int vrow = 8 * g4 + (l16 >> 2);
  const int vcol = 4 * (l16 & 3);
  const int nkb = pad_blocks(tr.nk[0]) + pad_blocks(tr.nk[1]) + pad_blocks(tr.nk[2]);

  // S^T of 32-key step s of the block in skb: tiles h = 0, 1 (C operand: the
  // shift tile, or zero for raw scores)
  auto scores_raw = [&](const __bf16* skb, int s, f32x4 (&sc)[2][NT], bool raw) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = 32 * s + krow0 + 4 * h;
        const bf16x8 kf = *(const bf16x8*)&skb[row * LDR + (((4 * ks + g4) ^ swz<D>(row)) * 8)];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          sc[h][nt] = mfma16(kf, qf[nt][ks], ks == 0 ? (raw ? f32x4{} : shift[nt]) : sc[h][nt]);
      }
  };

  // Exact row max of the whole tile (the rare second pass only): S^T with a
  // zero shift, reduced over every key.
  auto row_max = [&](float (&mx)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mx[nt] = -INFINITY;
    auto block = [&](int kb, const __bf16* skb, __bf16* skn, __bf16* svn) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int valid = cur_left;  // the cursor is on block kb
      if (kb + 1 < nkb) {
        cursor_next();
        fetch(skn, svn);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        f32x4 sc[2][NT];
        scores_raw(skb, s, sc, true);
        const int t = valid - 32 * s - 8 * g4;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * h + i < t)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) mx[nt] = fmaxf(mx[nt], sc[h][nt][i]);
      }
    };
    cursor_reset();
    fetch(sk0, sv0);
    for (int kb = 0; kb < nkb; kb += 2) {
      block(kb, sk0, sk1, sv1);
      if (kb + 1 < nkb) block(kb + 1, sk1, sk0, sv0);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mx[nt] = quad_max(mx[nt]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the tiles are free again
  };

  // One pass over the tile's keys with a fixed shift: p = exp2(acc), no max and
  // no rescale inside the loop.  preset=false: the shift is the exact row max
  // of the first 32 keys.  preset=true: the shift was set beforehand (the true
  // row max of the tile).
  //
  // Each 64-key block is one straight-line body of two 32-key steps,
  // specialised at compile time for the first block (FIRST: scores unshifted,
  // the max is taken): the score MFMAs of both steps are issued before the
  // first step's exp work, so the second step's MFMAs run while the VALU does
  // the first step's softmax.  Blocks that end inside a run's padding take the
  // same body.
  auto block = [&](int kb, const __bf16* skb, const __bf16* svb, __bf16* skn, __bf16* svn,
                   auto first_tag) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // this wave's copies into tile kb are done; after the barrier, everyone's are
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int valid = cur_left;  // the cursor is on block kb
    // a block that ends inside its run's padding (at most one per run)
    const bool part = PARTIAL && valid < kBN;
    if (kb + 1 < nkb) {
      cursor_next();
      fetch(skn, svn);
    }

    // Keys past the end of their run: entry i of tile h in lane group g4 is
    // key 8*g4 + 4h + i of step s; their scores become -inf.  Only blocks that
    // end inside a run's padding take this step, between the scheduled
    // regions, so full blocks and partial ones share one body.
    auto mask = [&](int s, f32x4 (&sc)[2][NT]) __attribute__((always_inline)) {
      const int t = valid - 32 * s - 8 * g4;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * h + i >= t)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sc[h][nt][i] = -INFINITY;
    };
    // O^T += V^T P^T over step s: per 16-dim tile one V^T fragment (keys
    // 8*g4 .. +8 of the step, from two transposed reads of four key rows);
    // then the row sums: ones * P^T adds the step's weights of each query
    auto pv = [&](int s, const bf16x8 (&p)[NT]) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int r0 = 32 * s + vrow, r1 = r0 + 4;
        const int col = 16 * dt + vcol;  // multiple of 4: one 8-byte half of a chunk
        const __bf16* p0p = &svb[r0 * LDR + (((col >> 3) ^ swz<D>(r0)) * 8) + (col & 7)];
        const __bf16* p1p = &svb[r1 * LDR + (((col >> 3) ^ swz<D>(r1)) * 8) + (col & 7)];
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0p);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1p);
        const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[dt][nt] = mfma16(vf, p[nt], o[dt][nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) l[nt] = mfma16(ones, p[nt], l[nt]);
    };

    f32x4 s0[2][NT], s1[2][NT];
    bf16x8 pa[NT], pb[NT];
    scores_raw(skb, 0, s0, FIRST);
    if (part) mask(0, s0);
    if (FIRST) {
      // the exact row max of the first 32 keys becomes the shift; step 1 then
      // takes the ordinary path with the shift inside its MFMA
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float m = fmaxf(max4(s0[0][nt]), max4(s0[1][nt]));
        m = quad_max(m);
        exp_pack(s0[0][nt], s0[1][nt], m, pa[nt]);
        shift[nt] = f32x4{-m, -m, -m, -m};
      }
      pv(0, pa);
      __builtin_amdgcn_sched_barrier(0);
      scores_raw(skb, 1, s1, false);
      if (part) mask(1, s1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) exp_pack0(s1[0][nt], s1[1][nt], pb[nt]);
      pv(1, pb);
      return;
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 1's score MFMAs run while the VALU turns step 0's scores into
    // weights (one region: the compiler interleaves them)
    scores_raw(skb, 1, s1, false);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) exp_pack0(s0[0][nt], s0[1][nt], pa[nt]);
    __builtin_amdgcn_sched_barrier(0);
    if (part) mask(1, s1);
    __builtin_amdgcn_sched_barrier(0);
    // step 0's PV MFMAs run while the VALU does step 1's weights (one region)
    pv(0, pa);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) exp_pack0(s1[0][nt], s1[1][nt], pb[nt]);
    __builtin_amdgcn_sched_barrier(0);
    pv(1, pb);
  };
  auto pass = [&](bool preset) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][nt] = f32x4{};
      l[nt] = f32x4{};
    }
    cursor_reset();
    fetch(sk0, sv0);
    if (preset)
      block(0, sk0, sv0, sk1, sv1, std::false_type{});
    else
      block(0, sk0, sv0, sk1, sv1, std::true_type{});
    for (int kb = 1; kb < nkb; kb += 2) {
      block(kb, sk1, sv1, sk0, sv0, std::false_type{});
      if (kb + 1 < nkb) block(kb + 1, sk0, sv0, sk1, sv1, std::false_type{});
    }
  };

  // The fast pass is kept unless some row sum leaves [1, 2^60] -- a later key
  // beating the first keys' max by ~60 in log2 units, or a non-finite input.
  // Then the workgroup computes every row's true max and runs the pass again
  // with that shift, where every weight is <= 1 and the max itself weighs 1.
  __shared__ int redo;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) shift[nt] = f32x4{};
  // At most two passes, one copy of the pass code: the second pass runs only
  // when the first one's row sums left [1, 2^60].
  bool preset = false;
  for (;;) {
    if (tid == 0) redo = 0;
    pass(preset);
    if (preset) break;
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bad |= !(l[nt][0] <= kOverflow);
    __syncthreads();
    if (wave_any(bad) && lane == 0) redo = 1;  // every writer stores 1
    __syncthreads();
    if (!redo) break;
    float mx[NT];
    row_max(mx);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) shift[nt] = f32x4{-mx[nt], -mx[nt], -mx[nt], -mx[nt]};
    preset = true;
  }

  // ---- normalise and store: lane (query l16, group g4) holds dims 16dt + 4g4 .. +4
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float inv = 1.0f / l[nt][0];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = o[dt][nt][i] * inv;
      const bf16x4 hv = __builtin_convertvector(v, bf16x4);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, hv), ro, qoff[nt] + (16 * dt + 4 * g4) * 2, 0,
                                            0);
    }
  }
}

}  // namespace

int attn_bf16_block_m(int head_dim, bool small) {
  if (head_dim == 64) return small ? 16 * Cfg<64, true>::WAVES * Cfg<64, true>::NT : 16 * Cfg<64, false>::WAVES * Cfg<64, false>::NT;
  if (head_dim == 128) return small ? 16 * Cfg<128, true>::WAVES * Cfg<128, true>::NT : 16 * Cfg<128, false>::WAVES * Cfg<128, false>::NT;
  return 0;
}

int attn_bf16_per_cu(int head_dim, bool small) {
  if (head_dim == 64) return small ? Cfg<64, true>::MINB : Cfg<64, false>::MINB;
  if (head_dim == 128) return small ? Cfg<128, true>::MINB : Cfg<128, false>::MINB;
  return 0;
}

template <int D, int MODE, bool SMALL>
void launch_dm(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.nblocks), block(64 * Cfg<D, SMALL>::WAVES);
  if (a.partial)
    hipLaunchKernelGGL((attn_bf16_kernel<D, MODE, true, SMALL>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, MODE, false, SMALL>), grid, block, 0, st, a);
}

template <int D, bool SMALL>
void launch_d(const AttnArgs& a, hipStream_t st) {
  const int mode = a.g.mode == NPA_MODE_STRIPS ? NPA_MODE_STRIPS : (a.g.T > 0 ? kModeJoint : NPA_MODE_WINDOW);
  if (mode == NPA_MODE_STRIPS)
    launch_dm<D, NPA_MODE_STRIPS, SMALL>(a, st);
  else if (mode == NPA_MODE_WINDOW)
    launch_dm<D, NPA_MODE_WINDOW, SMALL>(a, st);
  else
    launch_dm<D, kModeJoint, SMALL>(a, st);
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool small, hipStream_t st) {
  if (head_dim == 64) {
    if (small)
      launch_d<64, true>(a, st);
    else
      launch_d<64, false>(a, st);
  } else {
    if (small)
      launch_d<128, true>(a, st);
    else
      launch_d<128, false>(a, st);
  }
  return hipGetLastError();
}

}  // namespace npa
