// Host check of the workgroup -> (query block, tile, head, batch) map of the
// attention kernels: every map tile's query blocks, every (batch, head), and
// the text tile's blocks are each computed by exactly one workgroup, with and
// without the XCD dealing and the interior-first tile order; that order lists
// the tiles by class.  Prints "ok <cases>" or the first failure.
#include <cstdio>
#include <vector>

#include "npa_internal.hpp"

using namespace npa;

static bool check(int mode, int B, int Hh, int nr, int nc, int qblocks, int text_qblocks, bool remap, int lf) {
  AttnArgs a{};
  a.B = B;
  a.Hh = Hh;
  a.g.mode = mode;
  a.g.tiles_x = nc;
  a.g.n_img = mode == NPA_MODE_STRIPS ? nr : nr * nc;
  a.qblocks = qblocks;
  a.text_qblocks = text_qblocks;
  a.text_blocks = B * Hh * text_qblocks;
  a.nblocks = a.text_blocks + B * Hh * a.g.n_img * qblocks;
  a.largest_first = (mode == NPA_MODE_WINDOW && nr >= 3 && nc >= 3) ? lf : 0;
  set_divisors(a);
  const int tiles = a.g.n_img + (text_qblocks > 0);
  std::vector<int> seen((size_t)B * Hh * tiles * (qblocks > text_qblocks ? qblocks : text_qblocks), 0);
  for (int i = 0; i < a.nblocks; ++i) {
    const BlockCoord c = decode_block(a, i, remap);
    const int nq = c.tile == a.g.n_img ? text_qblocks : qblocks;
    if (c.b < 0 || c.b >= B || c.head < 0 || c.head >= Hh || c.tile < 0 || c.tile >= tiles || c.qb < 0 ||
        c.qb >= nq) {
      std::printf("out of range: mode %d B %d Hh %d grid %dx%d qblocks %d text %d remap %d block %d -> "
                  "qb %d tile %d head %d b %d\n",
                  mode, B, Hh, nr, nc, qblocks, text_qblocks, remap, i, c.qb, c.tile, c.head, c.b);
      return false;
    }
    const size_t slot = (((size_t)c.b * Hh + c.head) * tiles + c.tile) * (seen.size() / ((size_t)B * Hh * tiles)) + c.qb;
    if (seen[slot]++) {
      std::printf("twice: mode %d B %d Hh %d grid %dx%d qblocks %d text %d remap %d block %d\n", mode, B, Hh, nr,
                  nc, qblocks, text_qblocks, remap, i);
      return false;
    }
  }
  return true;
}

// tile_by_class lists a head's tiles interior, then edge, then corner.
static bool check_classes() {
  for (int tx = 3; tx <= 9; ++tx)
    for (int ty = 3; ty <= 9; ++ty) {
      AttnArgs a{};
      a.g.tiles_x = tx;
      a.g.n_img = tx * ty;
      a.B = a.Hh = a.qblocks = 1;
      set_divisors(a);
      const int n0 = (tx - 2) * (ty - 2), n1 = 2 * (tx - 2) + 2 * (ty - 2);
      for (int r = 0; r < tx * ty; ++r) {
        const int t = tile_by_class(a, r), ti = t / tx, tj = t % tx;
        const int cls = (ti == 0 || ti == ty - 1) + (tj == 0 || tj == tx - 1);
        if (cls != (r < n0 ? 0 : (r < n0 + n1 ? 1 : 2))) {
          std::printf("tile class: grid %dx%d rank %d -> tile %d\n", ty, tx, r, t);
          return false;
        }
      }
    }
  return true;
}

int main() {
  int cases = 0;
  if (!check_classes()) return 1;
  const int Bs[] = {1, 2, 3}, Hs[] = {1, 5, 10, 24}, qbs[] = {1, 4, 16, 7};
  for (int mode = 0; mode < 2; ++mode)
    for (int B : Bs)
      for (int Hh : Hs)
        for (int nr = 1; nr <= 9; ++nr)
          for (int nc = 1; nc <= (mode == NPA_MODE_STRIPS ? 1 : 9); ++nc)
            for (int qb : qbs)
              for (int tq = 0; tq <= (mode == NPA_MODE_STRIPS ? 0 : 2); ++tq)
                for (int remap = 0; remap < 2; ++remap)
                  for (int lf = 0; lf < 2; ++lf) {
                    if (!check(mode, B, Hh, nr, nc, qb, tq, remap, lf)) return 1;
                    ++cases;
                  }
  std::printf("ok %d\n", cases);
  return 0;
}
