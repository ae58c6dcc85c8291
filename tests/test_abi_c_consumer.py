"""The C ABI from plain C: a program compiled with gcc against include/npa.h and
linked to libnpa.so calls the host-only entry points (planner, useful flops,
argument validation) -- no GPU, no Python in between -- and its answers are
compared with the oracle's."""
import os
import subprocess
import tempfile

import pytest

from oracle import attention as A
from partial_context_patch_amd import npa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "npa.h"

static void layout(npa_layout_t* L, int b, int h, int d, int H, int W) {
  memset(L, 0, sizeof *L);
  L->batch = b; L->heads = h; L->head_dim = d; L->map_h = H; L->map_w = W;
  L->stride_h = d; L->stride_n = (long long)h * d; L->stride_b = (long long)H * W * h * d;
  L->dtype = NPA_BF16; L->scale = 0.0f;
}

int main(void) {
  npa_layout_t L;
  npa_halo_t h;
  int32_t n = 0;
  int64_t pairs = 0;
  npa_tile_desc_t tiles[64];

  /* strips: 32x32 map, 4 strips, p = 0.3 */
  layout(&L, 2, 3, 64, 32, 32);
  memset(&h, 0, sizeof h);
  h.mode = NPA_MODE_STRIPS; h.num_strips = 4; h.p = 0.3f; h.halo_rows = -1;
  if (npa_plan(&L, &h, tiles, 64, &n, &pairs) != NPA_OK) { printf("plan failed: %s\n", npa_last_error()); return 1; }
  printf("strips %d %lld %lld %d\n", n, (long long)pairs, (long long)npa_useful_flops(&L, &h), tiles[1].n_segments);

  /* windows with text tokens: 16x16 map, 4x4 tiles, halo 2, 10 text tokens */
  layout(&L, 1, 2, 128, 16, 16);
  memset(&h, 0, sizeof h);
  h.mode = NPA_MODE_WINDOW; h.tile_h = 4; h.tile_w = 4; h.halo_h = 2; h.halo_w = 2; h.text_tokens = 10;
  if (npa_plan(&L, &h, tiles, 64, &n, &pairs) != NPA_OK) { printf("plan failed: %s\n", npa_last_error()); return 1; }
  printf("joint %d %lld %lld %d %d\n", n, (long long)pairs, (long long)npa_useful_flops(&L, &h),
         tiles[n - 1].queries.row_len, tiles[n - 1].keys[0].row_len);

  /* a refused argument: tiles that do not divide the map */
  h.tile_h = 5;
  npa_status_t st = npa_attn_fwd((void*)16, (void*)32, (void*)48, 0, 0, &L, &h, (void*)64, 0);
  printf("refused %d %s\n", (int)st, strstr(npa_last_error(), "divide") ? "divide" : npa_last_error());
  return 0;
}
"""


@pytest.fixture(scope="module")
def lib_path():
    npa.load(build_if_missing=False)
    return npa.LIB_PATH


def test_c_program_uses_the_abi(lib_path):
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "consumer.c"), os.path.join(d, "consumer")
        open(c, "w").write(PROGRAM)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I" + os.path.join(ROOT, "include"), c,
                        lib_path, "-Wl,-rpath," + os.path.dirname(lib_path), "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    strips = out[0].split()
    assert strips[0] == "strips"
    spec = A.Strips(4, p=0.3)
    assert int(strips[1]) == 4
    assert int(strips[2]) == A.useful_pairs(32, 32, spec)
    assert int(strips[3]) == A.useful_flops(2, 3, 64, 32, 32, spec)
    assert int(strips[4]) == 3  # an inner strip: own rows plus a halo above and below
    joint = out[1].split()
    spec = A.Windows(4, 4, 2, 2, 10)
    assert joint[0] == "joint" and int(joint[1]) == 16 + 1
    assert int(joint[2]) == A.useful_pairs(16, 16, spec)
    assert int(joint[3]) == A.useful_flops(1, 2, 128, 16, 16, spec)
    assert int(joint[4]) == 10 and int(joint[5]) == 10 + 16 * 16  # the text tile: T queries, every token
    refused = out[2].split()
    assert refused[0] == "refused" and int(refused[1]) == npa.NPA_ERR_SHAPE and refused[2] == "divide"
