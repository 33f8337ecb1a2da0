"""The backward's work split for dK/dV, checked on the host by brute force (no
GPU): every visible (row, key) pair of the mask M[q,k] = 1[k<=q] AND
1[q-k<=w OR k<p] is counted exactly once, either by the dK/dV kernel (key
block kb, its query range from sa_dkdv_query_range) or, with the prefix fold
on, by the window dQ kernel (rows at or past the fold row of the first key
block, keys k < p).  The work-unit count of each block follows from its range.
And the window dQ kernel's key-tile lists fit the tiles it keeps in LDS.  The
schedule header is compiled with the host compiler; the mask predicate here
is written out independently of it."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sink_aware_masked_sinkattn_amd", "csrc")

SOURCE = r"""
#include <climits>
#include <cstdio>
#include "mask_tiles.h"

static bool visible(long long q, long long k, long long w, long long p) {
  return k <= q && (q - k <= w || k < p);
}

int main() {
  const int BKW = 128, BQ = 128;   // dK/dV key block and query tile
  const int ns[] = {1, 2, 31, 127, 128, 129, 255, 256, 257, 300, 383, 384, 385, 511, 640, 700};
  const int ws[] = {0, 1, 5, 31, 32, 63, 64, 100, 127, 128, 129, 200, 255, 256, 300, 1000, INT_MAX};
  const int ps[] = {0, 1, 3, 4, 15, 16, 17, 32, 100, 100000};
  const int groups[] = {1, 4, 8, 16};
  long long checked = 0;
  for (int n : ns)
    for (int w : ws)
      for (int p : ps)
        for (int fold = 0; fold < 2; ++fold) {
          // the fold runs only with every prefix key in the first 16 keys
          if (fold && !(p > 0 && p <= 16)) continue;
          const long long R = sa_prefix_fold_row(0, w, BKW, BQ);
          if (R % 32 != 0) { printf("fold row %lld not a multiple of 32\n", R); return 1; }
          for (int kb = 0; kb * BKW < n; ++kb) {
            int lo = 0, hi = -1;
            const bool has = sa_dkdv_query_range(kb, n, w, p, BQ, BKW, fold != 0, &lo, &hi);
            for (int k = kb * BKW; k < kb * BKW + BKW && k < n; ++k)
              for (int q = 0; q < n; ++q) {
                const bool in_range = has && lo <= q && q <= hi;
                const bool in_fold = fold && kb == 0 && q >= R && k < p && k < 16;
                const bool vis = visible(q, k, w, p);
                if (vis && in_range == in_fold) {
                  printf("n=%d w=%d p=%d fold=%d kb=%d q=%d k=%d: range %d fold %d\n", n, w, p,
                         fold, kb, q, k, (int)in_range, (int)in_fold);
                  return 1;
                }
                ++checked;
              }
            // rows the fold takes are not in the block's range (no double count)
            if (fold && kb == 0 && has && hi >= R) {
              printf("n=%d w=%d p=%d: block 0 range reaches the fold row\n", n, w, p);
              return 1;
            }
            for (int g : groups)
              for (int s = 0; s < 9; ++s) {
                const int c = sa_dkdv_block_chunks(kb, n, w, p, g, BQ, BKW, s, fold != 0);
                const int iters = has ? (hi / BQ - lo / BQ + 1) * g : 0;
                if (c != (iters + (1 << s) - 1) / (1 << s)) {
                  printf("chunks n=%d w=%d p=%d kb=%d g=%d s=%d: %d\n", n, w, p, kb, g, s, c);
                  return 1;
                }
              }
          }
        }
  printf("ok %lld\n", checked);
  return 0;
}
"""


# The resident-tile window dQ kernel holds a 32-row block's whole key-tile
# list in LDS (6 tiles of 32 keys).  The library runs it when
# ceil(min(p, T) / 32) + ceil(w / 32) + 1 <= 6 (w, p already clamped to the
# longest length T); then no block of any sequence of length <= T may list
# more than 6 tiles.
WIN_SOURCE = r"""
#include <cstdio>
#include "mask_tiles.h"

int main() {
  const int BK = 32, WIN_TILES = 6;
  long long checked = 0;
  for (int T = 1; T <= 700; T += (T < 80 ? 1 : 7))
    for (int w0 = 0; w0 <= 200; ++w0)
      for (int p0 = 0; p0 <= 200; p0 += (p0 < 70 ? 1 : 13)) {
        const int w = w0 < T ? w0 : T, p = p0 < T ? p0 : T;
        const int pre = (p + BK - 1) / BK, win = (w + BK - 1) / BK + 1;
        if (pre + win > WIN_TILES) continue;
        for (int len = 1; len <= T; len += (len < 70 ? 1 : 11))
          for (int q0 = 0; q0 < len; q0 += BK) {
            const int q1 = q0 + BK - 1 < len - 1 ? q0 + BK - 1 : len - 1;
            int seg[4];
            const int ns = sa_key_tile_segments(q0, q1, w, p, BK, seg);
            const int nt = (seg[1] - seg[0]) + (ns > 1 ? seg[3] - seg[2] : 0);
            if (nt > WIN_TILES) {
              printf("T=%d w=%d p=%d len=%d q0=%d: %d tiles\n", T, w, p, len, q0, nt);
              return 1;
            }
            ++checked;
          }
      }
  printf("ok %lld\n", checked);
  return 0;
}
"""


def _build(cxx, d, name, source):
    src = os.path.join(d, name + ".cpp")
    exe = os.path.join(d, name)
    with open(src, "w") as f:
        f.write(source)
    subprocess.run([cxx, "-std=c++17", "-O2", "-I", CSRC, src, "-o", exe], check=True)
    return exe


@pytest.fixture(scope="module")
def cover_binary():
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tempfile.mkdtemp(prefix="dkdv_cover_")
    yield {"cover": _build(cxx, d, "cover", SOURCE), "win": _build(cxx, d, "win", WIN_SOURCE)}
    shutil.rmtree(d, ignore_errors=True)


def test_dkdv_ranges_and_fold_cover_every_visible_pair_once(cover_binary):
    r = subprocess.run([cover_binary["cover"]], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_window_dq_tile_lists_fit_its_resident_tiles(cover_binary):
    r = subprocess.run([cover_binary["win"]], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
