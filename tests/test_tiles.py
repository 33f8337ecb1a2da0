"""The tile schedule the kernels use, checked against brute-force enumeration
of the mask M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p] (no GPU needed)."""
import itertools

import numpy as np
import pytest

from sink_aware_masked_sinkattn_amd import binding

INF = binding.WINDOW_INF


def _visible(n, w, p):
    q = np.arange(n)[:, None]
    k = np.arange(n)[None, :]
    return (k <= q) & ((q - k <= w) | (k < p))


@pytest.mark.parametrize("w,p", [(0, 0), (1, 0), (3, 2), (7, 0), (5, 9), (INF, 0), (INF, 3),
                                 (12, 1), (0, 20), (40, 0)])
def test_tile_class_matches_brute_force(w, p):
    n = 40
    m = _visible(n, w, p)
    for q0, k0 in itertools.product(range(0, n, 3), range(0, n, 3)):
        for hq, hk in ((1, 1), (4, 4), (8, 3), (2, 9)):
            q1, k1 = min(n - 1, q0 + hq - 1), min(n - 1, k0 + hk - 1)
            blk = m[q0:q1 + 1, k0:k1 + 1]
            c = binding.sinkattn_tile_class(q0, q1, k0, k1, w, p)
            if c == 0:
                assert not blk.any(), (q0, q1, k0, k1, w, p)
            elif c == 1:
                assert blk.all(), (q0, q1, k0, k1, w, p)
            else:
                assert c == 2
                # partial is exact when the block is neither empty nor full
                assert blk.any() and not blk.all(), (q0, q1, k0, k1, w, p)


@pytest.mark.parametrize("bk", [1, 4, 16, 64])
@pytest.mark.parametrize("w,p", [(0, 0), (3, 2), (16, 0), (5, 40), (INF, 0), (64, 4), (128, 16),
                                 (2, 70), (31, 1)])
def test_key_tile_segments_list_exactly_the_visible_tiles(bk, w, p):
    n = 200
    m = _visible(n, w, p)
    for q0 in range(0, n, 7):
        for rows in (1, 5, 64, 256):
            q1 = min(n - 1, q0 + rows - 1)
            segs = binding.sinkattn_key_tile_segments(q0, q1, w, p, bk)
            listed = [t for (b, e) in segs for t in range(b, e)]
            assert len(listed) == len(set(listed)), segs
            want = [t for t in range((n + bk - 1) // bk)
                    if m[q0:q1 + 1, t * bk:min(n, (t + 1) * bk)].any()]
            assert sorted(listed) == want, (q0, q1, w, p, bk, segs)
