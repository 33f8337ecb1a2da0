"""Host model of the MFMA register layouts the forward kernel's matrix-core
row sums rely on (CDNA3/CDNA4 ISA, matrix instructions: operand and result
layouts of v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16).

The forward keeps S^T = K Q^T in the 32x32 result layout (lane = query), turns
each 16-key half of it into a bf16x8 P^T register, and feeds that register to
a 16x16x32 MFMA against a constant 0/1 A operand.  This checks, on random
data, that the selector puts in register 0 of every lane the sum over the 16
keys for that lane's own query, and that no other choice of the ones' rows
among 0, 4, 8, 12 does.  The GPU parity tests check the kernel itself.
"""
import numpy as np


def c32_index(lane, i):
    """(row, col) of register i of lane in a 32x32 MFMA result."""
    return 8 * (i // 4) + 4 * (lane // 32) + i % 4, lane % 32


def mfma16x16x32(a_regs, b_regs):
    """D = A B for per-lane operands a_regs, b_regs [64, 8]; returns [64, 4]."""
    a = np.zeros((16, 32))
    b = np.zeros((32, 16))
    for lane in range(64):
        for e in range(8):
            a[lane % 16, 8 * (lane // 16) + e] = a_regs[lane, e]
            b[8 * (lane // 16) + e, lane % 16] = b_regs[lane, e]
    d = a @ b
    out = np.zeros((64, 4))
    for lane in range(64):
        for i in range(4):
            out[lane, i] = d[4 * (lane // 16) + i, lane % 16]
    return out


def selector(lane, rows=(0, 4, 8, 12)):
    m = lane % 16
    return 1.0 if m in rows and (m // 4) % 2 == (lane // 16) % 2 else 0.0


def p_registers(st, hh):
    """The bf16x8 P^T register hh of each lane: result elements 8hh .. 8hh+7."""
    regs = np.zeros((64, 8))
    for lane in range(64):
        for e in range(8):
            r, c = c32_index(lane, 8 * hh + e)
            regs[lane, e] = st[r, c]
    return regs


def test_row_sum_selector_gives_each_lane_its_query():
    rng = np.random.default_rng(7)
    st = rng.random((32, 32))            # [key, query] of one 32-key block
    sel = np.array([[selector(lane)] * 8 for lane in range(64)])
    total = np.zeros((64, 4))
    for hh in range(2):
        total += mfma16x16x32(sel, p_registers(st, hh))
    want = st.sum(axis=0)                # per query, over the block's 32 keys
    for lane in range(64):
        np.testing.assert_allclose(total[lane, 0], want[lane % 32], rtol=1e-13)


def test_each_half_register_covers_sixteen_distinct_keys():
    # a P^T register pair (hh = 0, 1) of one lane and its partner lane l ^ 32
    # covers each of the 32 keys of its query exactly once
    for lane in range(32):
        keys = []
        for ln in (lane, lane + 32):
            for i in range(16):
                r, c = c32_index(ln, i)
                assert c == lane
                keys.append(r)
        assert sorted(keys) == list(range(32))


def test_other_selector_rows_miss_queries():
    rng = np.random.default_rng(8)
    st = rng.random((32, 32))
    want = st.sum(axis=0)
    for rows in ((0,), (0, 4), (0, 1, 2, 3), (4, 8)):
        sel = np.array([[selector(lane, rows)] * 8 for lane in range(64)])
        total = sum(mfma16x16x32(sel, p_registers(st, hh)) for hh in range(2))
        got = np.array([total[lane, 0] for lane in range(64)])
        assert not np.allclose(got, want[np.arange(64) % 32])
