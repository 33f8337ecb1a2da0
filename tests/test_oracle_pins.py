"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

None of these compares the oracle with itself.  Each check is chosen so that a
plausible slip in the oracle (a dropped sink term, a wrong sign, an off-by-one
in the window or prefix, a transposed operand, the wrong GQA mapping) fails:

* mask: brute-force enumeration built from index *ranges* (not the
  predicate), plus the closed-form per-row and per-head visible counts;
* forward: an independent explicit-sink implementation (extra column of logit
  s and value 0, plain softmax), the s -> -inf / plain-causal reduction to
  torch's scaled_dot_product_attention, closed forms, hand-worked examples;
* backward: fp64 autograd through the explicit-sink formulation, central
  finite differences, and closed-form gradient identities.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import WINDOW_INF, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np64(x):
    return x.to(torch.float64).numpy()


# --------------------------------------------------------------------- mask

def _mask_from_ranges(n, w, p):
    """Visible set as a union of index ranges: for each row i the window keys
    [max(0, i - w), i] and the prefix keys [0, min(p, i + 1))."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        lo = max(0, i - min(w, n))
        m[i, lo:i + 1] = True
        m[i, 0:min(p, i + 1)] = True
    return m


def _row_count(i, w, p):
    return min(i + 1, w + p + 1)


def _head_count(n, w, p):
    c = w + p + 1
    if c >= n:
        return n * (n + 1) // 2
    return c * (c + 1) // 2 + (n - c) * c


@pytest.mark.parametrize("n", [1, 2, 7, 16, 33])
def test_mask_matches_range_enumeration(n):
    windows = list(range(0, n + 2)) + [WINDOW_INF]
    for w in windows:
        for p in range(0, n + 2):
            m = oracle.visible_mask(n, w, p)
            ref = _mask_from_ranges(n, w, p)
            assert np.array_equal(m, ref), (n, w, p)
            counts = m.sum(axis=1)
            assert all(counts[i] == _row_count(i, min(w, 10**9), p) for i in range(n))
            assert m.sum() == _head_count(n, min(w, 10**9), p)


def test_mask_structure_count_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "score_positions.json")))
    n = g["n"]
    assert n * n == g["positions_dense"]
    # every position of the causal half is reachable: w = inf, p = 0
    assert _head_count(n, WINDOW_INF, 0) == g["positions_causal"]
    m = oracle.visible_mask(n, WINDOW_INF, 0)
    assert int(m.sum(dtype=np.int64)) == g["positions_causal"]
    del m


# ------------------------------------------------------------ explicit sink

def _explicit_sink_attention(q, k, v, s, w, p, scale):
    """Independent form: append a sink column of logit s and value 0, then a
    plain softmax over [visible keys, sink] (arXiv 2608.10357 section 5,
    zero-value sink equivalence).  torch fp64, differentiable."""
    n = q.shape[0]
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    allowed = torch.zeros(n, n, dtype=torch.bool)
    for r in range(n):              # ranges, not the predicate
        allowed[r, max(0, r - min(w, n)):r + 1] = True
        allowed[r, :min(p, r + 1)] = True
    del i, j
    scores = scale * (q @ k.T)
    scores = scores.masked_fill(~allowed, float("-inf"))
    ext = torch.cat([scores, s.expand(n, 1)], dim=1)
    probs = torch.softmax(ext, dim=1)
    vals = torch.cat([v, torch.zeros(1, v.shape[1], dtype=v.dtype)], dim=0)
    return probs @ vals


CASES = [
    # n, d, w, p
    (9, 4, 2, 3),
    (16, 8, 0, 0),
    (16, 8, WINDOW_INF, 0),
    (13, 5, 1, 20),
    (20, 3, 4, 1),
    (1, 4, 0, 0),
]


@pytest.mark.parametrize("n,d,w,p", CASES)
@pytest.mark.parametrize("sink", [-1.3, 0.0, 2.5])
def test_forward_equals_explicit_sink(n, d, w, p, sink):
    g = torch.Generator().manual_seed(7 + n + d + p)
    q, k, v = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, l = oracle.attend_head(q.numpy(), k.numpy(), v.numpy(), sink, w, p, scale)
    ref = _explicit_sink_attention(q, k, v, torch.tensor(sink, dtype=torch.float64), w, p, scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)
    # l is the content-only log-sum-exp: alpha recovered from the explicit form
    # (1 - sink column probability) must equal sigmoid(l - s)
    alpha = 1.0 / (1.0 + np.exp(sink - l))
    scores = scale * (q @ k.T).numpy()
    vis = _mask_from_ranges(n, w, p)
    z = np.array([np.exp(scores[r][vis[r]]).sum() for r in range(n)])
    np.testing.assert_allclose(alpha, z / (z + math.exp(sink)), rtol=1e-12)
    np.testing.assert_allclose(l, np.log(z), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,d,w,p", CASES)
def test_backward_equals_explicit_sink_autograd(n, d, w, p):
    g = torch.Generator().manual_seed(100 + n * d + p)
    q, k, v, do = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(4))
    s = torch.tensor(0.7, dtype=torch.float64)
    scale = 1.0 / math.sqrt(d)
    qa, ka, va, sa = (t.clone().requires_grad_(True) for t in (q, k, v, s))
    out = _explicit_sink_attention(qa, ka, va, sa, w, p, scale)
    (out * do).sum().backward()
    dq, dk, dv, ds = oracle.attend_head_grad(q.numpy(), k.numpy(), v.numpy(), 0.7, w, p,
                                             scale, do.numpy())
    np.testing.assert_allclose(dq, qa.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, ka.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, va.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ds, sa.grad.item(), rtol=1e-10, atol=1e-12)


# ------------------------------------- row- and key-restricted forms
# rows_head / key_grads_head / sink_grad_head evaluate the same definition at
# chosen rows or keys only (what full-size GPU comparisons use); pinned here
# to the explicit-sink formulation and its fp64 autograd, on every row and key
# and on subsets, with small chunks so that the per-chunk candidate ranges are
# exercised.

RESTRICTED = [
    # n, d, w, p
    (23, 4, 2, 3),
    (30, 8, 0, 0),
    (30, 8, WINDOW_INF, 0),
    (17, 5, 1, 40),
    (40, 3, 6, 1),
    (25, 4, 9, 25),
    (1, 4, 0, 0),
]


@pytest.mark.parametrize("n,d,w,p", RESTRICTED)
def test_restricted_forms_equal_explicit_sink_autograd(n, d, w, p):
    g = torch.Generator().manual_seed(300 + n * d + p)
    q, k, v, do = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(4))
    sink = -0.4
    scale = 1.0 / math.sqrt(d)
    qa, ka, va, sa = (t.clone().requires_grad_(True) for t in (q, k, v,
                                                               torch.tensor(sink, dtype=torch.float64)))
    out = _explicit_sink_attention(qa, ka, va, sa, w, p, scale)
    (out * do).sum().backward()
    vis = _mask_from_ranges(n, w, p)
    scores = scale * (q @ k.T).numpy()
    l_ref = np.array([np.log(np.exp(scores[r][vis[r]]).sum()) for r in range(n)])
    rng = np.random.default_rng(n + p)
    qn, kn, vn, don = (t.numpy() for t in (q, k, v, do))
    for rows in (np.arange(n), rng.choice(n, size=max(1, n // 3), replace=False)):
        st = oracle.rows_head(qn, kn, vn, sink, w, p, scale, rows, do=don, chunk=4)
        np.testing.assert_allclose(st["o"], out.detach().numpy()[rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(st["l"], l_ref[rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st["dq"], qa.grad.numpy()[rows], rtol=1e-10, atol=1e-12)
    for keys in (np.arange(n), np.arange(max(0, n - 5), n), np.arange(0, min(n, 3)),
                 np.sort(rng.choice(n, size=max(1, n // 4), replace=False))):
        dk, dv = oracle.key_grads_head(qn, kn, vn, sink, w, p, scale, don, keys, chunk=4)
        np.testing.assert_allclose(dk, ka.grad.numpy()[keys], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, va.grad.numpy()[keys], rtol=1e-10, atol=1e-12)
        every = oracle.rows_head(qn, kn, vn, sink, w, p, scale, np.arange(n), do=don, chunk=5)
        dk2, dv2 = oracle.key_grads_head(qn, kn, vn, sink, w, p, scale, don, keys, chunk=3,
                                         row_stats=every)
        np.testing.assert_allclose(dk2, ka.grad.numpy()[keys], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv2, va.grad.numpy()[keys], rtol=1e-10, atol=1e-12)
    ds = oracle.sink_grad_head(qn, kn, vn, sink, w, p, scale, don)
    np.testing.assert_allclose(ds, sa.grad.item(), rtol=1e-10, atol=1e-12)


# ------------------------------------------- reduction to plain attention

@pytest.mark.parametrize("sink", [float("-inf"), -1.0e4])
@pytest.mark.parametrize("n,w,p", [(24, WINDOW_INF, 0), (24, 23, 0), (24, 100, 0),
                                   (24, 3, 24), (24, 0, 30)])
def test_reduces_to_causal_sdpa(sink, n, w, p):
    """s -> -inf gives alpha = 1; with w >= n-1 or p >= n the mask is plain
    causal, so the result is textbook causal attention."""
    d = 8
    g = torch.Generator().manual_seed(3 + n + p)
    q, k, v = (torch.randn(1, 1, n, d, generator=g, dtype=torch.float64) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    o, l = oracle.attend_head(q[0, 0].numpy(), k[0, 0].numpy(), v[0, 0].numpy(), sink, w,
                              p, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)
    lse_ref = torch.logsumexp((q[0, 0] @ k[0, 0].T / math.sqrt(d)).masked_fill(
        torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf")), dim=1)
    np.testing.assert_allclose(l, lse_ref.numpy(), rtol=1e-12)


@pytest.mark.parametrize("n,w,p", [(30, 4, 0), (30, 0, 5), (30, 7, 3)])
def test_masked_reduces_to_sdpa_with_mask(n, w, p):
    """s = -inf with a window/prefix mask equals SDPA given the same boolean
    mask (built from ranges)."""
    d = 6
    g = torch.Generator().manual_seed(n + w + p)
    q, k, v = (torch.randn(1, 1, n, d, generator=g, dtype=torch.float64) for _ in range(3))
    allowed = torch.from_numpy(_mask_from_ranges(n, w, p))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=allowed)
    o, _ = oracle.attend_head(q[0, 0].numpy(), k[0, 0].numpy(), v[0, 0].numpy(),
                              float("-inf"), w, p, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ closed forms

def test_diagonal_only_closed_form():
    n, d = 11, 5
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(n, d, generator=g, dtype=torch.float64).numpy() for _ in range(3))
    s, scale = 0.3, 0.5
    o, l = oracle.attend_head(q, k, v, s, 0, 0, scale)
    l_ref = scale * np.sum(q * k, axis=1)
    np.testing.assert_allclose(l, l_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o, (1 / (1 + np.exp(s - l_ref)))[:, None] * v, rtol=1e-13)


@pytest.mark.parametrize("w,p", [(3, 2), (0, 4), (WINDOW_INF, 0), (5, 0)])
def test_uniform_keys_closed_form(w, p):
    """All keys equal: l_i = scale q_i.k + ln(#visible_i); Obar_i is the mean
    of the visible values; dq_i = scale (1 - alpha_i) D_i k."""
    n, d = 17, 4
    g = torch.Generator().manual_seed(11)
    q, v, do = (torch.randn(n, d, generator=g, dtype=torch.float64).numpy() for _ in range(3))
    kvec = np.array([0.3, -1.2, 0.5, 2.0])
    k = np.tile(kvec, (n, 1))
    s, scale = -0.4, 0.5
    o, l = oracle.attend_head(q, k, v, s, w, p, scale)
    for i in range(n):
        cnt = _row_count(i, min(w, 10**9), p)
        assert math.isclose(l[i], scale * q[i] @ kvec + math.log(cnt), rel_tol=1e-13,
                            abs_tol=1e-13)
        keys = sorted(set(range(max(0, i - min(w, n)), i + 1)) | set(range(min(p, i + 1))))
        alpha = 1 / (1 + math.exp(s - l[i]))
        np.testing.assert_allclose(o[i], alpha * v[keys].mean(axis=0), rtol=1e-12)
    dq, dk, dv, ds = oracle.attend_head_grad(q, k, v, s, w, p, scale, do)
    alpha = 1 / (1 + np.exp(s - l))
    dd = np.sum(do * o, axis=1)
    np.testing.assert_allclose(dq, scale * ((1 - alpha) * dd)[:, None] * kvec[None, :],
                               rtol=1e-10, atol=1e-13)


def test_value_shift_invariant():
    """O(V + 1 c^T) = O + alpha c (softmax rows sum to one, sink value 0)."""
    n, d = 19, 6
    g = torch.Generator().manual_seed(12)
    q, k, v = (torch.randn(n, d, generator=g, dtype=torch.float64).numpy() for _ in range(3))
    c = np.linspace(-1, 2, d)
    o1, l = oracle.attend_head(q, k, v, 0.9, 4, 2, 0.4)
    o2, _ = oracle.attend_head(q, k, v + c[None, :], 0.9, 4, 2, 0.4)
    alpha = 1 / (1 + np.exp(0.9 - l))
    np.testing.assert_allclose(o2, o1 + alpha[:, None] * c[None, :], rtol=1e-12, atol=1e-13)


def test_hand_worked_examples():
    cases = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["cases"]
    for c in cases:
        q, k, v = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v"))
        o, l = oracle.attend_head(q, k, v, c["sink"], c["window"], c["prefix"], 1.0)
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=1e-13, atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(l, np.array(c["l"]), rtol=1e-13, atol=1e-14, err_msg=c["name"])
        if "dsink" in c:
            dq, dk, dv, ds = oracle.attend_head_grad(q, k, v, c["sink"], c["window"],
                                                     c["prefix"], 1.0, np.array(c["do"]))
            assert math.isclose(ds, c["dsink"], rel_tol=1e-12), c["name"]
            np.testing.assert_allclose(dv, np.array(c["dv"]), rtol=1e-12, err_msg=c["name"])


# ---------------------------------------------------------- finite differences

@pytest.mark.parametrize("w,p", [(2, 3), (0, 0), (WINDOW_INF, 0), (1, 20), (5, 1)])
def test_gradients_match_central_differences(w, p):
    """Loss = sum(O * dO) over a GQA call (Hq=4, Hkv=2), T=12, d=4."""
    inp = make_inputs(batch=1, seqlen=12, heads_q=4, heads_kv=2, head_dim=4, window=w,
                      prefix=p, seed=77 + p, std=1.0, dtype="fp32")
    q, k, v, do = (_np64(t) for t in (inp.q, inp.k, inp.v, inp.do))
    s = _np64(inp.sinks)
    sc = inp.scale

    def loss(q_, k_, v_, s_):
        o, _ = oracle.forward(q_, k_, v_, s_, w, p, sc)
        return float(np.sum(o * do))

    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, w, p, sc)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("s", s, ds)):
        num = np.zeros_like(arr)
        flat = arr.reshape(-1)
        nflat = num.reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + h
            lp = loss(q, k, v, s)
            flat[idx] = old - h
            lm = loss(q, k, v, s)
            flat[idx] = old
            nflat[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1e-3, np.max(np.abs(grad)))
        assert err < 1e-7, (name, err)


# ----------------------------------------------------- structural invariants

def test_varlen_equals_separate_runs():
    lengths = (5, 1, 12, 7)
    inp = make_inputs(batch=1, seqlen=0, heads_q=4, heads_kv=2, head_dim=3, window=2,
                      prefix=2, seed=5, dtype="fp32", lengths=lengths)
    q, k, v, do = (_np64(t) for t in (inp.q, inp.k, inp.v, inp.do))
    s = _np64(inp.sinks)
    cu = inp.cu_seqlens.numpy()
    o, lse = oracle.forward(q, k, v, s, 2, 2, inp.scale, cu_seqlens=cu)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, 2, 2, inp.scale, cu_seqlens=cu)
    ds_sum = np.zeros_like(ds)
    for i in range(len(lengths)):
        r = slice(cu[i], cu[i + 1])
        o1, l1 = oracle.forward(q[None, r], k[None, r], v[None, r], s, 2, 2, inp.scale)
        g1 = oracle.backward(q[None, r], k[None, r], v[None, r], s, do[None, r], 2, 2, inp.scale)
        np.testing.assert_allclose(o[r], o1[0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse[:, r], l1[0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dq[r], g1[0][0], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(dk[r], g1[1][0], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(dv[r], g1[2][0], rtol=1e-13, atol=1e-15)
        ds_sum += g1[3]
    np.testing.assert_allclose(ds, ds_sum, rtol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    inp = make_inputs(batch=2, seqlen=10, heads_q=6, heads_kv=2, head_dim=4, window=3,
                      prefix=1, seed=9, dtype="fp32")
    q, k, v, do = (_np64(t) for t in (inp.q, inp.k, inp.v, inp.do))
    s = _np64(inp.sinks)
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)   # head h -> kv h // 3
    o, lse = oracle.forward(q, k, v, s, 3, 1, inp.scale)
    o2, lse2 = oracle.forward(q, kr, vr, s, 3, 1, inp.scale)
    np.testing.assert_allclose(o, o2, rtol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, 3, 1, inp.scale)
    dq2, dk2, dv2, ds2 = oracle.backward(q, kr, vr, s, do, 3, 1, inp.scale)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(2, 10, 2, 3, 4).sum(axis=3), rtol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(2, 10, 2, 3, 4).sum(axis=3), rtol=1e-12)
    np.testing.assert_allclose(ds, ds2, rtol=1e-13)


def test_infinite_negative_sink_gives_zero_sink_gradient():
    inp = make_inputs(batch=1, seqlen=9, heads_q=2, heads_kv=1, head_dim=4, window=2,
                      prefix=1, seed=21, dtype="fp32", sink_values=(float("-inf"), 0.5))
    q, k, v, do = (_np64(t) for t in (inp.q, inp.k, inp.v, inp.do))
    s = _np64(inp.sinks)
    o, lse = oracle.forward(q, k, v, s, 2, 1, inp.scale)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, 2, 1, inp.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))
    assert ds[0] == 0.0 and ds[1] != 0.0


# ------------------------------------------------------------------- decode

def _decode_case(seed, lens, tmax, hq, hkv, d):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(len(lens), hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(len(lens), tmax, hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(len(lens), tmax, hkv, d, generator=g, dtype=torch.float64)
    s = torch.randn(hq, generator=g, dtype=torch.float64)
    return q.numpy(), k.numpy(), v.numpy(), s.numpy()


@pytest.mark.parametrize("w,p", [(WINDOW_INF, 0), (5, 0), (3, 2), (0, 0), (0, 4), (100, 100)])
def test_decode_equals_explicit_sink_row(w, p):
    # independent explicit-sink softmax over the visible keys of the last
    # position, built from index ranges (not the predicate)
    lens, tmax, hq, hkv, d = [1, 2, 9, 17], 20, 4, 2, 8
    q, k, v, s = _decode_case(11, lens, tmax, hq, hkv, d)
    scale = 0.3
    o, l = oracle.decode(q, k, v, lens, s, w, p, scale)
    for b, n in enumerate(lens):
        pos = n - 1
        keys = sorted(set(range(max(0, pos - min(w, n)), pos + 1)) | set(range(min(p, n))))
        for h in range(hq):
            kv = h // (hq // hkv)
            logits = np.array([scale * q[b, h] @ k[b, j, kv] for j in keys] + [s[h]])
            wts = np.exp(logits - logits.max())
            wts /= wts.sum()
            vals = np.vstack([v[b, keys, kv], np.zeros((1, d))])
            assert np.allclose(o[b, h], wts @ vals, atol=1e-12)
            content = logits[:-1]
            assert abs(l[b, h] - (content.max() + np.log(np.exp(content - content.max()).sum()))) < 1e-12


def test_decode_is_last_row_of_forward():
    # the rollout engine must reproduce the trainer's probabilities: decode on
    # a cache of n tokens equals row n - 1 of the forward on those n tokens
    for w, p in [(WINDOW_INF, 0), (6, 3), (2, 0)]:
        lens, hq, hkv, d = [1, 5, 12], 8, 2, 8
        q, k, v, s = _decode_case(12, lens, 12, hq, hkv, d)
        # training-side queries: the decode query is the last row, the others random
        qt = np.random.default_rng(3).standard_normal((len(lens), 12, hq, d))
        for b, n in enumerate(lens):
            qt[b, n - 1] = q[b]
        od, ld = oracle.decode(q, k, v, lens, s, w, p, 0.25)
        for b, n in enumerate(lens):
            of, lf = oracle.forward(qt[b:b + 1, :n], k[b:b + 1, :n], v[b:b + 1, :n], s, w, p, 0.25)
            assert np.allclose(od[b], of[0, n - 1], atol=1e-12)
            assert np.allclose(ld[b], lf[0, :, n - 1], atol=1e-12)


@pytest.mark.parametrize("w,p", [(WINDOW_INF, 0), (4, 2)])
def test_decode_infinite_negative_sink_reduces_to_sdpa(w, p):
    lens, tmax, hq, hkv, d = [3, 10, 16], 16, 4, 4, 8
    q, k, v, s = _decode_case(13, lens, tmax, hq, hkv, d)
    s[:] = -np.inf
    o, _ = oracle.decode(q, k, v, lens, s, w, p, 1.0 / math.sqrt(d))
    for b, n in enumerate(lens):
        mask = torch.zeros(1, n, dtype=torch.bool)
        mask[0, max(0, n - 1 - min(w, n)):n] = True
        mask[0, :min(p, n)] = True
        for h in range(hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h][None, None]), torch.from_numpy(k[b, :n, h][None].copy()),
                torch.from_numpy(v[b, :n, h][None].copy()), attn_mask=mask[None])
            assert np.allclose(o[b, h], ref[0, 0].numpy(), atol=1e-12)


def test_decode_closed_forms():
    lens, tmax, hq, hkv, d = [1, 7, 0], 8, 2, 1, 4
    q, k, v, s = _decode_case(14, lens, tmax, hq, hkv, d)
    # w = 0, p = 0: only the new token's own key is visible
    o, l = oracle.decode(q, k, v, lens, s, 0, 0, 0.5)
    for b, n in enumerate(lens[:2]):
        for h in range(hq):
            lh = 0.5 * q[b, h] @ k[b, n - 1, 0]
            assert abs(l[b, h] - lh) < 1e-12
            assert np.allclose(o[b, h], v[b, n - 1, 0] / (1.0 + np.exp(s[h] - lh)), atol=1e-12)
    # an empty cache: no keys, o = 0 and lse = -inf
    assert np.all(o[2] == 0) and np.all(np.isneginf(l[2]))
    # uniform keys: l = scale q.k + ln(count), o = alpha * mean of the visible values
    k[:] = k[:, :1]
    o, l = oracle.decode(q, k, v, lens, s, 2, 1, 0.5)
    n = 7
    keys = [0, 4, 5, 6]
    for h in range(hq):
        lh = 0.5 * q[1, h] @ k[1, 0, 0] + math.log(len(keys))
        assert abs(l[1, h] - lh) < 1e-12
        assert np.allclose(o[1, h], v[1, keys, 0].mean(axis=0) / (1.0 + np.exp(s[h] - lh)), atol=1e-12)
