"""Plain fp64 CPU oracle for sink-aware masked attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP library; the only thing the
two have in common is the seeded input generator module (``workloads.py``),
which holds no attention arithmetic.

Sources (cited by page title and section):
  [SUM]  "Efficient Reinforcement Learning for Long-Horizon Tool-Use Agentic
         Tasks" (summary page), paragraph on the sink-aware FlexAttention path:
         the mask M = 1[k <= q] AND 1[q - k <= w OR k < p], the attention call
         returning the output and an auxiliary log-sum-exp, and the sink
         scaling alpha = sigmoid(l - s) with l = log sum_i exp(q . k_i).
  [S5]   arXiv 2608.10357, section 5 "Sink-aware FlexAttention", paragraph
         "Zero-value sink equivalence": the explicit-sink output
         O_sink = (sum_i exp(q.k_i) v_i + exp(s) * 0) / (sum_i exp(q.k_i) + exp(s)).
  [RETRO] "GPT-OSS Agentic RL training: a practical retrospective", section on
         the FlashAttention v3 implementation: a backward pass that produces the
         gradient of the loss with respect to each head's sink logit S_h.

What is computed is the plain dense definition.  Everything is fp64, one
(sequence, query head) at a time, with the full score matrix of that head
formed explicitly (that is exactly what the GPU path must never do, and is
fine here).  Readings where the pages leave a step open:
  * scores are ``scale * q . k`` (the pages write q . k; scale = 1 is theirs);
  * the log-sum-exp runs over the visible keys only and is the content-only
    ``l`` (no sink term); natural log;
  * ``q - k <= w`` is inclusive, ``k < p`` strict; positions are local to each
    packed sequence; the q-head h reads kv-head h // group;
  * one fp32 sink logit per query head, shared by all rows and sequences.

Decode (the rollout side of the same attention; arXiv 2608.10357 section 4
"Rollout workers": sampling from the current policy; [RETRO], section on the
training-inference mismatch through attention sinks: the rollout engine must
give the trainer's token probabilities, sink included): one new query token
per sequence against its key/value cache of n tokens, the new token's own
key and value already at position n - 1.  The plain reading is that the
query sits at position n - 1 under the same mask, so the result is row
n - 1 of the forward on the whole sequence.

Backward (not printed on the pages; it is the chain rule through [S5]'s
softmax with one extra zero-valued column of logit s):
  L_i   = logaddexp(l_i, s)           (log of the sink-inclusive normaliser)
  P'_ij = exp(S_ij - L_i)             (sink-inclusive probabilities, = alpha_i P_ij)
  D_i   = dO_i . O_i
  dS_ij = P'_ij (dO_i . v_j - D_i)    (the sink column has value 0, so it only
                                       enters through D_i)
  dq_i  = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
  dv_j  = sum_i P'_ij dO_i,        ds   = -sum_i exp(s - L_i) D_i      [RETRO]
dk and dv of a kv-head are summed over the query heads that read it, and ds
over every row of every sequence.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np


def visible_mask(n: int, window: int, prefix: int) -> np.ndarray:
    """M[i, j] for one sequence of n tokens ([SUM], mask function)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & ((i - j <= window) | (j < prefix))


def attend_head(q, k, v, sink: float, window: int, prefix: int, scale: float):
    """Forward for one sequence and one query head.

    q [n, d], k [n, d], v [n, d] (any float type, used in fp64).
    Returns (o [n, d], l [n]) with o = sigmoid(l - s) * softmax(S) v   ([SUM]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    if n == 0:
        return np.zeros_like(q), np.zeros((0,), np.float64)
    m = visible_mask(n, window, prefix)
    s_mat = scale * (q @ k.T)
    s_mat = np.where(m, s_mat, -np.inf)
    rowmax = s_mat.max(axis=1)
    e = np.exp(s_mat - rowmax[:, None])
    z = e.sum(axis=1)
    l = rowmax + np.log(z)                       # content-only log-sum-exp
    o_bar = (e @ v) / z[:, None]                 # plain masked softmax attention
    alpha = 1.0 / (1.0 + np.exp(np.float64(sink) - l))   # sigmoid(l - s)
    return alpha[:, None] * o_bar, l


def attend_head_grad(q, k, v, sink: float, window: int, prefix: int, scale: float, do):
    """Backward for one sequence and one query head.

    Recomputes the forward, then applies the chain rule written in the module
    docstring.  Returns (dq [n, d], dk [n, d], dv [n, d], dsink float).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    if n == 0:
        z = np.zeros_like(q)
        return z, z.copy(), z.copy(), 0.0
    o, l = attend_head(q, k, v, sink, window, prefix, scale)
    m = visible_mask(n, window, prefix)
    s_mat = np.where(m, scale * (q @ k.T), -np.inf)
    big_l = np.logaddexp(l, np.float64(sink))
    p_prime = np.exp(s_mat - big_l[:, None])     # 0 where masked
    d_row = np.sum(do * o, axis=1)
    dp = do @ v.T
    ds_mat = p_prime * (dp - d_row[:, None])
    dq = scale * (ds_mat @ k)
    dk = scale * (ds_mat.T @ q)
    dv = p_prime.T @ do
    dsink = -float(np.sum(np.exp(np.float64(sink) - big_l) * d_row))
    return dq, dk, dv, dsink


def _candidate_keys(r_lo: int, r_hi: int, n: int, window: int, prefix: int) -> np.ndarray:
    """Every key that a row in [r_lo, r_hi] may see: the prefix keys [0, min(p, r_hi + 1))
    and the window keys [max(0, r_lo - w), r_hi] ([SUM] mask).  A superset; the mask
    itself is applied to every (row, key) pair afterwards."""
    pre = np.arange(min(prefix, r_hi + 1, n))
    win = np.arange(max(0, r_lo - window), min(r_hi, n - 1) + 1)
    return np.union1d(pre, win)


def rows_head(q, k, v, sink: float, window: int, prefix: int, scale: float, rows,
              do=None, chunk: int = 256):
    """Forward (and, with ``do``, dq and the row statistics) of one sequence and one
    query head at the given query rows only.

    The same definition as ``attend_head`` / ``attend_head_grad`` restricted to those
    rows: each row attends to its visible keys ([SUM] mask), gathered from the
    candidate range of its chunk of rows, so the cost is that of the visible pairs of
    the chosen rows.  Returns a dict with o [R, d], l [R] and, with do, dq [R, d],
    big_l [R] (logaddexp(l, s)) and d_row [R] (dO . O).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    out = {"o": np.zeros((rows.size, d)), "l": np.zeros(rows.size)}
    if do is not None:
        do = np.asarray(do, dtype=np.float64)
        out.update(dq=np.zeros((rows.size, d)), big_l=np.zeros(rows.size),
                   d_row=np.zeros(rows.size))
    order = np.argsort(rows, kind="stable")
    for c0 in range(0, rows.size, chunk):
        sel = order[c0:c0 + chunk]
        r = rows[sel]
        cand = _candidate_keys(int(r.min()), int(r.max()), n, window, prefix)
        vis = (cand[None, :] <= r[:, None]) & (
            (r[:, None] - cand[None, :] <= window) | (cand[None, :] < prefix))
        s_mat = np.where(vis, scale * (q[r] @ k[cand].T), -np.inf)
        rowmax = s_mat.max(axis=1)
        e = np.exp(s_mat - rowmax[:, None])
        z = e.sum(axis=1)
        l = rowmax + np.log(z)
        alpha = 1.0 / (1.0 + np.exp(np.float64(sink) - l))
        o = alpha[:, None] * ((e @ v[cand]) / z[:, None])
        out["o"][sel] = o
        out["l"][sel] = l
        if do is not None:
            big_l = np.logaddexp(l, np.float64(sink))
            p_prime = np.exp(s_mat - big_l[:, None])
            d_row = np.sum(do[r] * o, axis=1)
            ds_mat = p_prime * (do[r] @ v[cand].T - d_row[:, None])
            out["dq"][sel] = scale * (ds_mat @ k[cand])
            out["big_l"][sel] = big_l
            out["d_row"][sel] = d_row
    return out


def key_grads_head(q, k, v, sink: float, window: int, prefix: int, scale: float, do, keys,
                   chunk: int = 256, row_stats=None):
    """dk and dv of one sequence and one query head at the given key positions only.

    The rows that can see any of the keys are evaluated in full with ``rows_head`` (their
    l, O, L = logaddexp(l, s) and D = dO . O over all their visible keys); then, chunk by
    chunk of keys, on the rows that can see the chunk: P' = exp(S - L),
    dS = P' (dO . v - D), dk_j = scale sum_i dS_ij q_i and dv_j = sum_i P'_ij dO_i -- the
    chain rule of the module docstring restricted to the chosen keys.  ``row_stats``:
    the result of ``rows_head`` with ``do`` over every row 0 .. n-1 of the same
    inputs, to reuse instead of recomputing.  Returns (dk [K, d], dv [K, d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, d = q.shape
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((keys.size, d))
    dv = np.zeros((keys.size, d))
    if keys.size == 0:
        return dk, dv

    def rows_seeing(j_lo, j_hi):
        # rows i >= j_lo with i - j <= w for some key j <= j_hi, or every later row
        # when a prefix key is among them
        return j_lo, (n - 1 if j_lo < prefix else min(n - 1, j_hi + window))

    if row_stats is not None:
        r_lo, st = 0, row_stats
    else:
        r_lo, r_hi = rows_seeing(int(keys.min()), int(keys.max()))
        st = rows_head(q, k, v, sink, window, prefix, scale, np.arange(r_lo, r_hi + 1),
                       do=do, chunk=chunk)
    order = np.argsort(keys, kind="stable")
    for c0 in range(0, keys.size, chunk):
        sel = order[c0:c0 + chunk]
        j = keys[sel]
        a, b = rows_seeing(int(j.min()), int(j.max()))
        rows = np.arange(a, b + 1)
        big_l = st["big_l"][rows - r_lo]
        d_row = st["d_row"][rows - r_lo]
        vis = (j[None, :] <= rows[:, None]) & (
            (rows[:, None] - j[None, :] <= window) | (j[None, :] < prefix))
        s_mat = np.where(vis, scale * (q[rows] @ k[j].T), -np.inf)
        p_prime = np.exp(s_mat - big_l[:, None])
        ds_mat = p_prime * (do[rows] @ v[j].T - d_row[:, None])
        dk[sel] = scale * (ds_mat.T @ q[rows])
        dv[sel] = p_prime.T @ do[rows]
    return dk, dv


def sink_grad_head(q, k, v, sink: float, window: int, prefix: int, scale: float, do) -> float:
    """ds of one sequence and one query head: -sum_i exp(s - L_i) D_i over all its rows
    ([RETRO] per-head sink gradient), with every row evaluated by ``rows_head``."""
    n = np.asarray(q).shape[0]
    if n == 0:
        return 0.0
    st = rows_head(q, k, v, sink, window, prefix, scale, np.arange(n), do=do)
    return -float(np.sum(np.exp(np.float64(sink) - st["big_l"]) * st["d_row"]))


def _sequences(q, cu_seqlens):
    """Yield (batch_index_or_None, row_slice) for each sequence."""
    if cu_seqlens is None:
        for b in range(q.shape[0]):
            yield b, slice(None)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        for s in range(len(cu) - 1):
            yield None, slice(int(cu[s]), int(cu[s + 1]))


def _pick(x, b, rows, h):
    return x[b, :, h, :] if b is not None else x[rows, h, :]


def forward(q, k, v, sinks, window: int, prefix: int, scale: float,
            cu_seqlens=None, heads: Optional[Iterable[int]] = None):
    """Whole-call forward.

    q [B,T,Hq,d] (or [N,Hq,d] with cu_seqlens int[G+1]); k, v [B,T,Hkv,d]
    (or [N,Hkv,d]); sinks [Hq].  Returns (o like q, lse [B,Hq,T] or [Hq,N]),
    fp64.  ``heads`` restricts the work to some query heads (the others are
    left NaN), for spot checks at full size.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    sinks = np.asarray(sinks, dtype=np.float64)
    hq = q.shape[-2]
    group = hq // k.shape[-2]
    heads = list(range(hq)) if heads is None else list(heads)
    o = np.full(q.shape, np.nan, np.float64)
    if cu_seqlens is None:
        lse = np.full((q.shape[0], hq, q.shape[1]), np.nan, np.float64)
    else:
        lse = np.full((hq, q.shape[0]), np.nan, np.float64)
    for b, rows in _sequences(q, cu_seqlens):
        for h in heads:
            oh, lh = attend_head(_pick(q, b, rows, h), _pick(k, b, rows, h // group),
                                 _pick(v, b, rows, h // group), sinks[h], window,
                                 prefix, scale)
            if b is not None:
                o[b, :, h, :] = oh
                lse[b, h, :] = lh
            else:
                o[rows, h, :] = oh
                lse[h, rows] = lh
    return o, lse


def backward(q, k, v, sinks, do, window: int, prefix: int, scale: float,
             cu_seqlens=None, heads: Optional[Sequence[int]] = None):
    """Whole-call backward.  Returns (dq, dk, dv, dsinks), fp64.

    dk, dv of a kv-head sum the contributions of every query head in
    ``heads`` that reads it (complete only when ``heads`` covers the group);
    dsinks[h] sums over all rows of all sequences.  Heads left out are NaN in
    dq and dsinks.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    sinks = np.asarray(sinks, dtype=np.float64)
    hq = q.shape[-2]
    group = hq // k.shape[-2]
    heads = list(range(hq)) if heads is None else list(heads)
    dq = np.full(q.shape, np.nan, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    dsinks = np.full((hq,), np.nan, np.float64)
    for h in heads:
        dsinks[h] = 0.0
    for b, rows in _sequences(q, cu_seqlens):
        for h in heads:
            kv = h // group
            g_q, g_k, g_v, g_s = attend_head_grad(
                _pick(q, b, rows, h), _pick(k, b, rows, kv), _pick(v, b, rows, kv),
                sinks[h], window, prefix, scale, _pick(do, b, rows, h))
            if b is not None:
                dq[b, :, h, :] = g_q
                dk[b, :, kv, :] += g_k
                dv[b, :, kv, :] += g_v
            else:
                dq[rows, h, :] = g_q
                dk[rows, kv, :] += g_k
                dv[rows, kv, :] += g_v
            dsinks[h] += g_s
    return dq, dk, dv, dsinks


def decode(q, k_cache, v_cache, cache_seqlens, sinks, window: int, prefix: int,
           scale: float):
    """Decode: one query token per sequence against its key/value cache.

    q [B, Hq, d]; k_cache, v_cache [B, Tmax, Hkv, d]; cache_seqlens ints [B]
    (n_b cached tokens, the new token's key and value at position n_b - 1).
    The query at position n_b - 1 sees key j iff j <= n_b - 1 and
    (n_b - 1 - j <= w or j < p) ([SUM] mask) and gets
    o = sigmoid(l - s_h) * softmax(S) v with l the content-only log-sum-exp
    ([SUM]).  Returns (o [B, Hq, d], lse [B, Hq]), fp64.  A sequence with
    n_b = 0 has no keys: o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    sinks = np.asarray(sinks, dtype=np.float64)
    bsz, hq, d = q.shape
    group = hq // k_cache.shape[2]
    o = np.zeros((bsz, hq, d), np.float64)
    lse = np.full((bsz, hq), -np.inf, np.float64)
    for b in range(bsz):
        n = int(cache_seqlens[b])
        if n == 0:
            continue
        pos = n - 1
        j = np.arange(n)
        vis = (j <= pos) & ((pos - j <= window) | (j < prefix))
        for h in range(hq):
            kh = k_cache[b, :n, h // group, :]
            vh = v_cache[b, :n, h // group, :]
            sc = np.where(vis, scale * (kh @ q[b, h]), -np.inf)
            mx = sc.max()
            e = np.exp(sc - mx)
            z = e.sum()
            l = mx + np.log(z)
            alpha = 1.0 / (1.0 + np.exp(sinks[h] - l))      # sigmoid(l - s)
            o[b, h] = alpha * (e @ vh) / z
            lse[b, h] = l
    return o, lse

