"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs.  Tolerances are in tests/parity_util.py.

Small cases span several query and key tiles of both tile configurations
(narrow tiles for windows under 1024, wide ones otherwise) with ragged tails, every mask regime
(plain causal, window, prefix, window+prefix, w=0, prefix past the end), GQA
and varlen packing with empty, single-token and tile-edge lengths.  The
named workloads run at their full sizes and are compared on every head (see
the section on them below).
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, compare, log, run_gpu, run_oracle
from workloads import WINDOW_INF, WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu


SMALL = [
    # B, T, Hq, Hkv, w, p, std
    (2, 300, 8, 2, WINDOW_INF, 0, 0.5),
    (1, 333, 4, 1, 128, 0, 1.0),
    (2, 300, 8, 2, 128, 4, 0.5),
    (1, 257, 4, 4, 0, 0, 1.0),
    (1, 257, 4, 2, 1, 0, 1.0),
    (1, 400, 4, 2, 63, 1, 0.5),
    (1, 400, 4, 2, 64, 5, 0.5),
    (1, 300, 4, 2, 200, 300, 0.5),
    (1, 520, 4, 2, 5, 130, 0.5),
    (1, 64, 2, 1, 16, 4, 1.0),
    (3, 129, 16, 2, 31, 2, 0.5),
    (1, 1, 2, 1, 0, 0, 1.0),
    (2, 97, 8, 1, 0, 3, 1.0),      # four heads per forward workgroup, diagonal plus prefix
    # key block 0 split over several dK/dV work units (atomic flushes), the
    # later query tiles seeing only its prefix keys, p up to 32
    (1, 640, 8, 1, 100, 4, 0.5),
    (2, 700, 16, 2, 64, 16, 0.5),
    (1, 900, 8, 2, 40, 32, 0.5),
    # the prefix fold with key blocks split over two dK/dV work units (GQA
    # group of 16: the accumulating path), and p just past the fold's limit
    (1, 700, 16, 1, 128, 8, 0.5),
    (1, 600, 8, 2, 128, 17, 0.5),
    # many sequences of one length (grid y), window dQ kernel and fold
    (64, 300, 8, 2, 64, 4, 0.5),
    # windows >= 1024 after clamping run the wide-tile kernels (64-key forward /
    # dQ tiles, 128-row dK/dV tiles); shorter ones the narrow-tile kernels
    (1, 1100, 4, 2, WINDOW_INF, 0, 0.5),
    # large logits: frequent lazy rescales of the 64-key forward's output and
    # matrix-core row sums, probabilities spread over many binades
    (1, 1100, 4, 2, WINDOW_INF, 0, 2.0),
    (1, 1090, 4, 1, 1030, 70, 0.5),
    (2, 1200, 4, 2, 2000, 3, 0.5),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_T{}_H{}x{}_w{}_p{}_s{}".format(*c))
def test_bf16_small(case):
    b, t, hq, hkv, w, p, std = case
    inp = make_inputs(batch=b, seqlen=t, heads_q=hq, heads_kv=hkv, head_dim=64, window=w,
                      prefix=p, seed=hash(case) % 100000, std=std, dtype="bf16")
    log(f"case {case}")
    compare(run_gpu(inp), run_oracle(inp), "bf16", inp, label=str(case), scaled=True)


@pytest.mark.parametrize("lengths,w,p", [
    ((1, 63, 65, 255, 257, 300), 20, 3),
    ((0, 5, 0, 130), 4, 2),
    ((512, 1, 77), WINDOW_INF, 0),
    ((200, 300), 128, 16),
    ((1100, 37, 0, 1030), WINDOW_INF, 5),
    ((700, 300, 900), 50, 8),      # several dK/dV units per key block in the long sequences
    # packed grids sized from the token count: many short sequences, prefixes over
    # several 128-key blocks, empty and single-token sequences
    ((5, 0, 129, 1, 300, 64, 700, 33, 128, 2), 30, 200),
    ((1000, 999, 1, 0, 640), 128, 16),
    ((257,) * 12, 64, 130),
    # the prefix fold with sequences shorter than the prefix and than the fold row
    ((1, 5, 15, 16, 17, 0, 300, 40), 128, 16),
    # 150 packed sequences: the per-sequence scans of the work lists and the
    # fold's sum walk more than two 64-sequence steps
    (tuple((37 * i) % 97 + (260 if i % 10 == 0 else 0) for i in range(150)), 64, 8),
])
def test_bf16_varlen_small(lengths, w, p):
    inp = make_inputs(batch=0, seqlen=0, heads_q=8, heads_kv=2, head_dim=64, window=w, prefix=p,
                      seed=sum(lengths) + w, std=0.5, dtype="bf16", lengths=lengths)
    log(f"varlen {lengths} w={w} p={p}")
    compare(run_gpu(inp), run_oracle(inp), "bf16", inp, label=f"varlen{lengths}", scaled=True)


@pytest.mark.parametrize("lengths,hq,hkv,w,p", [
    # GQA group of 16 packed: the window dQ kernel takes four heads per wave
    # and the prefix fold runs with key blocks split over two dK/dV units
    ((700, 300, 129, 0, 520), 16, 1, 128, 8),
    # group of 12: the last round of each wave takes one head
    ((400, 33, 260), 12, 1, 96, 16),
])
def test_bf16_varlen_wide_groups(lengths, hq, hkv, w, p):
    inp = make_inputs(batch=0, seqlen=0, heads_q=hq, heads_kv=hkv, head_dim=64, window=w, prefix=p,
                      seed=sum(lengths) + hq, std=0.5, dtype="bf16", lengths=lengths)
    log(f"varlen {lengths} Hq={hq} Hkv={hkv} w={w} p={p}")
    compare(run_gpu(inp), run_oracle(inp), "bf16", inp, label=f"varlen{lengths}/{hq}", scaled=True)


@pytest.mark.parametrize("sinks", [(float("-inf"), -10.0, 0.0, 10.0)])
def test_bf16_sink_extremes(sinks):
    inp = make_inputs(batch=1, seqlen=200, heads_q=4, heads_kv=2, head_dim=64, window=30,
                      prefix=2, seed=5, std=1.0, dtype="bf16", sink_values=sinks)
    compare(run_gpu(inp), run_oracle(inp), "bf16", inp, label="sinks", scaled=True)


@pytest.mark.parametrize("d,case", [(32, (1, 128, 2, 2, 16, 4)), (32, (2, 200, 4, 2, 7, 0)),
                                    (64, (1, 150, 4, 1, WINDOW_INF, 0)),
                                    (32, (1, 90, 2, 1, 0, 50))])
def test_fp32_small(d, case):
    b, t, hq, hkv, w, p = case
    inp = make_inputs(batch=b, seqlen=t, heads_q=hq, heads_kv=hkv, head_dim=d, window=w,
                      prefix=p, seed=d + t, std=1.0, dtype="fp32")
    compare(run_gpu(inp), run_oracle(inp), "fp32", inp, label=f"fp32 d{d} {case}")


# Mask-edge sweep (the windows and prefixes around every tile size the kernels
# use: 32- and 64-key tiles, 32-row window dQ blocks, 64-row fp32 row blocks,
# 128-row dK/dV tiles), ragged lengths packed into one call, and the sink
# logits -inf, -10, 0, +10 on the four query heads.
SWEEP_SINKS = (float("-inf"), -10.0, 0.0, 10.0)
SWEEP_W = (0, 31, 32, 33, 63, 64, 65, 127, 128, 129, WINDOW_INF)
SWEEP_P = (0, 1, 32, 64, 128, 100000)


@pytest.mark.parametrize("w", SWEEP_W, ids=lambda w: f"w{w}")
@pytest.mark.parametrize("p", SWEEP_P, ids=lambda p: f"p{p}")
def test_fp32_mask_edge_sweep(w, p):
    lengths = (1, 63, 65, 129, 130)
    inp = make_inputs(batch=0, seqlen=0, heads_q=4, heads_kv=2, head_dim=32, window=w, prefix=p,
                      seed=w % 997 + p % 991, std=1.0, dtype="fp32", lengths=lengths,
                      sink_values=SWEEP_SINKS)
    compare(run_gpu(inp), run_oracle(inp), "fp32", inp, label=f"fp32 sweep w={w} p={p}",
            scaled=True)


@pytest.mark.parametrize("w", SWEEP_W + (1023, 1024, 1025), ids=lambda w: f"w{w}")
@pytest.mark.parametrize("p", SWEEP_P, ids=lambda p: f"p{p}")
def test_bf16_mask_edge_sweep(w, p):
    # the longest sequence (1090) puts windows >= 1024 on the 64-key kernels
    lengths = (1, 31, 33, 127, 129, 257, 1090)
    inp = make_inputs(batch=0, seqlen=0, heads_q=4, heads_kv=1, head_dim=64, window=w, prefix=p,
                      seed=w % 997 + 7 * (p % 991), std=1.0, dtype="bf16", lengths=lengths,
                      sink_values=SWEEP_SINKS)
    compare(run_gpu(inp), run_oracle(inp), "bf16", inp, label=f"bf16 sweep w={w} p={p}",
            scaled=True)


def test_fp32_varlen():
    inp = make_inputs(batch=0, seqlen=0, heads_q=2, heads_kv=1, head_dim=32, window=9, prefix=3,
                      seed=3, std=1.0, dtype="fp32", lengths=(17, 0, 64, 1))
    compare(run_gpu(inp), run_oracle(inp), "fp32", inp, label="fp32 varlen")


# ------------------------------------------------------------ named workloads

def test_workload_tiny_fp32():
    (inp,) = workload_inputs("tiny_fp32")
    compare(run_gpu(inp), run_oracle(inp), "fp32", inp, label="tiny_fp32")


# Full-size comparisons of the named workloads.  The GPU runs every head in the
# launch configuration the benchmark times; the oracle then checks every head:
#   * short-window layers (w=128): every row of every head (o, lse, dq, ds) and,
#     for every kv group, dk/dv at the prefix keys, keys around a 128-key dK/dV
#     block edge mid-sequence and the last keys; groups 0 and 7 at every key;
#   * full-causal layers: every head at sampled rows (tile edges, the prefix,
#     the last rows, random rows) and every kv group's last keys (few rows see
#     them); groups 0 and 7 in full with the dense oracle (every row and key,
#     ds of their heads).
# The short-window references use the oracle's row/key-restricted forms (the
# same definition over each row's visible band; pinned in
# test_oracle_pins.py), the dense ones oracle.forward / oracle.backward.

NAMED_LAYERS = [("gqa_swa_4096", 0), ("gqa_causal_4096", 0), ("long_8192", 0), ("long_8192", 1)]
_FULL = {}


def _full(name, layer):
    """GPU outputs of a named workload layer at full size (one layer cached at a time)."""
    key = (name, layer)
    if key not in _FULL:
        _FULL.clear()
        inp = workload_inputs(name)[layer]
        log(f"{name} layer {layer}: GPU run (full size, every head)")
        _FULL[key] = (inp, run_gpu(inp))
    return _FULL[key]


def _group_heads(inp, kv):
    return list(range(kv * inp.group, (kv + 1) * inp.group))


def _np_head(t, b, h):
    return t[b, :, h].to(torch.float64).numpy()


def _sample_rows(n, prefix, seed):
    edges = {0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513,
             n // 2 - 1, n // 2, n - 257, n - 256, n - 129, n - 128, n - 65, n - 64, n - 33,
             n - 32, n - 3, n - 2, n - 1}
    if prefix:
        edges |= {prefix - 1, prefix, prefix + 1}
    rnd = np.random.default_rng(seed).choice(n, size=min(n, 32), replace=False)
    return np.unique(np.array([r for r in edges if 0 <= r < n] + list(rnd), dtype=np.int64))


def _sample_keys(n, window, prefix):
    keys = set(range(max(0, n - 64), n))
    if window < n:   # short window: few rows see any key, so more blocks are cheap
        keys |= set(range(min(prefix, n)))
        keys |= set(range(max(0, n // 2 - 40), min(n, n // 2 + 40)))
        keys |= {j for j in (126, 127, 128, 129, 254, 255, 256, 257) if j < n}
    return np.array(sorted(keys), dtype=np.int64)


class _Errs:
    """Running max-abs errors per output, asserted at the end against the bf16 tolerances
    (scaled: the rule for cases outside the named workloads, max(tol, max|ref| / 64)
    on o, dq, dk, dv; see tests/parity_util.py)."""

    def __init__(self, label, scaled=False):
        self.label, self.e, self.m, self.scaled = label, {}, {}, scaled

    def add(self, name, gpu, ref):
        assert np.all(np.isfinite(gpu)), f"{self.label} {name}: non-finite GPU values"
        err = float(np.max(np.abs(gpu - ref))) if np.size(ref) else 0.0
        self.e[name] = max(self.e.get(name, 0.0), err)
        if np.size(ref):
            self.m[name] = max(self.m.get(name, 0.0), float(np.max(np.abs(ref))))

    def tol(self, name):
        t = TOL["bf16"][name]
        if self.scaled and name in ("o", "dq", "dk", "dv"):
            t = max(t, self.m.get(name, 0.0) / 64)
        return t

    def check(self, ds_gpu=None, ds_ref=None):
        if ds_ref is not None:
            self.e["ds"] = float(np.max(np.abs(ds_gpu - ds_ref)) / np.max(np.abs(ds_ref)))
        log(f"  {self.label} errors: " + ", ".join(f"{n}={e:.3g} (tol {self.tol(n):.3g})"
                                                   for n, e in self.e.items()))
        for n, e in self.e.items():
            assert e <= self.tol(n), f"{self.label} {n}: error {e:.3g} > {self.tol(n):.3g}"


@pytest.mark.slow
@pytest.mark.parametrize("name,layer", NAMED_LAYERS)
def test_workload_every_head(name, layer):
    """Every query head and every kv group of the layer against the oracle (see above)."""
    inp, gpu = _full(name, layer)
    n, hq, hkv = inp.q.shape[1], inp.q.shape[2], inp.k.shape[2]
    w, p, sc = inp.window, inp.prefix, inp.scale
    short = w < n
    rows = np.arange(n) if short else _sample_rows(n, p, seed=hq + n)
    keys = _sample_keys(n, w, p)
    errs = _Errs(f"{name}[{layer}] every head, {rows.size} rows, {keys.size} keys per kv group")
    ds_ref = np.zeros(hq)
    dk_ref = np.zeros((hkv, keys.size, inp.q.shape[3]))
    dv_ref = np.zeros_like(dk_ref)
    for h in range(hq):
        kv = h // inp.group
        q, k, v, do = (_np_head(t, 0, i) for t, i in ((inp.q, h), (inp.k, kv), (inp.v, kv),
                                                       (inp.do, h)))
        s = float(inp.sinks[h])
        st = oracle.rows_head(q, k, v, s, w, p, sc, rows, do=do)
        errs.add("o", gpu["o"][0, rows, h], st["o"])
        errs.add("lse", gpu["lse"][0, h, rows], st["l"])
        errs.add("dq", gpu["dq"][0, rows, h], st["dq"])
        if short:
            ds_ref[h] = -float(np.sum(np.exp(s - st["big_l"]) * st["d_row"]))
        dkh, dvh = oracle.key_grads_head(q, k, v, s, w, p, sc, do, keys,
                                         row_stats=st if short else None)
        dk_ref[kv] += dkh
        dv_ref[kv] += dvh
    for kv in range(hkv):
        errs.add("dk", gpu["dk"][0, keys, kv], dk_ref[kv])
        errs.add("dv", gpu["dv"][0, keys, kv], dv_ref[kv])
    errs.check(gpu["ds"] if short else None, ds_ref if short else None)


@pytest.mark.slow
@pytest.mark.parametrize("name,layer,kv", [(nm, ly, kv) for nm, ly in NAMED_LAYERS for kv in (0, 7)])
def test_workload_whole_group(name, layer, kv):
    """One whole GQA group (8 query heads and their kv head) at every row and key,
    including the sink gradient of its heads."""
    inp, gpu = _full(name, layer)
    heads = _group_heads(inp, kv)
    n = inp.q.shape[1]
    if inp.window < n:
        errs = _Errs(f"{name}[{layer}] kv{kv}")
        w, p, sc = inp.window, inp.prefix, inp.scale
        k, v = _np_head(inp.k, 0, kv), _np_head(inp.v, 0, kv)
        dk_ref = np.zeros((n, inp.q.shape[3]))
        dv_ref = np.zeros_like(dk_ref)
        ds_ref = np.zeros(len(heads))
        for i, h in enumerate(heads):
            q, do = _np_head(inp.q, 0, h), _np_head(inp.do, 0, h)
            s = float(inp.sinks[h])
            st = oracle.rows_head(q, k, v, s, w, p, sc, np.arange(n), do=do)
            errs.add("o", gpu["o"][0, :, h], st["o"])
            errs.add("lse", gpu["lse"][0, h], st["l"])
            errs.add("dq", gpu["dq"][0, :, h], st["dq"])
            ds_ref[i] = -float(np.sum(np.exp(s - st["big_l"]) * st["d_row"]))
            dkh, dvh = oracle.key_grads_head(q, k, v, s, w, p, sc, do, np.arange(n), row_stats=st)
            dk_ref += dkh
            dv_ref += dvh
        errs.add("dk", gpu["dk"][0, :, kv], dk_ref)
        errs.add("dv", gpu["dv"][0, :, kv], dv_ref)
        errs.check(gpu["ds"][heads], ds_ref)
        return
    log(f"{name} layer {layer}: dense oracle on heads {heads}")
    ref = run_oracle(inp, heads=heads)
    compare(gpu, ref, "bf16", inp, heads=heads, label=f"{name}[{layer}] kv{kv}")


@pytest.mark.slow
@pytest.mark.parametrize("t,w,p", [(131072, WINDOW_INF, 0), (65536, 128, 4)],
                         ids=["causal_T131072", "w128_p4_T65536"])
def test_long_sequence_sampled(t, w, p):
    """Sequences 8 and 16 times the benchmark's length (one GQA group of 8 heads):
    o, lse and dq of every head at sampled rows (tile edges, the prefix, the
    last rows, random rows), dk and dv at sampled keys, and for the short window
    the sink gradient from every row -- against the oracle's row- and
    key-restricted forms."""
    inp = make_inputs(batch=1, seqlen=t, heads_q=8, heads_kv=1, head_dim=64, window=w, prefix=p,
                      seed=t % 1000 + p, std=0.5, dtype="bf16")
    log(f"long sequence T={t} w={w} p={p}: GPU run")
    gpu = run_gpu(inp)
    short = w < t
    rows = np.arange(t) if short else _sample_rows(t, p, seed=t)
    keys = _sample_keys(t, w, p)
    # outside the named workloads: the scaled bound (a prefix key's dV here sums
    # the rows of eight times the benchmark's sequence, magnitude about 7)
    errs = _Errs(f"T={t} w={w} p={p}, {rows.size} rows, {keys.size} keys", scaled=True)
    ds_ref = np.zeros(8)
    dk_ref = np.zeros((keys.size, 64))
    dv_ref = np.zeros_like(dk_ref)
    k, v = _np_head(inp.k, 0, 0), _np_head(inp.v, 0, 0)
    for h in range(8):
        q, do = _np_head(inp.q, 0, h), _np_head(inp.do, 0, h)
        s = float(inp.sinks[h])
        st = oracle.rows_head(q, k, v, s, w, p, inp.scale, rows, do=do)
        errs.add("o", gpu["o"][0, rows, h], st["o"])
        errs.add("lse", gpu["lse"][0, h, rows], st["l"])
        errs.add("dq", gpu["dq"][0, rows, h], st["dq"])
        if short:
            ds_ref[h] = -float(np.sum(np.exp(s - st["big_l"]) * st["d_row"]))
        dkh, dvh = oracle.key_grads_head(q, k, v, s, w, p, inp.scale, do, keys,
                                         row_stats=st if short else None)
        dk_ref += dkh
        dv_ref += dvh
    errs.add("dk", gpu["dk"][0, keys, 0], dk_ref)
    errs.add("dv", gpu["dv"][0, keys, 0], dv_ref)
    errs.check(gpu["ds"] if short else None, ds_ref if short else None)


_VARLEN = {}


def _varlen_state():
    if "inp" not in _VARLEN:
        (inp,) = workload_inputs("varlen_grpo_g8")
        _VARLEN["inp"] = inp
        log(f"varlen_grpo_g8 lengths {inp.lengths}: GPU run")
        _VARLEN["gpu"] = run_gpu(inp)
        _VARLEN["ds_parts"] = {}
    return _VARLEN


VARLEN_GROUPS = (2, 7)


@pytest.mark.slow
@pytest.mark.parametrize("seq", list(range(8)))
def test_workload_varlen_per_sequence(seq):
    """Packed GRPO group (8 rollouts): the whole pack runs on the GPU in one call.  Per
    sequence the oracle checks every head at sampled rows, every kv group at sampled
    keys, and GQA groups 2 and 7 at every row and key (with their sink gradient,
    summed over the sequences once all eight have run)."""
    st_all = _varlen_state()
    inp, gpu = st_all["inp"], st_all["gpu"]
    cu = inp.cu_seqlens.numpy()
    r0, r1 = int(cu[seq]), int(cu[seq + 1])
    n = r1 - r0
    hq, hkv, d = inp.q.shape[1], inp.k.shape[1], inp.q.shape[2]
    w, p, sc = inp.window, inp.prefix, inp.scale
    errs = _Errs(f"varlen seq {seq} (len {n})")
    seqt = lambda t, h: t[r0:r1, h].to(torch.float64).numpy()  # noqa: E731
    rows = _sample_rows(n, p, seed=seq)
    keys = _sample_keys(n, w, p)
    full = set()
    for kv in VARLEN_GROUPS:
        full |= set(_group_heads(inp, kv))
    ds_part = np.zeros(hq)
    dk_ref = np.zeros((hkv, n, d))
    dv_ref = np.zeros_like(dk_ref)
    for h in range(hq):
        kv = h // inp.group
        q, k, v, do = seqt(inp.q, h), seqt(inp.k, kv), seqt(inp.v, kv), seqt(inp.do, h)
        s = float(inp.sinks[h])
        if h in full:
            st = oracle.rows_head(q, k, v, s, w, p, sc, np.arange(n), do=do)
            errs.add("o", gpu["o"][r0:r1, h], st["o"])
            errs.add("lse", gpu["lse"][h, r0:r1], st["l"])
            errs.add("dq", gpu["dq"][r0:r1, h], st["dq"])
            ds_part[h] = -float(np.sum(np.exp(s - st["big_l"]) * st["d_row"]))
            dkh, dvh = oracle.key_grads_head(q, k, v, s, w, p, sc, do, np.arange(n), row_stats=st)
            dk_ref[kv] += dkh
            dv_ref[kv] += dvh
        else:
            st = oracle.rows_head(q, k, v, s, w, p, sc, rows, do=do)
            errs.add("o", gpu["o"][r0 + rows, h], st["o"])
            errs.add("lse", gpu["lse"][h, r0 + rows], st["l"])
            errs.add("dq", gpu["dq"][r0 + rows, h], st["dq"])
            dkh, dvh = oracle.key_grads_head(q, k, v, s, w, p, sc, do, keys)
            dk_ref[kv, keys] += dkh
            dv_ref[kv, keys] += dvh
    for kv in range(hkv):
        sel = np.arange(n) if kv in VARLEN_GROUPS else keys
        errs.add("dk", gpu["dk"][r0 + sel, kv], dk_ref[kv, sel])
        errs.add("dv", gpu["dv"][r0 + sel, kv], dv_ref[kv, sel])
    errs.check()
    st_all["ds_parts"][seq] = ds_part
    if len(st_all["ds_parts"]) == 8:
        heads = sorted(full)
        ds_ref = sum(st_all["ds_parts"].values())[heads]
        err = float(np.max(np.abs(gpu["ds"][heads] - ds_ref)) / np.max(np.abs(ds_ref)))
        log(f"  varlen ds (all sequences, heads {heads}) norm-wise rel error {err:.3g}")
        assert err <= TOL["bf16"]["ds"]


# ------------------------------------------------------------------ invariants

def test_varlen_equals_separate_calls():
    lengths = (70, 300, 129)
    inp = make_inputs(batch=0, seqlen=0, heads_q=8, heads_kv=2, head_dim=64, window=40, prefix=3,
                      seed=17, std=0.5, dtype="bf16", lengths=lengths)
    full = run_gpu(inp)
    cu = inp.cu_seqlens.numpy()
    ds_sum = np.zeros_like(full["ds"])
    for i, L in enumerate(lengths):
        r = slice(int(cu[i]), int(cu[i + 1]))
        one = make_inputs(batch=1, seqlen=L, heads_q=8, heads_kv=2, head_dim=64, window=40,
                          prefix=3, seed=0, dtype="bf16")
        one.q, one.k, one.v, one.do = (t[r].unsqueeze(0) for t in (inp.q, inp.k, inp.v, inp.do))
        one.sinks = inp.sinks
        sep = run_gpu(one)
        np.testing.assert_array_equal(full["o"][r], sep["o"][0])
        np.testing.assert_array_equal(full["lse"][:, r], sep["lse"][0])
        for n in ("dq", "dk", "dv"):
            np.testing.assert_allclose(full[n][r], sep[n][0], atol=1e-2)
        ds_sum += sep["ds"]
    np.testing.assert_allclose(full["ds"], ds_sum, rtol=1e-3, atol=1e-3)


def test_gqa_equals_mha_with_repeated_kv():
    inp = make_inputs(batch=1, seqlen=300, heads_q=8, heads_kv=2, head_dim=64, window=100,
                      prefix=2, seed=23, std=0.5, dtype="bf16")
    gqa = run_gpu(inp)
    mha = make_inputs(batch=1, seqlen=300, heads_q=8, heads_kv=8, head_dim=64, window=100,
                      prefix=2, seed=0, dtype="bf16")
    mha.q, mha.do, mha.sinks = inp.q, inp.do, inp.sinks
    mha.k = inp.k.repeat_interleave(4, dim=2).contiguous()
    mha.v = inp.v.repeat_interleave(4, dim=2).contiguous()
    rep = run_gpu(mha)
    np.testing.assert_array_equal(gqa["o"], rep["o"])
    np.testing.assert_array_equal(gqa["lse"], rep["lse"])
    np.testing.assert_allclose(gqa["dq"], rep["dq"], atol=1e-2)
    for n in ("dk", "dv"):
        summed = rep[n].reshape(1, 300, 2, 4, 64).sum(axis=3)
        np.testing.assert_allclose(gqa[n], summed, atol=2e-2)


def test_memory_grows_linearly():
    """Peak device memory of fwd+bwd (workspace included) is O(T)."""
    peaks = {}
    for t in (2048, 4096, 8192, 16384):
        inp = make_inputs(batch=1, seqlen=t, heads_q=64, heads_kv=8, head_dim=64,
                          window=WINDOW_INF, prefix=0, seed=1, std=0.5, dtype="bf16")
        dev = torch.device("cuda:0")
        q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
        s = inp.sinks.to(dev)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        from sink_aware_masked_sinkattn_amd import sinkattn_bwd, sinkattn_fwd
        o, lse = sinkattn_fwd(q, k, v, s, inp.window, inp.prefix, inp.scale)
        grads = sinkattn_bwd(q, k, v, s, o, lse, do, inp.window, inp.prefix, inp.scale)
        torch.cuda.synchronize()
        peaks[t] = torch.cuda.max_memory_allocated() - base
        del o, lse, grads, q, k, v, do
        log(f"  T={t}: peak extra {peaks[t] / 2**20:.1f} MiB")
    # doubling T must not more than double (plus slack) the extra memory
    assert peaks[4096] <= 2.1 * peaks[2048]
    assert peaks[8192] <= 2.1 * peaks[4096]
    assert peaks[16384] <= 2.1 * peaks[8192]


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp32", 32)])
def test_bwd_phases_equal_single_call(dtype, d):
    from sink_aware_masked_sinkattn_amd import (BWD_DKDV, BWD_DQ, BWD_FINISH, BWD_PREPARE,
                                                sinkattn_bwd, sinkattn_bwd_phases, sinkattn_fwd)
    inp = make_inputs(batch=1, seqlen=700, heads_q=8, heads_kv=2, head_dim=d, window=100,
                      prefix=3, seed=31, std=0.5, dtype=dtype)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.do))
    s = inp.sinks.to(dev)
    o, lse = sinkattn_fwd(q, k, v, s, inp.window, inp.prefix, inp.scale)
    ref = sinkattn_bwd(q, k, v, s, o, lse, do, inp.window, inp.prefix, inp.scale)
    grads = tuple(torch.full_like(t, float("nan")) for t in ref)
    ws = torch.full((1 << 26,), 255, dtype=torch.uint8, device=dev)
    for ph in (BWD_PREPARE, BWD_DQ, BWD_DKDV, BWD_FINISH):
        sinkattn_bwd_phases(ph, q, k, v, s, o, lse, do, inp.window, inp.prefix, inp.scale,
                            workspace=ws, grads=grads)
    torch.cuda.synchronize()
    for a, b in zip(ref, grads):
        assert torch.isfinite(b).all()
        torch.testing.assert_close(a.float(), b.float(), atol=1e-3, rtol=1e-3)


@pytest.mark.parametrize("case", [(1, 700, 16, 2, 128, 4), (2, 300, 8, 1, WINDOW_INF, 0),
                                  (1, 400, 6, 2, 63, 5)],
                         ids=["win_dq", "causal", "group3"])
def test_repeat_calls_bitwise_equal(case):
    # o, lse, dq and the sink gradient involve no atomics: the sink gradient
    # is added from per-workgroup parts in a fixed order, so two calls on the
    # same inputs agree bit for bit.  dK/dV of key blocks split over several
    # work units are added with float atomics and may differ in the last bit;
    # in the short-window case every key block is one unit (stored whole, the
    # prefix fold's parts added in a fixed order), so dK and dV agree too.
    b, t, hq, hkv, w, p = case
    inp = make_inputs(batch=b, seqlen=t, heads_q=hq, heads_kv=hkv, head_dim=64, window=w,
                      prefix=p, seed=t + hq, std=0.5, dtype="bf16")
    first, second = run_gpu(inp), run_gpu(inp)
    names = ("o", "lse", "dq", "ds") + (("dk", "dv") if w == 128 else ())
    for name in names:
        np.testing.assert_array_equal(first[name], second[name], err_msg=f"{case} {name}")
