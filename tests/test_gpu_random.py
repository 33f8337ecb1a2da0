"""GPU parity on seeded random problem shapes: batch or packed lengths, GQA
group sizes 1..16, windows and prefixes around every tile width, value
scales 0.5 and 1 (bf16); small fp32 problems with head dims 32 and 64; and
rollout-decode batches of random cache lengths, capacities and group sizes.
Each case runs the HIP library through its C ABI and the fp64 oracle on the
same inputs and compares them under the tolerances of tests/parity_util.py
(the scaled bound for cases outside the named workloads).  The shapes are drawn once from a fixed seed, so the list is the
same on every run."""
import numpy as np
import pytest

from parity_util import compare, log, run_gpu, run_oracle
from workloads import WINDOW_INF, make_inputs

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 1, 2, 4]))
        group = int(rng.choice([1, 2, 3, 4, 8, 12, 16]))
        hq = hkv * group
        if hq > 32:
            hq, group = hkv * 8, 8
        w = int(rng.choice([0, 1, 7, 31, 32, 33, 64, 96, 127, 128, 129, 160, 300, 1023,
                            1024, 1500, WINDOW_INF]))
        p = int(rng.choice([0, 0, 1, 2, 4, 15, 16, 17, 32, 33, 100, 5000]))
        std = float(rng.choice([0.5, 1.0]))
        if rng.random() < 0.4:
            k = int(rng.integers(1, 9))
            lengths = tuple(int(x) for x in rng.integers(0, 700, size=k))
            out.append(dict(batch=0, seqlen=0, lengths=lengths, heads_q=hq, heads_kv=hkv,
                            window=w, prefix=p, std=std, seed=1000 + i))
        else:
            b = int(rng.integers(1, 4))
            t = int(rng.integers(1, 1200))
            out.append(dict(batch=b, seqlen=t, lengths=None, heads_q=hq, heads_kv=hkv,
                            window=w, prefix=p, std=std, seed=1000 + i))
    return out


CASES = _cases()


def _id(c):
    shape = f"L{len(c['lengths'])}" if c["lengths"] is not None else f"B{c['batch']}_T{c['seqlen']}"
    w = "inf" if c["window"] >= WINDOW_INF else c["window"]
    return f"{shape}_H{c['heads_q']}x{c['heads_kv']}_w{w}_p{c['prefix']}_s{c['std']}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape(case):
    kw = dict(case)
    lengths = kw.pop("lengths")
    inp = make_inputs(head_dim=64, dtype="bf16", lengths=lengths, **kw)
    log(f"random case {_id(case)} lengths={lengths}")
    compare(run_gpu(inp), run_oracle(inp), "bf16", inp, label=_id(case), scaled=True)


def _fp32_cases(n=12, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2, 4]))
        out.append(dict(batch=int(rng.integers(1, 3)), seqlen=int(rng.integers(1, 260)),
                        heads_q=hq, heads_kv=hkv, head_dim=int(rng.choice([32, 64])),
                        window=int(rng.choice([0, 1, 15, 63, 64, 65, 200, WINDOW_INF])),
                        prefix=int(rng.choice([0, 1, 3, 64, 1000])), seed=2000 + i))
    return out


FP32_CASES = _fp32_cases()


@pytest.mark.parametrize("case", FP32_CASES,
                         ids=[f"B{c['batch']}_T{c['seqlen']}_H{c['heads_q']}x{c['heads_kv']}_d"
                              f"{c['head_dim']}_w{c['window']}_p{c['prefix']}" for c in FP32_CASES])
def test_random_shape_fp32(case):
    inp = make_inputs(dtype="fp32", std=1.0, **case)
    log(f"random fp32 case {case}")
    compare(run_gpu(inp), run_oracle(inp), "fp32", inp, label=str(case), scaled=True)


def _decode_cases(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 8]))
        hq = hkv * int(rng.choice([1, 4, 8, 16]))
        if hq > 64:
            hq = hkv * 8
        cap = int(rng.integers(1, 3000))
        k = int(rng.integers(1, 40))
        lengths = tuple(int(x) for x in rng.integers(0, cap + 1, size=k))
        out.append((lengths, cap, hq, hkv,
                    int(rng.choice([0, 1, 31, 128, 1023, 2000, WINDOW_INF])),
                    int(rng.choice([0, 1, 4, 16, 100])), 3000 + i))
    return out


DECODE_CASES = _decode_cases()


@pytest.mark.parametrize("case", DECODE_CASES,
                         ids=[f"N{len(c[0])}_cap{c[1]}_H{c[2]}x{c[3]}_w{c[4]}_p{c[5]}"
                              for c in DECODE_CASES])
def test_random_decode(case):
    from test_gpu_decode import check, run_decode_gpu, run_decode_oracle
    from workloads import make_decode_inputs
    lengths, cap, hq, hkv, w, p, seed = case
    inp = make_decode_inputs(lengths=lengths, capacity=cap, heads_q=hq, heads_kv=hkv,
                             head_dim=64, window=w, prefix=p, seed=seed, std=1.0)
    log(f"random decode case {case[1:]} over {len(lengths)} caches")
    o, lse = run_decode_gpu(inp)
    ro, rl = run_decode_oracle(inp)
    check(o, lse, ro, rl, f"decode {case[1:]}", scaled=True)
