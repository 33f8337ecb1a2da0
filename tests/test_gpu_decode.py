"""GPU parity of the decode path (one query token per sequence against its
key/value cache) with the fp64 oracle, through the C ABI; and the
train-inference consistency the rollout engine needs: decode on a cache of n
tokens equals row n - 1 of the training forward kernel.

Tolerances as in tests/parity_util.py: O max-abs <= 2e-2 (max(2e-2,
max|ref|/64) for inputs outside the named workloads), lse <= 1e-3 (the decode
kernels sum the probabilities in fp32); against the training forward the
same 1e-3 on l, on sequences that run the forward's 32-key kernels (fp32 row
sums) and on sequences of 1024 tokens or more that run its 64-key kernel
(fp16 row sums).
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import DECODE_LSE_TOL, TOL, log
from sink_aware_masked_sinkattn_amd import sinkattn_decode, sinkattn_fwd
from workloads import (DECODE_WORKLOADS, WINDOW_INF, decode_workload_inputs, make_decode_inputs,
                       make_inputs)

pytestmark = pytest.mark.gpu


def run_decode_gpu(inp):
    dev = torch.device("cuda:0")
    o, lse = sinkattn_decode(inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev),
                             inp.cache_seqlens.to(dev), inp.sinks.to(dev), inp.window, inp.prefix,
                             inp.scale)
    torch.cuda.synchronize()
    return o.to("cpu", torch.float64).numpy(), lse.to("cpu", torch.float64).numpy()


def run_decode_oracle(inp, lengths=None):
    lens = inp.cache_seqlens.tolist() if lengths is None else lengths
    return oracle.decode(inp.q.to(torch.float64).numpy(), inp.k_cache.to(torch.float64).numpy(),
                         inp.v_cache.to(torch.float64).numpy(), lens,
                         inp.sinks.to(torch.float64).numpy(), inp.window, inp.prefix, inp.scale)


def check(o, lse, ro, rl, label, scaled):
    tol_o = TOL["bf16"]["o"]
    if scaled:
        tol_o = max(tol_o, float(np.abs(ro).max()) / 64)
    err_o = float(np.abs(o - ro).max()) if o.size else 0.0
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin), label
    err_l = float(np.abs(lse[fin] - rl[fin]).max()) if fin.any() else 0.0
    log(f"{label}: max|dO| {err_o:.3g} (tol {tol_o:.3g}), max|dl| {err_l:.3g}")
    assert err_o <= tol_o, label
    assert err_l <= DECODE_LSE_TOL, label


SMALL = [
    # lengths, capacity, Hq, Hkv, w, p
    ((1, 2, 63, 64, 65, 300), 300, 8, 1, WINDOW_INF, 0),
    ((1, 127, 128, 129, 257), 260, 16, 1, 128, 4),
    ((5, 700, 1000), 1024, 8, 2, 128, 130),
    ((1, 2, 3, 90), 90, 4, 4, 0, 0),
    ((31, 64, 200), 256, 4, 2, 1, 3),
    ((100, 513), 600, 12, 3, 63, 64),
    ((4096,), 4096, 8, 1, WINDOW_INF, 0),
    ((0, 17, 40), 64, 8, 1, 5, 2),          # an empty cache gives o = 0, lse = -inf
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "n{}_cap{}_H{}x{}_w{}_p{}".format(
    "-".join(map(str, c[0])), *c[1:]))
def test_decode_small(case):
    lengths, cap, hq, hkv, w, p = case
    inp = make_decode_inputs(lengths=lengths, capacity=cap, heads_q=hq, heads_kv=hkv,
                             head_dim=64, window=w, prefix=p, seed=sum(lengths) + hq, std=1.0)
    log(f"decode case {case}")
    o, lse = run_decode_gpu(inp)
    ro, rl = run_decode_oracle(inp)
    check(o, lse, ro, rl, str(case), scaled=True)


def test_decode_lengths_clamped_to_capacity():
    # cache_seqlens beyond the capacity read as the capacity, negative as 0
    inp = make_decode_inputs(lengths=(50, 10), capacity=40, heads_q=8, heads_kv=1, head_dim=64,
                             window=WINDOW_INF, prefix=0, seed=7, std=1.0)
    inp.cache_seqlens = torch.tensor([50, -3], dtype=torch.int32)
    o, lse = run_decode_gpu(inp)
    ro, rl = run_decode_oracle(inp, lengths=[40, 0])
    check(o, lse, ro, rl, "clamped", scaled=True)


def test_decode_many_sequences():
    # more sequences than one LDS scan window holds (1024): the single-pass
    # kernel walks its unit list window by window; lengths 0 .. capacity
    g = torch.Generator().manual_seed(5)
    lengths = tuple(int(x) for x in torch.randint(0, 97, (1100,), generator=g))
    inp = make_decode_inputs(lengths=lengths, capacity=96, heads_q=4, heads_kv=1, head_dim=64,
                             window=WINDOW_INF, prefix=0, seed=17, std=1.0)
    o, lse = run_decode_gpu(inp)
    ro, rl = run_decode_oracle(inp)
    check(o, lse, ro, rl, "1100 sequences", scaled=True)


def test_decode_stream_wide_batch():
    # the stream kernel near its batch bound (batch * heads_kv just under 1024):
    # many segments, blocks crossing sequence boundaries, some empty caches
    g = torch.Generator().manual_seed(6)
    lengths = tuple(int(x) for x in torch.randint(0, 600, (127,), generator=g))
    inp = make_decode_inputs(lengths=lengths, capacity=600, heads_q=64, heads_kv=8, head_dim=64,
                             window=WINDOW_INF, prefix=0, seed=18, std=1.0)
    o, lse = run_decode_gpu(inp)
    ro, rl = run_decode_oracle(inp)
    check(o, lse, ro, rl, "127 sequences x 8 kv heads", scaled=True)


@pytest.mark.parametrize("t,lengths,w,p", [
    (600, (600, 257, 1), WINDOW_INF, 0),
    (600, (600, 257, 1), 128, 4),
    (600, (600, 257, 1), 9, 70),
    # min(w, n) >= 1024: the forward's 64-key kernel (row sums on the matrix cores)
    (1300, (1300, 1100, 257), WINDOW_INF, 0),
    (1300, (1300, 1100, 1025), 1100, 16),
])
def test_decode_matches_training_forward_row(t, lengths, w, p):
    # the rollout engine must reproduce the trainer's probabilities: decode
    # over the first n tokens of a sequence equals row n - 1 of the forward
    # kernel run on those tokens
    hq, hkv = 16, 2
    tr = make_inputs(batch=len(lengths), seqlen=t, heads_q=hq, heads_kv=hkv, head_dim=64,
                     window=w, prefix=p, seed=41 + t, std=0.5, dtype="bf16")
    dev = torch.device("cuda:0")
    q_dec = torch.stack([tr.q[b, n - 1] for b, n in enumerate(lengths)])
    o_dec, l_dec = sinkattn_decode(q_dec.to(dev), tr.k.to(dev), tr.v.to(dev),
                                   torch.tensor(lengths, dtype=torch.int32, device=dev),
                                   tr.sinks.to(dev), w, p, tr.scale)
    worst_o = worst_l = 0.0
    for b, n in enumerate(lengths):
        o_fw, l_fw = sinkattn_fwd(tr.q[b:b + 1, :n].to(dev).contiguous(),
                                  tr.k[b:b + 1, :n].to(dev).contiguous(),
                                  tr.v[b:b + 1, :n].to(dev).contiguous(), tr.sinks.to(dev), w, p,
                                  tr.scale)
        worst_o = max(worst_o, float((o_dec[b].float() - o_fw[0, n - 1].float()).abs().max()))
        worst_l = max(worst_l, float((l_dec[b] - l_fw[0, :, n - 1]).abs().max()))
    log(f"decode vs forward row (T={t}, w={w}, p={p}): max|dO| {worst_o:.3g}, "
        f"max|dl| {worst_l:.3g}")
    assert worst_o <= TOL["bf16"]["o"]
    assert worst_l <= TOL["bf16"]["lse"]


@pytest.mark.slow
@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workload_full_size(name):
    for li, inp in enumerate(decode_workload_inputs(name)):
        log(f"{name} layer {li}: w={inp.window} p={inp.prefix}")
        o, lse = run_decode_gpu(inp)
        ro, rl = run_decode_oracle(inp)
        check(o, lse, ro, rl, f"{name}[{li}]", scaled=False)
