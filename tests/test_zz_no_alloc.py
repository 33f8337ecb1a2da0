"""The allocation-free decode entry point (sinkattn_decode_noalloc, for callers
that cannot allocate device memory) against sinkattn_decode, through the C ABI:
two calls in a row, the second smaller, each bitwise equal to the workspace
entry point's result and within the decode tolerances of the fp64 oracle
(O max-abs 2e-2, or max|ref|/64 for unit-scale inputs; lse 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import DECODE_LSE_TOL, TOL, log
from sink_aware_masked_sinkattn_amd import (SinkAttnError, sinkattn_decode,
                                            sinkattn_decode_noalloc)
from workloads import WINDOW_INF, decode_workload_inputs, make_decode_inputs

pytestmark = pytest.mark.gpu


def _call_both(inp):
    dev = torch.device("cuda:0")
    args = (inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev),
            inp.cache_seqlens.to(dev), inp.sinks.to(dev), inp.window, inp.prefix, inp.scale)
    o_ws, l_ws = sinkattn_decode(*args)
    # outputs allocated up front and poisoned, so nothing is allocated in the call and
    # stale values would show
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    torch.cuda.synchronize()
    sinkattn_decode_noalloc(*args, out=o_na, lse=l_na)
    torch.cuda.synchronize()
    return o_ws.cpu(), l_ws.cpu(), o_na.cpu(), l_na.cpu()


def _check(inp, label, scaled):
    o_ws, l_ws, o_na, l_na = _call_both(inp)
    assert torch.equal(o_ws, o_na), f"{label}: o differs from sinkattn_decode"
    assert torch.equal(l_ws, l_na), f"{label}: lse differs from sinkattn_decode"
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    ro, rl = oracle.decode(f64(inp.q), f64(inp.k_cache), f64(inp.v_cache),
                           inp.cache_seqlens.tolist(), f64(inp.sinks), inp.window, inp.prefix,
                           inp.scale)
    e_o = float(np.abs(f64(o_na) - ro).max())
    fin = np.isfinite(rl)
    e_l = float(np.abs(f64(l_na)[fin] - rl[fin]).max()) if fin.any() else 0.0
    assert np.all(np.isneginf(f64(l_na)[~fin]))
    tol_o = max(TOL["bf16"]["o"], float(np.abs(ro).max()) / 64) if scaled else TOL["bf16"]["o"]
    log(f"{label}: bitwise equal to sinkattn_decode; vs oracle max|dO| {e_o:.3g}, "
        f"max|dl| {e_l:.3g}")
    assert e_o <= tol_o and e_l <= DECODE_LSE_TOL, label


def test_decode_noalloc_two_calls_second_smaller():
    # first: the rollout-decode workload's full-causal layer (32 caches of up to 8192
    # tokens, stream kernel and combine, the largest use of the scratch here)
    big = decode_workload_inputs("decode_grpo_32")[1]
    assert big.window == WINDOW_INF
    _check(big, "decode_grpo_32 causal layer", scaled=False)
    # second, smaller: 5 caches, one empty, short lengths (fewer blocks; partials of the
    # first call left in the scratch must not leak into this one)
    small = make_decode_inputs(lengths=(700, 0, 1500, 65, 1), capacity=1500, heads_q=16,
                               heads_kv=2, head_dim=64, window=WINDOW_INF, prefix=0, seed=91,
                               std=1.0)
    _check(small, "5 short caches", scaled=True)


def test_decode_noalloc_single_pass_and_window():
    # short windows take the single-pass kernel (no scratch); same entry point
    inp = decode_workload_inputs("decode_grpo_32")[0]
    assert inp.window == 128
    _check(inp, "decode_grpo_32 window layer", scaled=False)


def test_decode_noalloc_empty_batch_and_errors():
    dev = torch.device("cuda:0")
    q = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((0, 16, 1, 64), dtype=torch.bfloat16, device=dev)
    lens = torch.zeros((0,), dtype=torch.int32, device=dev)
    s = torch.zeros(8, dtype=torch.float32, device=dev)
    o, lse = sinkattn_decode_noalloc(q, kc, kc, lens, s, 16, 0)
    assert o.shape == (0, 8, 64)
    with pytest.raises(SinkAttnError):
        sinkattn_decode_noalloc(q, kc, kc, lens, s, -1, 0)   # invalid window
