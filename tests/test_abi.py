"""C-ABI checks that need no GPU: the library loads, exports every function
that include/sinkattn.h declares, and rejects invalid calls on the host
(before any HIP call) with the documented status codes."""
import ctypes
import os
import re

import pytest

from sink_aware_masked_sinkattn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")

# fake device addresses: never dereferenced, validation fails before any HIP call
A = 0x7F0000000000


def _lib():
    return binding.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sinkattn_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _lib()
    names = _declared_functions()
    assert set(names) >= {"sinkattn_fwd", "sinkattn_bwd", "sinkattn_bwd_workspace_size",
                          "sinkattn_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = _lib()
    for code in range(9):
        s = lib.sinkattn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.sinkattn_status_string(99).decode() == "unknown status"


def _problem(**kw):
    pb = binding.Problem()
    pb.dtype = kw.get("dtype", binding.SINKATTN_BF16)
    pb.batch = kw.get("batch", 1)
    pb.seqlen = kw.get("seqlen", 256)
    pb.total_tokens = kw.get("total_tokens", 256)
    pb.heads_q = kw.get("heads_q", 8)
    pb.heads_kv = kw.get("heads_kv", 2)
    pb.head_dim = kw.get("head_dim", 64)
    pb.window = kw.get("window", 128)
    pb.prefix = kw.get("prefix", 4)
    pb.softmax_scale = kw.get("softmax_scale", 0.125)
    pb.cu_seqlens = kw.get("cu_seqlens", None)
    return pb


def _fwd(pb, q=A, k=A, v=A, s=A, o=A, lse=A):
    return _lib().sinkattn_fwd(ctypes.byref(pb), q, k, v, s, o, lse, None)


def _bwd(pb, ws=A, ws_bytes=1 << 40, **ptrs):
    p = {n: ptrs.get(n, A) for n in ("q", "k", "v", "s", "o", "lse", "do", "dq", "dk", "dv", "ds")}
    return _lib().sinkattn_bwd(ctypes.byref(pb), p["q"], p["k"], p["v"], p["s"], p["o"],
                               p["lse"], p["do"], p["dq"], p["dk"], p["dv"], p["ds"], ws,
                               ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(heads_q=6, heads_kv=4), 2),
    (dict(heads_kv=0), 2),
    (dict(batch=-1), 2),
    (dict(seqlen=-5), 2),
    (dict(softmax_scale=0.0), 2),
    (dict(softmax_scale=float("nan")), 2),
    (dict(window=-1), 3),
    (dict(prefix=-2), 3),
    (dict(head_dim=128), 4),
    (dict(dtype=7), 4),
    (dict(dtype=binding.SINKATTN_FP32, head_dim=48), 4),
    (dict(heads_q=(1 << 18) + 16, heads_kv=16), 2),   # Hq * d > 2^24
])
def test_invalid_problem_rejected(kw, code):
    pb = _problem(**kw)
    assert _fwd(pb) == code
    assert _bwd(pb) == code
    assert _lib().sinkattn_bwd_workspace_size(ctypes.byref(pb)) == 0


def test_null_and_misaligned_pointers():
    pb = _problem()
    assert _lib().sinkattn_fwd(None, A, A, A, A, A, A, None) == 1
    for name in ("q", "k", "v", "s", "o"):
        assert _fwd(pb, **{name: None}) == 1, name
        assert _fwd(pb, **{name: A + 2}) == 5, name
    assert _fwd(pb, lse=A + 4) == 5
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert _bwd(pb, **{name: None}) == 1, name
        assert _bwd(pb, **{name: A + 8}) == 5, name
    assert _bwd(pb, ds=None) == 1
    assert _bwd(pb, s=None) == 1


def test_workspace_checks():
    pb = _problem()
    need = _lib().sinkattn_bwd_workspace_size(ctypes.byref(pb))
    rows, hq, hkv, d = 256, 8, 2, 64
    # D and L stats, fp32 dK and dV accumulators
    assert need >= 4 * (2 * rows * hq + 2 * rows * hkv * d)
    assert _bwd(pb, ws=None) == 6
    assert _bwd(pb, ws_bytes=need - 1) == 6
    assert _bwd(pb, ws=A + 16, ws_bytes=need) == 5          # workspace must be 256-B aligned
    f32 = _problem(dtype=binding.SINKATTN_FP32, head_dim=32)
    need32 = _lib().sinkattn_bwd_workspace_size(ctypes.byref(f32))
    assert need32 >= 4 * 2 * rows * hq
    pb_var = _problem(cu_seqlens=A, batch=3, total_tokens=1000, seqlen=600)
    need_var = _lib().sinkattn_bwd_workspace_size(ctypes.byref(pb_var))
    assert need_var >= 4 * (2 * 1000 * hq + 2 * 1000 * hkv * d)
    bad_var = _problem(cu_seqlens=A, batch=3, total_tokens=-1)
    assert _fwd(bad_var) == 2


def test_empty_forward_is_a_no_op():
    # zero rows: valid, returns OK without touching the device
    assert _fwd(_problem(batch=0)) == 0
    assert _fwd(_problem(seqlen=0)) == 0
    assert _fwd(_problem(batch=0), q=None, k=None, v=None, s=None, o=None, lse=None) == 0


def test_bwd_phase_mask_validated():
    pb = _problem()
    lib = _lib()
    args = (ctypes.byref(pb),) + (A,) * 11 + (A, 1 << 40, None)
    assert lib.sinkattn_bwd_phases(0, *args) == 2
    assert lib.sinkattn_bwd_phases(16, *args) == 2
    assert lib.sinkattn_bwd_phases(1 | 32, *args) == 2
    # a valid mask still runs the same host checks first (window < 0 here)
    bad = _problem(window=-1)
    assert lib.sinkattn_bwd_phases(15, ctypes.byref(bad), *args[1:]) == 3


def test_tile_config():
    # short windows: 32-key forward / dQ tiles; dK/dV always 128-row tiles; the
    # window is clamped to the sequence length first (w >= T is plain causal)
    assert binding.sinkattn_tile_config(_problem(window=128, seqlen=8192)) == (32, 128)
    assert binding.sinkattn_tile_config(_problem(window=1023, seqlen=8192)) == (32, 128)
    assert binding.sinkattn_tile_config(_problem(window=1024, seqlen=8192)) == (64, 128)
    assert binding.sinkattn_tile_config(_problem(window=2**31 - 1, seqlen=8192)) == (64, 128)
    assert binding.sinkattn_tile_config(_problem(window=2**31 - 1, seqlen=300)) == (32, 128)
    with pytest.raises(binding.SinkAttnError):
        binding.sinkattn_tile_config(_problem(window=-1))
    assert _lib().sinkattn_tile_config(ctypes.byref(_problem()), None) == 1


def _dproblem(**kw):
    pb = binding.DecodeProblem()
    pb.batch = kw.get("batch", 4)
    pb.cache_capacity = kw.get("cache_capacity", 1024)
    pb.heads_q = kw.get("heads_q", 8)
    pb.heads_kv = kw.get("heads_kv", 1)
    pb.head_dim = kw.get("head_dim", 64)
    pb.window = kw.get("window", 128)
    pb.prefix = kw.get("prefix", 4)
    pb.softmax_scale = kw.get("softmax_scale", 0.125)
    return pb


def _decode(pb, ws=A, ws_bytes=1 << 40, **ptrs):
    p = {n: ptrs.get(n, A) for n in ("q", "k", "v", "lens", "s", "o", "lse")}
    return _lib().sinkattn_decode(ctypes.byref(pb), p["q"], p["k"], p["v"], p["lens"], p["s"],
                                  p["o"], p["lse"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(heads_q=6, heads_kv=4), 2),
    (dict(batch=-1), 2),
    (dict(cache_capacity=-1), 2),
    (dict(softmax_scale=0.0), 2),
    (dict(window=-1), 3),
    (dict(prefix=-1), 3),
    (dict(head_dim=128), 4),
    (dict(heads_q=32, heads_kv=1), 4),     # more than 16 query heads per kv head
    (dict(heads_q=(1 << 18) + 16, heads_kv=(1 << 14) + 1), 2),   # Hq * d > 2^24
])
def test_decode_invalid_problem_rejected(kw, code):
    pb = _dproblem(**kw)
    assert _decode(pb) == code
    assert _lib().sinkattn_decode_workspace_size(ctypes.byref(pb)) == 0


def test_decode_pointer_and_workspace_checks():
    pb = _dproblem()
    need = _lib().sinkattn_decode_workspace_size(ctypes.byref(pb))
    assert need > 0 and need % 256 == 0
    assert _lib().sinkattn_decode(None, A, A, A, A, A, A, A, A, need, None) == 1
    for name in ("q", "k", "v", "lens", "s", "o"):
        assert _decode(pb, **{name: None}) == 1, name
    for name in ("q", "k", "v", "s", "o", "lse"):
        assert _decode(pb, **{name: A + 8}) == 5, name
    assert _decode(pb, lens=A + 2) == 5
    assert _decode(pb, ws=None) == 6
    assert _decode(pb, ws_bytes=1) == 6
    assert _decode(pb, ws=A + 64, ws_bytes=need) == 5
    # no sequences: nothing to do, no pointer is touched
    assert _decode(_dproblem(batch=0), q=None, k=None, v=None, lens=None, s=None, o=None,
                   lse=None, ws=None, ws_bytes=0) == 0
    # the workspace grows with the batch and the cache length
    big = _lib().sinkattn_decode_workspace_size(ctypes.byref(_dproblem(batch=8, cache_capacity=8192,
                                                                      window=2**31 - 1, prefix=0)))
    assert big >= need


def _decode_noalloc(pb, **ptrs):
    p = {n: ptrs.get(n, A) for n in ("q", "k", "v", "lens", "s", "o", "lse")}
    return _lib().sinkattn_decode_noalloc(ctypes.byref(pb), p["q"], p["k"], p["v"], p["lens"],
                                          p["s"], p["o"], p["lse"], None)


def test_decode_noalloc_checks_before_any_device_work():
    # every status below is returned by host checks alone (no GPU here)
    lib = _lib()
    assert lib.sinkattn_decode_noalloc(None, A, A, A, A, A, A, A, None) == 1
    assert _decode_noalloc(_dproblem(batch=-1)) == 2
    assert _decode_noalloc(_dproblem(window=-1)) == 3
    assert _decode_noalloc(_dproblem(heads_q=32, heads_kv=1)) == 4
    for name in ("q", "k", "v", "lens", "s", "o"):
        assert _decode_noalloc(_dproblem(), **{name: None}) == 1, name
    for name in ("q", "k", "v", "s", "o", "lse"):
        assert _decode_noalloc(_dproblem(), **{name: A + 8}) == 5, name
    assert _decode_noalloc(_dproblem(batch=0), q=None, k=None, v=None, lens=None, s=None, o=None,
                           lse=None) == 0
    assert "static scratch" in lib.sinkattn_status_string(8).decode()
    # the static scratch covers every decode problem: the largest workspaces
    # (stream kernel, batch * heads_kv just under 1024, 16 heads per kv head,
    # long caches) stay within it
    limit = binding.SINKATTN_DECODE_SCRATCH_BYTES
    worst = 0
    for hkv in (1, 2, 8, 64, 1023):
        for batch in sorted({1, 7, max(1, 1023 // hkv), max(1, 1024 // hkv), 1024, 1025}):
            for group in (1, 8, 16):
                for cap, w, p in ((8192, 2**31 - 1, 0), (1 << 20, 2**31 - 1, 0),
                                  (65536, 128, 16), (300, 2**31 - 1, 0)):
                    pb = _dproblem(batch=batch, cache_capacity=cap, heads_q=hkv * group,
                                   heads_kv=hkv, window=w, prefix=p)
                    need = lib.sinkattn_decode_workspace_size(ctypes.byref(pb))
                    worst = max(worst, need)
                    assert 0 < need <= limit, (batch, hkv, group, cap, w, p)
    assert worst == 22282240


def test_header_states_the_scratch_size():
    src = open(HEADER).read()
    m = re.search(r"#define SINKATTN_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.SINKATTN_DECODE_SCRATCH_BYTES


def _gproblem(**kw):
    d = dict(num_rollouts=16, group_size=8, total_tokens=1000, kl_mode=0, eps_adv=1e-6,
             eps_clip=0.2, beta=0.04)
    d.update(kw)
    return binding.make_grpo_problem(d["num_rollouts"], d["group_size"], d["total_tokens"],
                                     d["eps_adv"], d["eps_clip"], d["beta"], d["kl_mode"])


def _grpo(pb, ws=A, ws_bytes=1 << 40, **ptrs):
    p = {n: ptrs.get(n, A) for n in ("new", "old", "ref", "mask", "rew", "cu", "loss", "grad",
                                      "adv")}
    return _lib().sinkattn_grpo_loss(ctypes.byref(pb), p["new"], p["old"], p["ref"], p["mask"],
                                     p["rew"], p["cu"], p["loss"], p["grad"], p["adv"], ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(num_rollouts=-8), dict(total_tokens=-1), dict(group_size=0), dict(group_size=1025,
                                                                           num_rollouts=1025),
    dict(num_rollouts=12),                      # not a multiple of the group size
    dict(num_rollouts=0, total_tokens=5),       # tokens without rollouts
    dict(kl_mode=2), dict(eps_adv=-1.0), dict(eps_adv=float("nan")), dict(eps_clip=1.0),
    dict(eps_clip=-0.1), dict(beta=float("inf")),
])
def test_grpo_invalid_problem_rejected(kw):
    pb = _gproblem(**kw)
    assert _grpo(pb) == 2
    assert _lib().sinkattn_grpo_workspace_size(ctypes.byref(pb)) == 0


def test_grpo_pointer_and_workspace_checks():
    pb = _gproblem()
    need = _lib().sinkattn_grpo_workspace_size(ctypes.byref(pb))
    assert need > 0 and need % 256 == 0
    assert _lib().sinkattn_grpo_loss(None, A, A, A, A, A, A, A, A, A, A, need, None) == 1
    for name in ("new", "old", "rew", "cu", "loss", "grad", "ref"):
        assert _grpo(pb, **{name: None}) == 1, name
    # no reference log-probs needed without a KL term
    pb0 = _gproblem(beta=0.0)
    assert _grpo(pb0, ref=None, ws=None) == 6
    for name in ("new", "old", "grad", "ref", "mask"):
        assert _grpo(pb, **{name: A + 4}) == 5, name
    for name in ("rew", "cu", "loss", "adv"):
        assert _grpo(pb, **{name: A + 2}) == 5, name
    assert _grpo(pb, ws=None) == 6
    assert _grpo(pb, ws_bytes=need - 1) == 6
    assert _grpo(pb, ws=A + 64, ws_bytes=need) == 5
    # the workspace grows with the rollouts and the tokens
    big = _lib().sinkattn_grpo_workspace_size(ctypes.byref(_gproblem(num_rollouts=4096,
                                                                     total_tokens=1 << 24)))
    assert big > need
