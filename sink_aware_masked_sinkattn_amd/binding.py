"""ctypes binding of libsinkattn.so (C ABI in include/sinkattn.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is not built, or a tensor
is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsinkattn.so")

WINDOW_INF = 2**31 - 1          # SINKATTN_WINDOW_INF
# size of the library's static per-GPU scratch (sinkattn_decode_noalloc)
SINKATTN_DECODE_SCRATCH_BYTES = 24 << 20

SINKATTN_BF16 = 0
SINKATTN_FP32 = 1

# backward phase flags (sinkattn_bwd_phases)
BWD_PREPARE = 1
BWD_DQ = 2
BWD_DKDV = 4
BWD_FINISH = 8
BWD_ALL = 15

STATUS = {
    0: "SINKATTN_OK",
    1: "SINKATTN_ERR_NULL_POINTER",
    2: "SINKATTN_ERR_BAD_SHAPE",
    3: "SINKATTN_ERR_BAD_MASK",
    4: "SINKATTN_ERR_UNSUPPORTED",
    5: "SINKATTN_ERR_MISALIGNED",
    6: "SINKATTN_ERR_WORKSPACE",
    7: "SINKATTN_ERR_HIP",
}


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        msg = STATUS.get(status, f"status {status}")
        if lib is not None:
            msg += ": " + lib.sinkattn_status_string(status).decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("prefix", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("cu_seqlens", ctypes.c_void_p),
    ]


class DecodeProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("prefix", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class GrpoProblem(ctypes.Structure):
    _fields_ = [
        ("num_rollouts", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("kl_mode", ctypes.c_int32),
        ("eps_adv", ctypes.c_float),
        ("eps_clip", ctypes.c_float),
        ("beta", ctypes.c_float),
    ]


_LIB = None


def load_library(path: str = LIB_PATH):
    """Load (once) and type the shared library.  Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -m sink_aware_masked_sinkattn_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    pp = ctypes.POINTER(Problem)
    lib.sinkattn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
    lib.sinkattn_fwd.restype = ctypes.c_int
    lib.sinkattn_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sinkattn_bwd.restype = ctypes.c_int
    lib.sinkattn_bwd_phases.argtypes = [ctypes.c_uint32, pp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, sz, vp]
    lib.sinkattn_bwd_phases.restype = ctypes.c_int
    lib.sinkattn_bwd_workspace_size.argtypes = [pp]
    lib.sinkattn_bwd_workspace_size.restype = sz
    lib.sinkattn_status_string.argtypes = [ctypes.c_int]
    lib.sinkattn_status_string.restype = ctypes.c_char_p
    lib.sinkattn_tile_class.argtypes = [i32] * 6
    lib.sinkattn_tile_class.restype = i32
    lib.sinkattn_key_tile_segments.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32)]
    lib.sinkattn_key_tile_segments.restype = i32
    lib.sinkattn_tile_config.argtypes = [pp, ctypes.POINTER(i32)]
    lib.sinkattn_tile_config.restype = ctypes.c_int
    dp = ctypes.POINTER(DecodeProblem)
    lib.sinkattn_decode_workspace_size.argtypes = [dp]
    lib.sinkattn_decode_workspace_size.restype = sz
    lib.sinkattn_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sinkattn_decode.restype = ctypes.c_int
    lib.sinkattn_decode_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sinkattn_decode_noalloc.restype = ctypes.c_int
    gp = ctypes.POINTER(GrpoProblem)
    lib.sinkattn_grpo_workspace_size.argtypes = [gp]
    lib.sinkattn_grpo_workspace_size.restype = sz
    lib.sinkattn_grpo_loss.argtypes = [gp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sinkattn_grpo_loss.restype = ctypes.c_int
    _LIB = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def make_problem(q: torch.Tensor, k: torch.Tensor, window: int, prefix: int,
                 softmax_scale: Optional[float] = None,
                 cu_seqlens: Optional[torch.Tensor] = None,
                 max_seqlen: Optional[int] = None) -> Problem:
    """Problem descriptor from tensor shapes (see include/sinkattn.h)."""
    dtype = {torch.bfloat16: SINKATTN_BF16, torch.float32: SINKATTN_FP32}.get(q.dtype)
    if dtype is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    pb = Problem()
    pb.dtype = dtype
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("q must be [B, T, Hq, d] (or [N, Hq, d] with cu_seqlens)")
        pb.batch, pb.seqlen, pb.heads_q, pb.head_dim = q.shape
        pb.total_tokens = q.shape[0] * q.shape[1]
        pb.heads_kv = k.shape[2]
        pb.cu_seqlens = None
    else:
        if q.dim() != 3:
            raise ValueError("varlen q must be [N, Hq, d]")
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        _dev(cu_seqlens, "cu_seqlens")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        pb.batch = cu_seqlens.numel() - 1
        pb.seqlen = int(max_seqlen)
        pb.total_tokens, pb.heads_q, pb.head_dim = q.shape
        pb.heads_kv = k.shape[1]
        pb.cu_seqlens = cu_seqlens.data_ptr()
    pb.window = int(min(window, WINDOW_INF))
    pb.prefix = int(prefix)
    pb.softmax_scale = float(softmax_scale if softmax_scale is not None
                             else 1.0 / math.sqrt(q.shape[-1]))
    return pb


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def sinkattn_bwd_workspace_size(pb: Problem) -> int:
    return int(load_library().sinkattn_bwd_workspace_size(ctypes.byref(pb)))


def sinkattn_fwd(q, k, v, sinks, window: int, prefix: int, softmax_scale=None,
                 cu_seqlens=None, max_seqlen=None, out=None, lse=None,
                 want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward: returns (o, lse).  lse is [B, Hq, T] (or [Hq, N]) fp32."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (sinks, "sinks")):
        _dev(t, n)
    pb = make_problem(q, k, window, prefix, softmax_scale, cu_seqlens, max_seqlen)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        shape = (pb.heads_q, pb.total_tokens) if cu_seqlens is not None else \
            (pb.batch, pb.heads_q, pb.seqlen)
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    st = lib.sinkattn_fwd(ctypes.byref(pb), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out),
                          _ptr(lse), _stream())
    if st != 0:
        raise SinkAttnError(st, "sinkattn_fwd", lib)
    return out, lse


def _bwd_call(phases: Optional[int], q, k, v, sinks, o, lse, dout, window, prefix,
              softmax_scale, cu_seqlens, max_seqlen, workspace, grads):
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (sinks, "sinks"), (o, "o"), (lse, "lse"),
                 (dout, "dout")):
        _dev(t, n)
    pb = make_problem(q, k, window, prefix, softmax_scale, cu_seqlens, max_seqlen)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsinks = torch.empty_like(sinks)
    else:
        dq, dk, dv, dsinks = grads
    need = int(lib.sinkattn_bwd_workspace_size(ctypes.byref(pb)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(pb), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o), _ptr(lse),
            _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), _ptr(workspace),
            workspace.numel(), _stream())
    if phases is None:
        st, entry = lib.sinkattn_bwd(*args), "sinkattn_bwd"
    else:
        st, entry = lib.sinkattn_bwd_phases(phases, *args), "sinkattn_bwd_phases"
    if st != 0:
        raise SinkAttnError(st, entry, lib)
    return dq, dk, dv, dsinks


def sinkattn_bwd(q, k, v, sinks, o, lse, dout, window: int, prefix: int, softmax_scale=None,
                 cu_seqlens=None, max_seqlen=None, workspace=None, grads=None):
    """Backward: returns (dq, dk, dv, dsinks).  ``workspace`` (uint8 GPU
    tensor) is allocated here when not given; ``grads`` may pass preallocated
    (dq, dk, dv, dsinks)."""
    return _bwd_call(None, q, k, v, sinks, o, lse, dout, window, prefix, softmax_scale,
                     cu_seqlens, max_seqlen, workspace, grads)


def sinkattn_bwd_phases(phases: int, q, k, v, sinks, o, lse, dout, window, prefix,
                        softmax_scale=None, cu_seqlens=None, max_seqlen=None, *, workspace,
                        grads):
    """Run some phases of the backward (OR of BWD_PREPARE, BWD_DQ, BWD_DKDV,
    BWD_FINISH, run in that order); the workspace and grads must be the same across the calls
    that make up one backward."""
    return _bwd_call(int(phases), q, k, v, sinks, o, lse, dout, window, prefix, softmax_scale,
                     cu_seqlens, max_seqlen, workspace, grads)


def sinkattn_tile_class(q0: int, q1: int, k0: int, k1: int, window: int, prefix: int) -> int:
    return int(load_library().sinkattn_tile_class(q0, q1, k0, k1, min(window, WINDOW_INF), prefix))


def sinkattn_key_tile_segments(q0: int, q1: int, window: int, prefix: int, block_k: int):
    out = (ctypes.c_int32 * 4)()
    n = load_library().sinkattn_key_tile_segments(q0, q1, min(window, WINDOW_INF), prefix,
                                                  block_k, out)
    if n < 0:
        raise ValueError("invalid arguments")
    return [(out[2 * i], out[2 * i + 1]) for i in range(n)]


def sinkattn_tile_config(pb: Problem):
    """(forward / dQ key-tile width, dK/dV query-tile height) the bf16
    kernels use for this problem; host only."""
    lib = load_library()
    out = (ctypes.c_int32 * 2)()
    st = lib.sinkattn_tile_config(ctypes.byref(pb), out)
    if st != 0:
        raise SinkAttnError(st, "sinkattn_tile_config", lib)
    return int(out[0]), int(out[1])


def make_decode_problem(q: torch.Tensor, k_cache: torch.Tensor, window: int, prefix: int,
                        softmax_scale: Optional[float] = None) -> DecodeProblem:
    """Decode problem from q [B, Hq, d] and k_cache [B, Tmax, Hkv, d]."""
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q and caches")
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, Tmax, Hkv, d]")
    pb = DecodeProblem()
    pb.batch, pb.heads_q, pb.head_dim = q.shape
    pb.cache_capacity = k_cache.shape[1]
    pb.heads_kv = k_cache.shape[2]
    pb.window = int(min(window, WINDOW_INF))
    pb.prefix = int(prefix)
    pb.softmax_scale = float(softmax_scale if softmax_scale is not None
                             else 1.0 / math.sqrt(q.shape[-1]))
    return pb


def sinkattn_decode_workspace_size(pb: DecodeProblem) -> int:
    return int(load_library().sinkattn_decode_workspace_size(ctypes.byref(pb)))


def sinkattn_decode(q, k_cache, v_cache, cache_seqlens, sinks, window: int, prefix: int,
                    softmax_scale=None, out=None, lse=None, want_lse: bool = True,
                    workspace=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode one query token per sequence against its cache: returns (o, lse),
    o [B, Hq, d] bf16, lse [B, Hq] fp32 (content-only log-sum-exp)."""
    lib = load_library()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (cache_seqlens, "cache_seqlens"), (sinks, "sinks")):
        _dev(t, n)
    if cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32")
    pb = make_decode_problem(q, k_cache, window, prefix, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((pb.batch, pb.heads_q), dtype=torch.float32, device=q.device)
    need = sinkattn_decode_workspace_size(pb)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.sinkattn_decode(ctypes.byref(pb), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                             _ptr(cache_seqlens), _ptr(sinks), _ptr(out), _ptr(lse),
                             _ptr(workspace), workspace.numel(), _stream())
    if st != 0:
        raise SinkAttnError(st, "sinkattn_decode", lib)
    return out, lse


def sinkattn_decode_noalloc(q, k_cache, v_cache, cache_seqlens, sinks, window: int, prefix: int,
                            softmax_scale=None, out=None, lse=None,
                            want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """sinkattn_decode through the allocation-free entry point: the library keeps the
    partials in its static per-GPU scratch.  Pass ``out`` (and ``lse``) to allocate
    nothing here either."""
    lib = load_library()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (cache_seqlens, "cache_seqlens"), (sinks, "sinks")):
        _dev(t, n)
    if cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32")
    pb = make_decode_problem(q, k_cache, window, prefix, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((pb.batch, pb.heads_q), dtype=torch.float32, device=q.device)
    st = lib.sinkattn_decode_noalloc(ctypes.byref(pb), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(cache_seqlens), _ptr(sinks), _ptr(out), _ptr(lse),
                                     _stream())
    if st != 0:
        raise SinkAttnError(st, "sinkattn_decode_noalloc", lib)
    return out, lse


def make_grpo_problem(num_rollouts: int, group_size: int, total_tokens: int, eps_adv: float,
                      eps_clip: float, beta: float, kl_mode: int = 0) -> GrpoProblem:
    pb = GrpoProblem()
    pb.num_rollouts, pb.group_size, pb.total_tokens = int(num_rollouts), int(group_size), \
        int(total_tokens)
    pb.kl_mode = int(kl_mode)
    pb.eps_adv, pb.eps_clip, pb.beta = float(eps_adv), float(eps_clip), float(beta)
    return pb


def sinkattn_grpo_workspace_size(pb: GrpoProblem) -> int:
    return int(load_library().sinkattn_grpo_workspace_size(ctypes.byref(pb)))


def sinkattn_grpo_loss(logp_new, logp_old, logp_ref, action_mask, rewards, cu_seqlens,
                       group_size: int, eps_adv: float, eps_clip: float, beta: float,
                       kl_mode: int = 0, loss=None, grad=None, advantages=None, workspace=None,
                       want_advantages: bool = True):
    """GRPO token loss (eq. 3-7 of arXiv 2608.10357 section 4): returns (loss [1], grad [N],
    advantages [B] or None), all fp32 GPU tensors.  logp_ref may be None when beta == 0,
    action_mask (uint8) None for every token optimised."""
    lib = load_library()
    for t, n in ((logp_new, "logp_new"), (logp_old, "logp_old"), (rewards, "rewards"),
                 (cu_seqlens, "cu_seqlens")):
        _dev(t, n)
    if logp_ref is not None:
        _dev(logp_ref, "logp_ref")
    if action_mask is not None:
        _dev(action_mask, "action_mask")
        if action_mask.dtype != torch.uint8:
            raise ValueError("action_mask must be uint8")
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    for t, n in ((logp_new, "logp_new"), (logp_old, "logp_old"), (rewards, "rewards")):
        if t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    pb = make_grpo_problem(cu_seqlens.numel() - 1, group_size, logp_new.numel(), eps_adv,
                           eps_clip, beta, kl_mode)
    dev = logp_new.device
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
    if grad is None:
        grad = torch.empty_like(logp_new)
    if advantages is None and want_advantages:
        advantages = torch.empty(pb.num_rollouts, dtype=torch.float32, device=dev)
    need = int(lib.sinkattn_grpo_workspace_size(ctypes.byref(pb)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.sinkattn_grpo_loss(ctypes.byref(pb), _ptr(logp_new), _ptr(logp_old), _ptr(logp_ref),
                                _ptr(action_mask), _ptr(rewards), _ptr(cu_seqlens), _ptr(loss),
                                _ptr(grad), _ptr(advantages), _ptr(workspace), workspace.numel(),
                                _stream())
    if st != 0:
        raise SinkAttnError(st, "sinkattn_grpo_loss", lib)
    return loss, grad, advantages
