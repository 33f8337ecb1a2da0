"""Seeded synthetic inputs for sink-aware masked attention.

This module holds no attention arithmetic.  It only names the workloads and
draws their tensors, so that the fp64 oracle (``oracle/``) and the HIP path
(``sink_aware_masked_sinkattn_amd``) can be fed the very same values without
sharing any code of the method itself.

Recipe (the same for every workload):
  * one ``torch.Generator`` (CPU) per workload, seeded with ``1000 + index``;
  * draws in this order per layer: Q, K, V, dO (each ``std * N(0, 1)`` in fp32),
    then the per-head sink logits ``s_h ~ N(0, 1)`` (fp32);
  * for bf16 workloads Q, K, V and dO are rounded once to bf16 (round to
    nearest even, torch's ``.to(torch.bfloat16)``); sinks stay fp32;
  * varlen workloads draw their G sequence lengths first, uniform on the
    closed range [lo, hi], and pack the sequences back to back
    (``cu_seqlens`` is the exclusive prefix sum of the lengths).

Layouts: Q, O, dO ``[B, T, Hq, d]`` (varlen ``[N, Hq, d]``); K, V
``[B, T, Hkv, d]`` (varlen ``[N, Hkv, d]``); sinks ``[Hq]``.  The q-head ``h``
reads kv-head ``h // (Hq // Hkv)``.

The shapes follow the attention layers of the workloads described for the
SinkFlex-RL method (64 query heads, 8 kv heads, head dim 64, alternating
128-token sliding-window and full-causal layers, GRPO groups of rollouts of
1k-8k tokens).  The pages measure on tau^2-Bench retail trajectories with an
unnamed MoE model; neither is available, so these seeded draws stand in for
their attention inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

# Window value meaning "no window limit" (plain causal plus prefix).  The C
# ABI uses the same value (INT32_MAX).
WINDOW_INF = 2**31 - 1


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                      # seed = 1000 + index
    dtype: str                      # "bf16" or "fp32"
    batch: int                      # B (ignored for varlen)
    seqlen: int                     # T (max length for varlen)
    heads_q: int
    heads_kv: int
    head_dim: int
    std: float                      # Q, K, V, dO ~ std * N(0, 1)
    layers: Tuple[Tuple[int, int], ...]   # (window, prefix) per layer
    varlen: Optional[Tuple[int, int, int]] = None  # (G, lo, hi)

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 0, "fp32", 1, 128, 2, 2, 32, 1.0, ((16, 4),)),
        Workload("gqa_swa_4096", 1, "bf16", 1, 4096, 64, 8, 64, 0.5, ((128, 0),)),
        Workload("gqa_causal_4096", 2, "bf16", 1, 4096, 64, 8, 64, 0.5, ((WINDOW_INF, 0),)),
        Workload("long_8192", 3, "bf16", 1, 8192, 64, 8, 64, 0.5,
                 ((128, 4), (WINDOW_INF, 0))),
        Workload("varlen_grpo_g8", 4, "bf16", 1, 8192, 64, 8, 64, 0.5, ((128, 16),),
                 varlen=(8, 1024, 8192)),
    ]
}


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    sinks: torch.Tensor
    window: int
    prefix: int
    scale: float
    group: int
    cu_seqlens: Optional[torch.Tensor] = None   # int32 [G+1] or None
    lengths: Optional[Tuple[int, ...]] = None
    meta: dict = field(default_factory=dict)

    @property
    def max_seqlen(self) -> int:
        if self.lengths is not None:
            return max(self.lengths) if self.lengths else 0
        return self.q.shape[1]


def _storage(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]


def draw(gen: torch.Generator, shape, std: float, dtype: str) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32) * std
    return x.to(_storage(dtype))


def draw_lengths(gen: torch.Generator, count: int, lo: int, hi: int) -> Tuple[int, ...]:
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (count,), generator=gen))


def make_inputs(*, batch: int, seqlen: int, heads_q: int, heads_kv: int, head_dim: int,
                window: int, prefix: int, seed: int, std: float = 1.0,
                dtype: str = "bf16", lengths: Optional[Tuple[int, ...]] = None,
                sink_values: Optional[Tuple[float, ...]] = None,
                gen: Optional[torch.Generator] = None) -> Inputs:
    """Draw one attention call's inputs.

    ``lengths`` given means varlen packing (``batch``/``seqlen`` ignored).
    ``sink_values`` overrides the drawn sinks (edge cases such as -inf).
    """
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    if lengths is not None:
        n = int(sum(lengths))
        qs, ks = (n, heads_q, head_dim), (n, heads_kv, head_dim)
    else:
        qs = (batch, seqlen, heads_q, head_dim)
        ks = (batch, seqlen, heads_kv, head_dim)
    q = draw(gen, qs, std, dtype)
    k = draw(gen, ks, std, dtype)
    v = draw(gen, ks, std, dtype)
    do = draw(gen, qs, std, dtype)
    sinks = torch.randn(heads_q, generator=gen, dtype=torch.float32)
    if sink_values is not None:
        sinks = torch.tensor(sink_values, dtype=torch.float32)
        assert sinks.numel() == heads_q
    cu = None
    if lengths is not None:
        offs = [0]
        for L in lengths:
            offs.append(offs[-1] + int(L))
        cu = torch.tensor(offs, dtype=torch.int32)
    return Inputs(q=q, k=k, v=v, do=do, sinks=sinks, window=int(window),
                  prefix=int(prefix), scale=1.0 / math.sqrt(head_dim),
                  group=heads_q // heads_kv, cu_seqlens=cu,
                  lengths=tuple(int(x) for x in lengths) if lengths is not None else None,
                  meta={"seed": seed, "std": std, "dtype": dtype})


def workload_inputs(name: str) -> list:
    """All layers' inputs of a named workload, drawn from its own generator."""
    wl = WORKLOADS[name]
    gen = torch.Generator().manual_seed(wl.seed)
    lengths = None
    if wl.varlen is not None:
        g, lo, hi = wl.varlen
        lengths = draw_lengths(gen, g, lo, hi)
    out = []
    for (w, p) in wl.layers:
        out.append(make_inputs(batch=wl.batch, seqlen=wl.seqlen, heads_q=wl.heads_q,
                               heads_kv=wl.heads_kv, head_dim=wl.head_dim, window=w,
                               prefix=p, seed=wl.seed, std=wl.std, dtype=wl.dtype,
                               lengths=lengths, gen=gen))
        out[-1].meta["workload"] = name
    return out


# ------------------------------------------------------------------ decode
#
# Rollout decode: one new query token per sequence against a key/value cache
# of up to ``capacity`` rows.  Recipe: one generator seeded ``2000 + index``;
# the cache lengths first (uniform on [lo, hi]), then per layer q [B, Hq, d],
# the K and V caches [B, capacity, Hkv, d] (``std * N(0, 1)``, rounded once
# to bf16; rows past a sequence's length are drawn too and must not matter),
# then the sinks ``N(0, 1)`` (fp32).

@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    index: int                      # seed = 2000 + index
    batch: int                      # sequences (rollouts) decoded together
    capacity: int                   # cache rows per sequence
    lengths: Tuple[int, int]        # cached tokens per sequence ~ U[lo, hi]
    heads_q: int
    heads_kv: int
    head_dim: int
    std: float
    layers: Tuple[Tuple[int, int], ...]   # (window, prefix) per layer

    @property
    def seed(self) -> int:
        return 2000 + self.index


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        # four GRPO groups of 8 rollouts, 1k-8k tokens each, the layer pair of
        # the long-context training workload
        DecodeWorkload("decode_grpo_32", 0, 32, 8192, (1024, 8192), 64, 8, 64, 0.5,
                       ((128, 4), (WINDOW_INF, 0))),
    ]
}


@dataclass
class DecodeInputs:
    q: torch.Tensor                 # [B, Hq, d]
    k_cache: torch.Tensor           # [B, capacity, Hkv, d]
    v_cache: torch.Tensor
    cache_seqlens: torch.Tensor     # int32 [B]
    sinks: torch.Tensor             # [Hq] fp32
    window: int
    prefix: int
    scale: float
    meta: dict = field(default_factory=dict)


def make_decode_inputs(*, lengths: Tuple[int, ...], capacity: int, heads_q: int, heads_kv: int,
                       head_dim: int, window: int, prefix: int, seed: int, std: float = 1.0,
                       gen: Optional[torch.Generator] = None) -> DecodeInputs:
    """Draw one decode call's inputs (bf16 q and caches, fp32 sinks)."""
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    b = len(lengths)
    q = draw(gen, (b, heads_q, head_dim), std, "bf16")
    k = draw(gen, (b, capacity, heads_kv, head_dim), std, "bf16")
    v = draw(gen, (b, capacity, heads_kv, head_dim), std, "bf16")
    sinks = torch.randn(heads_q, generator=gen, dtype=torch.float32)
    return DecodeInputs(q=q, k_cache=k, v_cache=v,
                        cache_seqlens=torch.tensor(lengths, dtype=torch.int32), sinks=sinks,
                        window=int(window), prefix=int(prefix),
                        scale=1.0 / math.sqrt(head_dim),
                        meta={"seed": seed, "std": std})


def decode_workload_inputs(name: str) -> list:
    """All layers' inputs of a named decode workload, from its own generator."""
    wl = DECODE_WORKLOADS[name]
    gen = torch.Generator().manual_seed(wl.seed)
    lengths = draw_lengths(gen, wl.batch, *wl.lengths)
    out = []
    for (w, p) in wl.layers:
        out.append(make_decode_inputs(lengths=lengths, capacity=wl.capacity, heads_q=wl.heads_q,
                                      heads_kv=wl.heads_kv, head_dim=wl.head_dim, window=w,
                                      prefix=p, seed=wl.seed, std=wl.std, gen=gen))
        out[-1].meta["workload"] = name
    return out


# ---------------------------------------------------------------------------
# GRPO token loss: packed per-token log-probs of a batch of rollout groups.
# Rollouts alternate environment-observation spans (action mask 0: tool
# outputs, user turns) with agent spans (mask 1: tokens the policy produced),
# as in the multi-turn, tool-heavy trajectories the pages describe; rewards are
# programmatic 0/1 outcomes.  Log-probs: old ~ -Exp(1) per token, the current
# and the reference policy drift from it by small Gaussian log-ratios.
@dataclass(frozen=True)
class GrpoWorkload:
    name: str
    index: int                      # seed = 3000 + index
    groups: int                     # prompts
    group_size: int                 # rollouts per prompt (G)
    lengths: Tuple[int, int]        # tokens per rollout ~ U[lo, hi]
    agent_span: Tuple[int, int]     # optimised span lengths ~ U[lo, hi]
    obs_span: Tuple[int, int]       # observation span lengths ~ U[lo, hi]
    new_drift: float                # std of logp_new - logp_old
    ref_drift: float                # std of logp_ref - logp_old
    reward_p: float                 # P(R = 1)
    eps_adv: float
    eps_clip: float
    beta: float
    kl_mode: int

    @property
    def seed(self) -> int:
        return 3000 + self.index


GRPO_WORKLOADS = {
    w.name: w
    for w in [
        # 64 prompts x 8 rollouts of 1k-8k tokens (about 2.4M packed tokens)
        GrpoWorkload("grpo_64x8", 0, 64, 8, (1024, 8192), (16, 256), (32, 512), 0.1, 0.1, 0.4,
                     1e-6, 0.2, 0.04, 0),
    ]
}


@dataclass
class GrpoInputs:
    logp_new: torch.Tensor          # [N] fp32
    logp_old: torch.Tensor          # [N] fp32
    logp_ref: torch.Tensor          # [N] fp32
    action_mask: torch.Tensor       # [N] uint8 (1 = optimised token)
    rewards: torch.Tensor           # [B] fp32
    cu_seqlens: torch.Tensor        # [B + 1] int32
    group_size: int
    eps_adv: float
    eps_clip: float
    beta: float
    kl_mode: int
    meta: dict = field(default_factory=dict)


def make_grpo_inputs(*, lengths: Tuple[int, ...], group_size: int, seed: int,
                     agent_span: Tuple[int, int] = (16, 256), obs_span: Tuple[int, int] = (32, 512),
                     new_drift: float = 0.1, ref_drift: float = 0.1, reward_p: float = 0.4,
                     eps_adv: float = 1e-6, eps_clip: float = 0.2, beta: float = 0.04,
                     kl_mode: int = 0) -> GrpoInputs:
    """Draw one batch of packed rollouts (rollout i has lengths[i] tokens)."""
    gen = torch.Generator().manual_seed(seed)
    n = int(sum(lengths))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    old = -torch.empty(n, dtype=torch.float32).exponential_(1.0, generator=gen)
    new = old + new_drift * torch.randn(n, generator=gen, dtype=torch.float32)
    ref = old + ref_drift * torch.randn(n, generator=gen, dtype=torch.float32)
    mask = torch.zeros(n, dtype=torch.uint8)
    for i, length in enumerate(lengths):
        pos, agent = int(cu[i]), False          # a rollout opens with an observation
        end = pos + int(length)
        while pos < end:
            lo, hi = agent_span if agent else obs_span
            span = int(torch.randint(lo, hi + 1, (1,), generator=gen))
            if agent:
                mask[pos:min(end, pos + span)] = 1
            pos += span
            agent = not agent
    rewards = (torch.rand(len(lengths), generator=gen) < reward_p).to(torch.float32)
    return GrpoInputs(logp_new=new, logp_old=old, logp_ref=ref, action_mask=mask,
                      rewards=rewards, cu_seqlens=cu, group_size=int(group_size),
                      eps_adv=eps_adv, eps_clip=eps_clip, beta=beta, kl_mode=kl_mode,
                      meta={"seed": seed})


def grpo_workload_inputs(name: str) -> GrpoInputs:
    w = GRPO_WORKLOADS[name]
    gen = torch.Generator().manual_seed(w.seed)
    lengths = draw_lengths(gen, w.groups * w.group_size, *w.lengths)
    return make_grpo_inputs(lengths=lengths, group_size=w.group_size, seed=w.seed + 1,
                            agent_span=w.agent_span, obs_span=w.obs_span, new_drift=w.new_drift,
                            ref_drift=w.ref_drift, reward_p=w.reward_p, eps_adv=w.eps_adv,
                            eps_clip=w.eps_clip, beta=w.beta, kl_mode=w.kl_mode)
