"""Plain fp64 CPU oracle for the GRPO token loss and group-normalised advantage.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP library.

Source: arXiv 2608.10357, "Efficient Reinforcement Learning for Long-Horizon
Tool-Use Agentic Tasks" (translated page), section 4 "Training pipeline",
paragraph "Policy update", eq. 3-7; the summary page's GRPO paragraph states
eq. 3 too.  For a prompt and its group of G rollouts sampled from the old
policy:

  eq. 3   A_i     = (R_i - mean(R_1..R_G)) / (std(R_1..R_G) + eps_A)
  eq. 4   rho_it  = pi_theta(y_it) / pi_old(y_it)
  eq. 5   rhob_it = clip(rho_it, 1 - eps_c, 1 + eps_c)
  eq. 6   J_it    = min(rho_it A_i, rhob_it A_i)
  eq. 7   L       = -(1 / sum_i T_i) sum_i sum_t J_it + beta D_KL(pi_theta || pi_ref)

with the same A_i for every optimised token of rollout i and T_i the number of
optimised tokens of rollout i.  The trainer receives token log-probabilities,
action masks and trajectory rewards (same section, "Rollout workers"), so the
inputs here are packed per-token log-probs of the current, old and reference
policies, a per-token action mask and one reward per rollout.

Readings where the pages leave a step open:
  * std is the population standard deviation of the group's G rewards; a
    reward equal to the group mean has advantage 0 (also for eps_A = 0 with
    all G rewards equal, where eq. 3 reads 0 / 0);
  * the optimised tokens are those whose action mask is 1;
  * D_KL(pi_theta || pi_ref) is estimated per optimised token and averaged
    like the J term (same 1 / sum_i T_i): kl_mode 0 takes the log-ratio
    logp_theta - logp_ref (the plain sample estimate of that KL), kl_mode 1
    takes exp(r) - r - 1 with r = logp_ref - logp_theta (a nonnegative form);
  * a batch of M groups (rollouts m*G .. m*G + G - 1 form group m): each
    group's loss is eq. 7 with its own normaliser, the batch loss is their
    mean, and a group without optimised tokens contributes 0;
  * the output besides the loss is dL / dlogp_theta per token (the only
    input that depends on theta).  J is continuous in rho but its derivative
    jumps where the clip becomes active: the clip counts as active when
    (A > 0 and rho > 1 + eps_c) or (A < 0 and rho < 1 - eps_c), and then
    dJ/dlogp = 0, else dJ/dlogp = A rho.  The decision is taken on the given
    log-probabilities in exact arithmetic: rho > 1 + eps_c is
    logp_theta - logp_old > log(1 + eps_c), with the difference of the two
    (fp32) inputs formed in fp64, where it is exact, and the bound
    log1p(eps_c) in fp64 (within one fp64 ulp of log(1 + eps_c); a
    difference that lands inside that ulp is not a case any fp32 input
    reaches except by construction).  The loss value itself is the literal
    min of eq. 6, in fp64.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def group_advantages(rewards, group_size: int, eps_adv: float) -> np.ndarray:
    """Eq. 3 for every rollout: (R_i - mean) / (population std + eps_A) over its group."""
    r_all = np.asarray(rewards, dtype=np.float64)
    g = int(group_size)
    if g <= 0 or r_all.size % g:
        raise ValueError("the number of rollouts must be a multiple of the group size")
    adv = np.empty_like(r_all)
    for m in range(r_all.size // g):
        r = r_all[m * g:(m + 1) * g]
        mu = r.sum() / g
        sigma = math.sqrt(((r - mu) ** 2).sum() / g)
        # a reward equal to the group mean has advantage 0, also when eps_A = 0 and all G
        # rewards are equal (eq. 3 would be 0 / 0 there; 0 is its limit for eps_A -> 0)
        with np.errstate(divide="ignore", invalid="ignore"):
            adv[m * g:(m + 1) * g] = np.where(r == mu, 0.0, (r - mu) / (sigma + eps_adv))
    return adv


def clip_thresholds(eps_clip: float):
    """The log-domain clip bounds log(1 + eps_c) and log(1 - eps_c), in fp64."""
    return math.log1p(eps_clip), math.log1p(-eps_clip)


def clip_active(logp_new: float, logp_old: float, adv: float, eps_clip: float) -> bool:
    """Whether the clipped term of eq. 6 is the strictly smaller one (see the header)."""
    hi, lo = clip_thresholds(eps_clip)
    d = float(logp_new) - float(logp_old)
    return bool((adv > 0 and d > hi) or (adv < 0 and d < lo))


def kl_term(logp_new: float, logp_ref: float, kl_mode: int):
    """Per-token KL estimate and its derivative in logp_new (see the header)."""
    if kl_mode == 0:
        return logp_new - logp_ref, 1.0
    if kl_mode == 1:
        r = logp_ref - logp_new
        e = math.exp(r)
        return e - r - 1.0, 1.0 - e
    raise ValueError("kl_mode must be 0 or 1")


def grpo_loss(logp_new, logp_old, logp_ref, action_mask, rewards, cu_seqlens: Sequence[int],
              group_size: int, eps_adv: float, eps_clip: float, beta: float, kl_mode: int = 0):
    """Eq. 3-7 over a packed batch.  Returns (loss, grad, advantages, group_losses), fp64.

    logp_* : [N] per-token log-probabilities (logp_ref may be None when beta == 0)
    action_mask : [N] 0/1 or None (every token optimised)
    rewards : [B], cu_seqlens : [B + 1] token offsets of the B rollouts.
    """
    new = np.asarray(logp_new, dtype=np.float64)
    old = np.asarray(logp_old, dtype=np.float64)
    n_tok = new.size
    ref = None if logp_ref is None else np.asarray(logp_ref, dtype=np.float64)
    if beta != 0.0 and ref is None:
        raise ValueError("a KL term needs the reference log-probs")
    mask = np.ones(n_tok, dtype=bool) if action_mask is None else \
        (np.asarray(action_mask) != 0)
    cu = [int(c) for c in cu_seqlens]
    n_roll = len(cu) - 1
    adv = group_advantages(rewards, group_size, eps_adv)
    if adv.size != n_roll:
        raise ValueError("one reward per rollout")
    g = int(group_size)
    n_groups = n_roll // g
    grad = np.zeros(n_tok)
    group_losses = np.zeros(n_groups)
    for m in range(n_groups):
        rolls = range(m * g, (m + 1) * g)
        s_m = sum(int(mask[cu[i]:cu[i + 1]].sum()) for i in rolls)   # sum_i T_i
        if s_m == 0:
            continue
        j_sum = 0.0
        kl_sum = 0.0
        hi, lo = clip_thresholds(eps_clip)
        for i in rolls:
            a = adv[i]
            sl = slice(cu[i], cu[i + 1])
            on = mask[sl]
            nw, od = new[sl][on], old[sl][on]
            rho = np.exp(nw - od)                                       # eq. 4
            rho_bar = np.clip(rho, 1.0 - eps_clip, 1.0 + eps_clip)      # eq. 5
            j_sum += np.minimum(rho * a, rho_bar * a).sum()             # eq. 6
            # clip decision on the exact log-ratio (clip_active, elementwise)
            d = nw - od
            active = (d > hi) if a > 0 else ((d < lo) if a < 0 else np.zeros(d.shape, bool))
            dj = np.where(active, 0.0, a * rho)
            dkl = np.zeros_like(rho)
            if beta != 0.0:
                rf = ref[sl][on]
                if kl_mode == 0:
                    kl, dkl = nw - rf, np.ones_like(rho)
                elif kl_mode == 1:
                    r = rf - nw
                    kl, dkl = np.exp(r) - r - 1.0, 1.0 - np.exp(r)
                else:
                    raise ValueError("kl_mode must be 0 or 1")
                kl_sum += kl.sum()
            g_roll = np.zeros(cu[i + 1] - cu[i])
            g_roll[on] = (-dj + beta * dkl) / (s_m * n_groups)
            grad[sl] = g_roll
        group_losses[m] = (-j_sum + beta * kl_sum) / s_m                # eq. 7
    loss = group_losses.mean() if n_groups else 0.0
    return loss, grad, adv, group_losses
