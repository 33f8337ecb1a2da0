"""Pins of the GRPO oracle (arXiv 2608.10357, section 4 "Training pipeline", paragraph
"Policy update", eq. 3-7) against what the equations and the mathematics fix: closed forms,
numpy's population standard deviation, central finite differences of the loss, and the
structure of the batch (mask, groups).  CPU only."""
import decimal
import math

import numpy as np
import pytest

import oracle


def test_advantage_closed_form():
    # rewards 1, 0, 0, 1: mean 1/2, population std 1/2
    adv = oracle.group_advantages([1.0, 0.0, 0.0, 1.0], 4, 1e-6)
    assert np.allclose(adv, np.array([0.5, -0.5, -0.5, 0.5]) / (0.5 + 1e-6), rtol=0, atol=1e-15)
    # a group with equal rewards has no advantage (0 / (0 + eps))
    assert np.array_equal(oracle.group_advantages([3.0, 3.0, 3.0], 3, 1e-4), np.zeros(3))
    assert np.array_equal(oracle.group_advantages([3.0, 3.0, 3.0], 3, 0.0), np.zeros(3))


def test_advantage_matches_numpy_population_std():
    rng = np.random.default_rng(1)
    r = rng.normal(size=24)
    adv = oracle.group_advantages(r, 6, 1e-3)
    for m in range(4):
        g = r[6 * m:6 * m + 6]
        assert np.allclose(adv[6 * m:6 * m + 6], (g - g.mean()) / (np.std(g, ddof=0) + 1e-3),
                           rtol=1e-13, atol=1e-13)


def test_advantage_invariants():
    rng = np.random.default_rng(2)
    r = rng.normal(size=16)
    a = oracle.group_advantages(r, 8, 1e-8)
    assert abs(a[:8].sum()) < 1e-12 and abs(a[8:].sum()) < 1e-12          # zero mean per group
    assert np.allclose(oracle.group_advantages(r + 7.5, 8, 1e-8), a, atol=1e-10)   # shift
    assert np.allclose(oracle.group_advantages(3 * r, 8, 1e-12), a, atol=1e-9)     # scale


def _batch(lengths, group, seed, mask_p=0.7, spread=0.3):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    n = int(cu[-1])
    old = -rng.gamma(2.0, 1.0, size=n).astype(np.float32)
    new = (old + rng.normal(scale=spread, size=n)).astype(np.float32)
    ref = (old + rng.normal(scale=spread, size=n)).astype(np.float32)
    mask = (rng.random(n) < mask_p).astype(np.uint8)
    rewards = rng.normal(size=len(lengths)).astype(np.float32)
    return new, old, ref, mask, rewards, cu


def test_unit_ratio_loss_is_minus_token_weighted_advantage():
    # rho = 1 everywhere and beta = 0: J = A_i, so L = -sum_i T_i A_i / sum_i T_i; with equal
    # T_i that is -mean(A) = 0
    lengths = [5, 9, 2, 4]
    new, old, ref, mask, rewards, cu = _batch(lengths, 4, 3)
    loss, grad, adv, _ = oracle.grpo_loss(new, new, None, None, rewards, cu, 4, 1e-6, 0.2, 0.0)
    t = np.array(lengths, dtype=np.float64)
    assert math.isclose(loss, -(t * adv).sum() / t.sum(), rel_tol=1e-12, abs_tol=1e-15)
    for i in range(4):
        assert np.allclose(grad[cu[i]:cu[i + 1]], -adv[i] / t.sum(), rtol=1e-12)
    loss_eq, _, _, _ = oracle.grpo_loss(new[:12], new[:12], None, None, rewards, [0, 3, 6, 9, 12],
                                        4, 1e-6, 0.2, 0.0)
    assert abs(loss_eq) < 1e-15


def test_clip_closed_forms():
    # group of 2 with rewards 1, 0: A = +-0.5 / (0.5 + eps) = +-1/(1 + 2 eps)
    eps_a, eps_c = 1e-6, 0.2
    a = 0.5 / (0.5 + eps_a)
    ln2 = math.log(2.0)
    # rollout 0 (A > 0): rho = 2 and 1/2; rollout 1 (A < 0): rho = 2 and 1/2
    old = np.zeros(4, dtype=np.float32)
    new = np.array([ln2, -ln2, ln2, -ln2], dtype=np.float32)
    rho = np.exp(new.astype(np.float64))
    loss, grad, _, _ = oracle.grpo_loss(new, old, None, None, [1.0, 0.0], [0, 2, 4], 2, eps_a,
                                        eps_c, 0.0)
    j = [1.2 * a, rho[1] * a, -rho[2] * a, -0.8 * a]   # min(rho A, clip(rho) A) by hand
    assert math.isclose(loss, -sum(j) / 4, rel_tol=1e-12)
    # the clip is active (zero gradient) for rho = 2 with A > 0 and rho = 1/2 with A < 0
    assert np.allclose(grad, np.array([0.0, -rho[1] * a, rho[2] * a, 0.0]) / 4, rtol=1e-12)


def test_kl_terms():
    assert oracle.kl_term(-1.5, -1.5, 0) == (0.0, 1.0)
    assert oracle.kl_term(-1.5, -1.5, 1) == (0.0, 0.0)
    for d in (-3.0, -0.1, 0.0, 0.2, 2.5):
        kl0, _ = oracle.kl_term(-1.0 + d, -1.0, 0)
        kl1, _ = oracle.kl_term(-1.0 + d, -1.0, 1)
        assert math.isclose(kl0, d, abs_tol=1e-15)
        assert kl1 >= 0.0 and math.isclose(kl1, math.exp(-d) + d - 1.0, rel_tol=1e-13, abs_tol=1e-15)
    # small differences: exp(r) - r - 1 = r^2 / 2 + O(r^3)
    kl1, _ = oracle.kl_term(-1.0 + 1e-4, -1.0, 1)
    assert math.isclose(kl1, 0.5e-8, rel_tol=1e-3)
    # with new == ref the KL part of the loss vanishes in both modes
    new, old, ref, mask, rewards, cu = _batch([6, 3, 7, 2], 2, 4)
    base, _, _, _ = oracle.grpo_loss(new, old, None, mask, rewards, cu, 2, 1e-6, 0.2, 0.0)
    for mode in (0, 1):
        with_kl, _, _, _ = oracle.grpo_loss(new, old, new, mask, rewards, cu, 2, 1e-6, 0.2, 0.3,
                                            mode)
        assert math.isclose(with_kl, base, rel_tol=1e-13, abs_tol=1e-16)


def _far_from_clip(new, old, eps_c, margin=1e-3):
    d = new.astype(np.float64) - old.astype(np.float64)
    return np.all(np.abs(d - math.log1p(eps_c)) > margin) and \
        np.all(np.abs(d - math.log1p(-eps_c)) > margin)


@pytest.mark.parametrize("kl_mode", [0, 1])
def test_gradient_matches_finite_differences(kl_mode):
    lengths = [4, 7, 3, 5, 6, 2]
    new, old, ref, mask, rewards, cu = _batch(lengths, 3, 5 + kl_mode, spread=0.4)
    assert _far_from_clip(new, old, 0.2)
    new64 = new.astype(np.float64)
    args = (old, ref, mask, rewards, cu, 3, 1e-4, 0.2, 0.05, kl_mode)
    _, grad, _, _ = oracle.grpo_loss(new64, *args)
    h = 1e-6
    for t in range(new.size):
        up, dn = new64.copy(), new64.copy()
        up[t] += h
        dn[t] -= h
        lu = oracle.grpo_loss(up, *args)[0]
        ld = oracle.grpo_loss(dn, *args)[0]
        assert math.isclose(grad[t], (lu - ld) / (2 * h), rel_tol=1e-6, abs_tol=1e-10), t


def test_masked_tokens_do_not_count():
    new, old, ref, mask, rewards, cu = _batch([8, 5, 9, 6], 2, 7)
    loss, grad, _, _ = oracle.grpo_loss(new, old, ref, mask, rewards, cu, 2, 1e-6, 0.2, 0.1)
    assert np.all(grad[mask == 0] == 0.0)
    new2 = new.copy()
    new2[mask == 0] += 5.0     # masked tokens' log-probs are irrelevant
    loss2, _, _, _ = oracle.grpo_loss(new2, old, ref, mask, rewards, cu, 2, 1e-6, 0.2, 0.1)
    assert loss2 == loss
    # a group with no optimised token contributes 0 to the batch mean
    mask0 = mask.copy()
    mask0[cu[0]:cu[2]] = 0
    loss0, grad0, _, gl = oracle.grpo_loss(new, old, ref, mask0, rewards, cu, 2, 1e-6, 0.2, 0.1)
    assert gl[0] == 0.0 and np.all(grad0[cu[0]:cu[2]] == 0.0)
    assert math.isclose(loss0, gl[1] / 2, rel_tol=1e-15)


def test_batch_is_mean_of_groups():
    lengths = [3, 6, 2, 5, 4, 7]
    new, old, ref, mask, rewards, cu = _batch(lengths, 2, 8)
    loss, grad, _, gl = oracle.grpo_loss(new, old, ref, mask, rewards, cu, 2, 1e-6, 0.2, 0.1, 1)
    assert math.isclose(loss, gl.mean(), rel_tol=1e-15)
    for m in range(3):
        sl = slice(int(cu[2 * m]), int(cu[2 * m + 2]))
        cu_m = np.array(cu[2 * m:2 * m + 3]) - cu[2 * m]
        lm, gm, _, _ = oracle.grpo_loss(new[sl], old[sl], ref[sl], mask[sl], rewards[2 * m:2 * m + 2],
                                        cu_m, 2, 1e-6, 0.2, 0.1, 1)
        assert math.isclose(lm, gl[m], rel_tol=1e-13)
        assert np.allclose(gm / 3, grad[sl], rtol=1e-13, atol=0)


def _exact_clip_active(new32, old32, adv, eps):
    """rho > 1 + eps (A > 0) or rho < 1 - eps (A < 0) decided with 60-digit decimals:
    the fp32 inputs are exact binary fractions and log(1 +- eps) is evaluated to far
    beyond any fp32 or fp64 rounding (eq. 5-6 of the "Policy update" paragraph)."""
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        d = decimal.Decimal(float(new32)) - decimal.Decimal(float(old32))
        e = decimal.Decimal(float(eps))
        hi = (1 + e).ln()
        lo = (1 - e).ln()
        return bool((adv > 0 and d > hi) or (adv < 0 and d < lo))


def test_clip_decision_is_exact_near_the_threshold():
    f32 = np.float32
    fp32_disagrees = 0
    for eps in (0.25, float(f32(0.2)), 0.125, float(f32(0.28))):
        cases = []
        for bound in (math.log1p(eps), math.log1p(-eps)):
            b32 = f32(bound)
            # fp32 log-probs bracketing the bound, as the difference from logp_old = 0 ...
            for x in (np.nextafter(b32, f32(-1)), b32, np.nextafter(b32, f32(1))):
                cases.append((f32(x), f32(0.0)))
            # ... and from a logp_old of another magnitude, where the fp32 difference rounds
            for old in (f32(-1e-3), f32(-3.7), f32(-0.0625)):
                new = f32(float(old) + bound)
                for x in (np.nextafter(new, f32(-10)), new, np.nextafter(new, f32(10))):
                    cases.append((f32(x), old))
        for new, old in cases:
            for adv in (1.0, -1.0, 0.0):
                want = _exact_clip_active(new, old, adv, eps)
                assert oracle.clip_active(float(new), float(old), adv, eps) == want, \
                    (eps, float(new), float(old), adv)
                d32 = f32(new - old)
                hi32, lo32 = f32(math.log1p(eps)), f32(math.log1p(-eps))
                fp32_rule = bool((adv > 0 and d32 > hi32) or (adv < 0 and d32 < lo32))
                fp32_disagrees += fp32_rule != want
    # the straddling cases include ones that a decision in fp32 gets wrong
    assert fp32_disagrees > 0


def test_clip_straddling_rollout_by_hand():
    # one group of two rollouts (rewards 1, 0: A = +1, -1 for eps_A = 0), beta = 0,
    # eps_c = 1/4: the clip bound is log(5/4) = 0.22314355131420976.  Rollout 0 holds two
    # tokens 2^-23 on either side of it (logp_old = 0); rollout 1 one token well inside.
    # By eq. 6: J = min(rho A, clip(rho) A); dJ/dlogp = A rho where the clip is inactive,
    # 0 where active; the loss gradient is -dJ/dlogp / S with S = 3 optimised tokens.
    below, above = 0.22314355131420976 - 2.0 ** -23, 0.22314355131420976 + 2.0 ** -23
    new = np.array([below, above, 0.1], np.float32)
    old = np.zeros(3, np.float32)
    loss, grad, adv, _ = oracle.grpo_loss(new, old, None, None, [1.0, 0.0], [0, 2, 3], 2,
                                          0.0, 0.25, 0.0)
    assert list(adv) == [1.0, -1.0]
    rho = np.exp(new.astype(np.float64))
    assert math.isclose(grad[0], -rho[0] / 3, rel_tol=1e-15)   # below the bound: A rho
    assert grad[1] == 0.0                                        # above it: clipped
    assert math.isclose(grad[2], rho[2] / 3, rel_tol=1e-15)    # A = -1, rho inside the band
    j = rho[0] + 1.25 - rho[2]
    assert math.isclose(loss, -j / 3, rel_tol=1e-15)


def test_token_counts_are_optimised_tokens():
    # rho = 1, beta = 0 with an action mask: J = A_i on optimised tokens only, so
    # L = -sum_i T_i A_i / sum_i T_i with T_i the optimised-token counts (not the lengths)
    lengths = [6, 4, 5, 3]
    new, old, ref, mask, rewards, cu = _batch(lengths, 4, 9, mask_p=0.5)
    t = np.array([mask[cu[i]:cu[i + 1]].sum() for i in range(4)], dtype=np.float64)
    assert not np.array_equal(t, np.array(lengths, dtype=np.float64))
    loss, grad, adv, _ = oracle.grpo_loss(new, new, None, mask, rewards, cu, 4, 1e-6, 0.2, 0.0)
    assert math.isclose(loss, -(t * adv).sum() / t.sum(), rel_tol=1e-12, abs_tol=1e-15)
    for i in range(4):
        sl = slice(int(cu[i]), int(cu[i + 1]))
        assert np.allclose(grad[sl], np.where(mask[sl] != 0, -adv[i] / t.sum(), 0.0), rtol=1e-12)
