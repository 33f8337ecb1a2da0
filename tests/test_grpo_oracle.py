"""Pins of the GRPO oracle (arXiv 2608.10357, section 4 "Training pipeline", paragraph
"Policy update", eq. 3-7) against what the equations and the mathematics fix: closed forms,
numpy's population standard deviation, central finite differences of the loss, and the
structure of the batch (mask, groups).  CPU only."""
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


def test_clip_decision_in_fp32_log_domain():
    hi, lo = oracle.clip_thresholds(0.2)
    assert hi == np.float32(math.log(1.2)) and lo == np.float32(math.log(0.8))
    # just above / below the upper bound, decided on the fp32 difference
    above = float(np.nextafter(hi, np.float32(1)))
    assert oracle.clip_active(above, 0.0, 1.0, 0.2)
    assert not oracle.clip_active(float(hi), 0.0, 1.0, 0.2)
    assert not oracle.clip_active(above, 0.0, -1.0, 0.2)
    below = float(np.nextafter(lo, np.float32(-1)))
    assert oracle.clip_active(below, 0.0, -1.0, 0.2)
    assert not oracle.clip_active(below, 0.0, 1.0, 0.2)
    assert not oracle.clip_active(5.0, 0.0, 0.0, 0.2)


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
