"""GPU parity of the GRPO token loss (arXiv 2608.10357, section 4 "Training pipeline",
paragraph "Policy update", eq. 3-7) with the fp64 oracle, through the C ABI.

Tolerances (fp32 arithmetic per token, one exp each; the loss terms summed in fp64): loss
within 1e-5 relative + 1e-9 absolute; advantages within
1e-6 x max|A| (fp64 group statistics, rounded once); gradients element by element within
2e-6 x max|grad|.  The oracle takes the clip decision of eq. 6 in exact arithmetic, the kernel
on the fp32 difference of the log-probs against fp32 bounds: the two can differ only for
tokens whose exact log-ratio lies within one fp32 ulp of log(1 +- eps_c), so tokens within
two fp32 ulps of either bound are left out of the gradient comparison (their number is
logged; the loss is continuous there and is compared in full).  eps_c reaches both sides as
the fp32 value the C ABI carries.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import log
from sink_aware_masked_sinkattn_amd import sinkattn_grpo_loss
from workloads import GRPO_WORKLOADS, grpo_workload_inputs, make_grpo_inputs

pytestmark = pytest.mark.gpu


def run_gpu(inp, use_mask=True, use_ref=True, workspace=None):
    dev = torch.device("cuda:0")
    loss, grad, adv = sinkattn_grpo_loss(
        inp.logp_new.to(dev), inp.logp_old.to(dev), inp.logp_ref.to(dev) if use_ref else None,
        inp.action_mask.to(dev) if use_mask else None, inp.rewards.to(dev),
        inp.cu_seqlens.to(dev), inp.group_size, inp.eps_adv, inp.eps_clip, inp.beta,
        inp.kl_mode, workspace=workspace)
    torch.cuda.synchronize()
    return float(loss.item()), grad.cpu().double().numpy(), adv.cpu().double().numpy()


def eps32(x: float) -> float:
    return float(np.float32(x))


def run_oracle(inp, use_mask=True, use_ref=True):
    return oracle.grpo_loss(inp.logp_new.numpy(), inp.logp_old.numpy(),
                            inp.logp_ref.numpy() if use_ref else None,
                            inp.action_mask.numpy() if use_mask else None, inp.rewards.numpy(),
                            inp.cu_seqlens.numpy(), inp.group_size, eps32(inp.eps_adv),
                            eps32(inp.eps_clip), eps32(inp.beta), inp.kl_mode)


def near_clip_bound(inp) -> np.ndarray:
    """Tokens whose exact log-ratio is within two fp32 ulps of log(1 +- eps_c)."""
    d = inp.logp_new.numpy().astype(np.float64) - inp.logp_old.numpy().astype(np.float64)
    near = np.zeros(d.shape, bool)
    for b in (np.log1p(eps32(inp.eps_clip)), np.log1p(-eps32(inp.eps_clip))):
        near |= np.abs(d - b) <= 2.0 * float(np.spacing(np.float32(abs(b))))
    return near


def check(gpu, ref, label, inp):
    loss, grad, adv = gpu
    r_loss, r_grad, r_adv, _ = ref
    near = near_clip_bound(inp)
    keep = ~near
    e_loss = abs(loss - r_loss)
    e_adv = float(np.abs(adv - r_adv).max()) if adv.size else 0.0
    e_grad = float(np.abs(grad[keep] - r_grad[keep]).max()) if keep.any() else 0.0
    g_scale = float(np.abs(r_grad).max()) if grad.size else 0.0
    a_scale = float(np.abs(r_adv).max()) if adv.size else 0.0
    log(f"{label}: loss {loss:.9g} vs {r_loss:.9g} (|d| {e_loss:.3g}), max|dA| {e_adv:.3g}, "
        f"max|dgrad| {e_grad:.3g} of {g_scale:.3g}; {int(near.sum())} tokens within two fp32 "
        f"ulps of a clip bound left out of the gradient comparison")
    assert e_loss <= 1e-5 * abs(r_loss) + 1e-9, label
    assert e_adv <= 1e-6 * max(a_scale, 1.0), label
    assert e_grad <= 2e-6 * g_scale + 1e-30, label


CASES = [
    # lengths, G, beta, kl_mode, eps_adv, eps_clip, new_drift, mask
    ((5, 7, 3, 9), 2, 0.04, 0, 1e-6, 0.2, 0.3, True),
    ((5, 7, 3, 9), 4, 0.1, 1, 1e-6, 0.2, 0.3, True),
    ((1, 0, 2, 0, 3, 1), 3, 0.04, 0, 1e-6, 0.2, 0.2, True),      # empty rollouts, N < 4
    ((4097, 5000, 3, 100), 2, 0.04, 1, 1e-6, 0.2, 0.2, True),    # several workgroups, ragged
    ((2000,) * 8, 8, 0.0, 0, 1e-6, 0.1, 0.3, False),             # no mask, no KL term
    ((300, 800, 77, 1200, 1, 9000), 1, 0.02, 1, 0.0, 0.28, 0.5, True),   # G = 1: A = 0
    ((640, 641, 642, 643, 9, 10, 11, 12), 4, 0.05, 0, 1e-4, 0.2, 0.05, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "n{}_G{}_b{}_kl{}".format(
    "-".join(map(str, c[0][:4])), c[1], c[2], c[3]))
def test_grpo_small(case):
    lengths, g, beta, mode, eps_a, eps_c, drift, mask = case
    inp = make_grpo_inputs(lengths=lengths, group_size=g, seed=sum(lengths) + g, beta=beta,
                           kl_mode=mode, eps_adv=eps_a, eps_clip=eps_c, new_drift=drift,
                           agent_span=(2, 40), obs_span=(2, 60))
    use_ref = beta != 0.0
    log(f"grpo case {case}")
    check(run_gpu(inp, mask, use_ref), run_oracle(inp, mask, use_ref), str(case), inp)


def test_grpo_equal_rewards_and_unoptimised_group():
    inp = make_grpo_inputs(lengths=(50, 60, 70, 80, 90, 100), group_size=2, seed=11, beta=0.04,
                           eps_adv=0.0)
    inp.rewards = torch.tensor([1.0, 1.0, 0.0, 1.0, 0.0, 0.0])   # groups 0 and 2: A = 0
    inp.action_mask[int(inp.cu_seqlens[2]):int(inp.cu_seqlens[4])] = 0   # group 1: no tokens
    gpu, ref = run_gpu(inp), run_oracle(inp)
    assert ref[3][1] == 0.0
    check(gpu, ref, "equal rewards, empty group", inp)
    assert np.all(gpu[1][int(inp.cu_seqlens[2]):int(inp.cu_seqlens[4])] == 0.0)


def test_grpo_deterministic_and_workspace_reuse():
    dev = torch.device("cuda:0")
    big = make_grpo_inputs(lengths=tuple(range(3000, 3016)), group_size=8, seed=21, kl_mode=1)
    small = make_grpo_inputs(lengths=(10, 20, 30, 40), group_size=4, seed=22)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    a = run_gpu(big, workspace=ws)
    b = run_gpu(big, workspace=ws)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    check(run_gpu(small, workspace=ws), run_oracle(small), "second, smaller call", small)
    check(a, run_oracle(big), "first call", big)


@pytest.mark.parametrize("name", list(GRPO_WORKLOADS))
def test_grpo_workload_full_size(name):
    inp = grpo_workload_inputs(name)
    log(f"{name}: {inp.logp_new.numel()} tokens, {inp.rewards.numel()} rollouts")
    check(run_gpu(inp), run_oracle(inp), name, inp)
