"""fp64 CPU oracle for sink-aware masked attention and the GRPO token loss.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library.
"""
from .grpo_ref import clip_active, clip_thresholds, group_advantages, grpo_loss, kl_term
from .sinkattn_ref import (attend_head, attend_head_grad, backward, decode, forward,
                           key_grads_head, rows_head, sink_grad_head, visible_mask)

__all__ = ["visible_mask", "attend_head", "attend_head_grad", "forward", "backward", "decode",
           "rows_head", "key_grads_head", "sink_grad_head",
           "group_advantages", "grpo_loss", "clip_active", "clip_thresholds", "kl_term"]
