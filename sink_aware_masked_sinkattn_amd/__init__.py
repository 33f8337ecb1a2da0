"""Sink-aware masked attention for MI355X (gfx950): forward, backward, rollout
decode, and the GRPO token loss of the same trainer.

The computation lives in ``libsinkattn.so`` (hand-written HIP kernels behind
the C ABI of ``include/sinkattn.h``); this package only binds it.
"""
from .binding import (BWD_ALL, BWD_DKDV, BWD_DQ, BWD_FINISH, BWD_PREPARE, WINDOW_INF,
                      DecodeProblem, GrpoProblem, Problem, SinkAttnError, load_library,
                      make_decode_problem, make_grpo_problem, make_problem, sinkattn_bwd,
                      sinkattn_bwd_phases, sinkattn_grpo_loss, sinkattn_grpo_workspace_size,
                      sinkattn_bwd_workspace_size, sinkattn_decode, sinkattn_decode_noalloc,
                      sinkattn_decode_workspace_size, sinkattn_fwd, sinkattn_key_tile_segments,
                      sinkattn_tile_class, sinkattn_tile_config)

__all__ = [
    "WINDOW_INF", "Problem", "SinkAttnError", "load_library", "make_problem",
    "BWD_PREPARE", "BWD_DKDV", "BWD_DQ", "BWD_FINISH", "BWD_ALL",
    "sinkattn_fwd", "sinkattn_bwd", "sinkattn_bwd_phases", "sinkattn_bwd_workspace_size",
    "sinkattn_tile_class", "sinkattn_key_tile_segments", "sinkattn_tile_config",
    "DecodeProblem", "make_decode_problem", "sinkattn_decode", "sinkattn_decode_workspace_size",
    "sinkattn_decode_noalloc",
    "GrpoProblem", "make_grpo_problem", "sinkattn_grpo_loss", "sinkattn_grpo_workspace_size",
]
