"""Batched speculative-sampling verification on AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels in ``libspecverify.so`` behind the
C ABI of ``include/spec_verify.h`` (verification), ``include/spec_bandit.h``
(online draft selection), ``include/spec_head.h`` (low-rank draft head with
its fused normaliser) and ``include/spec_tree.h`` (draft-tree pruning and
greedy tree verification); this package is a thin ctypes binding with
the same function names (``binding``) and the build script (``build``).
"""
from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, SPEC_BF16, SPEC_F32, Context, SpecVerifyError, dtype_code,
    load_library, spec_accept_logprobs, spec_verify, spec_verify_copy_lse, spec_verify_offset_ptr,
    spec_verify_destroy, spec_verify_enable_timing, spec_verify_get_geometry,
    spec_verify_init, spec_verify_philox_words, spec_verify_read_timing,
    spec_verify_set_stream, spec_verify_strerror, spec_verify_outcomes, SPEC_OUTCOME_MAX_F,
    spec_outcome_fanout, SPEC_FANOUT_MAX_LENGTHS,
    SPEC_BANDIT_MAX_ARMS, SPEC_BANDIT_THOMPSON, SPEC_BANDIT_UCB1, BanditContext,
    spec_bandit_destroy, spec_bandit_get_state, spec_bandit_init, spec_bandit_set_state,
    spec_bandit_set_stream, spec_bandit_step,
    HeadContext, spec_lowrank_head, spec_lowrank_head_copy_activation, spec_lowrank_head_destroy,
    spec_lowrank_head_init, spec_lowrank_head_set_stream,
    SPEC_TREE_MAX_NODES, TreeContext, spec_tree_prune, spec_tree_verify_destroy,
    spec_tree_verify_greedy, spec_tree_verify_init, spec_tree_verify_sample,
    spec_tree_verify_set_stream, spec_tree_verify_gave_up, spec_tree_verify_set_spin_limit,
    SPEC_ESCRATCH, SPEC_VERIFY_NOALLOC_SCRATCH_BYTES, spec_verify_noalloc, spec_hbm_read_probe,
)
