"""MI355X (gfx950) response-replay attention.

Exact attention of one causally masked response branch over a long, detached,
paged prompt K/V cache, split over prompt pages and merged through
log-sum-exp statistics, with a response-only backward (no prompt K/V
gradient).  The arithmetic lives in ``libls_replay.so`` (hand-written HIP
kernels behind the C ABI of ``include/ls_replay.h``); this package is its
binding, a small replay driver and the chunked capture that writes the
prompt's pages.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    LS_ACCUMULATE_KV,
    LS_SPLIT_BLOCK_CYCLIC,
    LS_SPLIT_CONTIGUOUS,
    LS_NOALLOC_SCRATCH_BYTES,
    LS_SPLIT_EXPLICIT,
    AttnShape,
    LsError,
    PageTable,
    lib,
    ls_calib_mfma,
    ls_kv_page_append,
    ls_kv_page_table,
    ls_lse_merge,
    ls_replay_attn_bwd,
    ls_replay_attn_bwd_workspace,
    ls_replay_attn_fwd,
    ls_replay_attn_fwd_members,
    ls_replay_attn_fwd_noalloc,
    ls_replay_attn_fwd_workspace,
    ls_status_string,
    ls_timing_enable,
    ls_timing_read,
    ls_timing_reset,
    ls_version,
    make_shape,
)
from .replay import (  # noqa: F401
    CaptureResult,
    ForwardResult,
    Member,
    PromptCache,
    block_bounds,
    capture_prefill,
    replay_backward,
    replay_forward,
    replay_group,
    replay_member,
    replay_token_blocks,
    score_group,
)
