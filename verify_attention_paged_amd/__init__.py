"""Paged decode/verify attention and speculative verification for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of ``include/vap.h``
(``lib/libvap.so``); this package is the thin Python binding over it.  PyTorch supplies device
memory and streams only.

    paged_attn_step(q, kv_pool, block_tables, ctx_lens, q_lens, out=None, *, scale=0.0)
    spec_verify(p, q, draft_ids, uniforms, out_ids=None, n_accepted=None)
    spec_verify_static(p, q, draft_ids, uniforms, out_ids, n_accepted)   (no workspace)
    spec_verify_tree(p, q, parents, tokens, uniforms)
    spec_verify_logits(target_logits, draft_logits, draft_ids, uniforms, temperatures)
    kv_append(k_new, v_new, kv_pool, block_tables, ctx_lens, q_lens)
    kv_commit(kv_pool, block_tables, ctx_lens, q_lens, n_accepted, path=None)
    (paged_attn_step also takes kv_scales= for an 8-bit cache and tree_mask= for token trees)
"""

from ._binding import (  # noqa: F401
    AttnShape,
    VapError,
    LIB_PATH,
    DERR_BLOCK_ID,
    DERR_LENS,
    DERR_TOTAL_Q,
    DERR_DRAFT_ID,
    DERR_EMPTY_ROW,
    DERR_TREE,
    DERR_TEMP,
    DERR_SYNC,
    TIMER_ATTENTION,
    TIMER_VERIFY,
    TIMER_TREE_VERIFY,
    TIMER_KV_APPEND,
    TIMER_KV_COMMIT,
    TIMER_LOGIT_STATS,
    TIMER_VERIFY_LOGITS,
    TIMER_TREE_DRAW,
    attn_shape,
    attn_workspace,
    device_info,
    get_device_error,
    header_functions,
    kv_append,
    kv_commit,
    kv_workspace,
    load_library,
    paged_attn_step,
    spec_verify,
    spec_verify_static,
    spec_verify_tree,
    spec_verify_logits,
    verify_logits_workspace,
    tree_verify_workspace,
    stream_copy,
    stream_read,
    timer_enable,
    timer_read,
    verify_workspace,
    workspace_init,
)
