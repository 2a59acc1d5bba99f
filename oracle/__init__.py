"""CPU oracle for the UniPrefill token-block pruning path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
calls it, and it shares no code with the GPU library.

Every function is a plain fp64 transcription of what the method computes, as
described on the UniPrefill article page "中国科学院与腾讯微信合作解决AI排队等待问题"
(sections 二 and 三 and its Q&A).  Two implementations of steps 1-5:
uniprefill_oracle.py (numpy) and uniprefill_oracle.cpp (plain single-threaded
C++17, reached through cxx.py); see those files for per-function citations.
"""
from .uniprefill_oracle import (  # noqa: F401
    widen_bf16,
    tail_range,
    tail_attention_probs,
    token_scores,
    block_offsets,
    block_scores,
    forced_blocks,
    select_request,
    select_topp,
    selection_trace,
    band_blocks,
    token_keep,
    compact,
    scatter_back,
    round_to_format,
    rms_normalize,
    compact_rmsnorm,
    gather_add,
    history_new,
    history_append,
    history_kv_len,
    run_chain,
)
