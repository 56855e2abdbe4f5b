"""CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
bench's cpu_baseline leg may import this package.  The GPU library never calls
it, and it imports nothing from the GPU library.
"""
from .verify_oracle import (  # noqa: F401
    FLAG_PROBE_TIE, FLAG_ACCEPT_TIE, FLAG_CDF_TIE, FLAG_DEGENERATE, FLAG_NO_CANDIDATE,
    FLAG_BAD_PAGE, FLAG_BAD_CTX, FLAG_BAD_TOKEN, FLAG_POOL_EMPTY,
    bf16_bits_to_f64, round_f64_to_bf16, as_f64,
    copy_match, copy_labels, probe_gate, verify_attention, verify_attention_layers,
    lm_head_full, lm_head_lowrank,
    head_softmax, reject_sample, reject_sample_multi, reject_sample_greedy, verify_step,
    kv_commit, kv_commit_layers, kv_truncate, gather_prefix, token_major, draft_sample, rho_tps,
)
