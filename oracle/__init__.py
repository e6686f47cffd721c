"""fp64 CPU oracle for context-parallel (CP) attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The GPU library never
calls it, and it imports nothing from the GPU library.

Everything here follows the G5 context-parallel modelling spec ("G5
上下文并行建模设计规格"): its Definitions table (CP, pass-KV, pass-Q, ring
step, partial attention with the online-softmax triple, balanced chunk split,
c_kv, d / n_h, CP=1 degeneration), its Formulas section (eq.
g5cp-passkv-bytes, eq. g5cp-step-flops, the pass-Q byte counts and the
per-rank memory) and its Acceptance table.

Parity pins: every function here is pinned by tests in tests/test_oracle_*.py
against hand-worked values, closed forms, brute force and invariants; none is
"parity unpinned".
"""
from .cp_oracle import (  # noqa: F401
    IDENTITY_M,
    account,
    attention_reference,
    attention_reference_rows,
    balanced_split,
    balanced_split_padded,
    brute_force_attention,
    canonical,
    decode_reference,
    finalize,
    merge,
    merge_tree,
    tree_rounds,
    merge_two,
    partial_attention,
    passq_decode,
    ring_prefill,
    ring_prefill_padded,
    ring_schedule,
    sequential_split,
    step_pair_counts,
    upcast,
)
