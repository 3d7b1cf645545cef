"""fp64 CPU oracle for the masked FlashAttention forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports, calls or links it,
and this package imports nothing from the product path.

What it computes is the plain definition of masked softmax attention: the
full ``[Lq, Lk]`` mask and softmax are materialised in fp64 (the unfused
"T x T score" method the InfiniTrain page, section "background", contrasts
with FlashAttention). FlashAttention reaches the same result exactly up to
rounding order, because its online softmax only rescales partial sums
(ExecuTorch page, "Summary"). A second route, the guarded chunked online
softmax, is kept here only to cross-check the first one.

Parity status of each function is stated in its docstring; every function
here is pinned by ``tests/test_oracle_pins.py`` (the varlen / paged-cache
functions by ``tests/test_oracle_paged_pins.py``, the score modifiers, per-head
masks and top-k variants of ``general.py`` by ``tests/test_oracle_general_pins.py``,
the gradients of ``backward.py`` by ``tests/test_oracle_backward_pins.py``).
"""
from .attention import (  # noqa: F401
    NEG_INF,
    query_positions,
    mask_matrix,
    attention_ref,
    attention_rows_ref,
    attention_chunked_ref,
    lse_merge_ref,
)
from .topk import (  # noqa: F401
    topk_kept_ref,
    topk_rank_ref,
    topk_tau_ref,
    kept_from_rank_tau,
    pack_keep_bits,
)
from .paged import gather_sequence_kv, paged_attention_ref  # noqa: F401
from .general import general_attention_ref, general_mask, general_scores  # noqa: F401
from .backward import attention_backward_ref, attention_backward_rows_ref  # noqa: F401
