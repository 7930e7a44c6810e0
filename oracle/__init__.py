"""Reference oracle for training-free block/stripe-sparse attention (CPU, numpy, fp64).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check of the package and the CPU
baseline leg of the benchmark may import or run anything in this package.  The product
path (the HIP library and its Python binding) never calls it and shares no code with it.

What it computes, in the pages' order and notation:

* ``estimate``  -- the estimation pass: the per-row anchor (max logit over the sink
  tokens and the causal local window, AnchorAttention Eq. 1, with the anchor read from the
  row-max buffer as the AnchorAttention referee's first major comment corrects), the
  block-averaged anchor and pooled query (Eq. 2), int8 quantisation of the pooled query
  and of key tiles (the low-precision Q.K^T estimate of SALE), the log-domain
  threshold compare ``avgpool(x_a) - avgpool(Q) K^T / sqrt(d) <= theta`` (Eq. 2), the
  union over the query heads that share a KV head (max aggregation, as the KVpop page
  does for grouped heads), forced sink and local blocks, and compaction into ascending
  per-row index lists (the index set I of Eq. 3).
* ``attention`` -- masked softmax attention under given lists: the plain definition.
* ``decode``    -- block-summary scoring, forced + top-K block selection and attention
  over the selected blocks for one query token per sequence.
* ``calibrate`` -- SALE's per-head threshold calibration: tau halved from 0.008 until the
  L1 output error against full attention meets a bound (theta = -ln tau).
* ``estimate_sale`` -- SALE's element-wise low-bit estimate with the relative attention
  score (the row's log-sum-exp over its sink-local area as the reference).
* ``anchor_state`` -- anchor-state reuse: the attention state over each row's anchor region
  (sink tokens and causal local window) and the sparse pass that resumes from it.

Parity pins: see ``tests/test_oracle_*.py``.  Every function is pinned by brute force,
closed forms, invariants or an independent library routine; none is "parity unpinned".
"""
from .estimate import (  # noqa: F401
    softmax_scale,
    anchor_rows,
    pool_queries,
    quantize_q8,
    quantize_key_tiles,
    forced_blocks,
    forced_columns,
    estimate_rows,
    estimate_all,
    group_step,
    AMBIGUITY_BAND,
)
from .attention import attention_rows, attention_all, dense_causal_reference_mask  # noqa: F401
from .decode import (block_summary, decode_select, decode_attention, quantize_summary_q4,  # noqa: F401
                     dequantize_summary_q4, pack_q4, quantize_summary_fp4,
                     dequantize_summary_fp4, pack_fp4)
from .diagnostics import pruned_mass_fraction, sparsity_from_kept, sale_log_margin  # noqa: F401
from .calibrate import full_lists, head_l1_error, calibrate_theta  # noqa: F401
from .estimate_sale import estimate_rows_sale, estimate_all_sale, relative_scores  # noqa: F401
from .anchor_state import anchor_region, anchor_state_rows, merge_partials, resume_rows  # noqa: F401
