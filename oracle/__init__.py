"""CPU oracle for CoSA block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  The oracle is a plain, slow, fp64 numpy
implementation of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, calls or links anything under ``oracle/``; the two share no code.
"""
from .cosa_oracle import (  # noqa: F401
    KapParams, OskParams, Shape, budget_count, dense_attention, kap_head, kap_kv_group,
    kap_unit, osk_unit, pool_rows, proxy_block_scores, restricted_attention,
    round_to_dtype, run_head, osk_walk, COMPUTED, VISITED, SKIP_OFF,
    SKIP_MAXDIFF, SKIP_MASS, STATUS_NOT_REACHED, STATUS_COMPUTED,
    STATUS_SKIPPED, POOL_MEAN, POOL_STRIDE, AGG_SUM, AGG_MAX, SEL_TOPK,
    SEL_CUMMASS, ORDER_HRM_FIRST, ORDER_SCORE,
)
