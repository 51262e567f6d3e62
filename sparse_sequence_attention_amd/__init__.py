"""MI355X (gfx950) Semi-Local Attention: HSTU pointwise SiLU attention over
jagged sequences under the ULTRA-HSTU semi-local mask, its backward, the STU
layer around it and attention truncation, as hand-written HIP kernels behind a
C ABI (include/sla.h).  This package is the Python binding of that library.
"""
from ._capi import (  # noqa: F401
    SLAError, SLA_OP_FWD, SLA_OP_BWD, SLA_OP_BWD_RECOMPUTE, SLA_NOALLOC_SCRATCH_BYTES, SLA_SCHED_RECORD_INTS, SLA_BWD_ALL, SLA_BWD_PREPARE,
    SLA_BWD_DKDV, SLA_BWD_DQ,
)
from .config import STUConfig  # noqa: F401
from .ops import (  # noqa: F401
    sla_fwd, sla_fwd_candidates, sla_bwd, sla_bwd_noalloc, sla_attention, sla_schedule, sla_schedule_host, schedule_tile, count_pairs_host, ds_blocks_host,
    probe_issue_rates,
    probe_mfma_peak,
    stu_layer_fwd, stu_layer_bwd, stu_layer_workspace_bytes, stu_quantize_rows_fp8,
    stu_layer_fwd_fp8, stu_gather_targets, stu_truncate, stu_truncate_bwd, make_problem,
    workspace_size,
)
from .stack import MoTChannel, STULayerWeights, mot_fwd, stu_stack_bwd, stu_stack_fwd  # noqa: F401
