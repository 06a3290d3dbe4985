"""CPU oracle for one EP rank's MoE-layer share.

TEST INFRASTRUCTURE ONLY: imported solely by the tests, the smoke check and
the benchmark's CPU-baseline leg. It shares no code with the HIP path.

moe_share: the share itself (routing, layout, schedule, segments, FFN,
transfer, weighted reduction). partition: the per-layer CU-split model.
"""
from .moe_share import (  # noqa: F401
    widen_bf16, route, local_histogram, counts_layout, row_layout, group_order, gather_rows,
    tile_schedule, segments, silu, expert_ffn, expert_outputs, combine_transfer,
    weighted_reduction, oracle_share, token_rows, Layout, Bands, Segments, ShareResult,
)
from .partition import Calib, Partition, partition_model, segment_bands, gemm_row_tiles  # noqa: F401
