"""Seeded synthetic inputs for MLA paged decode.

This package is shared by the tests, the benchmark and the smoke check. It
draws inputs only: sequence lengths, the physical page placement, BF16 query
and cache values, and the poison patterns used by tests. It performs none of
the attention arithmetic; the oracle (under ``oracle/``) and the HIP library
(under ``mla_paged_kv_02_amd/``) each do that on their own.
"""

from .gen import (  # noqa: F401
    HEAD_DIM,
    HEAD_DIM_V,
    PAGE_SIZE,
    WORKLOADS,
    Workload,
    MlaInputs,
    bf16_round_bits,
    bf16_bits_to_f32,
    make_inputs,
    make_workload_inputs,
    permute_pages,
    poison_page_tails,
    poison_block_table_padding,
    AppendInputs,
    APPEND_WORKLOADS,
    make_append_inputs,
    make_append_workload,
    ABSORB_WORKLOADS,
    AbsorbInputs,
    make_absorb_inputs,
    make_absorb_workload,
    FP8_PAGE_BYTES,
    make_fp8_cache,
    pack_fp8_pages,
    MhaInputs,
    MHA_WORKLOADS,
    make_mha_inputs,
    make_mha_workload,
)
from .roofline import (  # noqa: F401
    algorithmic_bytes,
    algorithmic_bytes_fp8,
    algorithmic_flops,
    visible_lengths,
    MI355X_HBM_GBPS,
    MI355X_BF16_TFLOPS,
)
