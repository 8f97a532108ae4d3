"""Plain FP64 CPU oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
load this package: only the tests, the smoke check and the benchmark's CPU
baseline use it. It shares no code with the HIP library and imports nothing
from it.

Every function here is the plain definition of what MLA decode computes,
written out in numpy float64 (or pure Python for the brute-force check).
Pins that tie it to the pages and to mathematics live in
``tests/test_oracle_pins.py``; there is no function here without a pin.
"""

from .mla_ref import (  # noqa: F401
    bf16_bits_to_f64,
    gather_sequence_rows,
    visible_length,
    attend_rows,
    mla_decode_ref,
    mla_decode_ref_f64,
    lse_combine_ref,
    mla_nonabsorbed_ref,
    mla_decode_bruteforce,
)
from .kv_append_ref import kv_append_ref  # noqa: F401
from .absorb_ref import absorb_q_ref, absorb_o_ref  # noqa: F401
from .fp8_ref import (  # noqa: F401
    e4m3_value,
    e4m3_decode,
    quantize_e4m3_rows,
    dequantize_fp8_cache,
    mla_decode_fp8_ref,
    kv_append_fp8_ref,
)
from .mha_ref import mha_decode_ref, mha_decode_bruteforce  # noqa: F401
