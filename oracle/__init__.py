"""Float64 CPU oracle for absorbed-MLA decode.

TEST INFRASTRUCTURE ONLY: imported by tests, by the package smoke check and by
the benchmark's CPU-baseline leg.  The product path never imports it."""

from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (absorb_q, absorbed_layer, attention_probs, bf16_to_f64,  # noqa: F401
                         cache_elements_per_token, combine_lse, decode_case_rows,
                         e4m3fn_to_f64, mha_mode_layer, mqa_decode_case, mqa_decode_rows,
                         paged_rows, project, rope, up_proj_v)
