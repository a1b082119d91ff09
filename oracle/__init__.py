"""CPU oracle for the KDA (Kimi Delta Attention / gated delta rule) decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may import, call or
execute this package; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP path
(``linear_attention_decode_amd``): the only module both sides use is ``synth``, which
draws seeded random inputs and holds none of the method's arithmetic.

Everything is plain numpy in float64, one token at a time, in the order the pages give
the step.  A library matrix-vector / matrix-matrix product serves as the projection
step; there is no blocking, fusion or reordering beyond that.

Pins (tests/test_oracle_*.py) tie each function to something other than itself; see
the docstring of each function for the pin that covers it.
"""
from .kda import (  # noqa: F401
    OracleLayer,
    bf16_round,
    q8_0_quantize,
    q8_0_dequantize,
    prepare_layer,
    layer_step,
    stack_step,
    rms_norm,
    decode_run,
    verify_run,
    prefill_run,
    silu,
    sigmoid,
    softplus,
)
