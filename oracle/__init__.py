"""CPU oracle for exact attention, in float64.

TEST INFRASTRUCTURE. This package is the slow, plain, obviously-correct
definition that the GPU path is checked against. Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import, call or run
anything in it. The product path (the HIP library and its Python binding)
never imports it and shares no code with it.

Every function materialises the score matrix S and the probability matrix P
for the rows it is asked about, exactly as the pages describe standard
attention, and works in float64 throughout.
"""

from .exact import (  # noqa: F401
    scores,
    visible,
    alibi_bias,
    attention_rows,
    attention,
    attention_dropout,
    attention_bwd,
    attention_varlen,
    attention_varlen_bwd,
    decode,
    decode_paged,
    partial,
    merge,
    finalize,
)
from .dropout import philox4x32, drop_threshold, keep_mask, keep_scale  # noqa: F401,E402
