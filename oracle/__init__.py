"""CPU oracle for frame-aligned attention (test infrastructure only).

Only tests/, the smoke check and bench.py's CPU-baseline leg may import this
package.  The product package never does.
"""
from .oracle import (  # noqa: F401
    Problem,
    attn,
    attn_rows,
    build,
    count,
    e4m3_decode,
    e4m3_encode,
    kmean,
    quant_e4m3,
    quant_int8,
    threads,
    FAO_TGT,
    FAO_SRC,
    FAO_REF,
)
