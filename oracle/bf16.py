"""bfloat16 rounding for the oracle.

Test infrastructure (see ``oracle/__init__``).

The two-layer bf16 network rounds the first layer's float32 output to
bfloat16 before the second layer reads it; the oracle does the same rounding
at the same place.  bfloat16 is the top 16 bits of an IEEE float32; the cast
rounds to nearest with ties to even on the dropped 16 bits.
"""

import numpy as np


def round_bf16(a):
    """Round to the nearest bfloat16 (ties to even); returns float64 values.

    The input is first rounded to float32 (nearest even, NumPy's cast), then
    the low 16 bits of the float32 pattern are rounded away.  NaN stays NaN.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    out = np.where(np.isnan(f), np.float32(np.nan), out)
    return out.astype(np.float64)
