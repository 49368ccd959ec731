"""Exact decoders for the stored number formats (oracle side; test infrastructure).

- bf16: the upper 16 bits of an IEEE float32; decoded exactly into float64.
- e4m3fn (OCP FP8, the "FP8 KV cache" of the HALOps README, Highlights): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, subnormals when the exponent field
  is 0, no infinities, and NaN for the all-ones exponent-and-mantissa pattern
  (0x7F / 0xFF). Largest finite magnitude: 1.75 * 2**8 = 448.

Both tables are written from the format definitions; nothing here is shared with
the HIP path.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def _build_e4m3fn_table():
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3FN_TABLE = _build_e4m3fn_table()


def e4m3fn_to_f64(codes):
    """uint8 e4m3fn codes -> float64 (exact)."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]

