"""Rows that see a few keys: the float32 model of the decode kernel's rounding
(tests/decode_rounding.py) over random two- to four-key rows with values spread over
[-6, 6] (CPU).

With P rounded to bf16 and nothing else, the weights of a row dominated by two or
three keys keep their 2^-9 relative rounding error, which can push the output past the
contract's 1e-2. With the low part of P multiplied into V on such chunks (as the
kernel does whenever a weight may exceed a quarter of its row's sum), every sampled row
stays within the tolerance and no error exceeds the bf16 output rounding of its value.
fp16 weights (2^-12 relative; the FP8-KV path) meet the bf16 tolerance without a low
part.
"""

import numpy as np
import pytest

from tests.decode_rounding import search_rows

SCALE = 1.0 / np.sqrt(128.0)


@pytest.mark.parametrize("keys", [2, 3, 4])
def test_low_part_keeps_few_key_rows_within_tolerance(keys):
    r = search_rows(SCALE, keys=keys, samples=300_000, seed=keys)
    # bf16 weights alone leave some rows past the tolerance ...
    assert r["max_excess_plain_all"] > 0
    # ... the low part keeps every row inside it, at least 2e-3 from its edge; fp16
    # weights (the FP8-KV path, whose own tolerance is 3e-2) at least 1e-3 from it.
    assert r["max_excess_low_all"] < -2e-3
    assert r["max_excess_f16_all"] < -1e-3
    # On the rows worst for bf16 weights the error drops to about the output's own
    # rounding (half a bf16 ulp, plus the low part's ~2^-16 relative remainder).
    _, e = np.frexp(np.abs(r["ref"]))
    half_ulp = np.ldexp(1.0, e - 9)
    assert np.all(r["err_low"] <= half_ulp + 2.0 ** -14 * np.abs(r["ref"]) + 1e-6)
