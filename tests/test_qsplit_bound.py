"""The fp8 decode carries a bf16 query as an e4m3 hi + lo pair after scaling each row by a
power of two s_q that puts its largest magnitude amax in [64, 128).  This pins what that
split keeps, with torch's own e4m3 cast (round to nearest even) as the rounding:

  * every bf16 element of magnitude >= 2^-2 / s_q is reproduced exactly by hi + lo;
  * every smaller element is off by at most 2^-10 / s_q <= 2^-16 amax (the lo term lands
    on the e4m3 subnormal grid of step 2^-9), and some are off by more than zero, so the
    pair is not exact for every bf16 query.

Every positive finite bf16 value up to amax is checked for several amax."""

import numpy as np
import pytest
import torch


def all_bf16_up_to(amax: float) -> torch.Tensor:
    bits = torch.arange(1, 0x7F80, dtype=torch.int32).to(torch.int16)   # positive finite
    vals = bits.view(torch.bfloat16).float()
    return vals[vals <= amax]


def row_scale(amax: float) -> float:
    # s_q = 2^(7 - E) with amax = f 2^E, f in [0.5, 1)
    _, e = np.frexp(np.float32(amax))
    return float(2.0 ** (7 - int(e)))


def split(y: torch.Tensor):
    hi = y.to(torch.float8_e4m3fn).float()
    lo = (y - hi).to(torch.float8_e4m3fn).float()
    return hi, lo


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4040, 0x3C23, 0x43E0, 0x3F7F, 0x2E80])
def test_hi_lo_split_exact_above_quarter_and_bounded_below(amax_bits):
    amax = float(torch.tensor([amax_bits], dtype=torch.int16).view(torch.bfloat16).float())
    s_q = row_scale(amax)
    assert 64.0 <= amax * s_q < 128.0
    x = all_bf16_up_to(amax)
    y = x * s_q                     # exact: power-of-two scale of a bf16 value
    hi, lo = split(y)
    err = (hi + lo - y).abs()       # fp32 sums of two e4m3 values near y: exact
    big = y >= 0.25
    assert big.any() and (~big).any()
    assert torch.all(err[big] == 0), "the pair must be exact for |y| >= 2^-2"
    assert float(err.max()) <= 2.0 ** -10
    # in units of the row: |x - (hi + lo) / s_q| <= 2^-16 amax
    assert float((err / s_q).max()) <= 2.0 ** -16 * amax
    # and the loss below the threshold is real: not every bf16 query is exact
    assert float(err[~big].max()) > 0.0
