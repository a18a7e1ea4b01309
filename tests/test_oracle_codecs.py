"""Pins of the oracle's closed-form code decoders (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import oracle
from tests.refdense import E2M1_SPEC, golden


def test_e4m3_all_codes_match_torch_float8():
    """All 256 e4m3 codes against torch's float8_e4m3fn cast (independent library)."""
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got = oracle.e4m3(c)
        want = float(lib[c])
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), c


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0),            # largest finite
    (0x08, 2.0 ** -6),        # smallest normal
    (0x01, 2.0 ** -9),        # smallest subnormal
    (0x07, 7 * 2.0 ** -9),    # largest subnormal
    (0x38, 1.0),
    (0x40, 2.0),
    (0x3C, 1.5),
    (0xC0, -2.0),
    (0x00, 0.0),
])
def test_e4m3_ocp_anchors(code, value):
    """OCP 8-bit floating point (OFP8) E4M3 anchors: bias 7, max 448, no infinities."""
    assert oracle.e4m3(code) == value


def test_e4m3_nan_and_structure():
    assert math.isnan(oracle.e4m3(0x7F)) and math.isnan(oracle.e4m3(0xFF))
    pos = [oracle.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "positive codes must be increasing"
    for c in range(0x7F):
        assert oracle.e4m3(c | 0x80) == -oracle.e4m3(c)


def test_e2m1_spec_grid():
    """OCP FP4 E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit."""
    for n in range(16):
        assert oracle.e2m1(n) == E2M1_SPEC[n], n
    assert sorted({abs(oracle.e2m1(n)) for n in range(16)}) == [0, .5, 1, 1.5, 2, 3, 4, 6]


def test_ue8m0():
    """UE8M0 scale 2^(b-127); the page's zero sentinel for byte 0; 255 is NaN."""
    assert oracle.ue8m0(127) == 1.0 and oracle.ue8m0(128) == 2.0 and oracle.ue8m0(126) == 0.5
    assert oracle.ue8m0(0) == 0.0 and math.isnan(oracle.ue8m0(255))
    for b in range(1, 255):
        assert oracle.ue8m0(b) == float(np.ldexp(1.0, b - 127))


def test_slot_content_matches_page_layout():
    lay = golden("p1_fp4_slot_layout.txt")
    assert oracle.slot_content_bytes(1, lay["head_dim"]) == lay["content_bytes"]
    assert oracle.slot_content_bytes(2, lay["head_dim"]) == lay["content_bytes"]
    assert oracle.slot_content_bytes(0, 128) == 256


def test_page_kv_byte_count():
    """81.6 MB of KV at batch 4 / 75k tokens / one kv head (FP4 D=256 page)."""
    g = golden("p1_kv_bytes.txt")
    lay = golden("p1_fp4_slot_layout.txt")
    total = g["batch"] * g["seq_len"] * g["kv_heads"] * oracle.slot_content_bytes(1, 256)
    assert abs(total / 1e6 - g["megabytes"]) < 0.05
    assert lay["content_bytes"] == oracle.slot_content_bytes(1, 256)
