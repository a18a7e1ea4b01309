"""Pins of the oracle's per-token-scaled fp8 decode (CPU).

Per-token mode of the pa_decode_tile PR (ROCm/FlyDSL #825, per_token_kv): every (token,
kv head) of the cache carries its own f32 K scale and V scale next to the e4m3 codes.
The scale tensors are [num_blocks, Hk, block_size], indexed by the token's physical
block, kv head and position in the block.

The references here do not re-type the oracle: torch's scaled_dot_product_attention
over a cache re-gathered and scaled with numpy fancy indexing, a one-hot gather that
must return exactly one token's scaled V row, the one-token closed form, and the
per-tensor special case of equal scales."""

import copy

import numpy as np
import pytest

from oracle import oracle
from quantized_paged_attention_amd import synth
from tests.refdense import dense_kv, sdpa_reference


def run(case, P=0):
    return oracle.decode(case.q, case.cache, case.block_table, case.seq_lens,
                         num_kv_heads=case.num_kv_heads, kv_format=case.kv_format,
                         softmax_scale=case.softmax_scale, k_scale=case.k_scale,
                         v_scale=case.v_scale, rot_signs=case.rot_signs, num_partitions=P,
                         query_len=case.query_len, k_scale_tok=case.k_scale_tok,
                         v_scale_tok=case.v_scale_tok)


def tok_case(seed=21, lens=(1, 15, 16, 17, 255, 256, 257, 700), hk=2, qg=4, bs=16, **kw):
    return synth.make_fp8_case("tok", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               block_size=bs, spare_blocks=5, scales="token", **kw)


@pytest.mark.parametrize("values,spread", [("normal", 0.75), ("uniform_codes", 0.5)])
@pytest.mark.parametrize("bs", [16, 64])
def test_per_token_matches_torch_sdpa(values, spread, bs):
    kw = dict(k_scale=0.05, v_scale=0.02) if values == "uniform_codes" else {}
    case = tok_case(values=values, tok_spread=spread, bs=bs, **kw)
    assert case.kv_format == oracle.FMT_FP8_E4M3_TOK
    got = run(case)
    want = sdpa_reference(case)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


def test_per_token_mtp_matches_torch_sdpa():
    case = tok_case(lens=(3, 40, 300), qg=2, values="normal", query_len=3, tok_spread=1.0)
    got = run(case)
    want = sdpa_reference(case)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


def test_per_token_v_ramp_matches_torch_sdpa():
    """V scales growing 2^(t/32) along each sequence (the GPU's running V reference is
    raised many times on such inputs)."""
    case = tok_case(lens=(700, 1000), values="normal", v_ramp=8.0)
    got = run(case)
    want = sdpa_reference(case)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


def test_single_token_returns_scaled_v_exactly():
    case = tok_case(lens=(1, 1, 1), values="uniform_codes", k_scale=0.05, v_scale=0.02)
    got = run(case)
    for b in range(case.B):
        blk = case.block_table[b, 0]
        for h in range(case.num_kv_heads):
            codes = case.cache[blk, 0, h, case.D:2 * case.D]
            from tests.refdense import e4m3_lib
            v0 = e4m3_lib(codes) * float(case.v_scale_tok[blk, h, 0])
            for g in range(case.QG):
                assert np.array_equal(got[b, h * case.QG + g], v0)


@pytest.mark.parametrize("bs", [16, 64])
def test_one_hot_gather_uses_the_tokens_own_scales(bs):
    """All K codes zero except token t* (K[0] = 448) and Q = 100 e0: every other weight
    underflows, so each head's output is exactly that token's V row times the V scale
    stored at [block of t*, head, position of t*]."""
    L = 3 * bs + 5
    case = tok_case(lens=(L,), hk=2, qg=2, bs=bs, values="normal")
    D = case.D
    case.q[:] = 0.0
    case.q[:, :, 0] = 100.0
    from tests.refdense import e4m3_lib
    for tstar in sorted({0, bs - 1, bs, 2 * bs + 3, L - 1}):
        c = copy.deepcopy(case)
        c.cache[..., :D] = 0
        blk = c.block_table[0, tstar // bs]
        pos = tstar % bs
        c.cache[blk, pos, :, 0] = 0x7E                   # 448 in both heads
        c.k_scale_tok[blk, :, pos] = 1.0
        got = run(c)
        for h in range(2):
            want = e4m3_lib(c.cache[blk, pos, h, D:2 * D]) * float(c.v_scale_tok[blk, h, pos])
            for g in range(2):
                assert np.array_equal(got[0, h * 2 + g], want), (tstar, h)


def test_equal_per_token_scales_equal_per_tensor_scales():
    """Every per-token scale equal to (ck, cv): the result is the per-tensor decode with
    k_scale = ck, v_scale = cv (an SDPA-pinned mode)."""
    case = tok_case(lens=(37, 300), values="uniform_codes", k_scale=0.05, v_scale=0.02)
    case.k_scale_tok[:] = np.float32(0.0625)
    case.v_scale_tok[:] = np.float32(0.03125)
    got = run(case)
    pt = copy.deepcopy(case)
    pt.kv_format, pt.k_scale, pt.v_scale = synth.FMT_FP8_E4M3, 0.0625, 0.03125
    pt.k_scale_tok = pt.v_scale_tok = None
    want = sdpa_reference(pt)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("P", [1, 3, 64])
def test_per_token_partials_reduce_to_full_output(P):
    case = tok_case(lens=(0, 1, 256, 257, 1000), values="normal")
    full, (pm, pl, po) = run(case, P)
    red = oracle.reduce(po, pm, pl, case.seq_lens)
    np.testing.assert_allclose(red, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())
