"""Pins of the oracle's multi-token query decode (query_len > 1) and its flash-combine
(CPU).

Query row j of sequence b sees the tokens t <= L_b - QL + j (the causal window of each
query row in the FlyDSL "pa_decode_tile" page's MTP path).  The references are torch's
scaled_dot_product_attention with an explicit boolean mask over a densely re-gathered
cache, the single-query decode of the same cache cut to the row's window, and the
reduce of the row's own partitions."""

import copy

import numpy as np
import pytest

from oracle import oracle
from quantized_paged_attention_amd import synth
from tests.refdense import sdpa_reference

LENS = (1, 2, 3, 4, 5, 255, 256, 257, 258, 259, 513, 700)


def run(case, P=0):
    return oracle.decode(case.q, case.cache, case.block_table, case.seq_lens,
                         num_kv_heads=case.num_kv_heads, kv_format=case.kv_format,
                         softmax_scale=case.softmax_scale, k_scale=case.k_scale,
                         v_scale=case.v_scale, rot_signs=case.rot_signs, num_partitions=P,
                         query_len=case.query_len)


def fp8_case(ql, qg=2, seed=31, lens=LENS, **kw):
    return synth.make_fp8_case("mtp8", seed + ql, seq_lens=list(lens), num_kv_heads=2, qg=qg,
                               block_size=16, spare_blocks=4, query_len=ql, **kw)


def fp4_case(ql, qg=4, seed=41, lens=LENS, kind="e4m3"):
    return synth.make_fp4_case("mtp4", seed + ql, seq_lens=list(lens), num_kv_heads=2, qg=qg,
                               head_dim=256, block_size=64, scale_kind=kind, rotate=True,
                               spare_blocks=3, query_len=ql)


@pytest.mark.parametrize("ql", [2, 3, 4])
@pytest.mark.parametrize("values,ks,vs", [("normal", 1.0, 1.0), ("uniform_codes", 0.05, 0.02)])
def test_fp8_mtp_matches_masked_sdpa(ql, values, ks, vs):
    case = fp8_case(ql, values=values, k_scale=ks, v_scale=vs)
    got = run(case)
    want = sdpa_reference(case)
    assert got.shape == (case.B * ql, case.Hq, case.D)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("ql", [2, 4])
@pytest.mark.parametrize("kind", ["e4m3", "ue8m0"])
def test_fp4_mtp_matches_masked_sdpa(ql, kind):
    case = fp4_case(ql, kind=kind)
    got = run(case)
    want = sdpa_reference(case)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("ql", [2, 3, 4])
def test_row_is_single_query_decode_of_its_window(ql):
    """Row j of sequence b equals a one-query decode of the same cache and table with
    length L_b - QL + 1 + j (zero when that is not positive)."""
    case = fp8_case(ql, values="normal")
    got = run(case)
    for j in range(ql):
        one = copy.deepcopy(case)
        one.query_len = 1
        one.q = case.q[j::ql].copy()
        one.seq_lens = np.maximum(case.seq_lens - ql + 1 + j, 0).astype(np.int32)
        want = run(one)
        np.testing.assert_array_equal(got[j::ql], want)


@pytest.mark.parametrize("ql", [2, 4])
@pytest.mark.parametrize("P", [1, 2, 3])
def test_partials_reduce_to_output(ql, P):
    """Each row's partitions (m, l, o), combined by the reduce, give the row's output;
    rows of a partition past their window are empty (m = -inf, l = 0)."""
    case = fp8_case(ql, values="normal")
    out, (pm, pl, po) = run(case, P)
    assert pm.shape == (case.B, case.num_kv_heads, P, ql * case.QG)
    red = oracle.reduce(po, pm, pl, case.seq_lens, query_len=ql)
    np.testing.assert_allclose(red, out, rtol=1e-12, atol=1e-14)
    empty = pl == 0
    assert np.all(pm[empty] == -np.inf)
    # the first sequence (L = 1) has tokens only for its last query row
    assert np.all(empty[0, :, :, :(ql - 1) * case.QG])
    assert not np.any(empty[0, :, 0, (ql - 1) * case.QG:])


def test_rows_without_tokens_are_zero():
    ql = 4
    case = fp8_case(ql, values="normal", lens=(1, 2, 3, 600))
    got = run(case)
    for b, L in enumerate(case.seq_lens):
        for j in range(ql):
            row = got[b * ql + j]
            if L - ql + 1 + j <= 0:
                assert np.all(row == 0)
            else:
                assert np.any(row != 0)


def test_query_len_one_is_the_decode():
    case = fp8_case(1, values="normal")
    got = run(case)
    np.testing.assert_allclose(got, sdpa_reference(case), rtol=1e-10, atol=1e-12)
