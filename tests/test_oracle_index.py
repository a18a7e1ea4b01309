"""Pins of the oracle's nvfp4 index scorer (CPU): a numpy brute-force per-page max over
pages decoded at the page's byte offsets, closed-form single-token pages, the QL=1
reduction to a plain page max, permutation invariance and untouched cells."""

import copy

import numpy as np
import pytest

from oracle import oracle
from quantized_paged_attention_amd import synth
from tests.refdense import e4m3_lib, golden, index_reference, unpack_e2m1


def small_index(ql=2, h=2, lens=(1, 127, 128, 129, 300, 1000), seed=21):
    lens = [max(L, ql) for L in lens]
    return synth.make_index_case("idx_small", seed, seq_lens=lens, query_len=ql, heads=h,
                                 max_pages=12)


def run(case, init=None):
    init = case.scores_init() if init is None else init
    return oracle.index_score(case.q, case.pages, case.block_table, case.seq_lens,
                              query_len=case.query_len, scores_init=init)


@pytest.mark.parametrize("ql,h", [(1, 1), (2, 2), (4, 1), (8, 4), (1, 4)])
def test_index_matches_bruteforce(ql, h):
    case = small_index(ql, h)
    got = run(case)
    want = index_reference(case)
    written = ~np.isnan(want)
    assert np.array_equal(written, ~np.isnan(got))
    assert np.array_equal(got[written], want[written])


def test_page_layout_constants():
    lay = golden("p2_index_page_layout.txt")
    assert lay["tokens_per_page"] * (lay["code_bytes_per_token"] + lay["scale_bytes_per_token"]) \
        == lay["page_bytes"]
    assert lay["tile_tokens"] * lay["code_bytes_per_token"] == lay["tile_code_stride"]
    assert lay["tokens_per_page"] * lay["code_bytes_per_token"] == lay["scale_region_offset"]
    assert lay["tile_tokens"] * lay["scale_bytes_per_token"] == lay["tile_scale_stride"]


def test_single_visible_token_page_is_its_dot_product():
    """L = 128 b + 1 with QL = 1: page b has one visible token, whose exact dot product
    (decoded at the page offsets) is the score."""
    case = small_index(1, 1, lens=(129, 257))
    got = run(case)
    lay = golden("p2_index_page_layout.txt")
    for r, L in enumerate(case.seq_lens):
        b = int(L) // 128
        pg = case.pages[case.block_table[r, b]]
        k = unpack_e2m1(pg[None, :64])[0] * np.repeat(
            e4m3_lib(pg[lay["scale_region_offset"]:lay["scale_region_offset"] + 8]), 16)
        assert got[0, r, b] == float(k @ e4m3_lib(case.q[r, 0]))


def test_ql1_is_plain_page_max():
    case = small_index(1, 2, lens=(500, 1024))
    got = run(case)
    q = e4m3_lib(case.q)
    lay = golden("p2_index_page_layout.txt")
    for r, L in enumerate(case.seq_lens):
        for b in range(-(-int(L) // 128)):
            pg = case.pages[case.block_table[r, b]]
            n = min(128, int(L) - 128 * b)
            k = unpack_e2m1(pg[:128 * 64].reshape(128, 64)) * np.repeat(
                e4m3_lib(pg[8192:8192 + 1024].reshape(128, 8)), 16, axis=1)
            for h in range(2):
                assert got[h, r, b] == max(float(k[t] @ q[r, h]) for t in range(n))
    assert lay["page_bytes"] == 9216


def test_causal_rows_see_fewer_tokens():
    """Row j of a request sees tokens t <= L - QL + j: with L = 128 b + QL - 1, row 0's
    last page holds no visible token (-inf) while the last row sees QL - 1 of them."""
    ql = 4
    case = small_index(ql, 1, lens=(128 + ql - 1,))
    got = run(case)
    assert got[0, 0, 1] == -np.inf
    assert np.isfinite(got[0, ql - 1, 1])


def test_permutation_invariance_and_untouched_cells():
    case = small_index(2, 2)
    base = run(case)
    rng = np.random.default_rng(3)
    perm = rng.permutation(case.pages.shape[0])
    c2 = copy.deepcopy(case)
    c2.pages = np.empty_like(case.pages)
    c2.pages[perm] = case.pages
    c2.block_table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)],
                              -1).astype(np.int32)
    got = run(c2)
    assert np.array_equal(np.isnan(got), np.isnan(base))
    assert np.array_equal(got[~np.isnan(got)], base[~np.isnan(base)])
    # cells of pages >= ceil(L/128) keep the pre-fill
    for r, L in enumerate(case.seq_lens):
        nb = -(-int(L) // 128)
        assert np.all(np.isnan(base[:, r * 2:(r + 1) * 2, nb:]))
