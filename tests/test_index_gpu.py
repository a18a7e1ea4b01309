"""GPU parity of the nvfp4 index scorer against the fp64 oracle: finite cells within
1e-4 of max|ref|, -inf cells exactly, cells past each request's pages bit-identical to
the NaN-payload pre-fill."""

import copy

import numpy as np
import pytest
import torch

from quantized_paged_attention_amd import synth
from tests.gpu_util import DEV, TOL_INDEX, log, need_gpu, uq

pytestmark = pytest.mark.gpu


def run_gpu(case, q=None, pages=None):
    q = q if q is not None else torch.from_numpy(case.q).to(DEV)
    pages = pages if pages is not None else torch.from_numpy(case.pages).to(DEV)
    bt = torch.from_numpy(case.block_table).to(DEV)
    sl = torch.from_numpy(case.seq_lens).to(DEV)
    scores = torch.from_numpy(case.scores_init().copy()).to(DEV)
    uq.index_score(q, pages, bt, sl, scores, query_len=case.query_len)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def run_oracle(case):
    from oracle import oracle
    return oracle.index_score(case.q, case.pages, case.block_table, case.seq_lens,
                              query_len=case.query_len, scores_init=case.scores_init())


def assert_index_match(got, ref, init, what):
    ref_bits = init.view(np.uint32)
    untouched = np.isnan(ref)
    # untouched cells: the pre-fill bit pattern, exactly
    assert np.array_equal(got.view(np.uint32)[untouched], ref_bits[untouched]), f"{what}: untouched"
    neg = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), neg), f"{what}: -inf cells"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite where the oracle is finite"
    scale = np.abs(ref[fin]).max() if fin.any() else 1.0
    err = float(np.abs(got[fin].astype(np.float64) - ref[fin]).max() / scale) if fin.any() else 0.0
    log(f"  {what}: max|err|/max|ref| = {err:.3e} over {int(fin.sum())} cells")
    assert err <= TOL_INDEX, f"{what}: {err:.3e} > {TOL_INDEX}"


@pytest.mark.parametrize("ql,h", synth.INDEX_COMBOS)
def test_index_config(ql, h):
    """32 requests, L ~ U[1024, 32768], D=128, every (query_len, heads) combination."""
    need_gpu()
    case = synth.nvfp4_index(ql, h)
    log(f"case nvfp4_index ql={ql} h={h} page_bytes={case.page_bytes()}")
    got = run_gpu(case)
    assert_index_match(got, run_oracle(case), case.scores_init(), f"ql={ql} h={h}")


@pytest.mark.parametrize("ql,h", [(1, 1), (4, 2), (8, 4), (2, 4)])
def test_edge_lengths(ql, h):
    """Lengths on and around page edges, including L = QL (the first rows see nothing of
    the only page beyond the first tokens)."""
    need_gpu()
    lens = [max(L, ql) for L in (1, 2, 8, 127, 128, 129, 255, 256, 257, 1000)]
    case = synth.make_index_case("idx_edges", 100 + ql * h, seq_lens=lens, query_len=ql,
                                 heads=h, max_pages=12)
    got = run_gpu(case)
    assert_index_match(got, run_oracle(case), case.scores_init(), f"edges ql={ql} h={h}")


def test_strided_query_and_padded_pages():
    """Query rows taken from a wider buffer (byte strides) and pages padded past 9216."""
    need_gpu()
    case = synth.make_index_case("idx_stride", 120, seq_lens=[300, 900, 129], query_len=2,
                                 heads=2, page_stride=9216 + 256, max_pages=10)
    R, H, D = case.q.shape
    wide = torch.zeros(R, H + 1, D + 64, dtype=torch.uint8)
    wide[:, :H, :D] = torch.from_numpy(case.q)
    q = wide.to(DEV)[:, :H, :D]
    got = run_gpu(case, q=q)
    assert_index_match(got, run_oracle(case), case.scores_init(), "strided")


def test_max_blocks_truncates():
    """A score row shorter than the request's page count: pages b >= S are not written."""
    need_gpu()
    case = synth.make_index_case("idx_trunc", 121, seq_lens=[2000, 700], query_len=1, heads=1,
                                 max_pages=16)
    full = run_oracle(case)
    short = copy.deepcopy(case)
    short.max_pages = 5
    got = run_gpu(short)
    assert got.shape[2] == 5
    assert_index_match(got, full[:, :, :5], short.scores_init(), "truncated")


def test_page_permutation_bit_identical():
    need_gpu()
    case = synth.make_index_case("idx_perm", 122, seq_lens=[500, 1300, 64], query_len=4,
                                 heads=2, max_pages=12)
    base = run_gpu(case)
    rng = np.random.default_rng(5)
    perm = rng.permutation(case.pages.shape[0])
    c2 = copy.deepcopy(case)
    c2.pages = np.empty_like(case.pages)
    c2.pages[perm] = case.pages
    c2.block_table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)],
                              -1).astype(np.int32)
    got = run_gpu(c2)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("ql,h", [(1, 1), (4, 2), (8, 4)])
def test_shared_prefix_pages(ql, h):
    """Requests whose first 64 pages are the same physical pages (a shared prefix): the
    result matches the oracle and is bit-identical to the same table pointing at private
    copies of those pages."""
    need_gpu()
    base = synth.make_index_case("shared", 77 + ql + h,
                                 seq_lens=np.random.default_rng(ql * 10 + h).integers(
                                     64 * 128 + 1, 20000, size=40).astype(np.int32),
                                 query_len=ql, heads=h, page_stride=9216)
    case = synth.index_shared_prefix(base, 64)
    log(f"case nvfp4_index shared prefix ql={ql} h={h} reqs={case.num_reqs}")
    got = run_gpu(case)
    assert_index_match(got, run_oracle(case), case.scores_init(), f"shared ql={ql} h={h}")
    # private copies: every request's prefix entries point at its own copy of the pages
    priv = copy.deepcopy(case)
    nref = case.pages.shape[0]
    extra = []
    for r in range(1, case.num_reqs):
        ids = case.block_table[r, :64]
        new_ids = nref + len(extra) + np.arange(64)
        extra.extend(case.pages[i] for i in ids)
        priv.block_table[r, :64] = new_ids
    priv.pages = np.concatenate([case.pages, np.stack(extra)], axis=0)
    got_priv = run_gpu(priv)
    assert np.array_equal(got.view(np.uint32), got_priv.view(np.uint32))


def test_shared_pages_across_windows_and_partial():
    """70 requests (two 64-request windows) sharing pages in irregular places: some
    requests share a page only at one block index, the shared last page of a request is
    partly visible, and requests in different windows share pages too."""
    need_gpu()
    rng = np.random.default_rng(123)
    lens = rng.integers(300, 3000, size=70).astype(np.int32)
    case = synth.make_index_case("shared_irreg", 124, seq_lens=lens, query_len=2, heads=2,
                                 page_stride=9216)
    bt = case.block_table
    for r in range(1, 70):
        if r % 3 == 0:           # share block 0 with the previous request
            bt[r, 0] = bt[r - 1, 0]
        if r % 5 == 0 and lens[r] > 128 and lens[r - 5] > 128:   # share block 1 with r - 5
            bt[r, 1] = bt[r - 5, 1]
    # request 69 maps request 1's pages at its first blocks (different windows)
    n = min(-(-int(lens[1]) // 128), -(-int(lens[69]) // 128)) - 1
    bt[69, :n] = bt[1, :n]
    log("case nvfp4_index irregular sharing, 70 requests")
    got = run_gpu(case)
    assert_index_match(got, run_oracle(case), case.scores_init(), "irregular sharing")


@pytest.mark.parametrize("ql,h", [(17, 1), (10, 2), (5, 4), (6, 4), (7, 4), (16, 2), (32, 1)])
def test_wide_column_counts(ql, h):
    """17-32 query columns (H * QL), each a 32 x 32 output tile, at counts other than 8 x 4:
    columns past H * QL unused, 21 requests whose pages meet inside workgroups, an empty
    request and page-edge lengths, the query rows taken from a wider buffer."""
    need_gpu()
    rng = np.random.default_rng(150 + ql * h + ql)
    lens = [max(ql, int(x)) for x in rng.integers(1, 3001, size=21)]
    lens[3], lens[7], lens[11], lens[12] = 0, ql, 128, 129
    case = synth.make_index_case("idx_wide", 151 + ql * h + ql, seq_lens=lens, query_len=ql,
                                 heads=h, max_pages=24)
    R, H, D = case.q.shape
    wide = torch.zeros(R, H + 1, D + 64, dtype=torch.uint8)
    wide[:, :H, :D] = torch.from_numpy(case.q)
    log(f"case index wide columns ql={ql} h={h}")
    got = run_gpu(case, q=wide.to(DEV)[:, :H, :D])
    assert_index_match(got, run_oracle(case), case.scores_init(), f"wide ql={ql} h={h}")


@pytest.mark.parametrize("R", [60, 300])
def test_many_requests_with_empty_ones(R):
    """Lengths from 0 to 3000.  60 requests: one wave per live page of the list built from
    the lengths, request boundaries anywhere; 300 requests (past the 64 lengths a wave
    holds): one wave per (request, page slot), the table read only for live pages."""
    need_gpu()
    rng = np.random.default_rng(130 + R)
    lens = rng.integers(1, 3001, size=R)
    lens[::23] = 0
    lens[1] = 1
    case = synth.make_index_case("idx_many", 131 + R, seq_lens=[int(x) for x in lens],
                                 query_len=1, heads=2, max_pages=24)
    got = run_gpu(case)
    assert_index_match(got, run_oracle(case), case.scores_init(), f"{R} requests")


@pytest.mark.parametrize("R,ql,h", [(64, 1, 1), (64, 8, 4), (64, 5, 4), (512, 1, 1)])
def test_long_page_lists(R, ql, h):
    """Requests of ~38k tokens whose tables all point at the same 300 pages.  64 requests:
    19k live pages, more than the waves of one launch, so each wave loops over several
    entries of the list (with 17-32 query columns every wave of a workgroup makes the same
    number of calls, those past the list idle); 512 requests: 150k page slots, one wave
    each."""
    need_gpu()
    base = synth.make_index_case("idx_long", 140, seq_lens=[300 * 128], query_len=1, heads=1,
                                 spare_pages=2)
    lens = np.array([300 * 128 - (r % 200) for r in range(R)], np.int32)
    rng = np.random.default_rng(141 + R + ql)
    q = synth.e4m3_encode(rng.standard_normal((R * ql, h, 128), dtype=np.float32))
    case = synth.IndexCase("idx_long", q, base.pages, np.repeat(base.block_table, R, axis=0),
                           lens, ql, h, 300)
    got = run_gpu(case)
    assert_index_match(got, run_oracle(case), case.scores_init(), f"long lists R={R} ql={ql}")
