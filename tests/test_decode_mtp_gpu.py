"""GPU parity of the multi-token query decode (query_len rows per sequence, each with its
own causal window) + reduce, through uq_paged_decode_mtp / uq_paged_reduce_mtp, against
the fp64 oracle."""

import copy

import numpy as np
import pytest

from quantized_paged_attention_amd import synth
from tests.gpu_util import (assert_decode_close, log, need_gpu, oracle_decode,
                            oracle_decode_seqs, run_decode)

pytestmark = pytest.mark.gpu

EDGE_LENS = (1, 2, 3, 4, 7, 255, 256, 257, 258, 259, 511, 1000, 3000)


def fp8(ql, qg, seed, lens=EDGE_LENS, hk=2, bs=16, **kw):
    return synth.make_fp8_case("mtp8", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               block_size=bs, spare_blocks=5, query_len=ql, **kw)


def fp4(ql, qg, seed, lens=EDGE_LENS, hk=2, kind="e4m3", **kw):
    return synth.make_fp4_case("mtp4", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               head_dim=256, block_size=64, rotate=True, spare_blocks=5,
                               scale_kind=kind, query_len=ql, **kw)


@pytest.mark.parametrize("ql,qg", [(2, 4), (4, 2), (3, 2), (8, 1), (2, 1)])
@pytest.mark.parametrize("P", [1, 4, 12])
def test_fp8_query_rows(ql, qg, P):
    need_gpu()
    case = fp8(ql, qg, seed=200 + 10 * ql + qg + P, k_scale=0.05, v_scale=0.02,
               values="uniform_codes")
    log(f"case fp8 mtp ql={ql} qg={qg} P={P}")
    got, _ = run_decode(case, P=P)
    assert got.shape == (case.B * ql, case.Hq, case.D)
    assert_decode_close(got, oracle_decode(case), f"fp8 mtp ql={ql} qg={qg} P={P}")


@pytest.mark.parametrize("ql,qg", [(2, 4), (4, 1)])
@pytest.mark.parametrize("P", [1, 12])
def test_fp8_query_rows_head_groups(ql, qg, P):
    """Query rows with Hk=4 (head-group workgroups)."""
    need_gpu()
    case = fp8(ql, qg, seed=260 + 10 * ql + qg + P, hk=4, k_scale=0.05, v_scale=0.02,
               values="uniform_codes")
    log(f"case fp8 mtp head groups ql={ql} qg={qg} P={P}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"fp8 mtp hg ql={ql} qg={qg} P={P}")


@pytest.mark.parametrize("kind", ["e4m3", "ue8m0"])
@pytest.mark.parametrize("ql,qg", [(2, 8), (4, 4), (2, 6), (4, 1), (3, 5)])
def test_fp4_query_rows(ql, qg, kind):
    need_gpu()
    case = fp4(ql, qg, seed=300 + 10 * ql + qg, kind=kind)
    log(f"case fp4 mtp ql={ql} qg={qg} scales={kind}")
    got, _ = run_decode(case, P=4)
    assert_decode_close(got, oracle_decode(case), f"fp4 mtp ql={ql} qg={qg} {kind}")


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_runs_ragged_batch(fmt):
    """A batch large enough for runs of several partitions per workgroup (merged into one
    partial), with lengths that end a row's window at every position of a run."""
    need_gpu()
    rng = np.random.default_rng(401)
    B = 32 if fmt == "fp8" else 16
    lens = rng.integers(1, 8193, size=B)
    lens[:8] = [1, 2, 3, 256, 257, 258, 1024, 8192]
    lens = tuple(int(x) for x in lens)
    if fmt == "fp8":
        case = fp8(4, 2, seed=402, lens=lens, hk=8, k_scale=0.05, v_scale=0.02)
        P = 32
    else:
        case = fp4(2, 8, seed=403, lens=lens, hk=2)
        P = 40
    log(f"case {fmt} mtp runs B={B}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"{fmt} mtp runs")


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_rows_without_tokens_are_zero(fmt):
    """Sequences shorter than query_len: the rows whose window is empty reduce to exactly
    0 and every other row is finite and matches."""
    need_gpu()
    ql = 4
    lens = (1, 2, 3, 300)
    case = fp8(ql, 2, seed=404, lens=lens) if fmt == "fp8" else fp4(ql, 4, seed=405, lens=lens)
    got, _ = run_decode(case, P=2)
    for b, L in enumerate(lens):
        for j in range(ql):
            if L - ql + 1 + j <= 0:
                assert np.all(got[b * ql + j] == 0), (b, j)
    assert_decode_close(got, oracle_decode(case), f"{fmt} mtp empty rows")


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_masked_bytes_bit_identical(fmt):
    """NaN codes in every slot past each sequence and in unused blocks leave the output
    bit for bit unchanged (per-row windows end inside blocks)."""
    need_gpu()
    lens = (3, 70, 129, 250, 513)
    case = fp8(3, 2, seed=406, lens=lens, bs=32) if fmt == "fp8" else fp4(2, 8, seed=407,
                                                                        lens=lens)
    base, _ = run_decode(case, P=2)
    assert np.isfinite(base).all()
    c2 = copy.deepcopy(case)
    used = np.zeros(c2.cache.shape[0], bool)
    for b, L in enumerate(c2.seq_lens):
        n = -(-int(L) // c2.block_size)
        used[c2.block_table[b, :n]] = True
        if L % c2.block_size:
            c2.cache[c2.block_table[b, L // c2.block_size], L % c2.block_size:] = 0x7F
        c2.block_table[b, n:] = 1 << 30
    c2.cache[~used] = 0xFF
    got, _ = run_decode(c2, P=2)
    assert np.array_equal(got, base)


def test_fp8_high_mtp_full():
    """The high-batch fp8 shape (B=128, L ~ U[4096, 16384], Hk=8) with 2 query rows x 4
    heads per kv head, at full size in the benchmark's launch configuration; every output
    row (both query rows of all 128 sequences) is compared with the oracle."""
    need_gpu()
    case = synth.fp8_high_mtp(2, 4)
    log(f"case fp8_high_mtp2_qg4 (full GPU run, full oracle) kv_bytes={case.kv_bytes()}")
    got, _ = run_decode(case)
    assert_decode_close(got, oracle_decode(case), "fp8_high_mtp")


@pytest.mark.parametrize("ql,qg", [(1, 16), (2, 8), (1, 12), (1, 32), (1, 64)])
def test_fp8_high_wide_groups_full(ql, qg):
    """The high-batch fp8 shape with 9-64 query rows per kv head (one f16 row tile of 16
    rows, two per wave, or two row slices per kv head), run at full size in the
    benchmark's launch configuration; every output row of every fourth sequence (32 of
    128, all their query rows and heads) is compared with the oracle."""
    need_gpu()
    case = synth.fp8_high_mtp(ql, qg)
    log(f"case fp8_high_mtp{ql}_qg{qg} (full GPU run, oracle on 32 sequences)")
    got, _ = run_decode(case)
    rows, ref = oracle_decode_seqs(case, np.arange(0, case.B, 4))
    assert_decode_close(got[rows], ref, f"fp8_high_mtp{ql}_qg{qg}")


@pytest.mark.parametrize("kind", ["e4m3", "ue8m0"])
def test_fp4_d256_mtp_full(kind):
    """B=4, Hk=2, L=75000, 512 partitions, 2 query rows x 8 heads (16 rows), rotation:
    the full output."""
    need_gpu()
    case = synth.fp4_d256_mtp(2, 8, kind)
    log(f"case fp4_d256_mtp2_qg8 scales={kind}")
    got, _ = run_decode(case)
    assert_decode_close(got, oracle_decode(case), f"fp4_d256_mtp {kind}")


@pytest.mark.parametrize("ql,qg,hk", [(2, 8, 2), (3, 5, 4), (4, 8, 4), (2, 16, 2)])
def test_fp8_query_rows_wide(ql, qg, hk):
    """Query rows x heads above 8: with hk = 2 (no head groups) two e4m3 row tiles of 8,
    and 32 rows in two passes; with hk = 4 f16 row tiles of 16 (15 rows in one, 32 in
    two)."""
    need_gpu()
    case = fp8(ql, qg, seed=280 + 10 * ql + qg + hk, hk=hk, k_scale=0.05, v_scale=0.02,
               values="uniform_codes", lens=(1, 2, 3, 7, 255, 256, 257, 1000))
    log(f"case fp8 mtp wide ql={ql} qg={qg} hk={hk}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"fp8 mtp wide ql={ql} qg={qg} hk={hk}")
