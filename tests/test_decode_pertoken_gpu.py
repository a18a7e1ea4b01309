"""GPU parity of the fp8 decode with per-token K/V scales (kv format
UQ_KV_FP8_E4M3_TOKSCALE; per_token_kv mode of the pa_decode_tile PR, ROCm/FlyDSL #825)
against the fp64 oracle, through the C ABI."""

import copy

import numpy as np
import pytest

from quantized_paged_attention_amd import synth
from tests.gpu_util import assert_decode_close, log, need_gpu, oracle_decode, run_decode

pytestmark = pytest.mark.gpu

EDGE_LENS = (1, 15, 16, 17, 31, 255, 256, 257, 513, 1000)


def tok(seed, lens=EDGE_LENS, hk=2, qg=8, bs=16, values="normal", **kw):
    if values == "uniform_codes":
        kw.setdefault("k_scale", 0.05)
        kw.setdefault("v_scale", 0.02)
    return synth.make_fp8_case("fp8_tok", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               block_size=bs, spare_blocks=7, scales="token", values=values,
                               **kw)


@pytest.mark.parametrize("P", [1, 2, 3, 7])
@pytest.mark.parametrize("values", ["normal", "uniform_codes"])
def test_edge_lengths_and_partitions(P, values):
    need_gpu()
    case = tok(61, values=values)
    log(f"case fp8 per-token edge lens P={P} values={values}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"per-token P={P} {values}")


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_block_sizes(bs):
    need_gpu()
    case = tok(62, lens=(1, bs - 1, bs, bs + 1, 5 * bs + 3, 700), bs=bs)
    log(f"case fp8 per-token block_size={bs}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"per-token bs={bs}")


@pytest.mark.parametrize("qg", [1, 2, 4, 8])
def test_query_groups(qg):
    need_gpu()
    case = tok(63, qg=qg, q_dtype="f32")
    log(f"case fp8 per-token qg={qg}")
    got, _ = run_decode(case, P=2)
    assert_decode_close(got, oracle_decode(case), f"per-token qg={qg}")


@pytest.mark.parametrize("ql,qg", [(2, 4), (4, 2), (3, 1)])
def test_query_rows(ql, qg):
    need_gpu()
    case = tok(64, qg=qg, query_len=ql, lens=(3, 17, 256, 257, 1000))
    log(f"case fp8 per-token query_len={ql} qg={qg}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"per-token ql={ql} qg={qg}")


@pytest.mark.parametrize("ramp", [1.0, 4.0])
def test_growing_v_scales(ramp):
    """V scales that grow 2^(ramp t / 256) along every sequence: the running V reference
    of each wave is raised many times, each time rescaling the accumulators."""
    need_gpu()
    case = tok(65, lens=(300, 1000, 2049), v_ramp=ramp, tok_spread=0.25)
    log(f"case fp8 per-token v_ramp={ramp}")
    got, _ = run_decode(case, P=2)
    assert_decode_close(got, oracle_decode(case), f"per-token v_ramp={ramp}")


@pytest.mark.parametrize("where", ["early", "late"])
def test_v_scale_outlier(where):
    """One token per sequence with a V scale 10^4 times the others, near the start (every
    later token's P is small against the reference) or near the end (the reference is
    raised last)."""
    need_gpu()
    case = tok(66, lens=(200, 1000, 1500))
    for b, L in enumerate(case.seq_lens):
        t = 5 if where == "early" else int(L) - 3
        blk = case.block_table[b, t // case.block_size]
        case.v_scale_tok[blk, :, t % case.block_size] *= np.float32(1e4)
    log(f"case fp8 per-token V-scale outlier {where}")
    got, _ = run_decode(case, P=1)
    assert_decode_close(got, oracle_decode(case), f"per-token outlier {where}")


def test_zero_scales():
    """All V scales of a sequence zero: its output is exactly zero.  All K scales of a
    sequence zero: every score is 0, so the output is the mean of its scaled V rows."""
    need_gpu()
    case = tok(67, lens=(40, 300, 513))
    bs = case.block_size
    for b, which in ((0, "v"), (2, "k")):
        L = int(case.seq_lens[b])
        blks = case.block_table[b, :-(-L // bs)]
        arr = case.v_scale_tok if which == "v" else case.k_scale_tok
        arr[blks] = 0.0
        arr[case.block_table[b, (L - 1) // bs], :, (L - 1) % bs + 1:] = np.nan   # past L
    log("case fp8 per-token zero scales")
    got, _ = run_decode(case, P=2)
    assert np.all(got[0] == 0)
    assert_decode_close(got, oracle_decode(case), "per-token zero scales")


def test_masked_scales_bit_identical():
    """Scales of slots past each sequence and of unused blocks (NaN from the generator)
    changed to other garbage leave every output bit unchanged."""
    need_gpu()
    case = tok(68, lens=(3, 20, 33, 250))
    base, _ = run_decode(case, P=2)
    assert np.isfinite(base).all()
    c2 = copy.deepcopy(case)
    for arr in (c2.k_scale_tok, c2.v_scale_tok):
        arr[np.isnan(arr)] = np.float32(np.inf)
    got, _ = run_decode(c2, P=2)
    assert np.array_equal(got, base)


def test_fp8_high_tok_full():
    """The high-batch fp8 shape (B=128, L ~ U[4096, 16384], Hk=8, QG=8, 64 partitions)
    with per-token scales, at full size in the benchmark's launch configuration; every
    output row is compared with the oracle."""
    need_gpu()
    case = synth.fp8_high_tok()
    log(f"case fp8_high_tok (full GPU run, full oracle) kv_bytes={case.kv_bytes()}")
    got, _ = run_decode(case)
    assert_decode_close(got, oracle_decode(case), "fp8_high_tok")


@pytest.mark.parametrize("P", [1, 64])
def test_head_groups_per_token(P):
    """Per-token scales with Hk=8 (head-group workgroups)."""
    need_gpu()
    case = tok(69, hk=8, qg=4, lens=(1, 17, 256, 257, 1000, 3000), v_ramp=1.0)
    log(f"case fp8 per-token head groups P={P}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"per-token head groups P={P}")


@pytest.mark.parametrize("qg", [12, 32, 64])
def test_balanced_row_slices_per_token(qg):
    """Per-token scales with f16 row tiles inside balanced slices (80 sequences, one of
    16384 tokens, Hk = 4): 12 rows in one tile, 32 in two, 64 in two row slices; fused
    and through decode + reduce."""
    need_gpu()
    rng = np.random.default_rng(370)
    lens = rng.integers(1, 300, size=80)
    lens[0] = 16384
    lens[[3, 40]] = 0
    case = tok(371 + qg, lens=tuple(int(x) for x in lens), hk=4, qg=qg)
    log(f"case fp8 per-token balanced row slices qg={qg}")
    ref = oracle_decode(case)
    got, _ = run_decode(case)
    assert_decode_close(got, ref, "per-token row slices fused")
    split, _ = run_decode(case, mode="split")
    assert_decode_close(split, ref, "per-token row slices split")


@pytest.mark.parametrize("qg,hk", [(16, 2), (16, 8), (32, 4)])
def test_wide_groups_per_token(qg, hk):
    """Per-token scales with query groups of 16 and 32 rows."""
    need_gpu()
    case = tok(90 + qg + hk, hk=hk, qg=qg, lens=(1, 17, 256, 257, 1500), v_ramp=1.0)
    log(f"case fp8 per-token wide qg={qg} hk={hk}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"per-token wide qg={qg} hk={hk}")


@pytest.mark.parametrize("hk,bs", [(3, 16), (1, 16), (3, 32)])
def test_odd_head_counts(hk, bs):
    """Odd kv head counts (runs of one head, no head groups) at block sizes 16 and 32."""
    need_gpu()
    case = tok(95 + hk + bs, hk=hk, qg=4, bs=bs, lens=(1, 15, 16, 17, 255, 257, 1000))
    log(f"case fp8 per-token odd hk={hk} bs={bs}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"per-token hk={hk} bs={bs}")
