"""GPU parity of the fp4 (e2m1 codes, e4m3 group scales) D=256 decode + reduce path,
with and without the in-kernel query rotation, against the fp64 oracle."""

import copy

import numpy as np
import pytest

from quantized_paged_attention_amd import synth
from tests.gpu_util import assert_decode_close, log, need_gpu, oracle_decode, rel_err, run_decode

pytestmark = pytest.mark.gpu

EDGE_LENS = (1, 63, 64, 65, 255, 256, 257, 1000, 3000)


KINDS = ["e4m3", "ue8m0"]   # group scale codes: e4m3 (the D=256 config) and UE8M0


def small(seed=61, lens=EDGE_LENS, hk=2, qg=8, bs=64, rotate=True, kind="e4m3", **kw):
    return synth.make_fp4_case("fp4_small", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               head_dim=256, block_size=bs, rotate=rotate, spare_blocks=5,
                               scale_kind=kind, **kw)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("qg", [1, 6, 8, 16])
@pytest.mark.parametrize("rotate", [True, False])
def test_edge_lengths_query_groups(qg, rotate, kind):
    need_gpu()
    case = small(qg=qg, rotate=rotate, seed=61 + qg, kind=kind)
    log(f"case fp4 edge lens qg={qg} rotate={rotate} scales={kind}")
    got, _ = run_decode(case, P=4)
    assert_decode_close(got, oracle_decode(case), f"fp4 qg={qg} rot={rotate} {kind}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("P", [1, 3, 12])
@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
def test_partition_counts(P, q_dtype, kind):
    """P = 1 and 3 put several strided tile-groups into one partition; P = 12 leaves
    trailing partitions empty for the shorter sequences."""
    need_gpu()
    case = small(q_dtype=q_dtype, seed=70 + P, kind=kind)
    log(f"case fp4 P={P} q={q_dtype} scales={kind}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"fp4 P={P} {q_dtype}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_block_sizes(bs, kind):
    need_gpu()
    case = small(bs=bs, lens=(5, 100, 700, 1500), seed=80 + bs, kind=kind)
    log(f"case fp4 block_size={bs}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"fp4 bs={bs}")


def test_partition_statistics():
    """part_max (true maximum, natural log), part_sum and part_out against the oracle's
    per-partition statistics."""
    need_gpu()
    case = small(lens=(300, 1000), qg=6, seed=90)
    P = 3
    _, (po, pm, pl) = run_decode(case, P=P, mode="split")
    _, (rm, rl, ro) = oracle_decode(case, P)
    pm, pl, po = pm.cpu().numpy(), pl.cpu().numpy(), po.float().cpu().numpy()
    live = np.isfinite(rm)
    np.testing.assert_allclose(pm[live], rm[live], rtol=2e-3, atol=2e-3)
    np.testing.assert_allclose(pl[live], rl[live], rtol=2e-2)
    assert rel_err(po[live], ro[live]) <= 1e-2


def test_zero_length_sequences():
    need_gpu()
    case = small(lens=(0, 77, 0), seed=91)
    got, _ = run_decode(case, P=2)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert_decode_close(got, oracle_decode(case), "fp4 zero length")


def test_one_hot_gather_bit_exact():
    """No rotation, Q = 100 e0 and one token whose K holds 6 * 448 in dim 0 (zero
    elsewhere): every other weight is exactly zero, and e2m1 * e4m3 values are exact in
    bf16, so the output equals v[t*] bit for bit."""
    need_gpu()
    bs = 64
    L = 3 * bs + 7
    case = small(lens=(L,), hk=1, qg=8, bs=bs, rotate=False, q_dtype="f32", seed=92)
    case.q[:] = 0.0
    case.q[:, :, 0] = 100.0
    from tests.refdense import dense_kv
    for tstar in (0, 63, 64, 65, 130, L - 1):
        c = copy.deepcopy(case)
        blk = c.block_table[0]
        for t in range(L):
            slot = c.cache[blk[t // bs], t % bs, 0]
            slot[:128] = 0                        # K codes zero
        slot = c.cache[blk[tstar // bs], tstar % bs, 0]
        slot[0] = 0x07                            # dim 0 code 6.0, dim 1 code 0
        slot[128] = 0x7E                          # group 0 scale 448
        got, _ = run_decode(c, P=1)
        _, v = dense_kv(c, 0, 0)
        for g in range(8):
            assert np.array_equal(got[0, g], v[tstar]), (tstar, g)


def test_block_permutation_bit_identical():
    need_gpu()
    case = small(lens=(17, 300, 513, 2000), seed=93)
    base, _ = run_decode(case, P=3)
    rng = np.random.default_rng(2)
    perm = rng.permutation(case.cache.shape[0])
    c2 = copy.deepcopy(case)
    c2.cache = np.empty_like(case.cache)
    c2.cache[perm] = case.cache
    c2.block_table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)],
                              -1).astype(np.int32)
    got, _ = run_decode(c2, P=3)
    assert np.array_equal(got, base)


@pytest.mark.parametrize("kind", KINDS)
def test_masked_bytes_bit_identical(kind):
    need_gpu()
    case = small(lens=(3, 70, 129, 250), seed=94, bs=32, kind=kind)
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


@pytest.mark.parametrize("qg,kind", [(6, "e4m3"), (8, "e4m3"), (16, "e4m3"), (6, "ue8m0"),
                                     (16, "ue8m0")])
def test_d256_config_full(qg, kind):
    """B=4, Hk=2, L=75000, block 64, 512 partitions, bf16 Q, rotation: the full output."""
    need_gpu()
    case = synth.fp4_d256(qg, kind)
    log(f"case fp4_d256 qg={qg} scales={kind} kv_bytes={case.kv_bytes()}")
    got, _ = run_decode(case)
    assert_decode_close(got, oracle_decode(case), f"fp4_d256 qg={qg} {kind}")


def test_ue8m0_one_hot_gather_bit_exact():
    """UE8M0 scales, no rotation, Q = 100 e0, one token whose K holds 6 x 2^8 in dim 0:
    every other weight is exactly zero and e2m1 x 2^k is exact in bf16, so the output
    equals v[t*] bit for bit."""
    need_gpu()
    bs = 64
    L = 3 * bs + 7
    case = small(lens=(L,), hk=1, qg=8, bs=bs, rotate=False, q_dtype="f32", seed=96,
                 kind="ue8m0")
    case.q[:] = 0.0
    case.q[:, :, 0] = 100.0
    from tests.refdense import dense_kv
    for tstar in (0, 63, 64, 130, L - 1):
        c = copy.deepcopy(case)
        blk = c.block_table[0]
        for t in range(L):
            c.cache[blk[t // bs], t % bs, 0][:128] = 0
        slot = c.cache[blk[tstar // bs], tstar % bs, 0]
        slot[0] = 0x07                            # dim 0 code 6.0
        slot[128] = 127 + 8                       # group 0 scale 2^8
        got, _ = run_decode(c, P=1)
        _, v = dense_kv(c, 0, 0)
        for g in range(8):
            assert np.array_equal(got[0, g], v[tstar]), (tstar, g)


@pytest.mark.parametrize("kind", KINDS)
def test_runs_ragged_batch(kind):
    """B=16 ragged lengths up to 40000 with 160 partitions: the launcher streams runs of
    several partitions per workgroup (five here), merged into one partial; lengths end a
    sequence at every position of a run."""
    need_gpu()
    rng = np.random.default_rng(97)
    lens = rng.integers(1, 40001, size=16)
    lens[:6] = [1, 256, 257, 5 * 256, 5 * 256 + 1, 40000]
    case = small(lens=tuple(int(x) for x in lens), hk=2, qg=8, seed=97, kind=kind)
    log(f"case fp4 runs ragged scales={kind}")
    got, _ = run_decode(case, P=160)
    assert_decode_close(got, oracle_decode(case), f"fp4 runs ragged {kind}")
