"""GPU parity of the fp8 e4m3 decode + reduce path against the fp64 oracle."""

import copy

import numpy as np
import pytest
import torch

from quantized_paged_attention_amd import synth
from tests.gpu_util import (assert_decode_close, device_case, log, need_gpu, oracle_decode,
                            q_tensor, rel_err, run_decode, uq)

pytestmark = pytest.mark.gpu

EDGE_LENS = (1, 15, 16, 17, 31, 255, 256, 257, 513, 1000)


def small(seed=31, lens=EDGE_LENS, hk=2, qg=8, bs=16, **kw):
    kw.setdefault("values", "uniform_codes")
    kw.setdefault("k_scale", 0.05)
    kw.setdefault("v_scale", 0.02)
    return synth.make_fp8_case("fp8_small", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               block_size=bs, spare_blocks=7, **kw)


def test_tiny_config():
    """B=2, Hk=1, QG=8, L={37, 200}, fp32 Q, one partition (the tiny workload)."""
    need_gpu()
    case = synth.tiny_fp8()
    log(f"case tiny_fp8 seq_lens={case.seq_lens.tolist()}")
    got, (po, pm, pl) = run_decode(case, mode="split")
    ref, (rm, rl, ro) = oracle_decode(case, case.num_partitions)
    assert_decode_close(got, ref, "tiny_fp8 out")
    # partition statistics themselves
    np.testing.assert_allclose(pm.cpu().numpy(), rm, rtol=2e-3, atol=2e-3)
    np.testing.assert_allclose(pl.cpu().numpy(), rl, rtol=2e-2)
    assert rel_err(po.float().cpu().numpy(), ro) <= 1e-2


@pytest.mark.parametrize("P", [1, 2, 3, 7])
@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
def test_edge_lengths_and_partitions(P, q_dtype):
    need_gpu()
    case = small(q_dtype=q_dtype)
    log(f"case fp8 edge lens P={P} q={q_dtype}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"edge P={P} {q_dtype}")


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_block_sizes(bs):
    need_gpu()
    case = small(bs=bs, lens=(3, 300, 700, 1200), seed=32 + bs)
    log(f"case fp8 block_size={bs}")
    got, _ = run_decode(case, P=2)
    assert_decode_close(got, oracle_decode(case), f"bs={bs}")


@pytest.mark.parametrize("qg", [1, 2, 4, 6, 8])
def test_query_groups(qg):
    need_gpu()
    case = small(qg=qg, hk=3, lens=(40, 600), seed=40 + qg)
    log(f"case fp8 qg={qg}")
    got, _ = run_decode(case, P=3)
    assert_decode_close(got, oracle_decode(case), f"qg={qg}")


def test_strided_query_from_fused_qkv():
    need_gpu()
    case = small(lens=(100, 777), seed=50)
    got, _ = run_decode(case, P=2, strided=True)
    assert_decode_close(got, oracle_decode(case), "strided q")


def test_normal_values_unit_scales():
    need_gpu()
    case = small(values="normal", k_scale=1.0, v_scale=1.0, seed=51, lens=(2000, 5, 4096))
    got, _ = run_decode(case, P=4)
    assert_decode_close(got, oracle_decode(case), "normal values")


def test_zero_length_sequences():
    need_gpu()
    case = small(lens=(0, 20, 0), seed=52)
    got, _ = run_decode(case, P=2)
    ref = oracle_decode(case)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert_decode_close(got, ref, "zero length")


def test_one_hot_gather_bit_exact():
    """Q = 100 e0, one key with K[0] = 448 and zeros elsewhere: every other weight is
    exactly zero, so the output must equal v[t*] bit for bit (v_scale = 1)."""
    need_gpu()
    bs = 16
    L = 10 * bs + 5
    case = small(lens=(L,), hk=1, qg=8, bs=bs, values="normal", k_scale=1.0, v_scale=1.0,
                 q_dtype="f32", seed=53)
    D = case.D
    case.q[:] = 0.0
    case.q[:, :, 0] = 100.0
    from tests.refdense import dense_kv
    for tstar in (0, 15, 16, 17, 31, 32, 100, L - 1):
        c = copy.deepcopy(case)
        c.cache[..., :D] = 0
        c.cache[c.block_table[0, tstar // bs], tstar % bs, 0, 0] = 0x7E
        got, _ = run_decode(c, P=1)
        _, v = dense_kv(c, 0, 0)
        for g in range(8):
            assert np.array_equal(got[0, g], v[tstar]), (tstar, g)


def test_block_permutation_bit_identical():
    need_gpu()
    case = small(lens=(17, 300, 513, 2000), seed=54)
    base, _ = run_decode(case, P=3)
    rng = np.random.default_rng(1)
    perm = rng.permutation(case.cache.shape[0])
    c2 = copy.deepcopy(case)
    c2.cache = np.empty_like(case.cache)
    c2.cache[perm] = case.cache
    c2.block_table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)],
                              -1).astype(np.int32)
    got, _ = run_decode(c2, P=3)
    assert np.array_equal(got, base)


def test_masked_bytes_bit_identical():
    """Slots past L (NaN-poisoned by the generator), unreferenced blocks and table tails
    changed to other garbage must not change a single output bit."""
    need_gpu()
    case = small(lens=(3, 20, 33, 250), seed=55)
    base, _ = run_decode(case, P=2)
    assert np.isfinite(base).all()
    c2 = copy.deepcopy(case)
    used = np.zeros(c2.cache.shape[0], bool)
    for b, L in enumerate(c2.seq_lens):
        n = -(-int(L) // c2.block_size)
        used[c2.block_table[b, :n]] = True
        if L % c2.block_size:
            c2.cache[c2.block_table[b, L // c2.block_size], L % c2.block_size:] = 0x7E
        c2.block_table[b, n:] = 1 << 30
    c2.cache[~used] = 0xFE
    got, _ = run_decode(c2, P=2)
    assert np.array_equal(got, base)


def test_reduce_against_oracle_partials():
    """The reduce kernel alone, fed the oracle's partials (rounded to the workspace
    types), including empty partitions (m = -inf, l = 0)."""
    need_gpu()
    from oracle import oracle
    case = small(lens=(0, 1, 256, 257, 1500), seed=56)
    P = 4
    _, (rm, rl, ro) = oracle_decode(case, P)
    po = torch.from_numpy(ro).to(torch.bfloat16)
    pm = torch.from_numpy(rm).to(torch.float32)
    pl = torch.from_numpy(rl).to(torch.float32)
    want = oracle.reduce(po.double().numpy(), pm.double().numpy(), pl.double().numpy(),
                         case.seq_lens)
    out = torch.empty(case.B, case.Hq, case.D, dtype=torch.float32, device="cuda")
    uq.paged_reduce(po.cuda(), pm.cuda(), pl.cuda(), torch.from_numpy(case.seq_lens).cuda(), out,
                    max_seq_len=case.max_seq_len)
    got = out.cpu().double().numpy()
    assert np.all(got[0] == 0)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6 * np.abs(want).max())


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_mid_config_full(mode):
    """B=16, Hk=8, QG=8, L=16384, bf16 Q, 64 partitions, k/v scales 0.05/0.02 (head-group
    runs: every sequence split into runs of partitions)."""
    need_gpu()
    case = synth.fp8_mid()
    log(f"case fp8_mid {mode} (full)")
    got, _ = run_decode(case, mode=mode)
    assert_decode_close(got, oracle_decode(case), f"fp8_mid {mode}")


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_high_config_full(mode):
    """B=128 with L ~ U[4096, 16384] at full size, in the benchmark's launch configuration
    (balanced slices: almost every sequence is split at some slice edge); every output row
    of all 128 sequences and 64 query heads is compared with the oracle.  fused: the one
    launch of uq_paged_attention; split: decode then reduce through partials."""
    need_gpu()
    case = synth.fp8_high()
    log(f"case fp8_high {mode} (full GPU run, full oracle) kv_bytes={case.kv_bytes()}")
    got, _ = run_decode(case, mode=mode)
    assert_decode_close(got, oracle_decode(case), f"fp8_high {mode}")


@pytest.mark.parametrize("B,run", [(32, 2), (128, 3)])
def test_partition_runs_ragged_batch(B, run):
    """Batches large enough that each wave streams a run of several partitions (Hk=8,
    P=32: B=32 gives 8192 (sequence, head, partition) items and runs of two, B=128 gives
    32768 and runs of three; four waves merge their runs): ragged lengths end a sequence
    at every position of a run and of a merged group, on and off tile-group edges."""
    need_gpu()
    rng = np.random.default_rng(57 + B)
    lens = rng.integers(1, 8193, size=B)
    lens[:8] = [1, 255, 256, 257, 511, 512, 8192, 4097]
    lens[8:20] = 256 * np.arange(1, 13) + 1       # 1..12 partitions + 1 token
    case = small(lens=tuple(int(x) for x in lens), hk=8, qg=8, seed=57 + B)
    log(f"case fp8 runs B={B} (run length {run})")
    got, _ = run_decode(case, P=32)
    assert_decode_close(got, oracle_decode(case), "runs ragged")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("P", [40, 130, 300, 700, 2100])
def test_reduce_skips_empty_partitions(D, P):
    """Synthetic partials with some partitions empty (l = 0, m = -inf) whose partial rows
    hold NaN: the reduce must not read them into the sum.  With 24 rows the launcher splits
    a row over 1, 2, 4, 8 and 16 waves for these P (at least 64 partitions per wave); P = 700
    and 2100 exceed the partitions the reduce keeps in registers (its batched path).
    Reference: the oracle's reduce on the same statistics with those rows zeroed (an empty
    partition's o is 0 there)."""
    need_gpu()
    from oracle import oracle
    rng = np.random.default_rng(58 + P + D)
    B, hk, qg = 3, 2, 4
    seq_lens = np.array([P * 256, 5 * 256 - 17, 0], np.int32)
    pm = rng.normal(0.0, 3.0, (B, hk, P, qg))
    pl = rng.uniform(0.5, 50.0, (B, hk, P, qg))
    po = rng.normal(0.0, 1.0, (B, hk, P, qg, D))
    empty = rng.random((B, hk, P, qg)) < 0.4
    empty[:, :, 0] = False
    pm[empty], pl[empty] = -np.inf, 0.0
    po_t = torch.from_numpy(po).to(torch.bfloat16)
    po_clean = po_t.double().numpy().copy()
    po_clean[empty] = 0.0
    po_t[torch.from_numpy(empty)] = float("nan")
    pm32 = torch.from_numpy(pm).float()
    pl32 = torch.from_numpy(pl).float()
    want = oracle.reduce(po_clean, pm32.double().numpy(), pl32.double().numpy(), seq_lens)
    out = torch.empty(B, hk * qg, D, dtype=torch.float32, device="cuda")
    uq.paged_reduce(po_t.cuda(), pm32.cuda(), pl32.cuda(), torch.from_numpy(seq_lens).cuda(), out,
                    max_seq_len=int(seq_lens.max()))
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    assert np.all(got[2] == 0)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6 * np.abs(want).max())


@pytest.mark.parametrize("fmt", ["fp8", "fp4", "fp8_tok_hg", "fp8_wide"])
def test_graph_replay_matches_eager(fmt):
    """decode + reduce captured in a HIP graph (torch.cuda.graph on the current stream):
    every one of several replays, with eager work and synchronisations in between, gives
    the eager result bit for bit (no memset nodes; all state lives in the partials).
    fp8_tok_hg: per-token scales with head-group workgroups; fp8_wide: a 32-row query
    group, two decode launches per step."""
    need_gpu()
    if fmt == "fp8":
        case = small(lens=(40, 700, 2049, 5000), seed=59, hk=2)
    elif fmt == "fp8_tok_hg":
        case = synth.make_fp8_case("tok_graph", 96, seq_lens=[40, 700, 2049, 5000],
                                   num_kv_heads=8, qg=4, spare_blocks=3, scales="token",
                                   values="normal")
    elif fmt == "fp8_wide":
        case = small(lens=(40, 700, 2049), seed=97, hk=4, qg=32)
    else:
        case = synth.make_fp4_case("fp4_graph", 95, seq_lens=[300, 1000, 3000], num_kv_heads=2,
                                   qg=8, head_dim=256, block_size=64, rotate=True, spare_blocks=3)
    dev = device_case(case)
    q = q_tensor(case)
    P = 8
    B, Hq, D = q.shape
    partials = uq.alloc_partials(B, case.num_kv_heads, Hq // case.num_kv_heads, D, P)
    out = torch.empty(B, Hq, D, dtype=q.dtype, device="cuda")
    eager, _ = run_decode(case, P=P, dev=dev, q=q, partials=partials, out=out)
    out.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        uq.paged_decode_reduce(q, dev["cache"], dev["bt"], dev["sl"], kv_format=case.kv_format,
                               max_seq_len=case.max_seq_len, num_partitions=P, partials=partials,
                               out=out, softmax_scale=case.softmax_scale, k_scale=dev["ks"],
                               v_scale=dev["vs"], rot_signs=dev["rot"])
    for i in range(4):
        out.fill_(float("nan"))
        partials[0].fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, eager), f"replay {i}"
        _ = (q.float() * 2).sum().item()      # eager work between replays


@pytest.mark.parametrize("hk", [4, 8])
@pytest.mark.parametrize("P", [1, 3, 64])
@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
def test_head_group_workgroups(hk, P, q_dtype):
    """Kv head counts that are multiples of 4 run as head groups (a workgroup's waves take
    4 neighbouring kv heads of one run of partitions); P = 1 and 3 make partitions own
    several strided tile-groups."""
    need_gpu()
    case = small(hk=hk, qg=8 if hk == 4 else 4, q_dtype=q_dtype, seed=70 + hk + P,
                 lens=(1, 16, 17, 255, 257, 700, 2049, 4000, 5000))
    log(f"case fp8 head groups hk={hk} P={P} q={q_dtype}")
    got, _ = run_decode(case, P=P)
    assert_decode_close(got, oracle_decode(case), f"head groups hk={hk} P={P} {q_dtype}")


def test_head_group_large_batch_runs():
    """Many sequences with Hk=8 so the launcher picks long runs of partitions per
    workgroup (the high-batch regime), lengths from 1 to 9000."""
    need_gpu()
    rng = np.random.default_rng(75)
    lens = list(rng.integers(1, 9000, size=96)) + [1, 255, 256, 257]
    case = small(hk=8, qg=8, lens=tuple(int(x) for x in lens), seed=76)
    log(f"case fp8 head groups B={case.B} hk=8 P=64")
    got, _ = run_decode(case, P=64)
    assert_decode_close(got, oracle_decode(case), "head groups large batch")


@pytest.mark.parametrize("qg", [12, 16, 24, 32, 64])
@pytest.mark.parametrize("hk", [2, 4])
def test_wide_query_groups(qg, hk):
    """Query groups above 8 rows (the pages' wide-GQA case).  hk = 4: head groups with f16
    row tiles of 16 rows, one wave per kv head up to 32 rows and two above.  hk = 2: no head
    groups up to 32 rows, so two e4m3 row tiles of 8 share one pass over the cache and
    wider groups run one pass per 16 rows; at 64 rows head groups of 2 kv heads."""
    need_gpu()
    case = small(hk=hk, qg=qg, seed=80 + qg + hk, q_dtype="f32" if qg == 12 else "bf16",
                 lens=(1, 17, 256, 257, 1000, 2500))
    log(f"case fp8 wide group qg={qg} hk={hk}")
    for P in (1, 3):
        got, _ = run_decode(case, P=P)
        assert_decode_close(got, oracle_decode(case), f"wide qg={qg} hk={hk} P={P}")


def _bal_lens(rng, B, zeros, lo, hi, long_len):
    lens = rng.integers(lo, hi, size=B)
    lens[rng.choice(B, zeros, replace=False)] = 0
    lens[0] = long_len
    return tuple(int(x) for x in lens)


@pytest.mark.parametrize("qg,hk", [(8, 4), (4, 8)])
def test_balanced_slices_sparse_batch(qg, hk):
    """Enough work for balanced slices (one workgroup per CU, each an equal share of all
    sequences' partitions) but mostly empty or tiny sequences, so fewer partitions than
    slices: empty slices, slices that start on empty sequences, units split at
    sequence boundaries."""
    need_gpu()
    rng = np.random.default_rng(90 + qg)
    lens = _bal_lens(rng, 300, 60, 1, 300, 16000)
    case = small(hk=hk, qg=qg, lens=lens, seed=91 + hk)
    log(f"case fp8 balanced sparse B={case.B} hk={hk} qg={qg}")
    got, _ = run_decode(case, P=64)
    assert_decode_close(got, oracle_decode(case), f"balanced sparse hk={hk}")


def test_balanced_slices_one_long_sequence():
    """A batch dominated by one 60000-token sequence: its partitions are split over many
    slices (one unit each), the other sequences share the rest."""
    need_gpu()
    rng = np.random.default_rng(93)
    lens = _bal_lens(rng, 120, 10, 1000, 3000, 60000)
    case = small(hk=8, qg=2, lens=lens, seed=94)
    log(f"case fp8 balanced long B={case.B}")
    got, _ = run_decode(case, P=256)
    assert_decode_close(got, oracle_decode(case), "balanced one long")


def test_balanced_slices_wide_group():
    """Balanced slices with a 24-row query group (two launches: rows 0-15, 16-23)."""
    need_gpu()
    rng = np.random.default_rng(95)
    lens = _bal_lens(rng, 200, 5, 100, 8000, 8000)
    case = small(hk=4, qg=24, lens=lens, seed=96)
    log(f"case fp8 balanced wide B={case.B} qg=24")
    got, _ = run_decode(case, P=64)
    assert_decode_close(got, oracle_decode(case), "balanced wide qg=24")


@pytest.mark.parametrize("B,qg", [(1000, 2), (1024, 16), (1000, 48), (1100, 8)])
def test_balanced_slices_many_sequences(B, qg):
    """Up to 1024 sequences (16 lengths per lane of the slice lookup), lengths 0..900 with
    a few long ones: balanced slices start in the middle of lanes' runs of sequences, with
    e4m3 row tiles (2 rows), one f16 tile (16) and row slices (48); 1100 sequences take
    the runs of head groups instead."""
    need_gpu()
    rng = np.random.default_rng(97 + qg)
    lens = rng.integers(0, 900, size=B)
    lens[rng.choice(B, 20, replace=False)] = rng.integers(4000, 9000, size=20)
    case = small(hk=4, qg=qg, lens=tuple(int(x) for x in lens), seed=98 + qg)
    log(f"case fp8 balanced B={case.B} qg={qg}")
    got, _ = run_decode(case, P=64)
    assert_decode_close(got, oracle_decode(case), f"balanced B={B} qg={qg}")
