"""uq_paged_attention: decode and flash-combine in one call.  With the fp8 formats and head
groups (num_kv_heads a multiple of 4, or of 2 for 33-64 rows) one launch does both: every
work unit that covers only part of its sequence leaves its softmax state in the workspace
and counts its partitions; the unit that completes the count merges the states and writes
the output rows.  These cases aim at the shapes of that bookkeeping (balanced slices that
split sequences, empty slices, sequences wholly inside one slice, zero-length sequences,
e4m3 and f16 row tiles, row slices, passes of 16 rows without head groups, float32
output) and at the workspace contract (counters back at zero after every call, reuse
across calls of other sizes, graph replay).  Every output is compared with the fp64
oracle."""

import numpy as np
import pytest
import torch

from quantized_paged_attention_amd import synth, uq
from tests.gpu_util import (assert_decode_close, device_case, log, need_gpu, oracle_decode,
                            q_tensor, run_decode)

pytestmark = pytest.mark.gpu


def fp8(lens, hk=4, qg=8, seed=0, **kw):
    kw.setdefault("k_scale", 0.05)
    kw.setdefault("v_scale", 0.02)
    return synth.make_fp8_case("fp8_fused", seed, seq_lens=[int(x) for x in lens],
                               num_kv_heads=hk, qg=qg, spare_blocks=5, **kw)


def counters_of(ws: torch.Tensor, B: int = 0, hk: int = 0) -> np.ndarray:
    """The whole fixed counter region at the start of the workspace (256 KiB)."""
    return ws[:256 << 10].view(torch.int32).cpu().numpy()


def sparse_lens(seed=300, B=80):
    """One 16k sequence among short and empty ones: with Hk = 4 the launcher takes
    balanced slices (80 x 64 partitions of work per head group exceed 16 per CU), but
    the sequences hold fewer partitions than there are slices, so many slices are empty
    and the long sequence is spread over dozens of one-partition units."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 300, size=B)
    lens[0] = 16384
    lens[[3, 17, 40]] = 0
    lens[5] = 256
    lens[6] = 257
    return lens


@pytest.mark.parametrize("qg,q_dtype", [(8, "bf16"), (8, "f32"), (16, "bf16"), (5, "f32"),
                                        (12, "f32")])
def test_balanced_sparse_slices(qg, q_dtype):
    """Balanced slices over a sparse batch (one long sequence, empty ones): e4m3 row
    tiles of 8 rows (QG 5, 8) and one f16 tile of 16 rows (QG 12, 16)."""
    need_gpu()
    case = fp8(sparse_lens(), hk=4, qg=qg, seed=301 + qg, q_dtype=q_dtype)
    log(f"case fused sparse slices qg={qg} q={q_dtype}")
    ws = uq.alloc_workspace(case.B, 4, 1, qg, 128, case.num_partitions, case.max_seq_len,
                            case.kv_format)
    got, _ = run_decode(case, workspace=ws)
    assert np.all(got[[3, 17, 40]] == 0)
    assert_decode_close(got, oracle_decode(case), f"fused sparse qg={qg}")
    assert not counters_of(ws, case.B, 4).any()


def test_balanced_whole_sequences_in_slices():
    """600 sequences of up to 2048 tokens (Hk=4, 8 partitions at most): about 10
    partitions per slice, so most sequences lie wholly inside one slice (written
    directly) and the others are split at slice edges."""
    need_gpu()
    rng = np.random.default_rng(310)
    lens = rng.integers(1, 2049, size=600)
    lens[::37] = 0
    lens[1] = 2048
    case = fp8(lens, hk=4, qg=8, seed=311)
    log("case fused 600 short sequences")
    ws = uq.alloc_workspace(case.B, 4, 1, 8, 128, case.num_partitions, case.max_seq_len,
                            case.kv_format)
    got, _ = run_decode(case, workspace=ws)
    assert np.all(got[::37] == 0)
    assert_decode_close(got, oracle_decode(case), "fused 600 sequences")
    assert not counters_of(ws, case.B, 4).any()


def test_workspace_reused_across_sizes():
    """One workspace for calls in a row, the second with a smaller batch and other
    lengths, the third with more arrival counters than either (sequences x kv heads):
    all match the oracle and the counters are zero after each."""
    need_gpu()
    big = fp8(sparse_lens(320), hk=8, qg=8, seed=321)
    ws = uq.alloc_workspace(big.B, 8, 1, 8, 128, big.num_partitions, big.max_seq_len,
                            big.kv_format)
    got, _ = run_decode(big, workspace=ws)
    assert_decode_close(got, oracle_decode(big), "fused reuse, first call")
    assert not counters_of(ws, big.B, 8).any()
    small = fp8((1, 300, 5000, 0, 4097, 256), hk=8, qg=8, seed=322)
    need = uq.attention_workspace_bytes(small.B, 8, 1, 8, 128, small.num_partitions,
                                       small.max_seq_len, small.kv_format)
    assert need <= ws.numel()
    got, _ = run_decode(small, workspace=ws)
    assert_decode_close(got, oracle_decode(small), "fused reuse, second call")
    assert not counters_of(ws, small.B, 8).any()
    grow = fp8(np.random.default_rng(323).integers(0, 2000, size=200), hk=8, qg=8, seed=324)
    need = uq.attention_workspace_bytes(grow.B, 8, 1, 8, 128, grow.num_partitions,
                                       grow.max_seq_len, grow.kv_format)
    assert need <= ws.numel()
    got, _ = run_decode(grow, workspace=ws)
    assert_decode_close(got, oracle_decode(grow), "fused reuse, third call")
    assert not counters_of(ws, grow.B, 8).any()


@pytest.mark.parametrize("ql,qg,q_dtype", [(1, 32, "bf16"), (1, 48, "f32"), (2, 32, "bf16"),
                                            (1, 64, "bf16")])
def test_balanced_row_slices(ql, qg, q_dtype):
    """Groups of 32-64 rows in f16 tiles of 16 rows: 32 rows as two tiles of one wave, 48
    and 64 rows split over two waves per kv head (row slices; at 48 rows the second
    wave's second tile is empty), inside balanced slices (the sparse batch at Hk = 4);
    through the fused step and through decode + reduce."""
    need_gpu()
    case = fp8(sparse_lens(360), hk=4, qg=qg, seed=361 + qg + ql, q_dtype=q_dtype,
               query_len=ql)
    log(f"case fused balanced row slices ql={ql} qg={qg} q={q_dtype}")
    ws = uq.alloc_workspace(case.B, 4, ql, qg, 128, case.num_partitions, case.max_seq_len,
                            case.kv_format)
    ref = oracle_decode(case)
    got, _ = run_decode(case, workspace=ws)
    assert_decode_close(got, ref, f"fused row slices ql={ql} qg={qg}")
    assert not counters_of(ws).any()
    split, _ = run_decode(case, mode="split")
    assert_decode_close(split, ref, f"split row slices ql={ql} qg={qg}")


@pytest.mark.parametrize("ql,qg,hk", [(2, 16, 4), (4, 8, 8), (1, 48, 4), (1, 12, 4), (1, 40, 6),
                                      (2, 16, 3)])
def test_fused_query_rows_and_passes(ql, qg, hk):
    """Head-group runs (short batch, 16 partitions) with f16 row tiles: one tile (12
    rows), two (32 rows), row slices (40 rows at Hk = 6, 48 at Hk = 4); and, without
    head groups (Hk = 3), 32 rows in two launches of 16 rows, each a complete
    flash-combine that leaves the counters at zero for the next."""
    need_gpu()
    lens = (1, 2, 3, 255, 256, 257, 1000, 3000, 9000)
    case = fp8(lens, hk=hk, qg=qg, seed=330 + ql + qg, query_len=ql)
    log(f"case fused rows ql={ql} qg={qg} hk={hk}")
    got, _ = run_decode(case, P=16)
    assert_decode_close(got, oracle_decode(case), f"fused rows ql={ql} qg={qg}")


@pytest.mark.parametrize("P", [1, 3])
def test_fused_strided_partitions(P):
    """Few partitions: each owns several strided tile-groups and a head-group workgroup
    takes one partition (units of one partition each, slots per partition)."""
    need_gpu()
    case = fp8((0, 1, 300, 2049, 5000, 9001), hk=4, qg=8, seed=340 + P)
    got, _ = run_decode(case, P=P)
    assert np.all(got[0] == 0)
    assert_decode_close(got, oracle_decode(case), f"fused strided P={P}")


@pytest.mark.parametrize("qg,layout", [(8, "sparse"), (32, "sparse"), (48, "ragged"),
                                       (16, "ragged")])
def test_fused_repeat_bit_identical(qg, layout):
    """Repeated calls give the same output bit for bit: the unit that completes a sequence
    merges its slots' states in slot order whichever unit finished last.  The sparse batch
    spreads one 16k sequence over dozens of units; the ragged one splits most sequences
    once or twice (e4m3 tiles at 8 rows, f16 tiles at 16 and 32, row slices at 48)."""
    need_gpu()
    lens = sparse_lens(371 + qg) if layout == "sparse" else np.random.default_rng(
        372 + qg).integers(0, 9000, size=96)
    case = fp8(lens, hk=4, qg=qg, seed=373 + qg)
    log(f"case fused repeat qg={qg} {layout}")
    dev = device_case(case)
    q = q_tensor(case)
    first, _ = run_decode(case, dev=dev, q=q)
    assert_decode_close(first, oracle_decode(case), f"fused repeat qg={qg}")
    for i in range(5):
        got, _ = run_decode(case, dev=dev, q=q)
        assert np.array_equal(got, first), f"call {i + 1}"


def test_fused_graph_replay():
    """uq_paged_attention captured in a HIP graph: every replay, with eager work and
    synchronisations in between, gives the eager result bit for bit (the counters return
    to zero inside each replay; no memset node)."""
    need_gpu()
    case = fp8(sparse_lens(350), hk=4, qg=8, seed=351)
    dev = device_case(case)
    q = q_tensor(case)
    B, Hq, D = q.shape
    P = case.num_partitions
    ws = uq.alloc_workspace(B, 4, 1, 8, D, P, case.max_seq_len, case.kv_format)
    out = torch.empty(B, Hq, D, dtype=q.dtype, device="cuda")
    kw = dict(kv_format=case.kv_format, max_seq_len=case.max_seq_len, num_partitions=P,
              out=out, workspace=ws, softmax_scale=case.softmax_scale, k_scale=dev["ks"],
              v_scale=dev["vs"])
    eager, _ = run_decode(case, dev=dev, q=q, out=out, workspace=ws)
    assert_decode_close(eager, oracle_decode(case), "fused graph eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        uq.paged_attention(q, dev["cache"], dev["bt"], dev["sl"], **kw)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, eager), f"replay {i}"
        assert not counters_of(ws, B, 4).any()
        _ = (q.float() * 2).sum().item()      # eager work between replays
