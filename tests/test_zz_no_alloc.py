"""uq_paged_attention_noalloc (the no-allocation variant of uq_paged_attention, its
workspace in the library's per-GPU scratch) against uq_paged_attention with a workspace
of its own, on two calls in a row, the second with a smaller input, then a third larger
than the first (more arrival counters than either: the counters sit in a fixed region
that no other data ever touches); all against the oracle as well.  Runs alone in a
fresh process and after the other tests."""

import numpy as np
import pytest
import torch

from quantized_paged_attention_amd import synth, uq
from tests.gpu_util import (assert_decode_close, device_case, log, need_gpu,
                            oracle_decode, q_tensor)

pytestmark = pytest.mark.gpu


def fp8_case(lens, hk, qg, seed):
    return synth.make_fp8_case("noalloc", seed, seq_lens=list(lens), num_kv_heads=hk, qg=qg,
                               spare_blocks=5, k_scale=0.05, v_scale=0.02)


def run_both(case):
    dev = device_case(case)
    q = q_tensor(case)
    kw = dict(kv_format=case.kv_format, max_seq_len=case.max_seq_len,
              num_partitions=case.num_partitions, softmax_scale=case.softmax_scale,
              k_scale=dev["ks"], v_scale=dev["vs"], rot_signs=dev["rot"],
              query_len=case.query_len)
    ref = uq.paged_attention(q, dev["cache"], dev["bt"], dev["sl"], **kw)
    got = uq.paged_attention_noalloc(q, dev["cache"], dev["bt"], dev["sl"], **kw)
    torch.cuda.synchronize()
    return (got.float().cpu().numpy().astype(np.float64),
            ref.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("kind", ["fp8_fused", "fp8_wide", "fp4_split"])
def test_noalloc_matches_workspace_entry(kind):
    """Calls in a row on the shared scratch, the second smaller, the third larger: each
    output equals the workspace entry point's bit for bit (the same kernels; the fused
    merge folds a sequence's states in slot order whichever unit finishes last, so the
    result does not depend on timing) and the oracle within the decode tolerance."""
    need_gpu()
    rng = np.random.default_rng(500)
    if kind == "fp8_fused":
        big = fp8_case(rng.integers(1, 9000, size=96), hk=8, qg=8, seed=501)
        small = fp8_case((1, 700, 5000, 0, 257), hk=8, qg=8, seed=502)
        grow = fp8_case(rng.integers(0, 3000, size=128), hk=8, qg=8, seed=505)
    elif kind == "fp8_wide":
        # f16 row tiles: two per wave (32 rows), one (16 rows), two row slices (48 rows)
        big = fp8_case(rng.integers(1, 9000, size=40), hk=4, qg=32, seed=507)
        small = fp8_case((1, 700, 5000, 0, 257), hk=4, qg=16, seed=508)
        grow = fp8_case(rng.integers(0, 6000, size=64), hk=4, qg=48, seed=509)
    else:
        big = synth.make_fp4_case("noalloc4", 503, seq_lens=[300, 5000, 20000, 64], num_kv_heads=2,
                                  qg=16, head_dim=256, block_size=64, rotate=True, spare_blocks=3)
        small = synth.make_fp4_case("noalloc4", 504, seq_lens=[1000, 33], num_kv_heads=2,
                                    qg=8, head_dim=256, block_size=64, rotate=True,
                                    spare_blocks=3)
        grow = synth.make_fp4_case("noalloc4", 506, seq_lens=[900, 3000, 12, 7000, 260, 5],
                                   num_kv_heads=4, qg=4, head_dim=256, block_size=64,
                                   rotate=True, spare_blocks=3)
    for i, case in enumerate((big, small, grow)):
        log(f"case noalloc {kind} call {i} B={case.B}")
        got, ref = run_both(case)
        assert np.isfinite(got).all()
        ndiff = int((got != ref).sum())
        log(f"  noalloc vs workspace entry: {ndiff} differing elements")
        assert ndiff == 0
        assert_decode_close(got, oracle_decode(case), f"noalloc {kind} call {i}")
