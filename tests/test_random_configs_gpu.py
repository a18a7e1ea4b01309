"""Seeded random configurations of the decode step against the fp64 oracle: kv head counts
with and without head groups, query rows x heads from 1 to 64 (every row tiling: e4m3
tiles of 8, f16 tiles of 16, row slices, passes of 16), block sizes, partition counts,
empty and ragged lengths, per-tensor and per-token fp8 scales, both query dtypes, the
fused step and decode + reduce; FP4 D=256 with both scale codes, with and without the
query rotation.  Every output element is compared."""

import numpy as np
import pytest

from quantized_paged_attention_amd import synth
from tests.gpu_util import assert_decode_close, log, need_gpu, oracle_decode, run_decode

pytestmark = pytest.mark.gpu


def _lens(rng, B, top):
    pool = [0, 1, 2, 15, 16, 17, 255, 256, 257, 511, 512, 1000, 2047, 2049, top]
    lens = [int(rng.choice(pool)) if rng.random() < 0.4 else int(rng.integers(1, top + 1))
            for _ in range(B)]
    return tuple(min(x, top) for x in lens)


def _fp8_configs(n=80, seed=9100):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ql = int(rng.choice([1, 1, 1, 2, 3, 4]))
        qg = int(rng.integers(1, 64 // ql + 1))
        out.append(dict(
            i=i, hk=int(rng.choice([1, 2, 3, 4, 6, 8])), ql=ql, qg=qg,
            bs=int(rng.choice([16, 32, 64, 128, 256])), B=int(rng.integers(1, 13)),
            P=int(rng.choice([1, 2, 3, 7, 16, 64])), tok=bool(rng.random() < 0.3),
            q=str(rng.choice(["bf16", "f32"])), mode=str(rng.choice(["fused", "split"])),
            top=int(rng.choice([300, 3000, 5000])), seed=seed + 1 + i))
    return out


def _fp4_configs(n=24, seed=9300):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ql = int(rng.choice([1, 1, 2]))
        qg = int(rng.integers(1, 16 // ql + 1))
        out.append(dict(
            i=i, hk=int(rng.choice([1, 2, 4])), ql=ql, qg=qg, B=int(rng.integers(1, 5)),
            P=int(rng.choice([1, 4, 16, 64])), kind=str(rng.choice(["e4m3", "ue8m0"])),
            rot=bool(rng.random() < 0.7), top=int(rng.choice([700, 4000, 6000])),
            seed=seed + 1 + i))
    return out


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k not in ("seed", "i"))


@pytest.mark.parametrize("c", _fp8_configs(), ids=_id)
def test_random_fp8(c):
    need_gpu()
    rng = np.random.default_rng(c["seed"])
    lens = _lens(rng, c["B"], c["top"])
    kw = dict(scales="token", values="normal") if c["tok"] else dict(
        k_scale=0.05, v_scale=0.02, values="uniform_codes")
    case = synth.make_fp8_case("rand8", c["seed"], seq_lens=list(lens), num_kv_heads=c["hk"],
                               qg=c["qg"], block_size=c["bs"], q_dtype=c["q"],
                               query_len=c["ql"], spare_blocks=3, **kw)
    log(f"case random fp8 {_id(c)} lens={lens}")
    got, _ = run_decode(case, P=c["P"], mode=c["mode"])
    assert_decode_close(got, oracle_decode(case), f"random fp8 {c['i']}")


@pytest.mark.parametrize("c", _fp4_configs(), ids=_id)
def test_random_fp4(c):
    need_gpu()
    rng = np.random.default_rng(c["seed"])
    lens = _lens(rng, c["B"], c["top"])
    case = synth.make_fp4_case("rand4", c["seed"], seq_lens=list(lens), num_kv_heads=c["hk"],
                               qg=c["qg"], scale_kind=c["kind"], rotate=c["rot"],
                               query_len=c["ql"], spare_blocks=3)
    log(f"case random fp4 {_id(c)} lens={lens}")
    got, _ = run_decode(case, P=c["P"])
    assert_decode_close(got, oracle_decode(case), f"random fp4 {c['i']}")
