"""The C ABI: libuq.so loads, exports every function include/uq_paged.h declares, and its
host-side validation rejects bad arguments before launching anything (CPU only: no call
here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from quantized_paged_attention_amd import uq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uq_paged.h")

# fake, never-dereferenced device addresses (validation fails before any use)
FAKE = 0x10000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uq_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(uq.LIB_PATH):
        pytest.skip("libuq.so not built")
    return uq.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(uq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def decode_args(**over):
    a = dict(query=FAKE, q_dtype=uq.UQ_BF16, q_ss=64 * 128, q_sh=128, cache=FAKE, nb=16, bs=16,
             hk=8, slot=256, fmt=uq.UQ_KV_FP8_E4M3, ks=None, vs=None, rot=None, bt=FAKE,
             bt_stride=1024, sl=FAKE, B=4, Hq=64, D=128, max_len=16384, scale=0.0, P=64,
             po=FAKE, pm=FAKE, pl=FAKE, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(Hq=60), uq.UQ_ERR_INVALID_ARG),                 # Hq not a multiple of Hk
    (dict(Hq=8 * 65), uq.UQ_ERR_INVALID_ARG),             # QG > 64
    (dict(Hq=8 * 17, fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=256, slot=272),
     uq.UQ_ERR_UNSUPPORTED),                              # fp4 QG up to 16
    (dict(q_dtype=7), uq.UQ_ERR_INVALID_ARG),
    (dict(bs=24), uq.UQ_ERR_INVALID_ARG),
    (dict(bs=512), uq.UQ_ERR_INVALID_ARG),
    (dict(slot=255), uq.UQ_ERR_INVALID_ARG),
    (dict(slot=258), uq.UQ_ERR_INVALID_ARG),              # not 4-aligned
    (dict(P=0), uq.UQ_ERR_INVALID_ARG),
    (dict(max_len=-1), uq.UQ_ERR_INVALID_ARG),
    (dict(bt_stride=10), uq.UQ_ERR_INVALID_ARG),          # table row too short for max_len
    (dict(query=None), uq.UQ_ERR_INVALID_ARG),
    (dict(po=None), uq.UQ_ERR_INVALID_ARG),
    (dict(q_sh=0), uq.UQ_ERR_INVALID_ARG),
    (dict(q_sh=129), uq.UQ_ERR_INVALID_ARG),              # stride not 16-byte aligned
    (dict(fmt=9), uq.UQ_ERR_INVALID_ARG),
    (dict(D=64, slot=128), uq.UQ_ERR_UNSUPPORTED),        # fp8 supports D=128 only
    (dict(Hq=8 * 64, D=64, slot=128), uq.UQ_ERR_UNSUPPORTED),  # fp8 needs D = 128
    (dict(rot=FAKE), uq.UQ_ERR_UNSUPPORTED),              # rotation needs an fp4 cache
    (dict(fmt=uq.UQ_KV_FP4_E2M1_UE8M0S, D=128, slot=144, Hq=8 * 8), uq.UQ_ERR_UNSUPPORTED),
    (dict(fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=128, slot=144, Hq=8 * 4), uq.UQ_ERR_UNSUPPORTED),
    (dict(fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=256, slot=272, Hq=8 * 8, rot=FAKE + 8),
     uq.UQ_ERR_INVALID_ARG),                              # rotation signs not 16-byte aligned
    (dict(fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=256, slot=272, Hq=8 * 8, ks=FAKE), uq.UQ_ERR_INVALID_ARG),
    (dict(fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=256, slot=268, Hq=8 * 8), uq.UQ_ERR_INVALID_ARG),
    (dict(fmt=uq.UQ_KV_FP8_E4M3_TOKSCALE), uq.UQ_ERR_INVALID_ARG),        # scales required
    (dict(fmt=uq.UQ_KV_FP8_E4M3_TOKSCALE, ks=FAKE), uq.UQ_ERR_INVALID_ARG),
    (dict(fmt=uq.UQ_KV_FP8_E4M3_TOKSCALE, ks=FAKE, vs=FAKE + 2), uq.UQ_ERR_INVALID_ARG),
    (dict(fmt=uq.UQ_KV_FP8_E4M3_TOKSCALE, ks=FAKE, vs=FAKE, D=64, slot=128),
     uq.UQ_ERR_UNSUPPORTED),
    (dict(fmt=uq.UQ_KV_FP8_E4M3_TOKSCALE, ks=FAKE, vs=FAKE, Hq=8 * 65), uq.UQ_ERR_INVALID_ARG),
])
def test_decode_validation(lib, over, status):
    st = lib.uq_paged_decode(*decode_args(**over))
    assert st == status, lib.uq_last_error()
    assert lib.uq_last_error().decode()


def test_decode_zero_sequences_is_a_no_op(lib):
    assert lib.uq_paged_decode(*decode_args(B=0)) == uq.UQ_OK
    assert lib.uq_last_error() == b""


def decode_mtp_args(QL=2, **over):
    """uq_paged_decode_mtp arguments: decode_args with query_len after num_seqs."""
    a = decode_args(**over)
    return a[:17] + [QL] + a[17:]


@pytest.mark.parametrize("QL,over,status", [
    (0, dict(), uq.UQ_ERR_INVALID_ARG),                    # query_len < 1
    (-3, dict(), uq.UQ_ERR_INVALID_ARG),
    (9, dict(), uq.UQ_ERR_UNSUPPORTED),                    # fp8: 9 x 8 rows > 64
    (3, dict(Hq=8 * 22), uq.UQ_ERR_UNSUPPORTED),           # fp8: 3 x 22 rows > 64
    (2, dict(fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=256, slot=272, Hq=8 * 16), uq.UQ_ERR_UNSUPPORTED),
    (5, dict(fmt=uq.UQ_KV_FP4_E2M1_UE8M0S, D=256, slot=272, Hq=8 * 4), uq.UQ_ERR_UNSUPPORTED),
    (2, dict(Hq=60), uq.UQ_ERR_INVALID_ARG),               # checks of uq_paged_decode apply
])
def test_decode_mtp_validation(lib, QL, over, status):
    assert lib.uq_paged_decode_mtp(*decode_mtp_args(QL, **over)) == status
    assert lib.uq_last_error().decode()


def test_decode_mtp_zero_sequences_is_a_no_op(lib):
    assert lib.uq_paged_decode_mtp(*decode_mtp_args(4, B=0, Hq=8 * 2)) == uq.UQ_OK
    assert lib.uq_paged_decode_mtp(
        *decode_mtp_args(4, B=0, fmt=uq.UQ_KV_FP4_E2M1_E4M3S, D=256, slot=272, Hq=8 * 4)) == uq.UQ_OK


def reduce_args(**over):
    a = dict(po=FAKE, pm=FAKE, pl=FAKE, sl=FAKE, B=4, hk=8, qg=8, D=128, P=64, max_len=100,
             out=FAKE, dt=uq.UQ_BF16, o_ss=64 * 128, o_sh=128, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(qg=0), uq.UQ_ERR_INVALID_ARG), (dict(qg=65), uq.UQ_ERR_INVALID_ARG),
    (dict(D=64), uq.UQ_ERR_UNSUPPORTED), (dict(P=0), uq.UQ_ERR_INVALID_ARG),
    (dict(dt=5), uq.UQ_ERR_INVALID_ARG), (dict(out=None), uq.UQ_ERR_INVALID_ARG),
    (dict(o_sh=4), uq.UQ_ERR_INVALID_ARG), (dict(max_len=-5), uq.UQ_ERR_INVALID_ARG),
])
def test_reduce_validation(lib, over, status):
    assert lib.uq_paged_reduce(*reduce_args(**over)) == status


@pytest.mark.parametrize("QL,qg,status", [
    (0, 8, uq.UQ_ERR_INVALID_ARG), (2, 33, uq.UQ_ERR_INVALID_ARG), (5, 13, uq.UQ_ERR_INVALID_ARG),
    (3, 0, uq.UQ_ERR_INVALID_ARG),
])
def test_reduce_mtp_validation(lib, QL, qg, status):
    a = reduce_args(qg=qg)
    assert lib.uq_paged_reduce_mtp(*(a[:6] + [QL] + a[6:])) == status


def test_reduce_mtp_zero_sequences_is_a_no_op(lib):
    a = reduce_args(B=0, qg=4)
    assert lib.uq_paged_reduce_mtp(*(a[:6] + [4] + a[6:])) == uq.UQ_OK


def index_args(**over):
    a = dict(q=FAKE, q_st=512, q_sh=128, pages=FAKE, pstride=9216, npages=100, bt=FAKE,
             bt_stride=256, sl=FAKE, R=32, QL=2, H=4, D=128, init=0, local=0, scores=FAKE,
             s_sh=64 * 256, s_st=256, max_blocks=256, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(H=3), uq.UQ_ERR_INVALID_ARG), (dict(QL=16, H=4), uq.UQ_ERR_INVALID_ARG),
    (dict(QL=0), uq.UQ_ERR_INVALID_ARG), (dict(D=64), uq.UQ_ERR_UNSUPPORTED),
    (dict(init=1), uq.UQ_ERR_UNSUPPORTED), (dict(local=2), uq.UQ_ERR_UNSUPPORTED),
    (dict(pstride=9200), uq.UQ_ERR_INVALID_ARG), (dict(pstride=9224), uq.UQ_ERR_INVALID_ARG),
    (dict(q_st=100), uq.UQ_ERR_INVALID_ARG), (dict(scores=None), uq.UQ_ERR_INVALID_ARG),
    (dict(npages=0), uq.UQ_ERR_INVALID_ARG),
    (dict(s_st=255), uq.UQ_ERR_INVALID_ARG),              # score rows overlap
    (dict(s_sh=63 * 256 + 255), uq.UQ_ERR_INVALID_ARG),   # heads' score planes overlap
    (dict(QL=32, H=1, q_st=1 << 27), uq.UQ_ERR_UNSUPPORTED),  # query rows past 2^31 bytes
])
def test_index_validation(lib, over, status):
    assert lib.uq_index_score(*index_args(**over)) == status


def test_workspace_bytes(lib):
    n = uq.decode_workspace_bytes(128, 8, 8, 128, 64)
    rows = 128 * 8 * 64 * 8
    assert n == rows * 128 * 2 + 2 * rows * 4
    assert uq.decode_workspace_bytes(1, 0, 8, 128, 64) == 0


def test_binding_rejects_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        uq.paged_decode(q, torch.zeros(1, 16, 1, 256, dtype=torch.uint8),
                        torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32),
                        kv_format=0, max_seq_len=1, num_partitions=1,
                        part_out=torch.zeros(1, 1, 1, 8, 128, dtype=torch.bfloat16),
                        part_max=torch.zeros(1, 1, 1, 8), part_sum=torch.zeros(1, 1, 1, 8))


def test_binding_rejects_column_sliced_tables(lib):
    """A column slice of a wider block table keeps the wide row stride, which is all the C
    ABI sees; the binding checks the view's own width."""
    import torch
    wide = torch.zeros(1, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="columns"):
        uq.paged_decode(torch.zeros(1, 8, 128, dtype=torch.bfloat16),
                        torch.zeros(8, 16, 1, 256, dtype=torch.uint8), wide[:, :2],
                        torch.ones(1, dtype=torch.int32), kv_format=0, max_seq_len=100,
                        num_partitions=1,
                        part_out=torch.zeros(1, 1, 1, 8, 128, dtype=torch.bfloat16),
                        part_max=torch.zeros(1, 1, 1, 8), part_sum=torch.zeros(1, 1, 1, 8))
    with pytest.raises(ValueError, match="columns"):
        uq.index_score(torch.zeros(1, 1, 128, dtype=torch.uint8),
                       torch.zeros(2, 9216, dtype=torch.uint8), wide[:, :2],
                       torch.ones(1, dtype=torch.int32), torch.zeros(1, 1, 4),
                       query_len=1)


def attention_args(ws_bytes=1 << 30, **over):
    """uq_paged_attention arguments: decode_mtp_args without the partials, then the
    workspace and the output."""
    a = dict(ws=FAKE * 16, ws_bytes=ws_bytes, out=FAKE, o_ss=64 * 128, o_sh=128, stream=None)
    d = {k: v for k, v in over.items() if k not in a}
    a.update({k: v for k, v in over.items() if k in a})
    base = decode_mtp_args(QL=1, **d)[:-4]          # drop part_out, part_max, part_sum, stream
    return base + list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(ws=None), uq.UQ_ERR_INVALID_ARG),
    (dict(ws=FAKE * 16 + 16), uq.UQ_ERR_INVALID_ARG),   # workspace not 256-byte aligned
    (dict(ws_bytes=4096), uq.UQ_ERR_INVALID_ARG),       # below what the call needs
    (dict(out=None), uq.UQ_ERR_INVALID_ARG),
    (dict(out=FAKE + 8), uq.UQ_ERR_INVALID_ARG),
    (dict(o_sh=100), uq.UQ_ERR_INVALID_ARG),
    (dict(o_ss=0), uq.UQ_ERR_INVALID_ARG),
    (dict(Hq=60), uq.UQ_ERR_INVALID_ARG),
    (dict(fmt=9), uq.UQ_ERR_INVALID_ARG),
    (dict(P=0), uq.UQ_ERR_INVALID_ARG),
    (dict(bs=24), uq.UQ_ERR_INVALID_ARG),               # decode checks still apply
    (dict(D=64, slot=128), uq.UQ_ERR_UNSUPPORTED),
])
def test_attention_validation(lib, over, status):
    st = lib.uq_paged_attention(*attention_args(**over))
    assert st == status, lib.uq_last_error()
    assert lib.uq_last_error().decode()


def test_attention_zero_sequences_is_a_no_op(lib):
    assert lib.uq_paged_attention(*attention_args(B=0, ws=None, out=None)) == uq.UQ_OK


def test_attention_workspace_bytes(lib):
    """A fixed 256 KiB counter region, then the fused states (fp8 head groups) or the
    decode partials.  With no GPU the planner assumes 256 compute units: the fp8
    high-batch shape takes balanced slices, 128 per head group, so 128 + 127 state slots
    of one row tile (8 rows of e4m3 codes, or 16 rows in f16 at QG=16); QG=32 takes two
    16-row tiles per state; QG=64 two row slices per kv head (four head groups of two
    heads, two workgroups per compute unit: still 128 slices per group)."""
    up = lambda x: (x + 255) // 256 * 256
    counters = 256 << 10
    state = 8 * 64 * 16 + 2 * 64 * 4
    n = uq.attention_workspace_bytes(128, 8, 1, 8, 128, 64, 16384, uq.UQ_KV_FP8_E4M3)
    assert n == counters + up(255 * 8 * 1 * state)
    n = uq.attention_workspace_bytes(128, 8, 1, 16, 128, 64, 16384, uq.UQ_KV_FP8_E4M3)
    assert n == counters + up(255 * 8 * 1 * state)
    n = uq.attention_workspace_bytes(128, 8, 1, 32, 128, 64, 16384, uq.UQ_KV_FP8_E4M3)
    assert n == counters + up(255 * 8 * 2 * state)
    n = uq.attention_workspace_bytes(128, 8, 1, 64, 128, 64, 16384, uq.UQ_KV_FP8_E4M3)
    assert n == counters + up(255 * 8 * 2 * 2 * state)
    # fp8 with an odd head count and fp4: decode partials after the counters
    for fmt, hk, D in ((uq.UQ_KV_FP8_E4M3, 3, 128), (uq.UQ_KV_FP4_E2M1_E4M3S, 2, 256)):
        n = uq.attention_workspace_bytes(4, hk, 2, 8, D, 512, 75000, fmt)
        assert n == counters + uq.decode_workspace_bytes(4, hk, 16, D, 512)
    # more arrival counters than the region holds: the decode + reduce layout
    n = uq.attention_workspace_bytes(9000, 8, 1, 8, 128, 64, 16384, uq.UQ_KV_FP8_E4M3)
    assert n == counters + uq.decode_workspace_bytes(9000, 8, 8, 128, 64)
    assert uq.attention_workspace_bytes(4, 2, 0, 8, 256, 512, 75000, 1) == 0


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """uq_paged_attention_noalloc refuses, before any HIP call, sizes whose workspace
    exceeds its 64 MiB scratch."""
    big_B = 1 << 20
    assert uq.attention_workspace_bytes(big_B, 2, 1, 16, 256, 512, 75000,
                                        uq.UQ_KV_FP4_E2M1_E4M3S) > (64 << 20)
    st = lib.uq_paged_attention_noalloc(
        FAKE, uq.UQ_BF16, 32 * 256, 256, FAKE, 1, 64, 2, 272, uq.UQ_KV_FP4_E2M1_E4M3S, None,
        None, None, FAKE, 1172, FAKE, big_B, 1, 32, 256, 75000, 0.0, 512, FAKE, 32 * 256, 256,
        None)
    assert st == uq.UQ_ERR_INVALID_ARG
    assert "no-allocation scratch" in lib.uq_last_error().decode()
