"""Every device buffer of a call placed where bit 31 of its address's low 32-bit word is
set.  The kernels build buffer resources from wave-uniform addresses split into two 32-bit
halves; a half widened as a signed int would spread that bit over the high word and point
the resource at the wrong address.  The caching allocator only sometimes hands out such
addresses, so each call here runs twice: once on buffers carved out of an arena at those
addresses, and once on ordinary allocations.  The two results must be bit-identical
(the kernels are deterministic), and each is compared with the oracle too."""

import numpy as np
import pytest
import torch

from quantized_paged_attention_amd import synth
from tests.gpu_util import (DEV, assert_decode_close, device_case, log, need_gpu, oracle_decode,
                            q_tensor, run_decode, uq)

pytestmark = pytest.mark.gpu

_HIGH = 1 << 31


class Arena:
    """A device allocation with a window of 2 GiB whose addresses all have bit 31 of the
    low word set; put() copies a tensor into the next 256-byte aligned spot of it."""

    def __init__(self):
        # 4 GiB + 2 GiB: a low word of exactly 0x80000000 lies within the first 4 GiB
        self.buf = torch.empty((1 << 32) + _HIGH, dtype=torch.uint8, device=DEV)
        base = self.buf.data_ptr()
        self.off = (_HIGH - (base & 0xFFFFFFFF)) % (1 << 32)
        self.end = self.off + _HIGH
        assert ((base + self.off) & 0xFFFFFFFF) == _HIGH

    def put(self, t):
        if t is None:
            return None
        t = t.contiguous()
        n = t.numel() * t.element_size()
        o = self.off
        assert o + n <= self.end, "arena window exhausted"
        self.off = (o + n + 255) & ~255
        v = self.buf[o:o + n].view(t.dtype).view(t.shape)
        v.copy_(t)
        assert (v.data_ptr() & _HIGH) and ((v.data_ptr() + max(n, 1) - 1) & _HIGH)
        return v


@pytest.fixture(scope="module")
def arena():
    need_gpu()
    a = Arena()
    yield a
    del a.buf
    torch.cuda.empty_cache()


def _decode_twice(arena, case, P, mode):
    """(high-address result, ordinary result) of one decode step."""
    dev_lo = device_case(case)
    q_lo = q_tensor(case)
    dev_hi = {k: arena.put(v) for k, v in dev_lo.items()}
    q_hi = arena.put(q_lo)
    rows, Hq, D = q_lo.shape
    out_hi = arena.put(torch.zeros(rows, Hq, D, dtype=q_lo.dtype, device=DEV))
    hk, QL = case.num_kv_heads, case.query_len
    kw = {}
    if mode == "split":
        kw["partials"] = tuple(arena.put(t)
                               for t in uq.alloc_partials(case.B, hk, QL * (Hq // hk), D, P))
    else:
        kw["workspace"] = arena.put(uq.alloc_workspace(case.B, hk, QL, Hq // hk, D, P,
                                                       case.max_seq_len, case.kv_format))
    hi, _ = run_decode(case, P=P, dev=dev_hi, q=q_hi, out=out_hi, mode=mode, **kw)
    lo, _ = run_decode(case, P=P, dev=dev_lo, q=q_lo, mode=mode)
    return hi, lo


def _check_pair(case, hi, lo, what):
    assert np.array_equal(hi, lo), f"{what}: high-address result differs from the ordinary one"
    assert_decode_close(hi, oracle_decode(case), what)


LENS = (1, 37, 200, 255, 256, 257, 1000, 3000)


@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("P,qg,scales", [(1, 8, "tensor"), (7, 8, "tensor"), (16, 32, "token"),
                                         (16, 4, "token")])
def test_fp8_high_addresses(arena, mode, P, qg, scales):
    kw = dict(scales="token", values="normal") if scales == "token" else dict(
        k_scale=0.05, v_scale=0.02, values="uniform_codes")
    case = synth.make_fp8_case("fp8_high_addr", 811 + P + qg, seq_lens=list(LENS),
                               num_kv_heads=2, qg=qg, q_dtype="f32", spare_blocks=5, **kw)
    log(f"case fp8 high addresses mode={mode} P={P} qg={qg} scales={scales}")
    hi, lo = _decode_twice(arena, case, P, mode)
    _check_pair(case, hi, lo, f"fp8 {mode} P={P} qg={qg}")


@pytest.mark.parametrize("rotate", [True, False])
def test_fp4_high_addresses(arena, rotate):
    case = synth.make_fp4_case("fp4_high_addr", 823, seq_lens=[1, 65, 300, 3000],
                               num_kv_heads=2, qg=8, rotate=rotate, spare_blocks=3)
    log(f"case fp4 high addresses rotate={rotate}")
    hi, lo = _decode_twice(arena, case, 16, "fused")
    _check_pair(case, hi, lo, f"fp4 rotate={rotate}")


def test_mtp_high_addresses(arena):
    case = synth.make_fp8_case("mtp_high_addr", 829, seq_lens=[5, 300, 2000], num_kv_heads=2,
                               qg=4, query_len=3, k_scale=0.05, v_scale=0.02, spare_blocks=3)
    log("case fp8 query_len=3 high addresses")
    hi, lo = _decode_twice(arena, case, 8, "split")
    _check_pair(case, hi, lo, "fp8 query_len=3")


def test_noalloc_high_addresses(arena):
    case = synth.make_fp8_case("noalloc_high_addr", 833, seq_lens=list(LENS), num_kv_heads=2,
                               qg=8, k_scale=0.05, v_scale=0.02, spare_blocks=3)
    log("case noalloc high addresses")
    dev_lo = device_case(case)
    q_lo = q_tensor(case)
    dev_hi = {k: arena.put(v) for k, v in dev_lo.items()}
    q_hi = arena.put(q_lo)
    out_hi = arena.put(torch.zeros_like(q_lo))
    kw = dict(kv_format=case.kv_format, max_seq_len=case.max_seq_len,
              num_partitions=case.num_partitions, softmax_scale=case.softmax_scale,
              query_len=case.query_len)
    uq.paged_attention_noalloc(q_hi, dev_hi["cache"], dev_hi["bt"], dev_hi["sl"], out=out_hi,
                               k_scale=dev_hi["ks"], v_scale=dev_hi["vs"], **kw)
    lo = uq.paged_attention_noalloc(q_lo, dev_lo["cache"], dev_lo["bt"], dev_lo["sl"],
                                    k_scale=dev_lo["ks"], v_scale=dev_lo["vs"], **kw)
    torch.cuda.synchronize()
    _check_pair(case, out_hi.double().cpu().numpy(), lo.double().cpu().numpy(), "noalloc")


@pytest.mark.parametrize("ql,h", [(1, 1), (8, 4)])
def test_index_high_addresses(arena, ql, h):
    from oracle import oracle
    case = synth.make_index_case("index_high_addr", 839 + ql, seq_lens=[1, 128, 129, 5000],
                                 query_len=ql, heads=h)
    log(f"case index high addresses ql={ql} h={h}")
    init = case.scores_init()
    res = []
    for put in (arena.put, lambda t: t):
        q = put(torch.from_numpy(case.q).to(DEV))
        pages = put(torch.from_numpy(case.pages).to(DEV))
        bt = put(torch.from_numpy(case.block_table).to(DEV))
        sl = put(torch.from_numpy(case.seq_lens).to(DEV))
        scores = put(torch.from_numpy(init.copy()).to(DEV))
        uq.index_score(q, pages, bt, sl, scores, query_len=ql)
        torch.cuda.synchronize()
        res.append(scores.cpu().numpy())
    assert np.array_equal(res[0].view(np.uint32), res[1].view(np.uint32))
    ref = oracle.index_score(case.q, case.pages, case.block_table, case.seq_lens,
                             query_len=ql, scores_init=init)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(res[0]), np.isneginf(ref))
    err = float(np.abs(res[0][fin] - ref[fin]).max() / np.abs(ref[fin]).max())
    log(f"  index ql={ql} h={h}: max|err|/max|ref| = {err:.3e}")
    assert err <= 1e-4
