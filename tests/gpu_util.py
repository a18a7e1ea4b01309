"""Helpers for the GPU parity tests: move a synthetic case to the device, run the HIP
path through the C ABI binding, and compare against the oracle."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from quantized_paged_attention_amd import synth

try:
    from quantized_paged_attention_amd import uq
except Exception:  # pragma: no cover
    uq = None

DEV = "cuda"
_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_value(name: str, key: str) -> float:
    """The number after `key` in tests/golden/<name> (lines starting with # are comments)."""
    with open(os.path.join(_GOLDEN, name)) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] == key:
                return float(parts[1])
    raise KeyError(f"{key} not in {name}")


# max|gpu - ref| <= TOL_DECODE max|ref|: the fp8 tolerance of the pa_decode_tile PR
TOL_DECODE = _golden_value("p3_fp8_tolerance.txt", "rel_to_max_abs_out")
TOL_INDEX = 1e-4       # relative to max|ref| over finite cells


def gpu_available() -> bool:
    return torch.cuda.is_available()


def need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def q_tensor(case, strided: bool = False) -> torch.Tensor:
    dt = torch.float32 if case.q_dtype == "f32" else torch.bfloat16
    q = torch.from_numpy(case.q).to(dt)
    if strided:
        # Q as a slice of a fused [B, Hq + 2 Hk, D] QKV projection
        B, Hq, D = q.shape
        big = torch.zeros(B, Hq + 2 * case.num_kv_heads, D, dtype=dt)
        big[:, :Hq] = q
        return big.to(DEV)[:, :Hq]
    return q.to(DEV)


def device_case(case):
    if case.kv_format == synth.FMT_FP8_E4M3:
        ks = torch.tensor([case.k_scale], dtype=torch.float32, device=DEV)
        vs = torch.tensor([case.v_scale], dtype=torch.float32, device=DEV)
    elif case.kv_format == synth.FMT_FP8_E4M3_TOK:
        ks = torch.from_numpy(case.k_scale_tok).to(DEV)
        vs = torch.from_numpy(case.v_scale_tok).to(DEV)
    else:
        ks = vs = None
    return dict(
        cache=torch.from_numpy(case.cache).to(DEV),
        bt=torch.from_numpy(case.block_table).to(DEV),
        sl=torch.from_numpy(case.seq_lens).to(DEV),
        ks=ks,
        vs=vs,
        rot=(torch.from_numpy(case.rot_signs).to(DEV) if case.rot_signs is not None else None),
    )


def run_decode(case, P=None, strided=False, dev=None, q=None, partials=None, out=None,
               mode=None, workspace=None):
    """HIP decode step; returns (out float64 numpy, partials or None).  mode "fused":
    uq_paged_attention (decode and flash-combine in one call, the default); "split":
    uq_paged_decode then uq_paged_reduce through partials (the default when partials are
    passed)."""
    dev = dev or device_case(case)
    P = P or case.num_partitions
    q = q if q is not None else q_tensor(case, strided)
    _, Hq, D = q.shape
    hk = case.num_kv_heads
    QL = case.query_len
    mode = mode or ("split" if partials is not None else "fused")
    kw = dict(kv_format=case.kv_format, max_seq_len=case.max_seq_len, num_partitions=P,
              out=out, softmax_scale=case.softmax_scale, k_scale=dev["ks"], v_scale=dev["vs"],
              rot_signs=dev["rot"], query_len=QL)
    if mode == "split":
        partials = partials or uq.alloc_partials(case.B, hk, QL * (Hq // hk), D, P)
        out = uq.paged_decode_reduce(q, dev["cache"], dev["bt"], dev["sl"], partials=partials,
                                     **kw)
    else:
        out = uq.paged_attention(q, dev["cache"], dev["bt"], dev["sl"], workspace=workspace, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), partials


def oracle_decode(case, P=0):
    from oracle import oracle
    return oracle.decode(case.q, case.cache, case.block_table, case.seq_lens,
                         num_kv_heads=case.num_kv_heads, kv_format=case.kv_format,
                         softmax_scale=case.softmax_scale, k_scale=case.k_scale,
                         v_scale=case.v_scale, rot_signs=case.rot_signs, num_partitions=P,
                         query_len=case.query_len, k_scale_tok=case.k_scale_tok,
                         v_scale_tok=case.v_scale_tok)


def oracle_decode_seqs(case, idx):
    """The oracle on the sequences idx only (all their query rows and heads): rows
    b * query_len + i of the output for b in idx, in that order."""
    from oracle import oracle
    idx = np.asarray(idx)
    QL = case.query_len
    rows = (idx[:, None] * QL + np.arange(QL)[None, :]).reshape(-1)
    ref = oracle.decode(case.q[rows], case.cache, case.block_table[idx], case.seq_lens[idx],
                        num_kv_heads=case.num_kv_heads, kv_format=case.kv_format,
                        softmax_scale=case.softmax_scale, k_scale=case.k_scale,
                        v_scale=case.v_scale, rot_signs=case.rot_signs, num_partitions=0,
                        query_len=QL, k_scale_tok=case.k_scale_tok,
                        v_scale_tok=case.v_scale_tok)
    return rows, ref


def rel_err(got, ref):
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def assert_decode_close(got, ref, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e = rel_err(got, ref)
    log(f"  {what}: max|err|/max|ref| = {e:.3e}")
    assert e <= TOL_DECODE, f"{what}: relative error {e:.3e} > {TOL_DECODE}"
    return e
