"""Benchmark of one quantized paged-attention decode step on one MI355X.

A step is uq_paged_decode + uq_paged_reduce over one batch of the high-batch fp8
workload (B=128, Hk=8, QG=8, D=128, L ~ U[4096, 16384], block 16, 64 partitions of 256
tokens, per-tensor e4m3 K/V).  Inputs are generated once, copied to HBM, and are
resident before the timed region starts.

Prints ONE JSON line: value = effective KV-stream GB/s (KV code bytes of every visible
(token, head) / step time), with the decode kernel's roofline (HIP events on the launch
stream) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import copy
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "µs/decode step + KV-stream GB/s (% of HBM peak) at B=128 ctx=16k"
CSRC = os.path.join(ROOT, "quantized_paged_attention_amd", "csrc")
# Sources that decide the decode kernel's code and launch shape.
DECODE_SRCS = ("decode_fp8.hip", "uq_device.h", "uq_kernels.h", "uq_abi.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_fp8_high_traffic.json")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SRCS:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(units_per_launch: float):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_source_sha256_16") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(case, n_seqs: int, min_seconds: float = 10.0):
    """fp64 oracle on the first n_seqs sequences (all kv heads) of the workload, repeated
    until at least min_seconds of wall time have been spent (at most 8 passes)."""
    from oracle import oracle
    sub = copy.copy(case)
    sub.q = case.q[:n_seqs]
    sub.block_table = case.block_table[:n_seqs]
    sub.seq_lens = case.seq_lens[:n_seqs]
    passes, t0 = 0, time.perf_counter()
    while passes < 8 and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.decode(sub.q, sub.cache, sub.block_table, sub.seq_lens,
                      num_kv_heads=sub.num_kv_heads, kv_format=sub.kv_format,
                      softmax_scale=sub.softmax_scale, k_scale=sub.k_scale,
                      v_scale=sub.v_scale)
        passes += 1
        print(f"cpu baseline: oracle pass {passes} done", file=sys.stderr, flush=True)
    dt = time.perf_counter() - t0
    threads = oracle.num_threads()
    return {"value": round(passes * sub.kv_bytes() / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"first {n_seqs} of {case.B} sequences, all {case.num_kv_heads} kv heads "
                      f"({sub.kv_bytes() / 1e6:.1f} MB of KV) x {passes} passes, fp64, "
                      f"{dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seqs", type=int, default=128,
                    help="sequences of the workload the CPU oracle baseline runs")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 launches), "
                         "the known-size kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only (the decode path needs no "
              "cross-GPU exchange); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_paged_attention_amd import synth, uq

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}),
              flush=True)
        return

    uq.load_library()
    dev = "cuda"
    case = synth.fp8_high()
    B, Hq, D, hk, P = case.B, case.Hq, case.D, case.num_kv_heads, case.num_partitions
    q = torch.from_numpy(case.q).to(torch.bfloat16).to(dev)
    cache = torch.from_numpy(case.cache).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seq_lens).to(dev)
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device=dev)
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device=dev)
    po, pm, pl = uq.alloc_partials(B, hk, case.QG, D, P, dev)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    max_len = case.max_seq_len
    stream = torch.cuda.current_stream()

    def decode():
        uq.paged_decode(q, cache, bt, sl, kv_format=case.kv_format, max_seq_len=max_len,
                        num_partitions=P, part_out=po, part_max=pm, part_sum=pl,
                        softmax_scale=case.softmax_scale, k_scale=ks, v_scale=vs,
                        stream=stream)

    def reduce():
        uq.paged_reduce(po, pm, pl, sl, out, max_seq_len=max_len, stream=stream)

    for _ in range(args.warmup):
        decode()
        reduce()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        decode()
        ev[i][1].record(stream)
        reduce()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dec_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    red_ms = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])
    step_ms = wall * 1e3 / K
    kv_bytes = case.kv_bytes()
    value = kv_bytes / (step_ms * 1e-3) / 1e9
    dec_avg = float(dec_ms.mean())
    achieved = kv_bytes / (dec_avg * 1e-3) / 1e9
    traffic = measured_traffic(1)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "us_per_step": round(step_ms * 1e3, 2),
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": "fp8_high: B=128 Hk=8 QG=8 D=128 L~U[4096,16384] block=16 P=64 "
                        "per-tensor e4m3 K/V, bf16 Q",
            "kv_bytes": kv_bytes,
            "global_batch": B,
            "seq_len_max": max_len,
        },
        "kernels_us": {"decode_fp8_avg": round(dec_avg * 1e3, 2),
                       "decode_fp8_median": round(float(np.median(dec_ms)) * 1e3, 2),
                       "reduce_avg": round(float(red_ms.mean()) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(case, min(args.cpu_seqs, B))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
