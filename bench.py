"""Benchmark of the quantized paged-attention hot path on one MI355X.

Default workload (the headline): one decode step = uq_paged_attention (decode and
flash-combine; one launch for the fp8 head-group kernels) over the high-batch fp8 batch
(B=128, Hk=8, QG=8, D=128, L ~ U[4096, 16384], block 16, 64 partitions of 256 tokens,
per-tensor e4m3 K/V).  Other workloads (--workload): fp8_mid (B=16, L=16384),
fp8_high_tok (the high-batch shape with per-token f32 K and V scales: 264 algorithmic bytes
per (token, head)), fp4_d256_qg{6,8,16} (B=4, Hk=2, D=256, L=75000, 512 partitions, e2m1 +
e4m3 group scales, in-kernel rotation; decode + reduce), the same fp8 and FP4 shapes with
QL query rows per sequence (fp8_high_mtp{QL}_qg{QG}, fp4_d256_mtp{QL}_qg{QG}: each row has
its own causal window), nvfp4_index_ql{QL}_h{H} (32 requests, L ~ U[1024, 32768]: one
uq_index_score call is a step).  Inputs are generated once, copied to HBM, and are
resident before the timed region starts.  The KV cache (or the index pages) is held in as
many copies as make at least 1 GiB, and step i reads copy i mod n: no step finds its bytes
in L2 or the 256 MB MALL left there by the step before, as after a >= 1 GiB cache flush,
while the timed steps still run back to back.

Order of the passes, each of K steps: W warm-up steps (more until 0.3 s of them have run);
an instrumented pass with a HIP event before each step and after each kernel (per-kernel
means and percentiles, the step's median / p10 / p90); the timed bare pass (`value`,
`ms_per_step`: K steps back to back between two synchronisations); a HIP graph of the K
steps, and one of K launches of the dominant kernel alone, each timed by HIP events
around one replay (`us_per_step_graph`, `dominant_kernel_us_graph`; the latter is the
roofline's kernel time).

Prints ONE JSON line: value = effective KV-stream GB/s (algorithmic bytes of every visible
(token, head) / step wall time of the bare pass), with the dominant kernel's roofline
(HIP events around K graph-replayed launches of it) and the fp64 CPU oracle timed on a
bounded sample of the same workload.
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
COLD_BYTES = 1 << 30   # KV bytes cycled through before a copy is read again
WARMUP_S = 0.3         # least wall time of warm-up steps before the passes
METRIC = "µs/decode step + KV-stream GB/s (% of HBM peak) at B=128 ctx=16k"
CSRC = os.path.join(ROOT, "quantized_paged_attention_amd", "csrc")
COMMON_SRCS = ("uq_device.h", "uq_kernels.h", "uq_abi.cpp")
# kernel source and committed rocprofv3 traffic record of each workload family
KERNEL_SRC = {"fp8": "decode_fp8.hip", "fp4": "decode_fp4.hip", "index": "index_score.hip"}


def family(workload: str) -> str:
    if workload.startswith("nvfp4_index"):
        return "index"
    return "fp4" if workload.startswith("fp4") else workload.split("_")[0]


def source_hash(fam: str = "fp8") -> str:
    h = hashlib.sha256()
    for name in (KERNEL_SRC[fam],) + COMMON_SRCS:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 PMC
    record of this workload, if it was taken on the current kernel sources; else None."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != source_hash(family(workload)):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed_passes(fn, min_seconds: float, max_passes: int = 8):
    passes, t0 = 0, time.perf_counter()
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        fn()
        passes += 1
        print(f"cpu baseline: oracle pass {passes} done", file=sys.stderr, flush=True)
    return passes, time.perf_counter() - t0


def cpu_baseline_decode(case, n_seqs: int, min_seconds: float = 10.0):
    """fp64 oracle on the first n_seqs sequences (all kv heads) of the workload, repeated
    until at least min_seconds of wall time have been spent (at most 8 passes)."""
    from oracle import oracle
    sub = copy.copy(case)
    sub.q = case.q[:n_seqs * case.query_len]
    sub.block_table = case.block_table[:n_seqs]
    sub.seq_lens = case.seq_lens[:n_seqs]
    passes, dt = _timed_passes(
        lambda: oracle.decode(sub.q, sub.cache, sub.block_table, sub.seq_lens,
                              num_kv_heads=sub.num_kv_heads, kv_format=sub.kv_format,
                              softmax_scale=sub.softmax_scale, k_scale=sub.k_scale,
                              v_scale=sub.v_scale, rot_signs=sub.rot_signs,
                              query_len=sub.query_len, k_scale_tok=sub.k_scale_tok,
                              v_scale_tok=sub.v_scale_tok), min_seconds)
    return {"value": round(passes * sub.kv_bytes() / dt / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {n_seqs} of {case.B} sequences, all {case.num_kv_heads} kv heads "
                      f"({sub.kv_bytes() / 1e6:.1f} MB of KV) x {passes} passes, fp64, "
                      f"{dt:.2f} s wall"}


def cpu_baseline_index(case, min_seconds: float = 10.0):
    """fp64 oracle scorer on the whole index workload, repeated as above."""
    from oracle import oracle
    passes, dt = _timed_passes(
        lambda: oracle.index_score(case.q, case.pages, case.block_table, case.seq_lens,
                                   query_len=case.query_len, scores_init=case.scores_init()),
        min_seconds)
    return {"value": round(passes * case.unique_page_bytes() / dt / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"all {case.num_reqs} requests ({case.page_bytes() / 1e6:.1f} MB of "
                      f"pages) x {passes} passes, fp64, {dt:.2f} s wall"}


def copies_for(nbytes: int) -> int:
    """Copies of an nbytes input that together stream at least COLD_BYTES."""
    return max(1, -(-COLD_BYTES // max(1, nbytes)))


def make_case(workload: str):
    from quantized_paged_attention_amd import synth
    if workload == "fp8_high":
        return synth.fp8_high(), ("fp8_high: B=128 Hk=8 QG=8 D=128 L~U[4096,16384] block=16 "
                                  "P=64 per-tensor e4m3 K/V, bf16 Q")
    if workload == "fp8_high_tok":
        return synth.fp8_high_tok(), ("fp8_high_tok: B=128 Hk=8 QG=8 D=128 L~U[4096,16384] "
                                      "block=16 P=64 e4m3 K/V with per-token f32 K and V "
                                      "scales, bf16 Q")
    if workload.startswith("fp8_high_mtp"):
        ql, qg = (int(x) for x in workload[len("fp8_high_mtp"):].split("_qg"))
        return synth.fp8_high_mtp(ql, qg), (
            f"{workload}: B=128 Hk=8 QL={ql} query rows x QG={qg} D=128 L~U[4096,16384] "
            "block=16 P=64 per-tensor e4m3 K/V, bf16 Q, causal window per query row")
    if workload.startswith("fp4_d256_mtp") or workload.startswith("fp4ue_d256_mtp"):
        ue = workload.startswith("fp4ue")
        ql, qg = (int(x) for x in workload.split("_mtp")[1].split("_qg"))
        return synth.fp4_d256_mtp(ql, qg, "ue8m0" if ue else "e4m3"), (
            f"{workload}: B=4 Hk=2 QL={ql} query rows x QG={qg} D=256 L=75000 block=64 "
            f"P=512 e2m1 K/V with {'UE8M0' if ue else 'e4m3'} group-of-32 scales, 272-byte "
            "slot, rotated keys, bf16 Q, causal window per query row")
    if workload == "fp8_mid":
        return synth.fp8_mid(), ("fp8_mid: B=16 Hk=8 QG=8 D=128 L=16384 block=16 P=64 "
                                 "per-tensor e4m3 K/V, bf16 Q")
    if workload.startswith("fp4_d256_qg") or workload.startswith("fp4ue_d256_qg"):
        ue = workload.startswith("fp4ue")
        qg = int(workload.split("_qg")[1])
        return synth.fp4_d256(qg, "ue8m0" if ue else "e4m3"), (
            f"{workload}: B=4 Hk=2 QG={qg} D=256 L=75000 block=64 P=512 e2m1 K/V with "
            f"{'UE8M0' if ue else 'e4m3'} group-of-32 scales, 272-byte slot, rotated keys, "
            "bf16 Q")
    if workload.startswith("nvfp4_index_shared_ql"):
        ql, h = workload[len("nvfp4_index_shared_ql"):].split("_h")
        case = synth.nvfp4_index_shared(int(ql), int(h))
        return case, (f"{workload}: 32 requests QL={ql} H={h} D=128 L~U[9216,32768] sharing "
                      "their first 64 nvfp4 pages (a prompt prefix), 9216-byte pages, e4m3 Q; "
                      "bytes = distinct pages read once")
    if workload.startswith("nvfp4_index_ql"):
        ql, h = workload[len("nvfp4_index_ql"):].split("_h")
        case = synth.nvfp4_index(int(ql), int(h))
        return case, (f"{workload}: 32 requests QL={ql} H={h} D=128 L~U[1024,32768] "
                      "128-token nvfp4 pages (9216 B), e4m3 Q")
    raise SystemExit(f"bench.py: unknown workload {workload!r}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fp8_high",
                    help="fp8_high (default), fp8_mid, fp8_high_tok, fp4_d256_qg{6,8,16}, "
                         "fp4ue_d256_qg{6,8,16}, "
                         "fp8_high_mtp{QL}_qg{QG} (QL*QG <= 64), "
                         "fp4[ue]_d256_mtp{QL}_qg{QG} (QL*QG <= 16), "
                         "nvfp4_index_ql{1,2,4,8}_h{1,2,4}, nvfp4_index_shared_ql{QL}_h{H}")
    ap.add_argument("--cpu-seqs", type=int, default=128,
                    help="sequences of a decode workload the CPU oracle baseline runs")
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

    from quantized_paged_attention_amd import uq

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
    workload = args.workload
    fam = family(workload)
    case, desc = make_case(workload)
    stream = torch.cuda.current_stream()

    if fam == "index":
        q = torch.from_numpy(case.q).to(dev)
        pages0 = torch.from_numpy(case.pages).to(dev)
        inputs = [pages0] + [pages0.clone() for _ in range(copies_for(pages0.nbytes) - 1)]
        bt = torch.from_numpy(case.block_table).to(dev)
        sl = torch.from_numpy(case.seq_lens).to(dev)
        scores = torch.from_numpy(case.scores_init().copy()).to(dev)

        def step(pages, st):
            uq.index_score(q, pages, bt, sl, scores, query_len=case.query_len, stream=st)
        kernel_calls = [step]       # one kernel per step
        algo_bytes = case.unique_page_bytes()   # = page_bytes() when no page is shared
        names = ("index_score",)
        dtype = "f16"
    else:
        B, Hq, D, hk, P = case.B, case.Hq, case.D, case.num_kv_heads, case.num_partitions
        QL = case.query_len
        qdt = torch.float32 if case.q_dtype == "f32" else torch.bfloat16
        q = torch.from_numpy(case.q).to(qdt).to(dev)
        cache0 = torch.from_numpy(case.cache).to(dev)
        inputs = [cache0] + [cache0.clone() for _ in range(copies_for(cache0.nbytes) - 1)]
        bt = torch.from_numpy(case.block_table).to(dev)
        sl = torch.from_numpy(case.seq_lens).to(dev)
        is_fp8 = fam == "fp8"
        if case.k_scale_tok is not None:      # per-token scale tensors
            ks = torch.from_numpy(case.k_scale_tok).to(dev)
            vs = torch.from_numpy(case.v_scale_tok).to(dev)
        elif is_fp8:
            ks = torch.tensor([case.k_scale], dtype=torch.float32, device=dev)
            vs = torch.tensor([case.v_scale], dtype=torch.float32, device=dev)
        else:
            ks = vs = None
        rot = torch.from_numpy(case.rot_signs).to(dev) if case.rot_signs is not None else None
        max_len = case.max_seq_len
        ws = uq.alloc_workspace(B, hk, QL, case.QG, D, P, max_len, case.kv_format, dev)
        out = torch.empty(B * QL, Hq, D, dtype=qdt, device=dev)
        # one launch per step when the decode finishes the flash-combine itself (fp8 head
        # groups), else decode + reduce inside the same call
        fused = is_fp8 and hk % 4 == 0
        kw = dict(kv_format=case.kv_format, max_seq_len=max_len, num_partitions=P,
                  softmax_scale=case.softmax_scale, k_scale=ks, v_scale=vs, rot_signs=rot,
                  query_len=QL)

        def step(cache, st):
            uq.paged_attention(q, cache, bt, sl, out=out, workspace=ws, stream=st, **kw)

        if fused:
            kernel_calls = [step]
            names = ("decode_fp8_fused",)
        else:
            # the same two kernels uq_paged_attention launches, called one at a time so
            # that an event can sit between them
            po, pm, pl = uq.alloc_partials(B, hk, QL * case.QG, D, P, dev)

            def dec(cache, st):
                uq.paged_decode(q, cache, bt, sl, part_out=po, part_max=pm, part_sum=pl,
                                stream=st, **kw)

            def red(cache, st):
                uq.paged_reduce(po, pm, pl, sl, out, max_seq_len=max_len, query_len=QL,
                                stream=st)
            kernel_calls = [dec, red]
            names = (f"decode_{fam}", "reduce")
        algo_bytes = case.kv_bytes()
        dtype = "fp8" if is_fp8 else "f16"

    n_in = len(inputs)
    K = args.steps
    # Warm-up: W steps, and more until WARMUP_S of steps have run.  Right after the inputs
    # are loaded the first tens of milliseconds of steps run slower on MI355X (measured:
    # the first 30-step pass after 10 warm-up steps 442 us per step against 415 us right
    # after it, fp8 high batch), so a few steps alone leave the timed pass in that ramp.
    t_w, i = time.perf_counter(), 0
    while i < args.warmup or time.perf_counter() - t_w < WARMUP_S:
        step(inputs[i % n_in], stream)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_steps = i

    # Instrumented pass (untimed for `value`): an event before each step and after each
    # kernel, on the launch stream, gives per-kernel times and the spread of the step.
    nk = len(kernel_calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        for j, call in enumerate(kernel_calls):
            call(inputs[i % n_in], stream)
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    k_ms = [np.array([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]) for j in range(nk)]
    step_ev_ms = np.array([ev[i][0].elapsed_time(ev[i][nk]) for i in range(K)])

    # Timed region: K steps back to back with nothing else on the stream.  A HIP event
    # record between kernels costs the stream about 4 us on MI355X, so the events live in
    # the pass above and this one is bare.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(inputs[i % n_in], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # HIP-graph passes (host launch overhead out of the way): one graph of K whole steps,
    # and one of K launches of the dominant kernel alone (the decode, or the scorer),
    # each replayed once between two HIP events after a warm-up replay.  The second gives the roofline's kernel time: the mean duration of K
    # back-to-back launches.
    cap = torch.cuda.Stream()

    def graph_us(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(K):
                for call in calls:
                    call(inputs[i % n_in], cap)
        g.replay()                   # (replays run on the current stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        e0.record(cur)
        g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    step_graph_us = graph_us(kernel_calls)
    dom_graph_us = step_graph_us if nk == 1 else graph_us(kernel_calls[:1])

    step_ms = wall * 1e3 / K
    value = algo_bytes / (step_ms * 1e-3) / 1e9
    achieved = algo_bytes / (dom_graph_us * 1e-6) / 1e9
    pct = lambda a, p: round(float(np.percentile(a, p)) * 1e3, 2)

    res = {
        "metric": (METRIC if workload == "fp8_high" else
                   "µs/index call + K-page GB/s (% of HBM peak)" if fam == "index" else
                   "µs/decode step + KV-stream GB/s (% of HBM peak)"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_steps,
        "ms_per_step": round(step_ms, 5),
        "us_per_step": round(step_ms * 1e3, 2),
        "us_per_step_instrumented": round(wall_ev * 1e6 / K, 2),
        "us_per_step_graph": round(step_graph_us, 2),
        "step_us_events": {"median": pct(step_ev_ms, 50), "p10": pct(step_ev_ms, 10),
                           "p90": pct(step_ev_ms, 90)},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": desc, "algorithmic_bytes": algo_bytes,
                   "input_copies_cycled": n_in},
        "kernels_us": {f"{nm}_avg": round(float(k_ms[j].mean()) * 1e3, 2)
                       for j, nm in enumerate(names)},
        "dominant_kernel_us_graph": round(dom_graph_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(workload)},
    }
    res["kernels_us"][f"{names[0]}_median"] = pct(k_ms[0], 50)
    res["kernels_us"][f"{names[0]}_p10"] = pct(k_ms[0], 10)
    res["kernels_us"][f"{names[0]}_p90"] = pct(k_ms[0], 90)
    if fam != "index":
        res["config"].update(global_batch=case.B, seq_len_max=case.max_seq_len,
                             query_len=case.query_len)
    if not args.no_cpu:
        res["cpu_baseline"] = (cpu_baseline_index(case) if fam == "index" else
                               cpu_baseline_decode(case, min(args.cpu_seqs, case.B)))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
