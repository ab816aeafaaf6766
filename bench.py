#!/usr/bin/env python3
"""Throughput of the In-Place TTT fast-weight MLP layer (forward) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode MODE]

One step = one call of the whole layer (S1 SwiGLU, S2 conv + target, the
chunk-wise fast-weight recurrence S3/S4) over one batch of synthetic inputs
that are already resident in HBM.  Prints ONE JSON line on stdout:
tokens/s over the timed steps, the roofline position of the dominant kernel
(timed with HIP events inside the library, on the stream it runs on), and the
fp64 CPU oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("chunk_wise_weight_chunked_amd/csrc/kernels.hip",
                "chunk_wise_weight_chunked_amd/csrc/gemm_core.h"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stage_work(w, group: int) -> dict:
    """Algorithmic flops per launch of each kernel (and the chunks it covers)."""
    B, T, C, d, f = w.batch, w.seq_len, w.chunk, w.d_model, w.d_ff
    tok = B * T
    chunk_tokens = B * min(group * C, T)  # tokens one prefix/down launch covers (full groups)
    return {
        "swiglu": 4.0 * tok * d * f,
        "target": 2.0 * tok * d * d,
        "prefix_update": 2.0 * chunk_tokens * d * f,
        "down_proj": 2.0 * chunk_tokens * d * f,
    }


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, inp) -> dict:
    """The oracle as it stands, sequential form, on the first chunk(s) of
    sequence 0 (a causal prefix of the same workload)."""
    import oracle
    from chunk_wise_weight_chunked_amd import synth

    oracle.build(force=False)
    per_tok = 8.0 * w.d_model * w.d_ff + 2.0 * w.d_model ** 2
    n = w.chunk
    # aim at ~10-30 s of host work at a conservative 1 GFLOP/s per thread
    threads = oracle.num_threads()
    budget = 15.0 * 1e9 * threads
    chunks = max(1, min(w.n_chunks, int(budget // (per_tok * n))))
    m = chunks * n
    ni = {k: synth.to_numpy_f32(inp[k][0, :m] if k in ("H", "X0") else inp[k])
          for k in ("H", "X0", "W_gate", "W_up", "W_down0", "taps", "W_target")}
    t0 = time.perf_counter()
    oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"], ni["taps"],
                   ni["W_target"], w.eta, w.chunk, form="sequential")
    dt = time.perf_counter() - t0
    return {"value": m / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"sequential fp64 oracle on the first {chunks} chunk(s) ({m} tokens) of "
                      f"sequence 0 of {w.name}; {dt:.1f} s",
            "seconds": dt}


def calib_copy(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {nbytes} bytes x {reps}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_4b_128k")
    ap.add_argument("--mode", default="auto", choices=["auto", "sequential", "chunk_parallel"])
    ap.add_argument("--max-group", type=int, default=0, help="chunks per group (0 = all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is described in DESIGN.md, not built)",
              file=sys.stderr)
        return 2

    import torch
    if args.calib_copy:
        calib_copy(args.calib_copy, max(1, args.steps))
        return 0

    from chunk_wise_weight_chunked_amd import synth
    from chunk_wise_weight_chunked_amd import ttt_mlp as tm

    w = synth.WORKLOADS[args.workload]
    if not torch.cuda.is_available():
        log("no GPU available")
        return 1
    tm.load()
    log(f"[bench] workload {w.name}: drawing inputs")
    inp = synth.workload_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items()}
    B, T, d, f, K = w.batch, w.seq_len, w.d_model, w.d_ff, w.conv_k
    desc = tm.make_desc(B, T, d, f, w.chunk, K, w.eta, w.dtype, args.mode, init_from_w0=1)
    ws = tm.alloc_workspace(desc, args.max_group)
    group = tm.ttt_mlp_group_size(desc, ws.numel())
    O = torch.empty_like(dev["H"])
    W = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        tm.ttt_mlp_forward_batched(desc, dev["H"], dev["X0"], dev["W_gate"], dev["W_up"],
                                   dev["W_down0"], dev["taps"], dev["W_target"], O, W, ws,
                                   stream=stream)

    log(f"[bench] warmup {args.warmup} (group {group} of {w.n_chunks} chunks)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tm.ttt_profile_read()  # drop anything recorded so far
    tm.ttt_profile_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    tm.ttt_profile_enable(False)
    ms_total = start.elapsed_time(end)
    stages = tm.ttt_profile_read()
    ms_step = ms_total / args.steps
    tokens = w.tokens
    value = tokens / (ms_step / 1e3)
    dtype = "bf16" if w.dtype == torch.bfloat16 else "f32"
    peak = PEAK_TFLOPS[dtype]
    log(f"[bench] {ms_step:.3f} ms/step, {value / 1e6:.3f} M tokens/s")

    work = stage_work(w, group)
    per_stage = {}
    for name, (ms, n) in stages.items():
        if n == 0:
            continue
        avg = ms / n
        entry = {"ms_per_launch": avg, "launches_per_step": n / args.steps}
        if name in work:
            tf = work[name] / (avg / 1e3) / 1e12
            entry.update({"tflops": tf, "frac_of_peak": tf / peak})
        per_stage[name] = entry
        log(f"  {name:14s} {avg:9.3f} ms x {n / args.steps:g}/step  "
            + (f"{entry['tflops']:8.1f} TFLOP/s ({entry['frac_of_peak']:.1%})" if "tflops" in entry else ""))
    dom = max((k for k in per_stage if k in work),
              key=lambda k: per_stage[k]["ms_per_launch"] * per_stage[k]["launches_per_step"])
    ach = per_stage[dom]["tflops"]
    roofline = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": peak,
                "unit": "TFLOP/s", "frac": ach / peak,
                "traffic": traffic_for(dom, w.name),
                "flops_per_launch": work[dom],
                "ms_per_launch": per_stage[dom]["ms_per_launch"]}
    layer_frac = w.flops() / (ms_step / 1e3) / (peak * 1e12)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle) ...")
        cpu = cpu_baseline(w, inp)
        log(f"[bench] oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": "TTT-MLP layer tokens/sec at d=2560,f=9728,128K ctx; % MFMA/HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": T, "chunk": w.chunk,
                   "d_model": d, "d_ff": f, "conv_k": K, "eta": w.eta, "mode": args.mode,
                   "group": group, "state": "fp32"},
        "layer_mfma_frac": layer_frac,
        "roofline": roofline,
        "stages": per_stage,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
