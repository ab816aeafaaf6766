#!/usr/bin/env python3
"""Throughput of the In-Place TTT fast-weight MLP layer (forward) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode MODE]

One step = one call of the whole layer (S1 SwiGLU, S2 conv + target, the
chunk-wise fast-weight recurrence S3/S4) over one batch of synthetic inputs
that are already resident in HBM.  With --segment L a step instead streams the
same sequences through the streaming entry point in calls of L tokens
(--segment-calls n: only the first n calls, e.g. a decode rate with L = 1).  Prints ONE JSON line on stdout:
tokens/s over the timed steps, the roofline position of the dominant kernel
(timed with HIP events inside the library, on the stream it runs on), and the
fp64 CPU oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
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
                "chunk_wise_weight_chunked_amd/csrc/gemm_core.h",
                "chunk_wise_weight_chunked_amd/csrc/epilogue.h"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _launches(w, group: int, split: bool, per_chunk: bool) -> list:
    """The group pipeline's launches in order, as the library issues them:
    (stage, (scan tokens, scan chunks), (output tokens, output chunks)), token
    and chunk counts over all sequences.  Launch g scans group g and computes
    the outputs of group g - 1; sequential mode (per_chunk) scans one chunk
    per launch, the first chunk's launch carrying the previous group's
    outputs.  split: the first launch also projects the later tokens."""
    B, T, C, N = w.batch, w.seq_len, w.chunk, w.n_chunks

    def toks(c0, cn):
        return B * (min(T, (c0 + cn) * C) - c0 * C)

    groups = -(-N // group)
    out = []
    for g in range(groups + 1):
        g0, a0 = g * group, (g - 1) * group
        gc = min(group, N - g0) if g < groups else 0
        ac = min(group, N - a0) if g > 0 else 0
        apply = (toks(a0, ac), ac * B) if ac else (0, 0)
        if per_chunk and gc > 1:
            for j in range(gc):
                o = apply if j == 0 else (0, 0)
                kind = "scan_target" if (g == 0 and j == 0 and split) else \
                    ("scan_apply" if o[0] else "prefix_update")
                out.append((kind, (toks(g0 + j, 1), B), o))
            continue
        scan = (toks(g0, gc), gc * B) if gc else (0, 0)
        if g == 0 and split:
            kind = "scan_target"
        else:
            kind = "scan_apply" if gc and ac else ("prefix_update" if gc else "down_proj")
        out.append((kind, scan, apply))
    return out


def _split_tokens(w, group: int) -> int:
    """Tokens (all sequences) the target stage projects when the rest of the
    projection runs next to the first group's scan (scan_target)."""
    return w.batch * min(w.seq_len, group * w.chunk)


def _pipeline_average(w, group, split, per_chunk, scan_cost, apply_cost) -> dict:
    """Per-launch averages over each pipeline stage's launches."""
    tot, cnt = {}, {}
    for kind, scan, apply in _launches(w, group, split, per_chunk):
        c = (scan_cost(*scan) if scan[0] else 0.0) + (apply_cost(*apply) if apply[0] else 0.0)
        tot[kind] = tot.get(kind, 0.0) + c
        cnt[kind] = cnt.get(kind, 0) + 1
    return {k: tot[k] / cnt[k] for k in tot}


def stage_work(w, group: int, split: bool = False, per_chunk: bool = False) -> dict:
    """Algorithmic flops per launch of each kernel.  split: the first group's
    scan ran next to the projection of the later tokens (scan_target);
    per_chunk: sequential mode's schedule."""
    B, T, d, f = w.batch, w.seq_len, w.d_model, w.d_ff
    tok = B * T
    out = {"swiglu": 4.0 * tok * d * f, "target": 2.0 * tok * d * d}
    out.update(_pipeline_average(w, group, split, per_chunk, lambda t, n: 2.0 * t * d * f,
                                 lambda t, n: 2.0 * t * d * f))
    if split:
        t0 = _split_tokens(w, group)
        out["target"] = 2.0 * t0 * d * d
        out["scan_target"] += 2.0 * (tok - t0) * d * d
    return out


def stage_bytes(w, group: int, split: bool = False, per_chunk: bool = False) -> dict:
    """Algorithmic HBM bytes per launch of each kernel: every operand read once
    and every result written once (the fp32 state once per scan launch)."""
    B, T, C, d, f = w.batch, w.seq_len, w.chunk, w.d_model, w.d_ff
    e = 2 if w.dtype == torch_bf16() else 4
    tok = B * T
    out = {
        "state_reset": e * d * f + 4 * B * d * f,
        "swiglu": e * tok * (d + f) + e * 2 * f * d,
        "target": e * tok * 2 * d + e * d * d,
    }
    out.update(_pipeline_average(
        w, group, split, per_chunk,
        lambda t, n: e * t * (d + f) + e * n * d * f + 8 * B * d * f,
        lambda t, n: e * t * (f + d) + e * n * d * f))
    if split:
        t0 = _split_tokens(w, group)
        out["target"] = e * t0 * 2 * d + e * d * d
        out["scan_target"] += e * (tok - t0) * 2 * d + e * d * d
    return out


def hbm_bound(flops: float, nbytes: float, dtype: str) -> bool:
    """A kernel is HBM-bound when its algorithmic flops per byte are below the
    ridge: the MFMA peak for its dtype over the HBM peak."""
    return flops / nbytes < PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)


def torch_bf16():
    import torch
    return torch.bfloat16


# layer stage -> the kernel's name as rocprofv3 prints it (prefix match)
# (the scan-only, fused and output-only launches of the group pipeline are
# one kernel; its median dispatch is a fused one when there are >= 3 groups)
STAGE_KERNELS = {
    "state_reset": "void ttt::state_reset_kernel",
    "swiglu": "void ttt::swiglu_kernel",
    "target": "void ttt::target_kernel",
    "scan_apply": "void ttt::scan_apply_kernel",
    "scan_target": "void ttt::scan_target_kernel",
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"layer_{workload}_traffic.json")


def traffic_for(stage: str, workload: str):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    counter runs, if they were taken on the current kernel sources; else None."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(stage)
    return None if k is None else k["bytes_per_launch"]


def _counter_medians(csv_path: str) -> dict:
    """Median counter value per kernel name of a rocprofv3 counter_collection.csv."""
    import csv
    import statistics
    vals = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def write_traffic(workload: str, fetch_csv: str, write_csv: str, cfetch_csv: str,
                  cwrite_csv: str, copy_bytes: int, commands: list) -> dict:
    """Turn four rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, in KiB per
    dispatch, on the layer and on a plain copy of copy_bytes) into bytes per
    launch of each stage's kernel, each counter scaled by copy_bytes over what
    it read for the copy."""
    def scale(csv_path):
        m = _counter_medians(csv_path)
        kib = next(v for k, v in m.items() if k.startswith(COPY_KERNEL))
        return kib, copy_bytes / (kib * 1024.0)
    cf_kib, f_scale = scale(cfetch_csv)
    cw_kib, w_scale = scale(cwrite_csv)
    fetch, write = _counter_medians(fetch_csv), _counter_medians(write_csv)
    kernels = {}
    for stage, prefix in STAGE_KERNELS.items():
        fk = [v for k, v in fetch.items() if k.startswith(prefix)]
        wk = [v for k, v in write.items() if k.startswith(prefix)]
        if not fk or not wk:
            continue
        fb, wb = fk[0] * 1024.0 * f_scale, wk[0] * 1024.0 * w_scale
        kernels[stage] = {"fetch_kib": fk[0], "write_kib": wk[0], "fetch_bytes": fb,
                          "write_bytes": wb, "bytes_per_launch": fb + wb}
    out = {"workload": workload, "source_hash": kernel_source_hash(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_kib": cf_kib, "write_kib": cw_kib,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": kernels, "commands": commands}
    with open(traffic_path(workload), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out


def cpu_baseline(w, inp, target: str = "conv_proj", align: str = "next") -> dict:
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
                   ni["W_target"], w.eta, w.chunk, form="sequential", target=target,
                   align=align)
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


def decode_roofline(w, L: int, us_per_call: float):
    """HBM roofline of decode-shaped streaming (bf16, L <= 16 rows per session,
    B*L <= 64): a decode call reads W_gate and W_up once for all sessions and
    each session's bf16 copy of its current weight once (2*f*d*2 + B*d*f*2
    bytes; the rows themselves are negligible).  The time per call includes
    the calls at chunk boundaries, which run the full layer."""
    import torch
    if w.dtype != torch.bfloat16 or L > 16 or w.batch * L > 64:
        return None
    d, f = w.d_model, w.d_ff
    nbytes = 2.0 * f * d * 2 + w.batch * d * f * 2.0
    gbs = nbytes / (us_per_call * 1e-6) / 1e9
    return {"kernel": "decode_swiglu + decode_down", "bound": "hbm", "achieved": gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": None, "algorithmic_bytes_per_call": nbytes}


def backward_bench(args, w, dev) -> int:
    """Tokens/s of the backward pass (ttt_mlp_backward_batched: the forward
    recomputed, the reverse scan, the GEMMs of every gradient) for a seeded
    dO and dW_final on the workload."""
    import torch
    from chunk_wise_weight_chunked_amd import ttt_mlp as tm

    B, T, d, f, K = w.batch, w.seq_len, w.d_model, w.d_ff, w.conv_k
    conv = args.target in ("conv_proj", "conv")
    proj = args.target in ("conv_proj", "proj")
    desc = tm.make_desc(B, T, d, f, w.chunk, K, w.eta, w.dtype, init_from_w0=1,
                        target=args.target, align=args.align)
    ws = torch.empty(tm.ttt_mlp_backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(12)
    dO = torch.randn((B, T, d), generator=gen, device="cuda").to(w.dtype)
    dWN = 0.01 * torch.randn((B, d, f), generator=gen, device="cuda")
    f32 = torch.float32
    outs = [torch.empty_like(dev["H"]), torch.empty_like(dev["H"]),
            torch.empty((f, d), dtype=f32, device="cuda"),
            torch.empty((f, d), dtype=f32, device="cuda"),
            torch.empty((B, d, f), dtype=f32, device="cuda"),
            torch.empty((d, K), dtype=f32, device="cuda") if conv else None,
            torch.empty((d, d), dtype=f32, device="cuda") if proj else None,
            torch.empty(1, dtype=f32, device="cuda")]
    stream = torch.cuda.current_stream()

    def step():
        tm.ttt_mlp_backward_batched(desc, dev["H"], dev["X0"], dev["W_gate"], dev["W_up"],
                                    dev["W_down0"], None, dev["taps"] if conv else None,
                                    dev["W_target"] if proj else None, dO, dWN, *outs, ws,
                                    stream=stream)

    log(f"[bench] backward: workspace {ws.numel() / 2**30:.1f} GiB, warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    value = w.tokens / (ms_step / 1e3)
    dtype = "bf16" if w.dtype == torch.bfloat16 else "f32"
    # contractions executed per token: the gate and up pre-activations (4df),
    # the forward's scan and the reverse scan (2 x 2df), dZ (4df), G (2df),
    # dH (4df), dW_gate and dW_up (4df); with the projection eta V^ (Vt), V^,
    # dU and dW_target (4 x 2d^2)
    flops = w.tokens * (22.0 * d * f + (8.0 * d * d if proj else 0.0))
    frac = flops / (ms_step / 1e3) / (PEAK_TFLOPS[dtype] * 1e12)
    log(f"[bench] backward {ms_step:.3f} ms/step, {value / 1e6:.3f} M tokens/s, "
        f"{frac:.1%} of the {dtype} MFMA peak")
    out = {
        "metric": "TTT-MLP layer backward tokens/sec",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": T, "chunk": w.chunk,
                   "d_model": d, "d_ff": f, "conv_k": K, "eta": w.eta, "target": args.target,
                   "align": args.align, "pass": "backward"},
        "executed_flops_per_step": flops,
        "layer_mfma_frac": frac,
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def stream_bench(args, w, dev, inp) -> int:
    """Tokens/s of the streaming entry point: each step feeds the B sequences
    from position 0 in calls of L tokens (the last call closes the streams
    when the whole sequence is fed)."""
    import torch
    from chunk_wise_weight_chunked_amd import ttt_mlp as tm

    B, T, d, f, K = w.batch, w.seq_len, w.d_model, w.d_ff, w.conv_k
    L = args.segment
    calls = [(p, min(L, T - p)) for p in range(0, T, L)]
    if args.segment_calls:
        calls = calls[:args.segment_calls]
    closing = calls[-1][0] + calls[-1][1] == T
    descs = {n: tm.make_desc(B, n, d, f, w.chunk, K, w.eta, w.dtype, args.mode, init_from_w0=1,
                             target=args.target, align=args.align)
             for n in {n for _, n in calls}}
    ws = torch.empty(tm.ttt_mlp_stream_workspace_size(descs[calls[0][1]], args.max_group),
                     dtype=torch.uint8, device="cuda")
    carry = torch.empty(tm.ttt_mlp_carry_size(descs[calls[0][1]]), dtype=torch.uint8,
                        device="cuda")
    segs = [(dev["H"][:, p:p + n].contiguous(), dev["X0"][:, p:p + n].contiguous())
            for p, n in calls]
    O = torch.empty((B, L, d), dtype=dev["H"].dtype, device="cuda")
    W = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        for i, ((p, n), (h, x0)) in enumerate(zip(calls, segs)):
            last = 1 if closing and i == len(calls) - 1 else 0
            tm.ttt_mlp_forward_stream(descs[n], p, last, h, x0, dev["W_gate"], dev["W_up"],
                                      dev["W_down0"], dev["taps"], dev["W_target"], O, W, carry,
                                      ws, stream=stream)

    log(f"[bench] streaming {len(calls)} calls of {L} tokens, warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    tokens = B * sum(n for _, n in calls)
    value = tokens / (ms_step / 1e3)
    log(f"[bench] {ms_step:.3f} ms/step, {value / 1e6:.4f} M tokens/s, "
        f"{ms_step * 1e3 / len(calls):.1f} us per call")
    out = {
        "metric": "TTT-MLP layer tokens/sec, streamed in segments",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": T, "chunk": w.chunk,
                   "d_model": d, "d_ff": f, "conv_k": K, "eta": w.eta, "mode": args.mode,
                   "target": args.target, "align": args.align, "segment": L,
                   "calls": len(calls),
                   "closing": closing},
        "us_per_call": ms_step * 1e3 / len(calls),
        "roofline": decode_roofline(w, L, ms_step * 1e3 / len(calls)),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_4b_128k")
    ap.add_argument("--mode", default="auto", choices=["auto", "sequential", "chunk_parallel"])
    ap.add_argument("--target", default="conv_proj", choices=["conv_proj", "proj", "conv", "embed"],
                    help="fast-weight target (the variants of the ablation table)")
    ap.add_argument("--align", default="next", choices=["next", "self"],
                    help="conv window ends at the next token (the method) or at the token "
                         "itself (the reconstruction alignment)")
    ap.add_argument("--max-group", type=int, default=0, help="chunks per group (0 = all)")
    ap.add_argument("--chunk", type=int, default=0, help="chunk size C (0 = the workload's)")
    ap.add_argument("--segment", type=int, default=0, metavar="L",
                    help="stream the sequences in calls of L tokens (0 = one call)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gradients of all inputs) instead")
    ap.add_argument("--segment-calls", type=int, default=0, metavar="N",
                    help="with --segment: time only the first N calls of each step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="write the traffic record of --workload from four rocprofv3 "
                         "counter_collection.csv files (layer FETCH_SIZE, layer WRITE_SIZE, "
                         "copy FETCH_SIZE, copy WRITE_SIZE) and exit; no GPU needed")
    ap.add_argument("--traffic-copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="command that produced the counter files (repeatable)")
    args = ap.parse_args()

    if args.traffic_from:
        t = write_traffic(args.workload, *args.traffic_from, args.traffic_copy_bytes,
                          args.traffic_command)
        print(json.dumps(t["kernels"], indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library runs the layer on one GPU; sharding across GPUs is not built)",
              file=sys.stderr)
        return 2

    import torch
    if args.calib_copy:
        calib_copy(args.calib_copy, max(1, args.steps))
        return 0

    from chunk_wise_weight_chunked_amd import synth
    from chunk_wise_weight_chunked_amd import ttt_mlp as tm

    w = synth.WORKLOADS[args.workload]
    default_config = (args.chunk in (0, w.chunk) and args.mode == "auto"
                      and args.target == "conv_proj" and args.align == "next"
                      and args.max_group == 0)
    if args.chunk:
        w = dataclasses.replace(w, chunk=args.chunk)
    if not torch.cuda.is_available():
        log("no GPU available")
        return 1
    tm.load()
    log(f"[bench] workload {w.name}: drawing inputs")
    inp = synth.workload_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items()}
    B, T, d, f, K = w.batch, w.seq_len, w.d_model, w.d_ff, w.conv_k
    desc = tm.make_desc(B, T, d, f, w.chunk, K, w.eta, w.dtype, args.mode, init_from_w0=1,
                        target=args.target, align=args.align)
    if args.segment:
        return stream_bench(args, w, dev, inp)
    if args.backward:
        return backward_bench(args, w, dev)
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
    # an event between steps (no synchronisation) gives each step's time too
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for k in range(args.steps):
        step()
        marks[k + 1].record(stream)
    torch.cuda.synchronize()
    tm.ttt_profile_enable(False)
    ms_total = marks[0].elapsed_time(marks[-1])
    per_step = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    stages = tm.ttt_profile_read()
    ms_step = ms_total / args.steps
    tokens = w.tokens
    value = tokens / (ms_step / 1e3)
    dtype = "bf16" if w.dtype == torch.bfloat16 else "f32"
    peak = PEAK_TFLOPS[dtype]
    log(f"[bench] {ms_step:.3f} ms/step (median {ms_median:.3f}), {value / 1e6:.3f} M tokens/s")

    split = stages.get("scan_target", (0.0, 0))[1] > 0
    per_chunk = args.mode == "sequential"
    work = stage_work(w, group, split, per_chunk)
    proj = args.target in ("conv_proj", "proj")
    if not proj:
        work.pop("target")  # no projection GEMM: the stage only moves rows
    nbytes = stage_bytes(w, group, split, per_chunk)
    if not proj:  # the stage reads X0 and writes one row per token, no weight
        nbytes["target"] = (2 if dtype == "bf16" else 4) * w.tokens * 2 * d
    per_stage = {}
    for name, (ms, n) in stages.items():
        if n == 0:
            continue
        avg = ms / n
        entry = {"ms_per_launch": avg, "launches_per_step": n / args.steps}
        if name in work:
            tf = work[name] / (avg / 1e3) / 1e12
            entry.update({"tflops": tf, "frac_of_peak": tf / peak})
        if name in nbytes:
            gbs = nbytes[name] / (avg / 1e3) / 1e9
            entry.update({"gbps": gbs, "frac_of_hbm": gbs / HBM_PEAK_GBS})
        per_stage[name] = entry
        log(f"  {name:14s} {avg:9.3f} ms x {n / args.steps:g}/step  "
            + (f"{entry['tflops']:8.1f} TFLOP/s ({entry['frac_of_peak']:.1%})" if "tflops" in entry else "")
            + (f"  {entry['gbps']:7.0f} GB/s ({entry['frac_of_hbm']:.1%})" if "gbps" in entry else ""))
    dom = max((k for k in per_stage if k in work),
              key=lambda k: per_stage[k]["ms_per_launch"] * per_stage[k]["launches_per_step"])
    is_hbm = hbm_bound(work[dom], nbytes[dom], dtype)
    if is_hbm:
        ach, pk, unit = per_stage[dom]["gbps"], HBM_PEAK_GBS, "GB/s"
    else:
        ach, pk, unit = per_stage[dom]["tflops"], peak, "TFLOP/s"
    roofline = {"kernel": dom, "bound": "hbm" if is_hbm else "mfma", "achieved": ach,
                "peak": pk, "unit": unit, "frac": ach / pk,
                "traffic": traffic_for(dom, w.name) if default_config else None,
                "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "flops_per_launch": work[dom],
                "algorithmic_bytes_per_launch": nbytes[dom],
                "ms_per_launch": per_stage[dom]["ms_per_launch"]}
    layer_flops = w.flops() - (0 if proj else 2.0 * w.tokens * d * d)
    layer_frac = layer_flops / (ms_step / 1e3) / (peak * 1e12)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle) ...")
        cpu = cpu_baseline(w, inp, args.target, args.align)
        log(f"[bench] oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": "TTT-MLP layer tokens/sec at d=2560,f=9728,128K ctx; % MFMA/HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": T, "chunk": w.chunk,
                   "d_model": d, "d_ff": f, "conv_k": K, "eta": w.eta, "mode": args.mode,
                   "group": group, "state": "fp32", "target": args.target,
                   "align": args.align},
        "layer_mfma_frac": layer_frac,
        "roofline": roofline,
        "stages": per_stage,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
