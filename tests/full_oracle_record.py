"""Full fp64 oracle runs of the full-size workloads against the GPU layer.

A record, not a test (minutes of host time per workload, so pytest does not
collect it): the GPU runs the layer as the benchmark does (one call, the
default group pipeline), the oracle runs the sequential form over every token,
and the relative errors of O, of the final weight and of its change are
printed, with the worst chunk of O.

    python tests/full_oracle_record.py [workload ...] [--sessions a:b]

--sessions a:b compares sequences a..b-1 only (the GPU still runs the whole
batch, as the benchmark does): the oracle's time is split over several runs.
"""
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from chunk_wise_weight_chunked_amd import synth  # noqa: E402
from chunk_wise_weight_chunked_amd import ttt_mlp as tm  # noqa: E402

from _common import numpy_inputs, rel, to_device, tol_for  # noqa: E402

DEFAULT = ["qwen3_4b_32k", "qwen3_4b_128k", "multi_session_16x8k", "small_4x128k"]


def record(name: str, sessions=None) -> bool:
    w = synth.WORKLOADS[name]
    b0, b1 = sessions if sessions else (0, w.batch)
    print(f"[record] {name}: inputs", flush=True)
    inp = synth.workload_inputs(w)
    dev = to_device(inp)
    O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                              dev["taps"], dev["W_target"], w.eta, w.chunk)
    torch.cuda.synchronize()
    O_gpu = O.float().cpu().numpy()
    W_gpu = W.cpu().numpy()
    del O, W, dev
    torch.cuda.empty_cache()
    ni = numpy_inputs(inp)
    if (b0, b1) != (0, w.batch):
        ni = dict(ni, H=ni["H"][b0:b1], X0=ni["X0"][b0:b1])
        O_gpu, W_gpu = O_gpu[b0:b1], W_gpu[b0:b1]
    print(f"[record] {name}: sequences {b0}..{b1 - 1}: oracle (sequential, fp64, "
          f"{oracle.num_threads()} threads)", flush=True)
    oracle.set_progress(max(1, w.n_chunks // 8))
    t0 = time.perf_counter()
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], w.eta, w.chunk)
    dt = time.perf_counter() - t0
    if Oo.ndim == 2:
        Oo, Wo = Oo[None], Wo[None]
    W0 = ni["W_down0"].astype(np.float64)[None]
    e_o, e_w, e_dw = rel(O_gpu, Oo), rel(W_gpu, Wo), rel(W_gpu - W0, Wo - W0)
    C = w.chunk
    worst = max(rel(O_gpu[b, i:i + C], Oo[b, i:i + C])
                for b in range(b1 - b0) for i in range(0, w.seq_len, C))
    tol = tol_for(w.dtype)
    ok = max(e_o, e_w, e_dw) <= tol
    print(f"[record] {name}: rel O {e_o:.3e}  rel W_final {e_w:.3e}  rel dW {e_dw:.3e}  "
          f"worst chunk of O {worst:.3e}  (tolerance {tol:g}; oracle {dt:.0f} s)  "
          f"{'PASS' if ok else 'FAIL'}", flush=True)
    return ok


def main() -> int:
    args = sys.argv[1:]
    sessions = None
    if "--sessions" in args:
        i = args.index("--sessions")
        a, b = args[i + 1].split(":")
        sessions = (int(a), int(b))
        del args[i:i + 2]
    names = args or DEFAULT
    oracle.build(force=False)
    tm.load()
    results = [record(n, sessions) for n in names]
    return 0 if all(results) else 1


if __name__ == "__main__":
    sys.exit(main())
