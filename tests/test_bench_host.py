"""Host-side checks of the benchmark's work and byte accounting (no GPU)."""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
from chunk_wise_weight_chunked_amd import synth  # noqa: E402


def test_stage_work_and_bytes_of_the_benchmark_workload():
    w = synth.WORKLOADS["qwen3_4b_128k"]
    BT, d, f, C = w.batch * w.seq_len, w.d_model, w.d_ff, w.chunk
    assert w.dtype == torch.bfloat16
    work = bench.stage_work(w, 32)
    nbytes = bench.stage_bytes(w, 32)
    # SwiGLU: gate and up products; operands H and the two weights, result Z
    assert work["swiglu"] == 4.0 * BT * d * f
    assert nbytes["swiglu"] == 2 * BT * (d + f) + 2 * 2 * f * d
    assert work["target"] == 2.0 * BT * d * d
    # four groups of 32 chunks: the fused launches each scan one group (2 C d f
    # per chunk) and compute the previous group's outputs (2 C d f per chunk)
    assert work["scan_apply"] == 2 * (2.0 * 32 * C * d * f)
    assert work["prefix_update"] == work["down_proj"] == 2.0 * 32 * C * d * f
    # per chunk: the scan reads C tokens of V^ and Z and writes one bf16 slot,
    # the outputs read C tokens of Z and the slot and write C rows of O; the
    # fp32 state is read and written once per group
    per_chunk = 2 * C * (d + f) + 2 * d * f
    assert nbytes["scan_apply"] == 2 * 32 * per_chunk + 8 * d * f
    # with the projection split, the first launch projects one group's tokens
    sw = bench.stage_work(w, 32, split=True)
    assert sw["target"] == 2.0 * 32 * C * d * d
    assert sw["scan_target"] == 2.0 * 32 * C * d * f + 2.0 * (BT - 32 * C) * d * d
    assert sum(sw[k] for k in ("target", "scan_target")) == work["target"] + work["prefix_update"]


def test_sequential_schedule_accounting():
    """Sequential mode scans one chunk per launch (the fp32 state read and
    written every time) and computes a group's outputs in the launch of the
    next group's first chunk."""
    w = synth.WORKLOADS["qwen3_4b_128k"]
    d, f, C = w.d_model, w.d_ff, w.chunk
    kinds = [k for k, _, _ in bench._launches(w, 32, False, True)]
    assert len(kinds) == 128 + 1
    assert kinds.count("scan_apply") == 3 and kinds.count("down_proj") == 1
    assert kinds.count("prefix_update") == 125
    work = bench.stage_work(w, 32, per_chunk=True)
    nbytes = bench.stage_bytes(w, 32, per_chunk=True)
    assert work["prefix_update"] == 2.0 * C * d * f
    assert work["scan_apply"] == 2.0 * C * d * f + 2.0 * 32 * C * d * f
    assert work["down_proj"] == 2.0 * 32 * C * d * f
    assert nbytes["prefix_update"] == 2 * C * (d + f) + 2 * d * f + 8 * d * f
    # with groups of one chunk the two schedules are the same
    assert bench._launches(w, 1, False, True) == bench._launches(w, 1, False, False)
    # split: the first chunk's launch projects the tokens after the first group
    sw = bench.stage_work(w, 32, split=True, per_chunk=True)
    assert sw["scan_target"] == 2.0 * C * d * f + 2.0 * (w.seq_len - 32 * C) * d * d


@pytest.mark.parametrize("name,stage,hbm", [
    ("qwen3_4b_128k", "swiglu", False),
    ("qwen3_4b_128k", "scan_apply", False),   # C = 1024: about 650 flop/B
    ("small_4x128k", "scan_apply", True),     # C = 256, d = 1024: below the ridge
    ("small_4x128k", "swiglu", False),
])
def test_roofline_bound_follows_the_ridge(name, stage, hbm):
    w = synth.WORKLOADS[name]
    group = -(-w.n_chunks // 4)
    work, nbytes = bench.stage_work(w, group), bench.stage_bytes(w, group)
    assert bench.hbm_bound(work[stage], nbytes[stage], "bf16") is hbm
    # the ridge itself: 2.5 PFLOP/s over 8 TB/s
    assert bench.hbm_bound(312.0, 1.0, "bf16") and not bench.hbm_bound(313.0, 1.0, "bf16")
