"""Seeded synthetic inputs for the TTT-MLP layer.

This module only draws random numbers; it holds none of the layer's arithmetic.
The tests feed the same tensors to the HIP library and to the CPU oracle, and the
benchmark uses the same recipe.

Recipe (per workload): a CPU ``torch.Generator`` seeded with the workload's seed
draws float32 standard normals in the fixed order H, X0, W_gate, W_up, W_down0,
taps, W_target; each is scaled by its standard deviation and, for bf16
workloads, rounded to bf16 (round-to-nearest-even).  Standard deviations:
H, X0 ~ N(0, 1); W_gate, W_up ~ N(0, 1/d); W_down0 ~ N(0, 1/f) (its fan-in is
f); W_target ~ N(0, 1/d); taps ~ N(0, 1/K).
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    chunk: int
    d_model: int
    d_ff: int
    conv_k: int
    eta: float
    dtype: torch.dtype  # activation and weight dtype; the fast-weight state is fp32
    seed: int

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def flops(self) -> float:
        """Algorithmic flops of one forward: five contractions per token
        (gate, up, down, target, update): 8*d*f + 2*d*d."""
        d, f = self.d_model, self.d_ff
        return float(self.tokens) * (8.0 * d * f + 2.0 * d * d)


# The five workloads, with the shapes and distributions stated for the layer.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1024, 128, 64, 256, 4, 1e-3, torch.float32, 1),
    "qwen3_4b_32k": Workload("qwen3_4b_32k", 1, 32768, 512, 2560, 9728, 4, 1e-3,
                             torch.bfloat16, 2),
    "qwen3_4b_128k": Workload("qwen3_4b_128k", 1, 131072, 1024, 2560, 9728, 4, 5e-4,
                              torch.bfloat16, 3),
    "multi_session_16x8k": Workload("multi_session_16x8k", 16, 8192, 512, 2560, 9728, 4,
                                    1e-3, torch.bfloat16, 4),
    "small_4x128k": Workload("small_4x128k", 4, 131072, 256, 1024, 4096, 8, 1e-3,
                             torch.bfloat16, 5),
}


def _normal(gen: torch.Generator, shape, std: float, dtype: torch.dtype,
            block_rows: int = 8192) -> torch.Tensor:
    """Draw N(0, std^2) of `shape` in row blocks (bounded temporary memory)."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], block_rows):
        r1 = min(r0 + block_rows, flat.shape[0])
        x = torch.randn((r1 - r0, shape[-1]), generator=gen, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1].copy_(x)  # RNE rounding for bf16
    return out


def make_inputs(batch: int, seq_len: int, d_model: int, d_ff: int, conv_k: int,
                dtype: torch.dtype, seed: int) -> dict:
    """Draw one set of layer inputs on the CPU.  Returns a dict of tensors:
    H, X0 [B][T][d]; W_gate, W_up [f][d]; W_down0 [d][f]; taps [d][K];
    W_target [d_in][d_out]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    B, T, d, f, K = batch, seq_len, d_model, d_ff, conv_k
    return {
        "H": _normal(g, (B, T, d), 1.0, dtype),
        "X0": _normal(g, (B, T, d), 1.0, dtype),
        "W_gate": _normal(g, (f, d), 1.0 / math.sqrt(d), dtype),
        "W_up": _normal(g, (f, d), 1.0 / math.sqrt(d), dtype),
        "W_down0": _normal(g, (d, f), 1.0 / math.sqrt(f), dtype),
        "taps": _normal(g, (d, K), 1.0 / math.sqrt(K), dtype),
        "W_target": _normal(g, (d, d), 1.0 / math.sqrt(d), dtype),
    }


def workload_inputs(w: Workload, seq_len: int | None = None, batch: int | None = None):
    """Inputs of a named workload (optionally with a different token count or
    batch, which draws a different set of values)."""
    return make_inputs(batch or w.batch, seq_len or w.seq_len, w.d_model, w.d_ff,
                       w.conv_k, w.dtype, w.seed)


def to_numpy_f32(t: torch.Tensor):
    """Exact float32 view of a bf16/fp32 tensor for the CPU oracle."""
    return t.detach().to("cpu", torch.float32).contiguous().numpy()
