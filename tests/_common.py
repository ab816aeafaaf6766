"""Shared helpers for the tests: relative errors, input conversion, device runs."""
from __future__ import annotations

import numpy as np
import torch

from chunk_wise_weight_chunked_amd import synth

# Tolerances on relative Frobenius error: fp32 end to end, and bf16 inputs with an
# fp32 fast-weight state.  The bf16 bound covers the roundings of Z, eta*V^, each
# chunk's weight and O (unit roundoff 2^-9 each; expected ~3e-3 in total).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2

INPUT_NAMES = ("H", "X0", "W_gate", "W_up", "W_down0", "taps", "W_target")


def rel(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def tol_for(dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def numpy_inputs(inp: dict) -> dict:
    """Exact float32 copies of the inputs for the CPU oracle."""
    return {k: synth.to_numpy_f32(inp[k]) for k in INPUT_NAMES}


def to_device(inp: dict, device="cuda") -> dict:
    return {k: inp[k].to(device).contiguous() for k in INPUT_NAMES}
