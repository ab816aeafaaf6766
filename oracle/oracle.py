"""Python side of the fp64 CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  It loads ``oracle/_build/libttt_oracle.so``, built
from ``ttt_oracle.c`` with gcc, and hands it numpy arrays.  It imports nothing
from the HIP package, and the HIP package imports nothing from here.

Inputs are passed as float32 arrays holding the exact values of the bf16/fp32
inputs; all arithmetic in the C code is double precision; outputs are float64.

Layouts (row-major): H, X0 [B][T][d]; W_gate, W_up [f][d]; W_down0 [d][f] or a
per-sequence starting state [B][d][f]; taps [d][K] (taps[c][k] multiplies
X0[t+1-k][c]); W_target [d][d] applied on the right (V^ = U @ W_target).
See ttt_oracle.c for the passages of the In-Place TTT page each form follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "libttt_oracle.so")
# A different build of the oracle (the mutation test plants slips in a copy of
# the source and points the pins at it through this variable).
_LIB_OVERRIDE = os.environ.get("TTT_ORACLE_LIB")

# x86-64-v3 (AVX2/FMA) so the library built here also runs on the GPU host.
_CFLAGS = ["-O2", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc; returns its path."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        fwd_args = [i64, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_double,
                    f32p, f32p, f32p, f32p, f32p, f32p, f32p, f64p, f64p]
        for name in ("oracle_forward_sequential", "oracle_forward_chunk_parallel",
                     "oracle_forward_dual"):
            fn = getattr(lib, name)
            fn.argtypes = fwd_args
            fn.restype = ctypes.c_int
        lib.oracle_gated_activations.argtypes = [i64, i64, i64, f32p, f32p, f32p, f64p]
        lib.oracle_gated_activations.restype = None
        lib.oracle_lm_target.argtypes = [i64, i64, i64, ctypes.c_int32, f32p, f32p, f32p,
                                         f64p]
        lib.oracle_lm_target.restype = ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_final_weight_grid.argtypes = [
            i64, i64, i64, ctypes.c_int32, ctypes.c_double, f32p, f32p, f32p, f32p, f32p,
            f32p, f32p, i64, i64p, i64, i64p, f64p]
        lib.oracle_final_weight_grid.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_progress.argtypes = [i64]
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        out = a.astype(np.float32)
        if not np.array_equal(out.astype(np.float64), a.astype(np.float64)):
            raise ValueError("oracle inputs must be exactly representable in float32")
        a = out
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def set_progress(every: int) -> None:
    """Print a progress line on stderr every `every` chunks of the sequential
    form (0: silent)."""
    _load().oracle_set_progress(int(every))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def gated_activations(H, W_gate, W_up) -> np.ndarray:
    """Z = silu(H W_gate^T) * (H W_up^T) for H of shape [rows][d]."""
    H, Wg, Wu = _f32(H), _f32(W_gate), _f32(W_up)
    rows, d = H.shape
    f = Wg.shape[0]
    assert Wg.shape == (f, d) and Wu.shape == (f, d)
    Z = np.empty((rows, f), dtype=np.float64)
    _load().oracle_gated_activations(rows, d, f, _ptr(H, ctypes.c_float),
                                     _ptr(Wg, ctypes.c_float), _ptr(Wu, ctypes.c_float),
                                     _ptr(Z, ctypes.c_double))
    return Z


# The target variants of the In-Place TTT page's ablation table (section 6):
# "w/o Conv" and "w/o Proj" leave out the conv or the projection of the
# section 3.3 target V^ = Conv1D(X0) W_target.  Read literally, a part left
# out is the identity: without the conv V^[t] = X0[t] W_target (the token's
# own embedding: the conv's tap k = 1 alone, X0[t+1-1]); without the
# projection V^ = Conv1D(X0) (W_target = I).  The oracle evaluates a variant
# as the method itself on those identity parts, which in fp64 is exact
# (multiplications by 1 and additions of 0).
TARGETS = ("conv_proj", "proj", "conv", "embed")
ALIGNS = ("next", "self")


def target_parts(target: str, taps, W_target, d: int, align: str = "next"):
    """(taps, W_target) that give `target` through the section 3.3 formula.
    align "self" (the reconstruction alignment of section 4's table) ends the
    conv's window at the token itself, U[t] = sum_k taps[k] X0[t-k]: the same
    sum as the section 3.3 conv over the taps with a zero tap put in front
    (tap k + 1 of the look-ahead form reads X0[t+1-(k+1)] = X0[t-k])."""
    if target not in TARGETS:
        raise ValueError(f"unknown target {target!r}")
    if align not in ALIGNS:
        raise ValueError(f"unknown align {align!r}")
    if target in ("proj", "embed"):       # no conv: U[t] = X0[t]
        taps = np.zeros((d, 2), dtype=np.float32)
        taps[:, 1] = 1.0
    elif align == "self":
        taps = _f32(taps)
        taps = np.concatenate([np.zeros((d, 1), dtype=np.float32), taps], axis=1)
    if target in ("conv", "embed"):       # no projection
        W_target = np.eye(d, dtype=np.float32)
    return taps, W_target


def lm_target(X0, taps, W_target, target: str = "conv_proj", align: str = "next") -> np.ndarray:
    """V^ = Conv1D(X0) W_target (or a variant, see TARGETS) for X0 of shape
    [B][T][d] (or [T][d])."""
    X0 = _f32(X0)
    squeeze = X0.ndim == 2
    if squeeze:
        X0 = X0[None]
    B, T, d = X0.shape
    taps, W_target = target_parts(target, taps, W_target, d, align)
    taps, Wt = _f32(taps), _f32(W_target)
    K = taps.shape[1]
    assert taps.shape == (d, K) and Wt.shape == (d, d)
    V = np.empty((B, T, d), dtype=np.float64)
    rc = _load().oracle_lm_target(B, T, d, K, _ptr(X0, ctypes.c_float),
                                  _ptr(taps, ctypes.c_float), _ptr(Wt, ctypes.c_float),
                                  _ptr(V, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"oracle_lm_target failed: {rc}")
    return V[0] if squeeze else V


_FORMS = {
    "sequential": "oracle_forward_sequential",
    "chunk_parallel": "oracle_forward_chunk_parallel",
    "dual": "oracle_forward_dual",
}


def forward(H, X0, W_gate, W_up, W_down0, taps, W_target, eta: float, chunk: int,
            form: str = "sequential", target: str = "conv_proj", align: str = "next"):
    """Run the layer; returns (O [B][T][d] float64, W_final [B][d][f] float64).

    H and X0 may be [T][d] (one sequence; outputs are then squeezed) or
    [B][T][d].  W_down0 may be [d][f] (shared starting weight) or [B][d][f]
    (one starting state per sequence).  `target` selects a variant of the
    fast weight's target (TARGETS); taps / W_target are ignored (may be None)
    when it leaves the conv / the projection out.
    """
    H, X0 = _f32(H), _f32(X0)
    squeeze = H.ndim == 2
    if squeeze:
        H, X0 = H[None], X0[None]
    B, T, d = H.shape
    assert X0.shape == (B, T, d)
    taps, W_target = target_parts(target, taps, W_target, d, align)
    Wg, Wu, taps, Wt = _f32(W_gate), _f32(W_up), _f32(taps), _f32(W_target)
    f = Wg.shape[0]
    K = taps.shape[1]
    assert Wg.shape == (f, d) and Wu.shape == (f, d)
    assert taps.shape == (d, K) and Wt.shape == (d, d)
    W0 = _f32(W_down0)
    if W0.ndim == 2:
        assert W0.shape == (d, f)
        W0 = np.ascontiguousarray(np.broadcast_to(W0, (B, d, f)))
    assert W0.shape == (B, d, f)
    O = np.empty((B, T, d), dtype=np.float64)
    W = np.empty((B, d, f), dtype=np.float64)
    fn = getattr(_load(), _FORMS[form])
    rc = fn(B, T, d, f, int(chunk), K, float(eta), _ptr(H, ctypes.c_float),
            _ptr(X0, ctypes.c_float), _ptr(Wg, ctypes.c_float), _ptr(Wu, ctypes.c_float),
            _ptr(W0, ctypes.c_float), _ptr(taps, ctypes.c_float), _ptr(Wt, ctypes.c_float),
            _ptr(O, ctypes.c_double), _ptr(W, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"{_FORMS[form]} failed: {rc}")
    if squeeze:
        return O[0], W[0]
    return O, W


def final_weight_grid(H, X0, W_gate, W_up, W_down0, taps, W_target, eta: float, ms, ns,
                      target: str = "conv_proj", align: str = "next"):
    """Entries W_final[m][n] for m in ms, n in ns of ONE sequence, by the closed
    form W0 + eta * sum_t V^[t][m] Z[t][n] (independent of the chunk size)."""
    H, X0 = _f32(H), _f32(X0)
    T, d = H.shape
    taps, W_target = target_parts(target, taps, W_target, d, align)
    Wg, Wu, W0, taps, Wt = (_f32(W_gate), _f32(W_up), _f32(W_down0), _f32(taps),
                            _f32(W_target))
    f = Wg.shape[0]
    K = taps.shape[1]
    ms = np.ascontiguousarray(np.asarray(ms, dtype=np.int64))
    ns = np.ascontiguousarray(np.asarray(ns, dtype=np.int64))
    out = np.empty((len(ms), len(ns)), dtype=np.float64)
    rc = _load().oracle_final_weight_grid(
        T, d, f, K, float(eta), _ptr(H, ctypes.c_float), _ptr(X0, ctypes.c_float),
        _ptr(Wg, ctypes.c_float), _ptr(Wu, ctypes.c_float), _ptr(W0, ctypes.c_float),
        _ptr(taps, ctypes.c_float), _ptr(Wt, ctypes.c_float), len(ms),
        _ptr(ms, ctypes.c_int64), len(ns), _ptr(ns, ctypes.c_int64),
        _ptr(out, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"oracle_final_weight_grid failed: {rc}")
    return out
