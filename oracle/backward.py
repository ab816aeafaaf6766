"""Backward pass of the In-Place TTT fast-weight MLP layer in fp64 numpy (test
infrastructure only: the test suite may import it, nothing in the HIP package
does).

The pages define the forward (In-Place TTT page, section 3.1: the gated MLP
whose down-projection is the fast weight; section 3.3: the target
V^ = Conv1D(X0) W_target and the update W^(i) = W^(i-1) + eta V^_iᵀ Z_i;
section 3.2: chunk i's outputs use the weight left by the chunks before it).
The pages' results come from training with the layer in place (section 5,
continual pretraining and training from scratch), which needs the gradient of
that forward.  This module is that gradient, by the chain rule through the
chunk recurrence, written plainly: one sequence at a time, one chunk at a time,
every product a numpy matmul in float64.

For a loss L with dL/dO = dO and dL/dW_final = dW_final, and chunks j of a
sequence with W^(-1) = W_down0:
  S_j   = dW_final + sum_{m > j} dO_mᵀ Z_m     (what flows into chunk j's update)
  dZ_j  = dO_j W^(j-1) + eta V^_j S_j
  dV^_j = eta Z_j S_jᵀ
  dW_down0 = S_{-1} = dW_final + sum_m dO_mᵀ Z_m
  deta  = sum_j <S_j, V^_jᵀ Z_j>_F
then through the SwiGLU (Z = SiLU(A_g) * A_u with A = H Wᵀ), the projection
(V^ = U W_target) and the depthwise conv (U[t][c] = sum_k taps[c][k]
X0[t + s - k][c], s = 1 for the next-token alignment, 0 for the
reconstruction one).
"""
from __future__ import annotations

import numpy as np

from .oracle import ALIGNS, TARGETS


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _conv(X0, taps, shift):
    """U[t][c] = sum_k taps[c][k] X0[t + shift - k][c], zero outside [0, T)."""
    T, d = X0.shape
    U = np.zeros((T, d))
    for k in range(taps.shape[1]):
        off = shift - k  # U[t] reads X0[t + off]
        lo, hi = max(0, -off), min(T, T - off)
        if lo < hi:
            U[lo:hi] += taps[:, k] * X0[lo + off:hi + off]
    return U


def _conv_backward(X0, taps, shift, dU):
    """Gradients of sum <dU, U> with respect to X0 and taps."""
    T, d = X0.shape
    dX0 = np.zeros((T, d))
    dtaps = np.zeros_like(taps)
    for k in range(taps.shape[1]):
        off = shift - k
        lo, hi = max(0, -off), min(T, T - off)
        if lo < hi:
            dX0[lo + off:hi + off] += taps[:, k] * dU[lo:hi]
            dtaps[:, k] = (dU[lo:hi] * X0[lo + off:hi + off]).sum(axis=0)
    return dX0, dtaps


def backward(H, X0, W_gate, W_up, W_down0, taps, W_target, eta: float, chunk: int, dO,
             dW_final=None, target: str = "conv_proj", align: str = "next") -> dict:
    """Gradients of L = <dO, O> + <dW_final, W_final> for the layer run on
    H, X0 [B][T][d] from W_down0 ([d][f], shared, or [B][d][f], one starting
    state per sequence).  Returns float64 arrays: H, X0 [B][T][d]; W_gate,
    W_up [f][d]; W_state0 [B][d][f] (per sequence) and W_down0 [d][f] (their
    sum); taps [d][K] (None without the conv); W_target [d][d] (None without
    the projection); eta (a float); eta_scale = ||V^||_F ||G||_F with
    G_j = Z_j S_jᵀ (eta's gradient is the inner product <V^, G>: the bound of
    its rounding error scales with these norms, not with the result, whose
    terms largely cancel)."""
    if target not in TARGETS or align not in ALIGNS:
        raise ValueError(f"unknown target/align {target!r}/{align!r}")
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    shift = 1 if align == "next" else 0
    H, X0, dO = _f64(H), _f64(X0), _f64(dO)
    if H.ndim == 2:
        H, X0, dO = H[None], X0[None], dO[None]
    B, T, d = H.shape
    Wg, Wu, W0 = _f64(W_gate), _f64(W_up), _f64(W_down0)
    f = Wg.shape[0]
    if W0.ndim == 2:
        W0 = np.broadcast_to(W0, (B, d, f))
    tp = _f64(taps) if conv else None
    Wt = _f64(W_target) if proj else None
    dWN = np.zeros((B, d, f)) if dW_final is None else np.broadcast_to(_f64(dW_final), (B, d, f))
    C = int(chunk)
    N = -(-T // C)

    g = {"H": np.zeros((B, T, d)), "X0": np.zeros((B, T, d)), "W_gate": np.zeros((f, d)),
         "W_up": np.zeros((f, d)), "W_state0": np.zeros((B, d, f)),
         "taps": np.zeros_like(tp) if conv else None,
         "W_target": np.zeros((d, d)) if proj else None, "eta": 0.0}
    v2 = g2 = 0.0
    for b in range(B):
        # forward, keeping what the backward reads
        Ag, Au = H[b] @ Wg.T, H[b] @ Wu.T
        sig = 1.0 / (1.0 + np.exp(-Ag))
        Z = Ag * sig * Au
        U = _conv(X0[b], tp, shift) if conv else X0[b]
        V = U @ Wt if proj else U
        W_used = []  # W^(j-1), the weight chunk j's outputs use
        W = W0[b].copy()
        for j in range(N):
            W_used.append(W.copy())
            r = slice(j * C, min(T, (j + 1) * C))
            W = W + eta * V[r].T @ Z[r]
        # backward through the chunks, last to first
        S = dWN[b].copy()
        dZ = np.zeros_like(Z)
        G = np.zeros((T, d))  # Z_j S_jᵀ: dV^ = eta G
        for j in reversed(range(N)):
            r = slice(j * C, min(T, (j + 1) * C))
            dZ[r] = dO[b][r] @ W_used[j] + eta * V[r] @ S
            G[r] = Z[r] @ S.T
            g["eta"] += float(np.sum(S * (V[r].T @ Z[r])))
            S = S + dO[b][r].T @ Z[r]
        g["W_state0"][b] = S
        v2 += float(np.sum(V * V))
        g2 += float(np.sum(G * G))
        dV = eta * G
        # SwiGLU: dZ/dA_g = A_u * SiLU'(A_g), dZ/dA_u = SiLU(A_g)
        dAg = dZ * Au * sig * (1.0 + Ag * (1.0 - sig))
        dAu = dZ * Ag * sig
        g["H"][b] = dAg @ Wg + dAu @ Wu
        g["W_gate"] += dAg.T @ H[b]
        g["W_up"] += dAu.T @ H[b]
        if proj:
            g["W_target"] += U.T @ dV
            dU = dV @ Wt.T
        else:
            dU = dV
        if conv:
            dX, dt = _conv_backward(X0[b], tp, shift, dU)
            g["X0"][b] = dX
            g["taps"] += dt
        else:
            g["X0"][b] = dU
    g["W_down0"] = g["W_state0"].sum(axis=0)
    g["eta_scale"] = float(np.sqrt(v2) * np.sqrt(g2))
    return g


def sampled_weight_grads(H, X0, W_gate, W_up, W_down0, taps, W_target, eta: float, chunk: int,
                         dO, features, dW_final=None, target: str = "conv_proj",
                         align: str = "next") -> dict:
    """Rows `features` of dW_gate and dW_up and columns `features` of each
    sequence's dW_start, at a cost of O(T d) per feature (plus V^ once), for
    checking full-size runs.  Column f' of every W^(j) and S_j only involves
    column f' of Z:  W^(j)[:, f'] = W0[:, f'] + eta sum_{m <= j} V^_mᵀ Z_m[:, f'],
    S_j[:, f'] = dW_final[:, f'] + sum_{m > j} dO_mᵀ Z_m[:, f'], so
    dZ[t][f'] = dO[t] . W^(j-1)[:, f'] + eta V^[t] . S_j[:, f'] needs no other
    feature; then dA_g, dA_u for that feature and their products with H.
    Returns W_gate, W_up [len(features)][d] and W_start [B][d][len(features)]."""
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    shift = 1 if align == "next" else 0
    H, X0, dO = _f64(H), _f64(X0), _f64(dO)
    if H.ndim == 2:
        H, X0, dO = H[None], X0[None], dO[None]
    B, T, d = H.shape
    Wg, Wu, W0 = _f64(W_gate), _f64(W_up), _f64(W_down0)
    f = Wg.shape[0]
    if W0.ndim == 2:
        W0 = np.broadcast_to(W0, (B, d, f))
    F = np.asarray(features, dtype=np.int64)
    dWN = np.zeros((B, d, f)) if dW_final is None else np.broadcast_to(_f64(dW_final), (B, d, f))
    C = int(chunk)
    N = -(-T // C)
    out = {"W_gate": np.zeros((len(F), d)), "W_up": np.zeros((len(F), d)),
           "W_start": np.zeros((B, d, len(F)))}
    for b in range(B):
        U = _conv(X0[b], _f64(taps), shift) if conv else X0[b]
        V = U @ _f64(W_target) if proj else U
        Ag, Au = H[b] @ Wg[F].T, H[b] @ Wu[F].T          # [T][|F|]
        sig = 1.0 / (1.0 + np.exp(-Ag))
        Z = Ag * sig * Au
        # per chunk: V^_jᵀ Z_j[:, F] and dO_jᵀ Z_j[:, F]  ([d][|F|] each)
        inc_w = np.stack([V[j * C:(j + 1) * C].T @ Z[j * C:(j + 1) * C] for j in range(N)])
        inc_s = np.stack([dO[b][j * C:(j + 1) * C].T @ Z[j * C:(j + 1) * C] for j in range(N)])
        W_used = W0[b][:, F] + eta * (np.cumsum(inc_w, axis=0) - inc_w)          # W^(j-1)
        S = dWN[b][:, F] + (inc_s.sum(axis=0) - np.cumsum(inc_s, axis=0))       # S_j
        dZ = np.zeros_like(Z)
        for j in range(N):
            r = slice(j * C, min(T, (j + 1) * C))
            dZ[r] = dO[b][r] @ W_used[j] + eta * V[r] @ S[j]
        dAg = dZ * Au * sig * (1.0 + Ag * (1.0 - sig))
        dAu = dZ * Ag * sig
        out["W_gate"] += dAg.T @ H[b]
        out["W_up"] += dAu.T @ H[b]
        out["W_start"][b] = dWN[b][:, F] + inc_s.sum(axis=0)
    return out
