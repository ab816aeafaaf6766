"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Every check here compares the oracle with something it does not compute: values
worked by hand (tests/golden), library routines (numpy matmul, numpy
correlate, torch.nn.functional.silu, torch autograd), closed forms implied by
the update rule, and invariants (agreement of three differently structured forms,
causality, linearity, batching).  A plausible slip in the oracle -- a dropped
term, a sign, an index shift, a transposed operand, output-after-update -- fails
at least one of them (tests/test_oracle_mutants.py plants such slips and checks).

Citations: In-Place TTT page (zhichai.net), section 3.1 (gated MLP with W_down as
the fast weight), section 3.2 (chunk-wise schedule, three-step parallel form),
section 3.3 (LM-aligned target, Frobenius loss and its one-step update rule),
section 4 (Theorem 1 contrasts the next-token target V_t = E_{x_{t+1}} with the
reconstruction target V_t = E_{x_t}).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_inputs(B, T, d, f, K, seed, scale_w0=1.0):
    """Small float32 inputs (exact for the oracle)."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    return dict(
        H=rng.standard_normal((B, T, d)).astype(f32),
        X0=rng.standard_normal((B, T, d)).astype(f32),
        W_gate=(rng.standard_normal((f, d)) / np.sqrt(d)).astype(f32),
        W_up=(rng.standard_normal((f, d)) / np.sqrt(d)).astype(f32),
        W_down0=(scale_w0 * rng.standard_normal((d, f)) / np.sqrt(f)).astype(f32),
        taps=(rng.standard_normal((d, K)) / np.sqrt(K)).astype(f32),
        W_target=(rng.standard_normal((d, d)) / np.sqrt(d)).astype(f32),
    )


def run(inp, eta, C, form="sequential"):
    return oracle.forward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"],
                          inp["taps"], inp["W_target"], eta, C, form=form)


def silu_lib(x):
    return torch.nn.functional.silu(torch.from_numpy(np.asarray(x, np.float64))).numpy()


def static_mlp_lib(H, Wg, Wu, W0):
    """Section 3.1 gated MLP with library routines (torch silu, numpy matmul)."""
    H = H.astype(np.float64)
    a = H @ Wg.astype(np.float64).T
    u = H @ Wu.astype(np.float64).T
    return (silu_lib(a) * u) @ W0.astype(np.float64).T


def rel(a, b):
    return float(np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300))


# ---------------------------------------------------------------- hand-worked examples
@pytest.mark.parametrize("form", ["sequential", "chunk_parallel", "dual"])
def test_hand_examples(form):
    data = json.load(open(GOLDEN))
    for ex in data["examples"]:
        s = ex["shape"]
        inp = {k: np.asarray(v, np.float32) for k, v in ex["inputs"].items()}
        inp["H"] = inp["H"].reshape(1, s["T"], s["d"])
        inp["X0"] = inp["X0"].reshape(1, s["T"], s["d"])
        O, W = run(inp, ex["eta"], s["C"], form)
        np.testing.assert_allclose(O[0], np.asarray(ex["expected"]["O"]), rtol=1e-13,
                                   atol=1e-13, err_msg=ex["name"])
        np.testing.assert_allclose(W[0], np.asarray(ex["expected"]["W_final"]),
                                   rtol=1e-13, atol=1e-13, err_msg=ex["name"])


# ---------------------------------------------------------------- section 3.1: static MLP
@pytest.mark.parametrize("B,T,d,f,K,C", [(1, 37, 8, 24, 4, 8), (2, 20, 16, 8, 3, 5)])
def test_eta_zero_is_static_gated_mlp(B, T, d, f, K, C):
    inp = rand_inputs(B, T, d, f, K, seed=11)
    O, W = run(inp, 0.0, C)
    for b in range(B):
        ref = static_mlp_lib(inp["H"][b], inp["W_gate"], inp["W_up"], inp["W_down0"])
        assert rel(O[b], ref) < 1e-13
        assert np.array_equal(W[b], inp["W_down0"].astype(np.float64))


def test_gated_activations_library():
    inp = rand_inputs(1, 19, 12, 20, 2, seed=3)
    Z = oracle.gated_activations(inp["H"][0], inp["W_gate"], inp["W_up"])
    H = inp["H"][0].astype(np.float64)
    ref = silu_lib(H @ inp["W_gate"].astype(np.float64).T) * (H @ inp["W_up"].astype(np.float64).T)
    assert rel(Z, ref) < 1e-14


# ---------------------------------------------------------------- section 3.2: chunk 0
@pytest.mark.parametrize("C", [1, 4, 16])
def test_first_chunk_uses_w_down0(C):
    inp = rand_inputs(1, 40, 8, 16, 4, seed=5)
    O, _ = run(inp, 0.7, C)
    ref = static_mlp_lib(inp["H"][0], inp["W_gate"], inp["W_up"], inp["W_down0"])
    assert rel(O[0, :C], ref[:C]) < 1e-13
    # and the second chunk does not (eta != 0 changes the weight)
    assert rel(O[0, C:2 * C], ref[C:2 * C]) > 1e-6


# ---------------------------------------------------------------- section 3.3: conv target
@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_conv_one_hot_alignment(k):
    """One-hot tap k with W_target = I gives V^[t] = X0[t+1-k] (0 outside the
    sequence).  k=0 is the next-token target of section 4, k=1 the
    reconstruction target."""
    T, d, K = 11, 5, 4
    rng = np.random.default_rng(7)
    X0 = rng.standard_normal((2, T, d)).astype(np.float32)
    taps = np.zeros((d, K), np.float32)
    taps[:, k] = 1.0
    V = oracle.lm_target(X0, taps, np.eye(d, dtype=np.float32))
    for b in range(2):
        exp = np.zeros((T, d))
        for t in range(T):
            s = t + 1 - k
            if 0 <= s < T:
                exp[t] = X0[b, s]
        np.testing.assert_array_equal(V[b], exp)
    if k == 0:
        assert np.all(V[:, T - 1] == 0.0)  # right zero pad: no token after the last


def test_conv_general_taps_numpy_correlate():
    """General depthwise taps against numpy.correlate on each zero-padded channel,
    and W_target applied on the right (a cyclic shift matrix pins orientation)."""
    T, d, K = 13, 6, 5
    rng = np.random.default_rng(9)
    X0 = rng.standard_normal((T, d)).astype(np.float32)
    taps = rng.standard_normal((d, K)).astype(np.float32)
    P = np.zeros((d, d), np.float32)
    for c in range(d):
        P[c, (c + 1) % d] = 1.0  # V^[t][j] = U[t][j-1]
    V = oracle.lm_target(X0, taps, P)
    U = np.zeros((T, d))
    for c in range(d):
        # U[t] = sum_k taps[k] X0[t+1-k]: correlate the padded signal with the
        # reversed taps (window X0[t+2-K .. t+1]).
        x = np.concatenate([np.zeros(K - 2 if K >= 2 else 0), X0[:, c].astype(np.float64),
                            np.zeros(1)])
        if K == 1:
            x = x[1:]
        U[:, c] = np.correlate(x, taps[c, ::-1].astype(np.float64), mode="valid")[:T]
    np.testing.assert_allclose(V, np.roll(U, 1, axis=1), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- section 3.3: update rule
def test_update_is_one_gradient_step_of_frobenius_loss():
    """W^(1) = W^(0) - eta * dL/dW with L = -<V^_0, Z_0 W^T>_F (torch autograd),
    and chunk 1's output is made with that weight."""
    B, d, f, K, C = 1, 6, 10, 3, 7
    T = 2 * C
    inp = rand_inputs(B, T, d, f, K, seed=21)
    eta = 0.3
    O, Wfin = run(inp, eta, C)
    Z = oracle.gated_activations(inp["H"][0], inp["W_gate"], inp["W_up"])
    V = oracle.lm_target(inp["X0"][0], inp["taps"], inp["W_target"])
    W0 = torch.tensor(inp["W_down0"], dtype=torch.float64, requires_grad=True)
    Zt = torch.from_numpy(Z[:C])
    Vt = torch.from_numpy(V[:C])
    L = -(Vt * (Zt @ W0.T)).sum()
    (g,) = torch.autograd.grad(L, W0)
    W1 = (W0 - eta * g).detach().numpy()
    O1 = Z[C:] @ W1.T
    assert rel(O[0, C:], O1) < 1e-13
    # second step with the second chunk
    W1t = torch.tensor(W1, requires_grad=True)
    L2 = -(torch.from_numpy(V[C:]) * (torch.from_numpy(Z[C:]) @ W1t.T)).sum()
    (g2,) = torch.autograd.grad(L2, W1t)
    assert rel(Wfin[0], (W1t - eta * g2).detach().numpy()) < 1e-13


@pytest.mark.parametrize("C", [1, 3, 7, 64])
def test_final_weight_closed_form_independent_of_chunk(C):
    """Summing the rule over chunks: W^(N) = W^(0) + eta * V^^T Z over all tokens."""
    inp = rand_inputs(1, 45, 8, 12, 4, seed=13)
    eta = 0.05
    _, W = run(inp, eta, C)
    Z = oracle.gated_activations(inp["H"][0], inp["W_gate"], inp["W_up"])
    V = oracle.lm_target(inp["X0"][0], inp["taps"], inp["W_target"])
    ref = inp["W_down0"].astype(np.float64) + eta * V.T @ Z
    assert rel(W[0], ref) < 1e-13


def test_final_weight_grid_matches_full():
    inp = rand_inputs(1, 33, 10, 14, 3, seed=17)
    eta = 0.02
    _, W = run(inp, eta, 8)
    ms, ns = [0, 3, 9], [1, 2, 13]
    g = oracle.final_weight_grid(inp["H"][0], inp["X0"][0], inp["W_gate"], inp["W_up"],
                                 inp["W_down0"], inp["taps"], inp["W_target"], eta, ms, ns)
    assert rel(g, W[0][np.ix_(ms, ns)]) < 1e-13


# ---------------------------------------------------------------- section 3.2: three forms
SHAPES = [
    # B, T, d, f, K, C
    (1, 32, 8, 16, 4, 8),     # even chunks
    (1, 37, 8, 16, 4, 8),     # ragged tail chunk
    (2, 23, 6, 10, 3, 5),     # batched, ragged
    (1, 17, 4, 8, 2, 1),      # per-token updates (C = 1)
    (1, 12, 4, 8, 4, 12),     # C = T: one chunk
    (1, 12, 4, 8, 4, 50),     # C > T
    (1, 21, 4, 8, 1, 4),      # K = 1
    (1, 21, 4, 8, 9, 4),      # K > C
    (3, 9, 5, 7, 6, 2),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_sequential_chunk_parallel_dual_agree(shape):
    B, T, d, f, K, C = shape
    inp = rand_inputs(B, T, d, f, K, seed=sum(shape))
    eta = 0.1
    Os, Ws = run(inp, eta, C, "sequential")
    Op, Wp = run(inp, eta, C, "chunk_parallel")
    Od, Wd = run(inp, eta, C, "dual")
    assert rel(Op, Os) < 1e-12 and rel(Wp, Ws) < 1e-12
    assert rel(Od, Os) < 1e-12 and rel(Wd, Ws) < 1e-12


def test_chunk_at_least_T_is_static_output_but_updated_weight():
    inp = rand_inputs(1, 10, 4, 6, 3, seed=2)
    O, W = run(inp, 0.5, 10)
    O0, _ = run(inp, 0.0, 10)
    assert rel(O, O0) < 1e-14
    assert rel(W[0], inp["W_down0"].astype(np.float64)) > 1e-3


# ---------------------------------------------------------------- causality
@pytest.mark.parametrize("C", [1, 4, 6])
def test_causality_bitwise(C):
    B, T, d, f, K = 1, 24, 6, 10, 4
    inp = rand_inputs(B, T, d, f, K, seed=31)
    eta = 0.2
    O, _ = run(inp, eta, C)
    rng = np.random.default_rng(1)
    for t in [0, 5, 11, 17]:
        for name in ("H", "X0"):
            p = {k: v.copy() for k, v in inp.items()}
            p[name][0, t + 1:] += rng.standard_normal(p[name][0, t + 1:].shape).astype(np.float32)
            Op, _ = run(p, eta, C)
            assert np.array_equal(Op[0, :t + 1], O[0, :t + 1]), (name, t)


def test_chunk_start_token_reaches_previous_update():
    """X0 at a chunk start feeds the target of the previous chunk's last token
    (tap 0 looks one ahead), so it changes the current chunk's outputs."""
    B, T, d, f, K, C = 1, 16, 6, 10, 4, 4
    inp = rand_inputs(B, T, d, f, K, seed=41)
    O, _ = run(inp, 0.2, C)
    p = {k: v.copy() for k, v in inp.items()}
    p["X0"][0, 8] += 1.0  # first token of chunk 2
    Op, _ = run(p, 0.2, C)
    assert np.array_equal(Op[0, :8], O[0, :8])
    assert not np.array_equal(Op[0, 8:12], O[0, 8:12])


# ---------------------------------------------------------------- linearity, batching
def test_linear_in_eta():
    inp = rand_inputs(1, 30, 6, 10, 4, seed=8)
    O0, W0 = run(inp, 0.0, 7)
    O1, W1 = run(inp, 0.05, 7)
    O2, W2 = run(inp, 0.1, 7)
    assert rel(O2 - O0, 2 * (O1 - O0)) < 1e-12
    assert rel(W2 - W0, 2 * (W1 - W0)) < 1e-12


def test_batched_equals_single_calls_and_own_states():
    B, T, d, f, K, C = 3, 19, 6, 8, 3, 4
    inp = rand_inputs(B, T, d, f, K, seed=4)
    rng = np.random.default_rng(5)
    Winit = (rng.standard_normal((B, d, f)) * 0.1).astype(np.float32)
    O, W = oracle.forward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], Winit,
                          inp["taps"], inp["W_target"], 0.1, C)
    for b in range(B):
        Ob, Wb = oracle.forward(inp["H"][b], inp["X0"][b], inp["W_gate"], inp["W_up"],
                                Winit[b], inp["taps"], inp["W_target"], 0.1, C)
        assert np.array_equal(O[b], Ob) and np.array_equal(W[b], Wb)


def test_rejects_inexact_inputs():
    inp = rand_inputs(1, 4, 2, 2, 1, seed=0)
    inp["H"] = inp["H"].astype(np.float64) + 1e-12
    with pytest.raises(ValueError):
        run(inp, 0.1, 2)


# ------------------------------------------ ablation targets (section 6 table)
def test_target_variants_are_their_definitions():
    """Without the conv V^ = X0 W_target; without the projection V^ = Conv1D(X0);
    without both V^ = X0 (exactly); the conv checked against numpy.correlate."""
    T, d, K = 11, 5, 3
    rng = np.random.default_rng(31)
    X0 = rng.standard_normal((T, d)).astype(np.float32)
    taps = rng.standard_normal((d, K)).astype(np.float32)
    Wt = rng.standard_normal((d, d)).astype(np.float32)
    assert np.array_equal(oracle.lm_target(X0, None, None, target="embed"), X0.astype(np.float64))
    np.testing.assert_allclose(oracle.lm_target(X0, None, Wt, target="proj"),
                               X0.astype(np.float64) @ Wt.astype(np.float64),
                               rtol=1e-13, atol=1e-13)
    U = np.zeros((T, d))
    for c in range(d):
        x = np.concatenate([np.zeros(K - 2), X0[:, c].astype(np.float64), np.zeros(1)])
        U[:, c] = np.correlate(x, taps[c, ::-1].astype(np.float64), mode="valid")[:T]
    np.testing.assert_allclose(oracle.lm_target(X0, taps, None, target="conv"), U,
                               rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.lm_target(X0, taps, Wt, target="nope")


def test_reconstruction_alignment_is_the_window_shifted_by_one():
    """The reconstruction alignment (section 4's table: V_t from the token's own
    embedding) ends the conv's window at t: a one-hot tap 0 gives V^ = X0
    exactly, the general conv is sum_k taps[k] X0[t-k] (explicit loops), and
    every row is the next-token alignment's previous row."""
    T, d, K = 9, 4, 3
    rng = np.random.default_rng(35)
    X0 = rng.standard_normal((T, d)).astype(np.float32)
    taps = rng.standard_normal((d, K)).astype(np.float32)
    Wt = rng.standard_normal((d, d)).astype(np.float32)
    one_hot = np.zeros((d, K), dtype=np.float32)
    one_hot[:, 0] = 1.0
    assert np.array_equal(oracle.lm_target(X0, one_hot, None, target="conv", align="self"),
                          X0.astype(np.float64))
    U = np.zeros((T, d))
    for t in range(T):
        for c in range(d):
            for k in range(K):
                if t - k >= 0:
                    U[t, c] += float(taps[c, k]) * float(X0[t - k, c])
    V_self = oracle.lm_target(X0, taps, Wt, align="self")
    np.testing.assert_allclose(V_self, U @ Wt.astype(np.float64), rtol=1e-12, atol=1e-12)
    V_next = oracle.lm_target(X0, taps, Wt)
    np.testing.assert_allclose(V_self[1:], V_next[:-1], rtol=1e-13, atol=1e-13)
    # the variants without a conv do not depend on the alignment
    for target in ("proj", "embed"):
        assert np.array_equal(oracle.lm_target(X0, taps, Wt, target=target, align="self"),
                              oracle.lm_target(X0, taps, Wt, target=target))
    with pytest.raises(ValueError):
        oracle.lm_target(X0, taps, Wt, align="prev")


def test_reconstruction_alignment_layer_closed_form():
    """With the reconstruction alignment the update rule is unchanged:
    W_final = W0 + eta V^^T Z with V^ from the shifted window; forms agree."""
    inp = rand_inputs(1, 29, 8, 12, 4, seed=36)
    eta, C = 0.05, 6
    outs = [oracle.forward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"],
                           inp["taps"], inp["W_target"], eta, C, form=form, align="self")
            for form in ("sequential", "chunk_parallel", "dual")]
    for O, W in outs[1:]:
        assert rel(O, outs[0][0]) < 1e-12 and rel(W, outs[0][1]) < 1e-12
    X0 = inp["X0"][0].astype(np.float64)
    taps = inp["taps"].astype(np.float64)
    U = np.zeros_like(X0)
    for k in range(taps.shape[1]):
        U[k:] += taps[:, k] * X0[:X0.shape[0] - k]
    V = U @ inp["W_target"].astype(np.float64)
    Z = oracle.gated_activations(inp["H"][0], inp["W_gate"], inp["W_up"])
    ref = inp["W_down0"].astype(np.float64) + eta * V.T @ Z
    assert rel(outs[0][1][0], ref) < 1e-13
    # chunk 0's outputs use W0 in either alignment
    O0 = Z[:C] @ inp["W_down0"].astype(np.float64).T
    assert rel(outs[0][0][0][:C], O0) < 1e-13


@pytest.mark.parametrize("target", ["proj", "conv", "embed"])
def test_target_variant_layer_closed_form_and_forms_agree(target):
    """Every variant still follows the update rule: W_final = W0 + eta V^^T Z, and
    the three evaluation forms agree."""
    inp = rand_inputs(1, 37, 8, 12, 3, seed=33)
    eta, C = 0.05, 8
    outs = [oracle.forward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"],
                           inp["taps"], inp["W_target"], eta, C, form=form, target=target)
            for form in ("sequential", "chunk_parallel", "dual")]
    for O, W in outs[1:]:
        assert rel(O, outs[0][0]) < 1e-12 and rel(W, outs[0][1]) < 1e-12
    X0 = inp["X0"][0].astype(np.float64)
    V = {"proj": X0 @ inp["W_target"].astype(np.float64),
         "embed": X0,
         "conv": oracle.lm_target(inp["X0"][0], inp["taps"], None, target="conv")}[target]
    Z = oracle.gated_activations(inp["H"][0], inp["W_gate"], inp["W_up"])
    ref = inp["W_down0"].astype(np.float64) + eta * V.T @ Z
    assert rel(outs[0][1][0], ref) < 1e-13
