"""Pins of the oracle's backward pass (CPU).

The backward is checked against two things it shares no code with: central
finite differences of the C oracle's forward (an independent implementation
of the layer), and torch autograd through a forward written here with torch
ops.  Plus structural facts: with eta = 0 nothing flows into X0, taps or
W_target and the weight gradient is dW_final + sum_t dO[t]ᵀ Z[t]."""
import numpy as np
import pytest
import torch

import oracle
from oracle.backward import backward

H_STEP = 2.0 ** -10  # x +- H_STEP is exact in float32 for |x| < 2^13


def rand_case(B, T, d, f, K, seed, per_seq_w0=False):
    rng = np.random.default_rng(seed)
    f32 = np.float32
    inp = dict(
        H=rng.standard_normal((B, T, d)).astype(f32),
        X0=rng.standard_normal((B, T, d)).astype(f32),
        W_gate=(rng.standard_normal((f, d)) / np.sqrt(d)).astype(f32),
        W_up=(rng.standard_normal((f, d)) / np.sqrt(d)).astype(f32),
        W_down0=(rng.standard_normal((B, d, f) if per_seq_w0 else (d, f)) / np.sqrt(f)).astype(f32),
        taps=(rng.standard_normal((d, K)) / np.sqrt(K)).astype(f32),
        W_target=(rng.standard_normal((d, d)) / np.sqrt(d)).astype(f32),
    )
    dO = rng.standard_normal((B, T, d)).astype(f32)
    dWN = rng.standard_normal((B, d, f)).astype(f32)
    return inp, dO, dWN


def loss(inp, eta, C, dO, dWN, target, align):
    O, W = oracle.forward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"],
                          inp["taps"], inp["W_target"], eta, C, target=target, align=align)
    return float(np.sum(O * dO) + np.sum(W * dWN))


CASES = [
    # B, T, d, f, K, C, target, align, per-sequence W0
    (1, 13, 4, 6, 3, 4, "conv_proj", "next", False),
    (2, 11, 4, 6, 4, 3, "conv_proj", "self", False),
    (2, 9, 3, 5, 2, 4, "conv_proj", "next", True),
    (1, 10, 4, 6, 3, 3, "proj", "next", False),
    (1, 10, 4, 6, 3, 3, "conv", "self", False),
    (1, 10, 4, 6, 3, 20, "embed", "next", False),   # one chunk
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[1]}C{c[5]}-{c[6]}-{c[7]}")
def test_backward_matches_finite_differences_of_the_c_forward(case):
    B, T, d, f, K, C, target, align, per_seq = case
    inp, dO, dWN = rand_case(B, T, d, f, K, seed=101 + T, per_seq_w0=per_seq)
    eta = 0.3
    g = backward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
                 inp["W_target"], eta, C, dO, dWN, target=target, align=align)
    rng = np.random.default_rng(7)
    names = ["H", "X0", "W_gate", "W_up", "W_down0"]
    if target in ("conv_proj", "conv"):
        names.append("taps")
    if target in ("conv_proj", "proj"):
        names.append("W_target")
    for name in names:
        x = inp[name]
        grad = g["W_state0"] if (name == "W_down0" and per_seq) else g[name]
        assert grad.shape == x.shape, name
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            plus, minus = dict(inp), dict(inp)
            plus[name], minus[name] = x.copy(), x.copy()
            plus[name][idx] += H_STEP
            minus[name][idx] -= H_STEP
            fd = (loss(plus, eta, C, dO, dWN, target, align) -
                  loss(minus, eta, C, dO, dWN, target, align)) / (2 * H_STEP)
            assert abs(fd - grad[idx]) <= 2e-5 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    for name in ("taps", "W_target"):
        if name not in names:
            assert g[name] is None
    fd = (loss(inp, eta + 1e-4, C, dO, dWN, target, align) -
          loss(inp, eta - 1e-4, C, dO, dWN, target, align)) / 2e-4
    assert abs(fd - g["eta"]) <= 1e-6 * max(1.0, abs(fd)), (fd, g["eta"])


def torch_forward(H, X0, Wg, Wu, W0, taps, Wt, eta, C, shift):
    """The layer with torch ops, float64: one chunk at a time."""
    B, T, d = H.shape
    K = taps.shape[1]
    outs, finals = [], []
    for b in range(B):
        Z = torch.nn.functional.silu(H[b] @ Wg.T) * (H[b] @ Wu.T)
        pad = torch.nn.functional.pad(X0[b], (0, 0, K, K))
        U = sum(taps[:, k] * pad[K + shift - k:K + shift - k + T] for k in range(K))
        V = U @ Wt
        W = W0[b] if W0.dim() == 3 else W0
        o = []
        for j in range(0, T, C):
            o.append(Z[j:j + C] @ W.T)
            W = W + eta * V[j:j + C].T @ Z[j:j + C]
        outs.append(torch.cat(o))
        finals.append(W)
    return torch.stack(outs), torch.stack(finals)


@pytest.mark.parametrize("align", ["next", "self"])
def test_backward_matches_torch_autograd(align):
    B, T, d, f, K, C = 2, 23, 8, 12, 4, 5
    inp, dO, dWN = rand_case(B, T, d, f, K, seed=202)
    eta = 0.2
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    te = torch.tensor(eta, dtype=torch.float64, requires_grad=True)
    O, W = torch_forward(t["H"], t["X0"], t["W_gate"], t["W_up"], t["W_down0"], t["taps"],
                         t["W_target"], te, C, 1 if align == "next" else 0)
    L = (O * torch.tensor(dO, dtype=torch.float64)).sum() + \
        (W * torch.tensor(dWN, dtype=torch.float64)).sum()
    L.backward()
    g = backward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
                 inp["W_target"], eta, C, dO, dWN, align=align)
    for k in inp:
        ref = t[k].grad.numpy()
        got = g[k]
        assert np.linalg.norm(got - ref) <= 1e-11 * np.linalg.norm(ref), k
    assert abs(g["eta"] - te.grad.item()) <= 1e-11 * abs(te.grad.item())


def test_backward_with_eta_zero():
    """eta = 0: the static MLP.  The target gets no gradient, and the weight's
    gradient is dW_final + sum over all tokens of dO[t]ᵀ Z[t]."""
    B, T, d, f, K, C = 1, 17, 4, 6, 3, 5
    inp, dO, dWN = rand_case(B, T, d, f, K, seed=303)
    g = backward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
                 inp["W_target"], 0.0, C, dO, dWN)
    assert not g["X0"].any() and not g["taps"].any() and not g["W_target"].any()
    Z = oracle.gated_activations(inp["H"][0], inp["W_gate"], inp["W_up"])
    ref = dWN[0].astype(np.float64) + dO[0].astype(np.float64).T @ Z
    np.testing.assert_allclose(g["W_down0"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("target,align", [("conv_proj", "next"), ("conv", "self"),
                                          ("embed", "next")])
def test_sampled_weight_grads_match_the_full_backward(target, align):
    """The per-feature form used on full-size runs gives the full backward's
    rows of dW_gate / dW_up and columns of dW_start."""
    from oracle.backward import sampled_weight_grads
    B, T, d, f, K, C = 2, 29, 8, 12, 3, 6
    inp, dO, dWN = rand_case(B, T, d, f, K, seed=404)
    eta = 0.1
    g = backward(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
                 inp["W_target"], eta, C, dO, dWN, target=target, align=align)
    F = [0, 5, 11]
    s = sampled_weight_grads(inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"],
                             inp["taps"], inp["W_target"], eta, C, dO, F, dWN, target=target,
                             align=align)
    np.testing.assert_allclose(s["W_gate"], g["W_gate"][F], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s["W_up"], g["W_up"][F], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s["W_start"], g["W_state0"][:, :, F], rtol=1e-11, atol=1e-11)
