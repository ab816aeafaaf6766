"""Backward pass on the GPU against the oracle's backward (fp64): every
gradient (H, X0, W_gate, W_up, the starting weight, taps, W_target, eta) to
the activation dtype's tolerance, on shapes that span several tiles and a
ragged last chunk, for both scan tile shapes (64 x 64 when 256 does not divide
d and f, 256 x 256 otherwise), every target variant and both alignments."""
import numpy as np
import pytest
import torch

from oracle.backward import _conv as oracle_conv
from oracle.backward import backward as oracle_backward
from chunk_wise_weight_chunked_amd import synth
from chunk_wise_weight_chunked_amd import ttt_mlp as tm

from _common import numpy_inputs, rel, to_device, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tm.load()


CASES = [
    # B, T, d, f, K, C, dtype, target, align, per-sequence start, dW_final
    (2, 333, 128, 192, 4, 100, torch.bfloat16, "conv_proj", "next", False, True),
    (1, 300, 192, 256, 4, 64, torch.float32, "conv_proj", "next", False, True),
    (2, 600, 256, 512, 4, 128, torch.bfloat16, "conv_proj", "next", False, False),  # 256-tiles
    (1, 257, 256, 256, 3, 256, torch.float32, "conv_proj", "self", True, True),
    (2, 200, 128, 192, 8, 64, torch.bfloat16, "conv_proj", "self", True, False),
    (1, 300, 128, 192, 4, 50, torch.bfloat16, "proj", "next", False, True),
    (1, 300, 128, 192, 4, 50, torch.float32, "conv", "next", False, True),
    (2, 150, 64, 128, 2, 1000, torch.bfloat16, "embed", "next", False, True),   # one chunk
    (1, 1, 64, 64, 1, 1, torch.bfloat16, "conv_proj", "next", False, True),     # T = 1
    (2, 70, 64, 128, 4, 1, torch.float32, "conv_proj", "next", False, True),    # C = 1
    (1, 130, 128, 64, 1, 65, torch.bfloat16, "conv_proj", "self", False, True),  # K = 1, C odd
    # gate/up weight rows longer than 4 KB (stored in tiles)
    (1, 150, 2112, 128, 4, 64, torch.bfloat16, "conv_proj", "next", False, True),
    (1, 150, 1088, 128, 4, 64, torch.float32, "conv_proj", "next", False, True),
]


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _keep(x):
    return x


def deta_with_roundings(ni, eta, C, dO, dWN, target, align, rz=_keep, ru=_keep, rv=_keep,
                        rs=_keep):
    """eta's gradient sum_j <S_j, V^_jᵀ Z_j> in fp64, with the operands passed
    through the given roundings at the points where a bf16 pipeline rounds
    them: Z, the conv output U, V^ = U W_target, and each S_j (the reversed
    scan's slots)."""
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    shift = 1 if align == "next" else 0
    H, X0 = ni["H"].astype(np.float64), ni["X0"].astype(np.float64)
    Wg, Wu = ni["W_gate"].astype(np.float64), ni["W_up"].astype(np.float64)
    B, T, d = H.shape
    f = Wg.shape[0]
    N = -(-T // C)
    total = 0.0
    for b in range(B):
        Ag, Au = H[b] @ Wg.T, H[b] @ Wu.T
        Z = rz(Ag / (1.0 + np.exp(-Ag)) * Au)
        U = ru(oracle_conv(X0[b], ni["taps"].astype(np.float64), shift)) if conv else X0[b]
        V = rv(U @ ni["W_target"].astype(np.float64)) if proj else U
        S = np.zeros((d, f)) if dWN is None else dWN[b].astype(np.float64).copy()
        for j in reversed(range(N)):
            r = slice(j * C, min(T, (j + 1) * C))
            total += float(np.sum(V[r] * (Z[r] @ rs(S).T)))
            S = S + dO[b][r].T.astype(np.float64) @ Z[r]
    return total


def bf16_deta_spread(ni, eta, C, dO, dWN, target, align, exact):
    """How far bf16 rounding moves eta's gradient, relative to it: each
    rounding point's own shift (Z, U with a conv, V^ with a projection, S),
    combined in quadrature as independent errors are (their actual sum can
    cancel by chance, which would make a bound on it too tight), or their
    actual joint shift if that is larger."""
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    points = [{"rz": _bf16}, {"rs": _bf16}]
    if conv:
        points.append({"ru": _bf16})
    if proj:
        points.append({"rv": _bf16})
    shifts = [abs(deta_with_roundings(ni, eta, C, dO, dWN, target, align, **p) - exact)
              for p in points]
    together = abs(deta_with_roundings(ni, eta, C, dO, dWN, target, align,
                                       **{k: v for p in points for k, v in p.items()}) - exact)
    spread = max(float(np.sqrt(np.sum(np.square(shifts)))), together)
    return spread / max(abs(exact), 1e-30)


def _id(c):
    return (f"B{c[0]}T{c[1]}d{c[2]}f{c[3]}C{c[5]}{str(c[6])[6:]}-{c[7]}-{c[8]}"
            f"{'-W' if c[9] else ''}{'-dWN' if c[10] else ''}")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_matches_oracle(case):
    B, T, d, f, K, C, dtype, target, align, per_seq, with_dwn = case
    print(f"[backward] {_id(case)}", flush=True)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=55)
    gen = torch.Generator().manual_seed(56)
    dO = torch.randn((B, T, d), generator=gen).to(dtype)
    dWN = (0.1 * torch.randn((B, d, f), generator=gen)) if with_dwn else None
    W_start = (inp["W_down0"].float()[None].repeat(B, 1, 1)
               + 0.01 * torch.randn((B, d, f), generator=gen)) if per_seq else None
    dev = to_device(inp)
    eta = 2e-2
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    g = tm.backward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                            dev["taps"] if conv else None, dev["W_target"] if proj else None,
                            eta, C, dO.cuda(),
                            dW_final=None if dWN is None else dWN.cuda(),
                            W_start=None if W_start is None else W_start.cuda(),
                            target=target, align=align, conv_k=K)
    torch.cuda.synchronize()
    ni = numpy_inputs(inp)
    w0 = ni["W_down0"] if W_start is None else W_start.numpy()
    ref = oracle_backward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], w0, ni["taps"],
                          ni["W_target"], eta, C, dO.float().numpy(),
                          None if dWN is None else dWN.numpy(), target=target, align=align)
    tol = tol_for(dtype)
    pairs = [("H", "H"), ("X0", "X0"), ("W_gate", "W_gate"), ("W_up", "W_up"),
             ("W_start", "W_state0")]
    if conv:
        pairs.append(("taps", "taps"))
    if proj:
        pairs.append(("W_target", "W_target"))
    errs = {}
    for mine, theirs in pairs:
        errs[mine] = rel(g[mine].float().cpu().numpy().astype(np.float64), ref[theirs])
    # eta's gradient is one inner product <V^, G> whose terms cancel (by ~5000x
    # at these shapes): its rounding error is bounded by the operands' norms
    d_eta = abs(g["eta"].item() - ref["eta"])
    # (V^ = 0, e.g. one token whose only tap reads the next one: eta's gradient is 0)
    e_eta = d_eta / ref["eta_scale"] if ref["eta_scale"] > 0 else d_eta
    e_eta_plain = d_eta / max(abs(ref["eta"]), 1e-30)
    bound = 1e-3
    if dtype == torch.bfloat16:
        # the plain relative bound: three times what the bf16 roundings of
        # the operands alone move eta's gradient (0.1%-16% at these shapes)
        spread = bf16_deta_spread(ni, eta, C, dO.float().numpy(),
                                  None if dWN is None else dWN.numpy(), target, align, ref["eta"])
        bound = 3.0 * spread + 2e-3
    print("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) +
          f"  eta {e_eta:.2e} (plain relative {e_eta_plain:.2e}, bound {bound:.2e})", flush=True)
    for k, v in errs.items():
        assert v <= tol, (k, v)
    assert e_eta <= tol, e_eta
    assert e_eta_plain <= bound, (e_eta_plain, bound)


def test_backward_is_deterministic():
    B, T, d, f, K, C = 1, 300, 256, 256, 4, 64
    inp = synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=57)
    dev = to_device(inp)
    dO = torch.randn((B, T, d), generator=torch.Generator().manual_seed(58)).to(torch.bfloat16)
    runs = [tm.backward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                                dev["taps"], dev["W_target"], 1e-2, C, dO.cuda())
            for _ in range(2)]
    torch.cuda.synchronize()
    for k, v in runs[0].items():
        assert torch.equal(v, runs[1][k]), k


def test_backward_rejects_bad_arguments():
    B, T, d, f, K, C = 1, 64, 64, 128, 4, 16
    inp = synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=59)
    dev = to_device(inp)
    dO = torch.zeros_like(dev["H"])
    desc = tm.make_desc(B, T, d, f, C, K, 1e-2, torch.bfloat16)
    ws = torch.empty(tm.ttt_mlp_backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = [torch.empty_like(dev["H"]), torch.empty_like(dev["H"])] + \
        [torch.empty(s, dtype=torch.float32, device="cuda")
         for s in ((f, d), (f, d), (B, d, f), (d, K), (d, d), (1,))]
    args = [dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"], None, dev["taps"],
            dev["W_target"], dO, None] + out
    with pytest.raises(tm.TTTError) as e:
        tm.ttt_mlp_backward_batched(desc, *args, ws, ws_bytes=ws.numel() - 256)
    assert e.value.status == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    bad = list(args)
    bad[10] = dev["H"]  # dH on top of H
    with pytest.raises(tm.TTTError) as e:
        tm.ttt_mlp_backward_batched(desc, *bad, ws)
    assert "overlaps" in str(e.value)
    bad = list(args)
    bad[8] = None  # no dO
    with pytest.raises(tm.TTTError) as e:
        tm.ttt_mlp_backward_batched(desc, *bad, ws)
    assert "dO is NULL" in str(e.value)


@pytest.mark.parametrize("name", ["qwen3_4b_128k", "multi_session_16x8k"])
def test_backward_full_size_sampled(name):
    """The backward at a full workload size, as `bench.py --backward` runs it:
    rows of dW_gate / dW_up and columns of dW_start for a few features against
    the oracle's per-feature form (which needs only those features of Z)."""
    from oracle.backward import sampled_weight_grads
    w = synth.WORKLOADS[name]
    print(f"[backward full] {name}: drawing inputs", flush=True)
    inp = synth.workload_inputs(w)
    gen = torch.Generator().manual_seed(60)
    B, T, d, f = w.batch, w.seq_len, w.d_model, w.d_ff
    dO = torch.randn((B, T, d), generator=gen).to(w.dtype)
    dWN = 0.01 * torch.randn((B, d, f), generator=gen)
    dev = to_device(inp)
    g = tm.backward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                            dev["taps"], dev["W_target"], w.eta, w.chunk, dO.cuda(),
                            dW_final=dWN.cuda())
    torch.cuda.synchronize()
    F = [0, 4097, f - 1]
    got = {"W_gate": g["W_gate"][F].cpu().numpy(), "W_up": g["W_up"][F].cpu().numpy(),
           "W_start": g["W_start"][:, :, F].cpu().numpy()}
    del g, dev
    torch.cuda.empty_cache()
    print(f"[backward full] {name}: oracle on features {F}", flush=True)
    ni = numpy_inputs(inp)
    ref = sampled_weight_grads(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                               ni["taps"], ni["W_target"], w.eta, w.chunk,
                               dO.float().numpy(), F, dWN.numpy())
    errs = {k: rel(got[k], ref[k]) for k in got}
    print("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol_for(w.dtype), (k, v)
