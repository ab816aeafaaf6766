"""Shares of a sequence on one GPU: the per-device parts of the chunk-wise
update's context-parallel form (In-Place TTT page, section 3.2: every device
sums the increments of its own chunks, one exclusive prefix sum over the
devices gives each its starting weight, then every device outputs its
chunks).  A sequence is cut into consecutive shares of whole chunks; each
share's increment sum S_r comes from ttt_mlp_share_increment, the prefix sum
over shares is formed here (the collective's part), and ttt_mlp_share_forward
gives each share's outputs from W_down0 + S_0 + ... + S_{r-1}.  The joined
outputs and the last share's weight are checked against the oracle (small
shapes) and against one call over the whole sequence (full size)."""
import numpy as np
import pytest
import torch

import oracle
from chunk_wise_weight_chunked_amd import synth
from chunk_wise_weight_chunked_amd import ttt_mlp as tm

from _common import numpy_inputs, rel, to_device, tol_for

pytestmark = pytest.mark.gpu

HALO = 7  # X0 rows a share passes from before its first token


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tm.load()


def _halos(X0, t0, t1):
    """(X0_left [B][7][d] or None, X0_right [B][d] or None) of share [t0, t1)."""
    B, T, d = X0.shape
    left = None
    if t0 > 0:
        left = torch.zeros((B, HALO, d), dtype=X0.dtype, device=X0.device)
        n = min(HALO, t0)
        left[:, HALO - n:] = X0[:, t0 - n:t0]
    right = X0[:, t1].contiguous() if t1 < T else None
    return left, right


def run_shares(dev, bounds, eta, C, target="conv_proj", align="next", K=4, reuse=True,
               mode="auto"):
    """Runs the shares [bounds[r], bounds[r+1]) of every sequence; returns
    (O joined [B][T][d], weight after the last share [B][d][f], [S_r])."""
    H, X0 = dev["H"], dev["X0"]
    B, T, d = H.shape
    f = dev["W_gate"].shape[0]
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    taps = dev["taps"] if conv else None
    Wt = dev["W_target"] if proj else None
    parts = []
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        desc = tm.make_desc(B, t1 - t0, d, f, C, K, eta, H.dtype, mode, target=target,
                            align=align)
        left, right = _halos(X0, t0, t1)
        share = tm.make_share(left, right)
        Hr, Xr = H[:, t0:t1].contiguous(), X0[:, t0:t1].contiguous()
        ws = tm.alloc_workspace(desc)
        S = torch.empty((B, d, f), dtype=torch.float32, device=H.device)
        tm.ttt_mlp_share_increment(desc, share, Hr, Xr, dev["W_gate"], dev["W_up"], taps, Wt,
                                   S, ws)
        parts.append((desc, share, left, right, Hr, Xr, ws, S))
    # the exclusive prefix sum over the shares (a collective across devices)
    W0 = dev["W_down0"].float()[None].expand(B, d, f)
    starts, acc = [], torch.zeros((B, d, f), dtype=torch.float32, device=H.device)
    for p in parts:
        starts.append(W0 + acc)
        acc = acc + p[7]
    outs = []
    W = None
    for (desc, share, left, right, Hr, Xr, ws, S), Win in zip(parts, starts):
        O = torch.empty_like(Hr)
        W = Win.contiguous()
        tm.ttt_mlp_share_forward(desc, share, 1 if reuse else 0, Hr, Xr, dev["W_gate"],
                                 dev["W_up"], taps, Wt, O, W, ws)
        outs.append(O)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), W, [p[7] for p in parts]


CASES = [
    # B, T, d, f, K, C, dtype, target, align, share bounds
    (2, 700, 256, 512, 4, 64, torch.bfloat16, "conv_proj", "next", [0, 192, 448, 700]),
    (1, 600, 128, 192, 8, 64, torch.bfloat16, "conv_proj", "self", [0, 128, 256, 600]),
    (2, 513, 192, 256, 5, 100, torch.float32, "conv_proj", "next", [0, 100, 300, 513]),
    (1, 300, 128, 192, 4, 4, torch.bfloat16, "conv", "next", [0, 4, 8, 300]),   # shares < halo
    (1, 400, 128, 256, 4, 64, torch.bfloat16, "proj", "next", [0, 256, 400]),
    (1, 260, 64, 128, 8, 20, torch.float32, "conv", "self", [0, 20, 40, 60, 260]),
]


def _id(c):
    return f"B{c[0]}T{c[1]}d{c[2]}f{c[3]}K{c[4]}C{c[5]}{str(c[6])[6:]}-{c[7]}-{c[8]}-{len(c[9]) - 1}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_shares_match_oracle(case):
    B, T, d, f, K, C, dtype, target, align, bounds = case
    print(f"[share] {_id(case)}", flush=True)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=301)
    dev = to_device(inp)
    eta = 2e-2
    O, W, S = run_shares(dev, bounds, eta, C, target, align, K)
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C, target=target, align=align)
    W0 = ni["W_down0"].astype(np.float64)
    Og = O.float().cpu().numpy()
    Wg = W.cpu().numpy()
    Ssum = sum(s.double() for s in S).cpu().numpy()
    tol = tol_for(dtype)
    e_o, e_w, e_dw = rel(Og, Oo), rel(Wg, Wo), rel(Wg - W0, Wo - W0)
    e_s = rel(Ssum, Wo - W0)
    worst = max(rel(Og[b, i:i + C], Oo[b, i:i + C]) for b in range(B) for i in range(0, T, C))
    print(f"  rel O {e_o:.3e} (worst chunk {worst:.3e})  W {e_w:.3e}  dW {e_dw:.3e}  "
          f"sum S_r {e_s:.3e}", flush=True)
    assert max(e_o, worst, e_w, e_dw, e_s) <= tol, (e_o, worst, e_w, e_dw, e_s)
    # recomputing S1 and S2 in the forward call gives the same bits as reusing them
    O2, W2, _ = run_shares(dev, bounds, eta, C, target, align, K, reuse=False)
    assert torch.equal(O2, O) and torch.equal(W2, W)


def test_one_share_is_the_batched_call():
    """A single share covering the sequence (no halo rows) is the batched
    forward from W_down0, bit for bit; its increment sum is the weight change."""
    B, T, d, f, K, C = 2, 600, 256, 512, 4, 64
    inp = synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=302)
    dev = to_device(inp)
    eta = 2e-2
    O, W, S = run_shares(dev, [0, T], eta, C)
    O1, W1 = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                                dev["taps"], dev["W_target"], eta, C)
    torch.cuda.synchronize()
    assert torch.equal(O, O1) and torch.equal(W, W1)
    dW = (W1 - dev["W_down0"].float()[None]).double().cpu().numpy()
    e = rel(S[0].double().cpu().numpy(), dW)
    print(f"  increment sum vs weight change: rel {e:.3e}", flush=True)
    assert e <= 1e-5


def test_full_size_eight_shares():
    """qwen3_4b_32k (32768 tokens, C = 512) as eight shares of 4096 tokens in
    the bench's launch configuration: the joined outputs and the last share's
    weight against one call over the whole sequence, and sampled entries of the
    final weight against the oracle's closed form."""
    w = synth.WORKLOADS["qwen3_4b_32k"]
    print(f"[share full] {w.name}: drawing inputs", flush=True)
    inp = synth.workload_inputs(w)
    dev = to_device(inp)
    T, C = w.seq_len, w.chunk
    bounds = list(range(0, T + 1, T // 8))
    O, W, S = run_shares(dev, bounds, w.eta, C, K=w.conv_k)
    print(f"[share full] {w.name}: shares done", flush=True)
    O1, W1 = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                                dev["taps"], dev["W_target"], w.eta, C)
    torch.cuda.synchronize()
    e_o = rel(O.float().cpu().numpy(), O1.float().cpu().numpy())
    diff = (O.float() - O1.float()).reshape(T // C, C, -1)
    ref = O1.float().reshape(T // C, C, -1)
    worst = float((diff.norm(dim=(1, 2)) / ref.norm(dim=(1, 2))).max())
    W0 = dev["W_down0"].float()[None]
    e_w = rel(W.cpu().numpy(), W1.cpu().numpy())
    e_dw = rel((W - W0).cpu().numpy(), (W1 - W0).cpu().numpy())
    print(f"  vs one call: rel O {e_o:.3e} (worst chunk {worst:.3e})  W {e_w:.3e}  dW {e_dw:.3e}",
          flush=True)
    # the prefix sums differ from the one call's only in fp32 summation order;
    # a bf16 weight slot may round the other way where they differ
    assert e_o <= 1e-3 and worst <= 1e-3 and e_dw <= 1e-4
    del dev
    ni = numpy_inputs(inp)
    rng = np.random.default_rng(1)
    ms = np.sort(rng.choice(w.d_model, 3, replace=False))
    ns = np.sort(rng.choice(w.d_ff, 6, replace=False))
    Wg = oracle.final_weight_grid(ni["H"][0], ni["X0"][0], ni["W_gate"], ni["W_up"],
                                  ni["W_down0"], ni["taps"], ni["W_target"], w.eta, ms, ns)
    got = W[0].cpu().numpy()[np.ix_(ms, ns)]
    W0s = ni["W_down0"].astype(np.float64)[np.ix_(ms, ns)]
    e_g, e_gd = rel(got, Wg), rel(got - W0s, Wg - W0s)
    print(f"  W_final sample vs oracle: rel {e_g:.3e}, dW rel {e_gd:.3e}", flush=True)
    assert e_g <= tol_for(w.dtype) and e_gd <= tol_for(w.dtype)
