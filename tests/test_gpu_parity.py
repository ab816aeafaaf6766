"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Every case draws seeded inputs (chunk_wise_weight_chunked_amd.synth), runs the
library on the GPU and the oracle on the host, and compares output O, the final
fast weight, and the weight change W_final - W_down0 by relative Frobenius
error: <= 1e-4 for fp32 workloads, <= 2e-2 for bf16 inputs with the fp32 state.
Small shapes span several 256-row tiles, ragged tails, padded chunks and
partial weight tiles; the five named workloads run at full size with the
oracle on a causal prefix plus sampled entries of the final weight (closed
form), in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
from chunk_wise_weight_chunked_amd import synth
from chunk_wise_weight_chunked_amd import ttt_mlp as tm

from _common import numpy_inputs, rel, to_device, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tm.load()
    yield
    torch.cuda.synchronize()


def run_gpu(inp_dev, eta, C, mode="auto", max_group=0, W_state=None):
    B = inp_dev["H"].shape[0]
    O, W = tm.forward_batched(inp_dev["H"], inp_dev["X0"], inp_dev["W_gate"], inp_dev["W_up"],
                              inp_dev["W_down0"], inp_dev["taps"], inp_dev["W_target"], eta, C,
                              W_state=W_state, mode=mode, max_group=max_group)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), W.cpu().numpy()


def worst_chunk(O, Oo, C):
    """The largest relative error of one chunk of one sequence's outputs (late
    chunks have larger outputs and dominate the global norm; this catches an
    error confined to a few chunks)."""
    B, T = Oo.shape[:2]
    return max(rel(O[b, i:i + C], Oo[b, i:i + C]) for b in range(B) for i in range(0, T, C))


def check_against_oracle(inp, eta, C, dtype, mode="auto", max_group=0, label=""):
    print(f"[parity] {label} B,T,d,f,K={tuple(inp['H'].shape)},{inp['W_gate'].shape[0]},"
          f"{inp['taps'].shape[1]} C={C} eta={eta} mode={mode} G={max_group}", flush=True)
    dev = to_device(inp)
    O, W = run_gpu(dev, eta, C, mode, max_group)
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C)
    tol = tol_for(dtype)
    W0 = ni["W_down0"].astype(np.float64)
    e_o, e_w, e_dw = rel(O, Oo), rel(W, Wo), rel(W - W0, Wo - W0)
    worst = worst_chunk(O, Oo, C)
    print(f"  rel O {e_o:.3e} (worst chunk {worst:.3e})  W {e_w:.3e}  dW {e_dw:.3e}  (tol {tol})",
          flush=True)
    assert e_o <= tol and e_w <= tol and worst <= tol, (e_o, e_w, worst)
    if eta != 0.0:
        assert e_dw <= tol, e_dw
    else:
        assert np.array_equal(W, np.broadcast_to(W0, W.shape).astype(np.float32))
    return O, W


# --------------------------------------------------------------- tiny fp32 workload
def test_tiny_fp32_workload_full():
    w = synth.WORKLOADS["tiny_fp32"]
    inp = synth.workload_inputs(w)
    check_against_oracle(inp, w.eta, w.chunk, w.dtype, label=w.name)


# --------------------------------------------------------------- small shapes
SMALL = [
    # B, T, d, f, K, C, dtype, eta
    (1, 700, 256, 512, 4, 128, torch.bfloat16, 1e-2),   # ragged T vs 256-row tiles
    (2, 333, 128, 192, 3, 100, torch.bfloat16, 2e-2),   # padded chunks, partial tiles
    (1, 517, 64, 320, 8, 64, torch.bfloat16, 1e-2),     # K = 8, d = 64
    (1, 70, 128, 128, 4, 1, torch.bfloat16, 5e-3),      # per-token updates
    (1, 300, 128, 256, 1, 1000, torch.bfloat16, 1e-2),  # C > T, K = 1
    (3, 260, 192, 256, 2, 37, torch.float32, 1e-2),     # fp32, odd chunk
    (1, 1, 64, 64, 4, 16, torch.float32, 1e-1),         # a single token
    (2, 513, 320, 384, 5, 256, torch.float32, 1e-2),    # fp32, several tiles
    (1, 600, 320, 128, 4, 128, torch.bfloat16, 1e-2),   # d > f: conv output wider than Z
    # gate/up weight rows longer than 4 KB (stored in tiles), 64 x 64 scan tiles
    (1, 300, 2112, 128, 4, 128, torch.bfloat16, 1e-2),
    (1, 200, 1088, 192, 4, 64, torch.float32, 1e-2),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}T{c[1]}d{c[2]}f{c[3]}K{c[4]}C{c[5]}{str(c[6])[6:]}")
def test_small_shapes(case):
    B, T, d, f, K, C, dtype, eta = case
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=B * 1000 + T)
    check_against_oracle(inp, eta, C, dtype, label="small")


def test_eta_zero_static_mlp():
    inp = synth.make_inputs(1, 300, 128, 256, 4, torch.bfloat16, seed=77)
    check_against_oracle(inp, 0.0, 64, torch.bfloat16, label="eta0")


# --------------------------------------------------------------- invariants
def _inp_small(dtype=torch.bfloat16, B=2, T=600, d=128, f=256, K=4, seed=5):
    return to_device(synth.make_inputs(B, T, d, f, K, dtype, seed))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_modes_and_group_sizes_bitwise_equal(dtype):
    dev = _inp_small(dtype)
    ref = run_gpu(dev, 1e-2, 64, mode="chunk_parallel")
    # sequential: groups of 3 (its default here: 10 chunks) and of 1 -- one
    # launch per chunk's update either way, the outputs batched per group
    for mode, g in (("sequential", 0), ("sequential", 1), ("chunk_parallel", 1),
                    ("chunk_parallel", 3), ("auto", 0)):
        O, W = run_gpu(dev, 1e-2, 64, mode=mode, max_group=g)
        assert np.array_equal(O, ref[0]) and np.array_equal(W, ref[1]), (mode, g)


@pytest.mark.parametrize("target,T,C,dtype,split_group",
                         [("conv_proj", 1300, 64, torch.bfloat16, 8),
                          ("proj", 1300, 100, torch.bfloat16, 6),
                          ("conv_proj", 1300, 100, torch.float32, 6),
                          ("conv_proj", 1300, 256, torch.bfloat16, 2)])
def test_projection_split_bitwise_equal(target, T, C, dtype, split_group):
    """With 256-divisible weights, more than one group and a first group of at
    least 2 d tokens, the projection of the later tokens runs inside the first
    pipeline launch (stage scan_target); otherwise it runs whole before the
    scans.  Both give the same bits, over several sequences, padded chunks and
    a ragged last tile.  (Chunk-parallel mode takes one group of all chunks
    when the workspace holds them, so split_group < N / 2 forces groups of
    split_group.)"""
    B, d, f = 2, 256, 512
    dev = to_device(synth.make_inputs(B, T, d, f, 4, dtype, seed=41))
    if target == "proj":
        dev["taps"] = None

    def run(mode, g):
        tm.ttt_profile_read()
        tm.ttt_profile_enable(True)
        O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"],
                                  dev["W_down0"], dev["taps"], dev["W_target"], 1e-2, C,
                                  mode=mode, max_group=g, target=target)
        torch.cuda.synchronize()
        tm.ttt_profile_enable(False)
        split = tm.ttt_profile_read()["scan_target"][1] > 0
        return O.float().cpu().numpy(), W.cpu().numpy(), split

    ref = run("chunk_parallel", 0)  # one group: no split
    assert not ref[2]
    # auto and sequential mode take a quarter of the chunks per group at most
    # (sequential scans them one chunk per launch; its first chunk's launch
    # carries the projection); the split needs a group of 2 d tokens or more
    N = -(-T // C)

    def splits(g):
        return g * C >= 2 * d and -(-N // g) > 1

    quarter = -(-N // 4)
    for mode, g, expect_split in (("chunk_parallel", split_group, True),
                                  ("sequential", 0, splits(quarter)),
                                  ("sequential", split_group, splits(min(quarter, split_group))),
                                  ("auto", 0, splits(quarter))):
        O, W, split = run(mode, g)
        assert split == expect_split, (mode, g)
        assert np.array_equal(O, ref[0]) and np.array_equal(W, ref[1]), (mode, g)


def test_repeat_call_bitwise_deterministic():
    dev = _inp_small()
    a = run_gpu(dev, 1e-2, 96)
    b = run_gpu(dev, 1e-2, 96)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_batched_equals_single_calls():
    dev = _inp_small(B=3)
    Ob, Wb = run_gpu(dev, 1e-2, 128)
    for b in range(3):
        O, W = tm.forward(dev["H"][b], dev["X0"][b], dev["W_gate"], dev["W_up"], dev["W_down0"],
                          dev["taps"], dev["W_target"], 1e-2, 128)
        torch.cuda.synchronize()
        assert np.array_equal(O.float().cpu().numpy(), Ob[b])
        assert np.array_equal(W.cpu().numpy(), Wb[b])


def test_causality_bitwise():
    inp = synth.make_inputs(1, 512, 128, 256, 4, torch.bfloat16, seed=9)
    dev = to_device(inp)
    O, _ = run_gpu(dev, 2e-2, 64)
    g = torch.Generator().manual_seed(3)
    for t in (0, 63, 64, 200, 450):
        for name in ("H", "X0"):
            p = dict(dev)
            x = inp[name].clone()
            x[0, t + 1:] += torch.randn(x[0, t + 1:].shape, generator=g).to(x.dtype)
            p[name] = x.cuda()
            Op, _ = run_gpu(p, 2e-2, 64)
            assert np.array_equal(Op[0, :t + 1], O[0, :t + 1]), (name, t)


def test_state_reset_and_carried_state():
    """ttt_fastweight_state_reset followed by a batched call that starts from
    the buffers (init_from_w0 = 0) equals a call with init_from_w0 = 1."""
    dev = _inp_small(B=2, T=256)
    B, T, d = dev["H"].shape
    f = dev["W_gate"].shape[0]
    O1, W1 = run_gpu(dev, 1e-2, 64)
    Ws = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    tm.ttt_fastweight_state_reset(Ws, dev["W_down0"], dev["W_down0"].dtype, B, d, f)
    O2, W2 = run_gpu(dev, 1e-2, 64, W_state=Ws)
    assert np.array_equal(O1, O2) and np.array_equal(W1, W2)
    # the reset value itself
    tm.ttt_fastweight_state_reset(Ws, dev["W_down0"], dev["W_down0"].dtype, B, d, f)
    torch.cuda.synchronize()
    assert np.array_equal(Ws.cpu().numpy(),
                          np.broadcast_to(dev["W_down0"].float().cpu().numpy(), (B, d, f)))


def test_error_leaves_outputs_untouched():
    dev = _inp_small(B=1, T=128)
    H = dev["H"][0]
    T, d = H.shape
    f = dev["W_gate"].shape[0]
    desc = tm.make_desc(1, T, d, f, 64, 4, 1e-2, H.dtype)
    small = torch.empty(tm.ttt_mlp_workspace_size(desc, 1) - 256, dtype=torch.uint8, device="cuda")
    O = torch.full_like(H, 7.0)
    W = torch.full((d, f), 3.0, device="cuda")
    with pytest.raises(tm.TTTError) as ei:
        tm.ttt_mlp_forward(desc, H, dev["X0"][0], dev["W_gate"], dev["W_up"], dev["W_down0"],
                           dev["taps"], dev["W_target"], O, W, small)
    assert ei.value.status == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((O == 7.0).all()) and bool((W == 3.0).all())


def test_nan_input_propagates_without_fault():
    inp = synth.make_inputs(1, 256, 64, 128, 4, torch.bfloat16, seed=1)
    inp["H"][0, 70, 5] = float("nan")
    dev = to_device(inp)
    O, W = run_gpu(dev, 1e-2, 64)
    assert np.isnan(O[0, 70]).all()          # its own row
    assert not np.isnan(O[0, :64]).any()      # chunk 0 is untouched
    assert np.isnan(O[0, 128:]).any()         # later chunks see the updated weight


# --------------------------------------------------- ablation targets (section 6)
TARGET_CASES = [
    # B, T, d, f, K, C, dtype
    (2, 333, 128, 192, 3, 100, torch.bfloat16),
    (1, 300, 192, 256, 4, 64, torch.float32),
]


@pytest.mark.parametrize("target", ["proj", "conv", "embed"])
@pytest.mark.parametrize("case", TARGET_CASES, ids=lambda c: f"T{c[1]}d{c[2]}{str(c[6])[6:]}")
def test_target_variants(case, target):
    """The ablation targets against the oracle; the inputs a variant leaves out
    are passed as NULL."""
    B, T, d, f, K, C, dtype = case
    print(f"[parity] target={target} B,T,d,f,K,C={B},{T},{d},{f},{K},{C} {dtype}", flush=True)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=77)
    dev = to_device(inp)
    taps = None if target in ("proj", "embed") else dev["taps"]
    Wt = None if target in ("conv", "embed") else dev["W_target"]
    eta = 2e-2
    O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                              taps, Wt, eta, C, target=target, conv_k=K)
    torch.cuda.synchronize()
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C, target=target)
    W0 = ni["W_down0"].astype(np.float64)
    Og, Wg = O.float().cpu().numpy(), W.cpu().numpy()
    e_o, e_dw = rel(Og, Oo), rel(Wg - W0, Wo - W0)
    print(f"  rel O {e_o:.3e}  dW {e_dw:.3e}", flush=True)
    assert e_o <= tol_for(dtype) and e_dw <= tol_for(dtype), (e_o, e_dw)


ALIGN_CASES = [
    # B, T, d, f, K, C, dtype, target
    (2, 333, 128, 192, 8, 100, torch.bfloat16, "conv_proj"),   # window reaches back 7 rows
    (1, 300, 192, 256, 4, 64, torch.float32, "conv_proj"),
    (1, 257, 128, 192, 1, 32, torch.bfloat16, "conv"),         # K = 1: V^ = taps * X0
    (2, 200, 64, 128, 5, 7, torch.float32, "conv"),
]


@pytest.mark.parametrize("case", ALIGN_CASES,
                         ids=lambda c: f"T{c[1]}K{c[4]}{str(c[6])[6:]}-{c[7]}")
def test_reconstruction_alignment(case):
    """The conv window ending at the token itself (the reconstruction target of
    section 4's table) against the oracle."""
    B, T, d, f, K, C, dtype, target = case
    print(f"[parity] align=self target={target} B,T,d,f,K,C={B},{T},{d},{f},{K},{C} {dtype}",
          flush=True)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=78)
    dev = to_device(inp)
    Wt = None if target == "conv" else dev["W_target"]
    eta = 2e-2
    O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                              dev["taps"], Wt, eta, C, target=target, align="self")
    O_next, _ = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"],
                                   dev["W_down0"], dev["taps"], Wt, eta, C, target=target)
    torch.cuda.synchronize()
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C, target=target, align="self")
    W0 = ni["W_down0"].astype(np.float64)
    Og, Wg = O.float().cpu().numpy(), W.cpu().numpy()
    e_o, e_dw = rel(Og, Oo), rel(Wg - W0, Wo - W0)
    print(f"  rel O {e_o:.3e}  dW {e_dw:.3e}", flush=True)
    assert e_o <= tol_for(dtype) and e_dw <= tol_for(dtype), (e_o, e_dw)
    # chunk 0 uses W0 in both alignments; later chunks see different updates
    assert torch.equal(O[:, :C], O_next[:, :C])
    assert not torch.equal(O[:, C:], O_next[:, C:])


# --------------------------------------------------------------- full-size workloads
FULL = ["qwen3_4b_32k", "qwen3_4b_128k", "multi_session_16x8k", "small_4x128k"]
# two chunks everywhere: chunk 1's outputs come from a weight the scan has
# updated, at the benchmark's chunk size, group and launch shapes
PREFIX_CHUNKS = {"qwen3_4b_32k": 2, "qwen3_4b_128k": 2, "multi_session_16x8k": 2,
                 "small_4x128k": 2}
PREFIX_SEQS = {"multi_session_16x8k": (0, 15), "small_4x128k": (0, 3)}


@pytest.mark.parametrize("name", FULL)
def test_full_workload_prefix_and_final_weight(name):
    """Full-size run as the benchmark runs it.  O on the first chunks of chosen
    sequences vs the oracle on that causal prefix (O[0:mC] depends only on the
    first mC tokens); sampled entries of the final weight and of its change vs
    the closed form W0 + eta * V^^T Z over every token."""
    w = synth.WORKLOADS[name]
    print(f"[full] {name}: drawing inputs", flush=True)
    inp = synth.workload_inputs(w)
    dev = to_device(inp)
    O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                              dev["taps"], dev["W_target"], w.eta, w.chunk)
    torch.cuda.synchronize()
    print(f"[full] {name}: GPU done", flush=True)
    del dev
    ni = numpy_inputs(inp)
    m = PREFIX_CHUNKS[name] * w.chunk
    seqs = PREFIX_SEQS.get(name, (0,))
    for b in seqs:
        Oo, _ = oracle.forward(ni["H"][b, :m], ni["X0"][b, :m], ni["W_gate"], ni["W_up"],
                               ni["W_down0"], ni["taps"], ni["W_target"], w.eta, w.chunk)
        Og = O[b, :m].float().cpu().numpy()
        e = rel(Og, Oo)
        per_chunk = [rel(Og[i:i + w.chunk], Oo[i:i + w.chunk]) for i in range(0, m, w.chunk)]
        print(f"  seq {b} O[0:{m}] rel {e:.3e}, per chunk "
              + " ".join(f"{x:.3e}" for x in per_chunk), flush=True)
        assert e <= tol_for(w.dtype) and max(per_chunk) <= tol_for(w.dtype)
        # chunk 1 used an updated weight: its outputs differ from W_down0's
        Ostatic = oracle.gated_activations(ni["H"][b, w.chunk:m], ni["W_gate"], ni["W_up"]) \
            @ ni["W_down0"].astype(np.float64).T
        moved = rel(Ostatic, Oo[w.chunk:m])
        print(f"  seq {b} chunk 1 with W_down0 instead: rel {moved:.3e}", flush=True)
        assert moved > 10 * per_chunk[1]
    rng = np.random.default_rng(0)
    ms = np.sort(rng.choice(w.d_model, 3, replace=False))
    ns = np.sort(rng.choice(w.d_ff, 6, replace=False))
    b = seqs[-1]
    Wg = oracle.final_weight_grid(ni["H"][b], ni["X0"][b], ni["W_gate"], ni["W_up"],
                                  ni["W_down0"], ni["taps"], ni["W_target"], w.eta, ms, ns)
    Wgpu = W[b].cpu().numpy()[np.ix_(ms, ns)]
    W0 = ni["W_down0"].astype(np.float64)[np.ix_(ms, ns)]
    e_w, e_dw = rel(Wgpu, Wg), rel(Wgpu - W0, Wg - W0)
    print(f"  seq {b} W_final sample rel {e_w:.3e}, dW rel {e_dw:.3e}", flush=True)
    assert e_w <= tol_for(w.dtype) and e_dw <= tol_for(w.dtype)


@pytest.mark.parametrize("name", ["qwen3_4b_32k", "small_4x128k", "qwen3_4b_128k"])
def test_full_size_sequential_mode_bitwise(name):
    """Sequential mode at full size (one launch per chunk's read-modify-write of
    the fp32 state, the single-chunk update tiles, a group's outputs batched)
    against the default chunk-parallel groups: the fp32 state sums run in the
    same order, so outputs and final weights are the same bits."""
    w = synth.WORKLOADS[name]
    dev = to_device(synth.workload_inputs(w))
    runs = []
    for mode in ("auto", "sequential"):
        O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"],
                                  dev["W_down0"], dev["taps"], dev["W_target"], w.eta, w.chunk,
                                  mode=mode)
        torch.cuda.synchronize()
        runs.append((O, W))
        print(f"[full] {name} {mode}: done", flush=True)
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("dtype,C,T", [(torch.bfloat16, 1024, 2500), (torch.float32, 512, 1100)],
                         ids=["bf16", "f32"])
def test_sequential_update_many_tiles_bitwise(dtype, C, T):
    """Sequential mode with chunks of 16 k-tiles, more single-chunk update
    tiles than the GPU holds at once (four sequences of a 1024 x 4096 weight)
    and a ragged last chunk, against the chunk-parallel groups: the same
    bits."""
    dev = to_device(synth.make_inputs(4, T, 1024, 4096, 4, dtype, seed=31))
    ref = run_gpu(dev, 1e-2, C, mode="chunk_parallel")
    got = run_gpu(dev, 1e-2, C, mode="sequential")
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


# ------------------------------------------------- coherent-accumulation stress
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_repeated_block_stress(dtype):
    """An induction-head-like input: every token's H and X0 rows come from a
    table of 48 rows, in a block of 64 tokens that repeats, so every chunk's
    increment points the same way and the fast weight grows linearly with the
    chunk index instead of like its square root.  Checks range and tolerance
    (and prints the worst chunk of O)."""
    B, T, d, f, K, C = 1, 4096, 256, 512, 4, 256
    g = torch.Generator().manual_seed(71)
    table_h = torch.randn((48, d), generator=g)
    table_x = torch.randn((48, d), generator=g)
    block = torch.randint(0, 48, (64,), generator=g)
    idx = block.repeat(T // 64)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=72)
    inp["H"] = table_h[idx][None].to(dtype)
    inp["X0"] = table_x[idx][None].to(dtype)
    dev = to_device(inp)
    eta = 2e-3
    O, W = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                              dev["taps"], dev["W_target"], eta, C)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all() and torch.isfinite(W).all()
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C)
    Og, Wg = O.float().cpu().numpy()[0], W.cpu().numpy()[0]
    Oo, Wo = Oo[0], Wo[0]
    W0 = ni["W_down0"].astype(np.float64)
    grow = np.linalg.norm(Wo - W0) / np.linalg.norm(W0)
    e_o, e_dw = rel(Og, Oo), rel(Wg - W0, Wo - W0)
    worst = max(rel(Og[i:i + C], Oo[i:i + C]) for i in range(0, T, C))
    print(f"  |W_final - W0| / |W0| = {grow:.1f}; rel O {e_o:.2e} (worst chunk {worst:.2e}), "
          f"rel dW {e_dw:.2e}", flush=True)
    assert grow > 1.0  # the update dominates the starting weight
    tol = tol_for(dtype)
    assert e_o <= tol and e_dw <= tol and worst <= tol, (e_o, e_dw, worst)
