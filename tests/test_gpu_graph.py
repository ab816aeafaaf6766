"""The entry points under HIP graph capture: a captured forward, decode call
and backward are replayed several times, with eager work and
synchronisations in between, and every replay equals the eager result bit
for bit (the calls allocate nothing and issue no memsets, so capture records
only kernels and device copies)."""
import pytest
import torch

from chunk_wise_weight_chunked_amd import synth
from chunk_wise_weight_chunked_amd import ttt_mlp as tm

from _common import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tm.load()


def _replays(graph, outs, refs, scratch):
    for r in range(3):
        scratch.mul_(1.5).add_(r)          # unrelated eager work between replays
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), r


def test_forward_graph_replays_equal_eager():
    B, T, d, f, K, C = 2, 600, 256, 512, 4, 128
    inp = to_device(synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=61))
    desc = tm.make_desc(B, T, d, f, C, K, 1e-2, torch.bfloat16)
    ws = tm.alloc_workspace(desc, 0)
    O = torch.empty_like(inp["H"])
    W = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    args = (desc, inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
            inp["W_target"], O, W, ws)
    tm.ttt_mlp_forward_batched(*args)
    torch.cuda.synchronize()
    O_ref, W_ref = O.clone(), W.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tm.ttt_mlp_forward_batched(*args, stream=s)
    _replays(g, [O, W], [O_ref, W_ref], torch.ones(1 << 20, device="cuda"))


def test_forward_with_projection_split_graph_replays_equal_eager():
    # groups of 8 chunks of 64 tokens (512 >= 2 d): the later rows' projection
    # runs inside the first pipeline launch
    B, T, d, f, K, C = 1, 1300, 256, 512, 4, 64
    inp = to_device(synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=65))
    desc = tm.make_desc(B, T, d, f, C, K, 1e-2, torch.bfloat16, "chunk_parallel")
    ws = tm.alloc_workspace(desc, 8)
    O = torch.empty_like(inp["H"])
    W = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    args = (desc, inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
            inp["W_target"], O, W, ws)
    tm.ttt_profile_read()
    tm.ttt_profile_enable(True)
    tm.ttt_mlp_forward_batched(*args)
    torch.cuda.synchronize()
    tm.ttt_profile_enable(False)
    assert tm.ttt_profile_read()["scan_target"][1] == 1
    O_ref, W_ref = O.clone(), W.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tm.ttt_mlp_forward_batched(*args, stream=s)
    _replays(g, [O, W], [O_ref, W_ref], torch.ones(1 << 20, device="cuda"))


def test_decode_call_graph_replays_equal_eager():
    B, L, d, f, K, C = 4, 1, 256, 512, 4, 64
    inp = to_device(synth.make_inputs(B, 40, d, f, K, torch.bfloat16, seed=62))
    st = tm.Stream(inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"], inp["W_target"],
                   1e-2, C, B)
    st.step(inp["H"][:, :37].contiguous(), inp["X0"][:, :37].contiguous())  # pos 37
    desc = tm.make_desc(B, L, d, f, C, K, 1e-2, torch.bfloat16)
    ws = torch.empty(tm.ttt_mlp_stream_workspace_size(desc), dtype=torch.uint8, device="cuda")
    h, x = inp["H"][:, 37:38].contiguous(), inp["X0"][:, 37:38].contiguous()
    O = torch.empty_like(h)
    carry0 = st.carry.clone()
    args = (desc, 37, 0, h, x, inp["W_gate"], inp["W_up"], inp["W_down0"], inp["taps"],
            inp["W_target"], O, st.state, st.carry, ws)
    tm.ttt_mlp_forward_stream(*args)
    torch.cuda.synchronize()
    O_ref, carry_ref = O.clone(), st.carry.clone()
    st.carry.copy_(carry0)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tm.ttt_mlp_forward_stream(*args, stream=s)
    for r in range(3):
        st.carry.copy_(carry0)
        O.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref) and torch.equal(st.carry, carry_ref), r


def test_backward_graph_replays_equal_eager():
    B, T, d, f, K, C = 1, 300, 256, 256, 4, 64
    inp = to_device(synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=63))
    dO = torch.randn((B, T, d), generator=torch.Generator().manual_seed(64)).to(
        torch.bfloat16).cuda()
    desc = tm.make_desc(B, T, d, f, C, K, 1e-2, torch.bfloat16)
    ws = torch.empty(tm.ttt_mlp_backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(inp["H"]), torch.empty_like(inp["H"]), torch.empty((f, d), **f32),
            torch.empty((f, d), **f32), torch.empty((B, d, f), **f32), torch.empty((d, K), **f32),
            torch.empty((d, d), **f32), torch.empty(1, **f32)]
    args = (desc, inp["H"], inp["X0"], inp["W_gate"], inp["W_up"], inp["W_down0"], None,
            inp["taps"], inp["W_target"], dO, None, *outs, ws)
    tm.ttt_mlp_backward_batched(*args)
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tm.ttt_mlp_backward_batched(*args, stream=s)
    _replays(g, outs, refs, torch.ones(1 << 20, device="cuda"))
