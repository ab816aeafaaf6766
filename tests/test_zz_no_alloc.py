"""The allocation-free decode entry point (ttt_mlp_forward_stream_decode_noalloc,
whose gated activations live in a static device buffer) against the same
decode calls made through ttt_mlp_forward_stream_ragged with a workspace:
outputs, fast-weight states and carries bit for bit, over two calls in a row,
the second with fewer rows; and a call the decode kernels do not serve is
refused with nothing written."""
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


@pytest.mark.parametrize("B,d,f,C,calls", [(4, 256, 512, 64, [16, 5]),
                                           (4, 2560, 9728, 64, [16, 3])],
                         ids=["small", "qwen3-4b-mlp"])
def test_noalloc_decode_equals_workspace_call(B, d, f, C, calls):
    K, eta, dtype = 4, 2e-2, torch.bfloat16
    T = sum(calls)
    print(f"[noalloc] B={B} d={d} f={f} C={C} calls={calls}", flush=True)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=401)
    dev = to_device(inp)
    w = (dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"])
    desc0 = tm.make_desc(B, calls[0], d, f, C, K, eta, dtype)
    nbytes = tm.ttt_mlp_carry_size(desc0)
    carry_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    carry_b = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    state_a = torch.zeros((B, d, f), dtype=torch.float32, device="cuda")
    state_b = torch.zeros((B, d, f), dtype=torch.float32, device="cuda")
    p = 0
    for L in calls:
        desc = tm.make_desc(B, L, d, f, C, K, eta, dtype)
        ws = torch.empty(tm.ttt_mlp_stream_workspace_size(desc), dtype=torch.uint8,
                         device="cuda")
        H = dev["H"][:, p:p + L].contiguous()
        X0 = dev["X0"][:, p:p + L].contiguous()
        pos, last = [p] * B, [0] * B
        Oa = torch.empty((B, L, d), dtype=dtype, device="cuda")
        Ob = torch.full((B, L, d), 7.0, dtype=dtype, device="cuda")
        tm.ttt_mlp_forward_stream_ragged(desc, pos, last, H, X0, *w, Oa, state_a, carry_a, ws)
        tm.ttt_mlp_forward_stream_decode_noalloc(desc, pos, last, H, X0, *w, Ob, state_b,
                                                 carry_b)
        torch.cuda.synchronize()
        assert torch.equal(Oa, Ob), (L, (Oa.float() - Ob.float()).abs().max().item())
        assert torch.equal(state_a, state_b), L
        assert torch.equal(carry_a, carry_b), L
        print(f"  call of {L} rows at {p}: bitwise equal", flush=True)
        p += L


def test_noalloc_refuses_calls_that_need_the_full_path():
    B, d, f, K, C = 2, 256, 512, 4, 16
    inp = synth.make_inputs(B, 20, d, f, K, torch.bfloat16, seed=402)
    dev = to_device(inp)
    w = (dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"])
    carry = torch.zeros(tm.ttt_mlp_carry_size(tm.make_desc(B, 4, d, f, C, K, 1e-2,
                                                           torch.bfloat16)),
                        dtype=torch.uint8, device="cuda")
    state = torch.full((B, d, f), 3.0, dtype=torch.float32, device="cuda")
    outs = []
    for L, last in ((4, 1), (20, 0)):  # a closing call; more rows than a decode call takes
        desc = tm.make_desc(B, L, d, f, C, K, 1e-2, torch.bfloat16)
        O = torch.full((B, L, d), 7.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(tm.TTTError) as e:
            tm.ttt_mlp_forward_stream_decode_noalloc(
                desc, [0] * B, [last] * B, dev["H"][:, :L].contiguous(),
                dev["X0"][:, :L].contiguous(), *w, O, state, carry)
        msg = str(e.value)
        assert e.value.status == tm.TTT_ERR_UNSUPPORTED, msg
        assert ("full path" in msg) if last else ("at most" in msg), msg
        outs.append(O)
    torch.cuda.synchronize()
    assert all(bool((O == 7.0).all()) for O in outs)
    assert bool((state == 3.0).all()) and bool((carry == 0).all())
