"""Streaming continuation on the GPU: sessions fed over consecutive calls give
the final weights of one call over the whole sequence bit for bit, and its
outputs bit for bit except for the rows of decode calls (a few rows that do
not complete a chunk: computed by the decode kernels, equal to rounding)."""
import numpy as np
import pytest
import torch

import oracle
from chunk_wise_weight_chunked_amd import synth
from chunk_wise_weight_chunked_amd import ttt_mlp as tm

from _common import numpy_inputs, rel, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tm.load()


def decode_call(B, L, pos, C, last, dtype):
    """Which calls the library serves with its decode kernels: bf16, not the
    closing call, at most 16 new rows per session and 64 in all, and the new
    rows stay inside the pending chunk."""
    n_pend = 0 if pos == 0 else pos - (pos - 1) // C * C
    return (dtype == torch.bfloat16 and not last and L <= 16 and B * L <= 64
            and n_pend + L <= C)


# Decode rows against the one-call run: the same weight, a different
# summation order (measured <= 4e-5).
DECODE_TOL = 1e-3


def stale_weight_error(inp, eta, C, dec, O1, target="conv_proj", align="next"):
    """How far the decode rows of chunks >= 1 would move had they used the
    weight one chunk older (W^(i-2) instead of W^(i-1)): row t of chunk i
    changes by eta Z_t Z_{i-1}ᵀ V^_{i-1}; relative to the rows' outputs.  None
    if no decode row lies past chunk 0."""
    ni = numpy_inputs(inp)
    B, T = inp["H"].shape[:2]
    rows = [t for t in range(C, T) if dec[t]]
    if not rows:
        return None
    num = den = 0.0
    for b in range(B):
        Z = oracle.gated_activations(ni["H"][b], ni["W_gate"], ni["W_up"])
        V = oracle.lm_target(ni["X0"][b], ni["taps"], ni["W_target"], target, align)
        Ob = O1[b].double().cpu().numpy()
        for t in rows:
            i = t // C
            prev = slice((i - 1) * C, i * C)
            diff = eta * (Z[t] @ Z[prev].T) @ V[prev]
            num += float(diff @ diff)
            den += float(Ob[t] @ Ob[t])
    return (num / den) ** 0.5


CASES = [
    # B, T, d, f, K, C, dtype, call lengths, target
    (2, 700, 128, 192, 4, 128, torch.bfloat16, [700], "conv_proj"),
    (2, 700, 128, 192, 4, 128, torch.bfloat16, [128, 572], "conv_proj"),
    (2, 700, 128, 192, 4, 128, torch.bfloat16, [100, 300, 300], "conv_proj"),
    (1, 300, 128, 256, 8, 4, torch.bfloat16, [3, 1, 50, 246], "conv_proj"),   # C < halo
    (1, 64, 64, 128, 4, 16, torch.bfloat16, [1] * 64, "conv_proj"),           # decoding
    (1, 200, 64, 64, 3, 1, torch.bfloat16, [7, 13, 180], "conv_proj"),        # C = 1
    (2, 513, 192, 256, 5, 100, torch.float32, [200, 313], "conv_proj"),
    (1, 300, 128, 192, 4, 64, torch.bfloat16, [50, 250], "conv"),
    (1, 300, 128, 192, 4, 64, torch.bfloat16, [50, 250], "proj"),
    # decode calls: one group of 16 tokens (B*L = 64), two groups (21), mixed
    (4, 200, 128, 256, 4, 64, torch.bfloat16, [16, 16, 16, 15, 1, 1, 135], "conv_proj"),
    (3, 150, 192, 320, 4, 32, torch.bfloat16, [7, 7, 7, 11, 1, 16, 101], "conv_proj"),
    (2, 90, 256, 512, 8, 16, torch.bfloat16, [1] * 40 + [50], "conv"),
    (1, 120, 128, 192, 4, 128, torch.bfloat16, [16] * 7 + [8], "embed"),
    # reconstruction alignment: the halo holds K - 1 = 7 rows
    (2, 300, 128, 192, 8, 4, torch.bfloat16, [3, 1, 50, 246], "conv_proj@self"),
    (1, 200, 128, 192, 8, 64, torch.float32, [70, 1, 129], "conv@self"),
    (2, 100, 128, 256, 8, 32, torch.bfloat16, [1] * 40 + [60], "conv_proj@self"),
]


def _id(c):
    return f"B{c[0]}T{c[1]}C{c[5]}{str(c[6])[6:]}-{len(c[7])}calls-{c[8].replace('@', '-')}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_stream_equals_one_call(case):
    B, T, d, f, K, C, dtype, calls, target = case
    target, _, align = target.partition("@")
    align = align or "next"
    assert sum(calls) == T
    print(f"[stream] {_id(case)}", flush=True)
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=91)
    dev = to_device(inp)
    eta = 2e-2
    O1, W1 = tm.forward_batched(dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"],
                                dev["taps"], dev["W_target"], eta, C, target=target, align=align)
    st = tm.Stream(dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"], eta,
                   C, B, target=target, align=align)
    outs, p = [], 0
    dec = torch.zeros(T, dtype=torch.bool)
    for i, L in enumerate(calls):
        last = i == len(calls) - 1
        dec[p:p + L] = decode_call(B, L, p, C, last, dtype)
        outs.append(st.step(dev["H"][:, p:p + L].contiguous(), dev["X0"][:, p:p + L].contiguous(),
                            last=last))
        p += L
    torch.cuda.synchronize()
    Os = torch.cat(outs, dim=1)
    assert torch.equal(st.state, W1), (st.state - W1).abs().max().item()
    rows = ~dec.cuda()
    assert torch.equal(Os[:, rows], O1[:, rows]), \
        (Os[:, rows].float() - O1[:, rows].float()).abs().max().item()
    if dec.any():
        a = Os[:, dec.cuda()].double().cpu().numpy()
        b = O1[:, dec.cuda()].double().cpu().numpy()
        e = rel(a, b)
        print(f"  {int(dec.sum())} decode rows: rel to one call {e:.3e}", flush=True)
        assert e <= DECODE_TOL
        stale = stale_weight_error(inp, eta, C, dec, O1, target, align)
        if stale is not None:
            print(f"  the same rows with the weight one chunk older: rel {stale:.3e}", flush=True)
            assert stale > 10 * DECODE_TOL


def test_stream_state_between_calls_matches_oracle():
    """After a call that ends inside a chunk, the state is the weight after the
    chunks before the pending one: the next call's outputs, made with it,
    match the oracle on the whole sequence."""
    B, T, d, f, K, C, dtype = 1, 400, 128, 192, 4, 64, torch.bfloat16
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=92)
    dev = to_device(inp)
    eta = 2e-2
    st = tm.Stream(dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"], eta,
                   C, B)
    O_a = st.step(dev["H"][:, :150].contiguous(), dev["X0"][:, :150].contiguous())
    O_b = st.step(dev["H"][:, 150:].contiguous(), dev["X0"][:, 150:].contiguous(), last=True)
    torch.cuda.synchronize()
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C)
    O = torch.cat([O_a, O_b], dim=1).float().cpu().numpy()
    W0 = ni["W_down0"].astype(np.float64)
    e_o, e_dw = rel(O, Oo), rel(st.state.cpu().numpy() - W0, Wo - W0)
    print(f"  rel O {e_o:.3e}  dW {e_dw:.3e}", flush=True)
    assert e_o <= 2e-2 and e_dw <= 2e-2


def test_decode_at_model_size_matches_oracle():
    """Token-by-token decoding at the Qwen3-4B MLP shape (d = 2560, f = 9728)
    for two sessions over 40 tokens with C = 16: the decode kernels' outputs
    and the updates made at the chunk boundaries against the oracle."""
    B, T, d, f, K, C, dtype = 2, 40, 2560, 9728, 4, 16, torch.bfloat16
    inp = synth.make_inputs(B, T, d, f, K, dtype, seed=94)
    dev = to_device(inp)
    eta = 1e-3
    st = tm.Stream(dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"], eta,
                   C, B)
    outs = [st.step(dev["H"][:, t:t + 1].contiguous(), dev["X0"][:, t:t + 1].contiguous(),
                    last=t == T - 1) for t in range(T)]
    torch.cuda.synchronize()
    O = torch.cat(outs, dim=1).double().cpu().numpy()
    ni = numpy_inputs(inp)
    Oo, Wo = oracle.forward(ni["H"], ni["X0"], ni["W_gate"], ni["W_up"], ni["W_down0"],
                            ni["taps"], ni["W_target"], eta, C)
    W0 = ni["W_down0"].astype(np.float64)
    e_o = rel(O, Oo)
    e_dw = rel(st.state.cpu().numpy() - W0[None], Wo - W0[None])
    print(f"  rel O {e_o:.3e}  dW {e_dw:.3e}", flush=True)
    assert e_o <= 2e-2 and e_dw <= 2e-2


def test_stream_rejects_bad_arguments():
    B, T, d, f, K, C = 1, 64, 64, 128, 4, 16
    inp = synth.make_inputs(B, T, d, f, K, torch.bfloat16, seed=93)
    dev = to_device(inp)
    desc = tm.make_desc(B, T, d, f, C, K, 1e-2, torch.bfloat16)
    ws = torch.empty(tm.ttt_mlp_stream_workspace_size(desc), dtype=torch.uint8, device="cuda")
    carry = torch.zeros(tm.ttt_mlp_carry_size(desc), dtype=torch.uint8, device="cuda")
    W = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    O = torch.empty_like(dev["H"])
    args = (dev["H"], dev["X0"], dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"],
            dev["W_target"], O, W)
    for pos, last, c, word in ((-1, 0, carry, "pos"), (0, 2, carry, "last"),
                               (16, 0, None, "carry")):
        with pytest.raises(tm.TTTError) as e:
            tm.ttt_mlp_forward_stream(desc, pos, last, *args, c, ws)
        assert word in str(e.value)
    with pytest.raises(tm.TTTError) as e:
        tm.ttt_mlp_forward_stream(desc, 0, 0, *args, carry, ws, ws_bytes=1024)
    assert e.value.status == tm.TTT_ERR_WORKSPACE_TOO_SMALL


# Three slots over eight calls of L tokens: slot 0 runs sequence 0 (40 tokens)
# then sequence 3 (24 tokens) from a fresh start; slot 1 runs sequence 1 (64
# tokens); slot 2 runs two one-call sequences (4, 5) and then sequence 2 (48
# tokens).  Each call passes every slot's own position and closing flag.
RAGGED_SLOTS = [[(0, 40), (3, 24)], [(1, 64)], [(4, 8), (5, 8), (2, 48)]]


@pytest.mark.parametrize("dtype,L,C", [(torch.bfloat16, 8, 16), (torch.float32, 8, 16),
                                       (torch.bfloat16, 24, 16)],
                         ids=["bf16-decode", "f32", "bf16-L24"])
def test_ragged_sessions_equal_their_own_runs(dtype, L, C):
    d, f, K = 128, 192, 4
    scale = L // 8
    slots = [[(q, n * scale) for q, n in s] for s in RAGGED_SLOTS]
    B = len(slots)
    inp = synth.make_inputs(6, 64 * scale, d, f, K, dtype, seed=95)
    dev = to_device(inp)
    eta = 2e-2
    w = (dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"])
    ref = {}
    for q in range(6):
        n = max(m for s in slots for (qq, m) in s if qq == q)
        ref[q] = tm.forward_batched(dev["H"][q:q + 1, :n].contiguous(),
                                    dev["X0"][q:q + 1, :n].contiguous(), *w, eta, C)
    calls = sum(m for _, m in slots[0]) // L
    desc = tm.make_desc(B, L, d, f, C, K, eta, dtype)
    ws = torch.empty(tm.ttt_mlp_stream_workspace_size(desc), dtype=torch.uint8, device="cuda")
    carry = torch.empty(tm.ttt_mlp_carry_size(desc), dtype=torch.uint8, device="cuda")
    state = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    outs = {q: [] for q in range(6)}
    finals, dec_rows = {}, {q: [] for q in range(6)}
    cursor = [[0, 0] for _ in range(B)]  # (index of the slot's sequence, its position)
    for j in range(calls):
        pos, last, hs, xs, seqs = [], [], [], [], []
        for b in range(B):
            k, p = cursor[b]
            q, n = slots[b][k]
            pos.append(p)
            last.append(1 if p + L == n else 0)
            hs.append(dev["H"][q, p:p + L])
            xs.append(dev["X0"][q, p:p + L])
            seqs.append(q)
            n_pend = 0 if p == 0 else p - (p - 1) // C * C
            dec = dtype == torch.bfloat16 and L <= 16 and B * L <= 64 and not last[-1] \
                and n_pend + L <= C
            dec_rows[q] += [dec] * L
        O = torch.empty((B, L, d), dtype=dtype, device="cuda")
        tm.ttt_mlp_forward_stream_ragged(desc, pos, last, torch.stack(hs).contiguous(),
                                         torch.stack(xs).contiguous(), *w, O, state, carry, ws)
        for b in range(B):
            outs[seqs[b]].append(O[b].clone())
            if last[b]:
                finals[seqs[b]] = state[b].clone()
                cursor[b] = [cursor[b][0] + 1, 0]
            else:
                cursor[b][1] += L
    torch.cuda.synchronize()
    for q in range(6):
        Oq = torch.cat(outs[q])
        O1, W1 = ref[q]
        assert torch.equal(finals[q], W1[0]), q
        dec = torch.tensor(dec_rows[q], device="cuda")
        assert torch.equal(Oq[~dec], O1[0][~dec]), q
        if dec.any():
            e = rel(Oq[dec].double().cpu().numpy(), O1[0][dec].double().cpu().numpy())
            assert e <= DECODE_TOL, (q, e)
    print(f"  decode rows: {sum(sum(v) for v in dec_rows.values())}", flush=True)


@pytest.mark.parametrize("seed", [1, 2])
def test_ragged_random_schedule(seed):
    """Four slots over 30 calls with a random number of new tokens per call
    (1..20, the same for every slot) and sequences that end at random (or at
    their drawn length) and are replaced by new ones; each finished sequence
    is compared with its own one-call run."""
    import random
    rnd = random.Random(seed)
    B, d, f, K, C, dtype = 4, 128, 192, 4, 16, torch.bfloat16
    eta = 2e-2
    n_seq, max_len, calls = 4 + 4 * 30, 160, 30
    inp = synth.make_inputs(n_seq, max_len, d, f, K, dtype, seed=96 + seed)
    dev = to_device(inp)
    w = (dev["W_gate"], dev["W_up"], dev["W_down0"], dev["taps"], dev["W_target"])
    length = [rnd.randint(1, max_len) for _ in range(n_seq)]
    desc_max = tm.make_desc(B, 20, d, f, C, K, eta, dtype)
    ws = torch.empty(tm.ttt_mlp_stream_workspace_size(desc_max), dtype=torch.uint8,
                     device="cuda")
    carry = torch.empty(tm.ttt_mlp_carry_size(desc_max), dtype=torch.uint8, device="cuda")
    state = torch.empty((B, d, f), dtype=torch.float32, device="cuda")
    slot = [[b, 0] for b in range(B)]  # (sequence, position)
    nxt = B
    outs = {q: [] for q in range(n_seq)}
    dec_rows = {q: [] for q in range(n_seq)}
    finals = {}
    for _ in range(calls):
        L = rnd.randint(1, min(20, min(max_len - p for _, p in slot)))
        pos, last, hs, xs = [], [], [], []
        for b in range(B):
            q, p = slot[b]
            closing = p + L >= length[q] or rnd.random() < 0.15
            if closing:
                length[q] = p + L
            pos.append(p)
            last.append(1 if closing else 0)
            hs.append(dev["H"][q, p:p + L])
            xs.append(dev["X0"][q, p:p + L])
            n_pend = 0 if p == 0 else p - (p - 1) // C * C
            dec_rows[q] += [B * L <= 64 and L <= 16 and not closing and n_pend + L <= C] * L
        desc = tm.make_desc(B, L, d, f, C, K, eta, dtype)
        O = torch.empty((B, L, d), dtype=dtype, device="cuda")
        tm.ttt_mlp_forward_stream_ragged(desc, pos, last, torch.stack(hs).contiguous(),
                                         torch.stack(xs).contiguous(), *w, O, state, carry, ws)
        for b in range(B):
            q, p = slot[b]
            outs[q].append(O[b].clone())
            if last[b]:
                finals[q] = state[b].clone()
                slot[b] = [nxt, 0]
                nxt += 1
            else:
                slot[b][1] = p + L
    torch.cuda.synchronize()
    assert len(finals) >= 6
    for q, Wq in finals.items():
        n = length[q]
        O1, W1 = tm.forward_batched(dev["H"][q:q + 1, :n].contiguous(),
                                    dev["X0"][q:q + 1, :n].contiguous(), *w, eta, C)
        Oq = torch.cat(outs[q])
        assert Oq.shape[0] == n, (q, Oq.shape, n)
        assert torch.equal(Wq, W1[0]), q
        dec = torch.tensor(dec_rows[q], device="cuda")
        assert torch.equal(Oq[~dec], O1[0][~dec]), q
        if dec.any():
            assert rel(Oq[dec].double().cpu().numpy(), O1[0][dec].double().cpu().numpy()) <= DECODE_TOL
    print(f"  {len(finals)} sequences finished, "
          f"{sum(sum(dec_rows[q]) for q in finals)} of their rows decoded", flush=True)
