"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, plans workspaces, and rejects bad
arguments with the documented status before touching the device.  Invalid
calls use fake (never dereferenced) device addresses."""
import ctypes
import os
import re
import threading

import pytest

from chunk_wise_weight_chunked_amd import ttt_mlp as tm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt_mlp.h")


@pytest.fixture(scope="module")
def lib():
    return tm.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tm.EXPORTS)


def desc(**kw):
    base = dict(batch=1, seq_len=4096, d_model=256, d_ff=512, chunk=512, conv_k=4, eta=1e-3,
                dtype=tm.TTT_BF16, mode="auto", init_from_w0=1)
    base.update(kw)
    return tm.make_desc(**base)


def test_workspace_plan():
    # T = 4096, C = 512: N = 8 chunks.  One slot set if a group covers every
    # chunk, else two (the scan of group g+1 runs next to the outputs of g).
    d = desc()
    slot = 256 * 512 * 2
    w1 = tm.ttt_mlp_workspace_size(d, 1)           # groups of 1: 2 sets of 1
    fixed = w1 - 2 * slot
    assert tm.ttt_mlp_workspace_size(d, 0) == fixed + 2 * 2 * slot   # auto: 4 groups of 2
    w_all = tm.ttt_mlp_workspace_size(d, 8)
    assert w_all == fixed + 8 * slot               # one group, one set
    assert tm.ttt_mlp_workspace_size(d, 100) == w_all
    assert tm.ttt_mlp_workspace_size(d, 3) == fixed + 2 * 3 * slot
    cp, seq = desc(mode="chunk_parallel"), desc(mode="sequential")
    assert tm.ttt_mlp_workspace_size(cp, 0) == w_all
    assert tm.ttt_mlp_workspace_size(seq, 0) == tm.ttt_mlp_workspace_size(d, 0)  # auto's groups
    # auto takes a quarter of the chunks at most
    assert tm.ttt_mlp_group_size(d, w_all) == 2
    assert tm.ttt_mlp_group_size(d, w1) == 1
    assert tm.ttt_mlp_group_size(d, w1 + slot) == 1   # 3 slots: still 2 sets of 1
    # chunk-parallel takes as much as fits
    assert tm.ttt_mlp_group_size(cp, w_all) == 8
    assert tm.ttt_mlp_group_size(cp, w_all - 1) == 3  # 7 slots: 2 sets of 3
    assert tm.ttt_mlp_group_size(cp, w1) == 1
    assert tm.ttt_mlp_group_size(seq, w_all) == 2
    assert tm.ttt_mlp_group_size(seq, w1) == 1
    with pytest.raises(tm.TTTError) as e:
        tm.ttt_mlp_group_size(d, w1 - 1)
    assert e.value.status == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    # a single chunk needs one slot
    one = desc(seq_len=300)
    assert tm.ttt_mlp_workspace_size(one, 1) == tm.ttt_mlp_workspace_size(one, 0)
    assert tm.ttt_mlp_group_size(one, tm.ttt_mlp_workspace_size(one, 0)) == 1


def test_auto_mode_takes_one_group_for_many_sequences():
    # the scan of one group has B * ceil(d/256) * ceil(f/256) weight tiles:
    # from 1024 tiles on, auto takes one group of all chunks, else four
    many = desc(batch=16, seq_len=8192, d_model=2560, d_ff=9728, chunk=512)  # 6080 tiles
    few = desc(batch=2, seq_len=8192, d_model=2560, d_ff=9728, chunk=512)    # 760 tiles
    assert tm.ttt_mlp_workspace_size(many, 0) == tm.ttt_mlp_workspace_size(many, 16)
    assert tm.ttt_mlp_group_size(many, tm.ttt_mlp_workspace_size(many, 0)) == 16
    assert tm.ttt_mlp_group_size(few, tm.ttt_mlp_workspace_size(few, 0)) == 4
    edge = desc(batch=64, d_model=1024, d_ff=1024)  # 64 * 4 * 4 = 1024 tiles, N = 8
    assert tm.ttt_mlp_group_size(edge, tm.ttt_mlp_workspace_size(edge, 0)) == 8
    below = desc(batch=63, d_model=1024, d_ff=1024)
    assert tm.ttt_mlp_group_size(below, tm.ttt_mlp_workspace_size(below, 0)) == 2


def test_workspace_fixed_part_matches_layout():
    # bf16: U [T][d] + Zt [f][P] + Vt [d][P] + WgU [2f][d] + WtT [d][d]
    # + tapsT [8][d] fp32 + 2 slot sets of 1 (Z is kept only token-major);
    # fp32 adds the row-major Z [T][f] in front
    d = desc(seq_len=1000, chunk=100)  # padded chunks: Cp = 128, P = 10 * 128
    for es, dt in ((2, tm.TTT_BF16), (4, tm.TTT_F32)):
        parts = [1000 * 256 * es, 512 * 1280 * es, 256 * 1280 * es,
                 2 * 512 * 256 * es, 256 * 256 * es, 8 * 256 * 4, 2 * 256 * 512 * es]
        if es == 4:
            parts.insert(0, 1000 * 512 * es)
        expect = sum((p + 255) // 256 * 256 for p in parts)
        assert tm.ttt_mlp_workspace_size(desc(seq_len=1000, chunk=100, dtype=dt), 1) == expect


def test_workspace_conv_output_has_its_own_region():
    # d > f: the conv output U [T][d] has its own region (Zt keeps f rows)
    d = desc(d_model=512, d_ff=256, seq_len=1000, chunk=100)
    es = 2
    parts = [1000 * 512 * es, 256 * 1280 * es, 512 * 1280 * es,
             2 * 256 * 512 * es, 512 * 512 * es, 8 * 512 * 4, 2 * 512 * 256 * es]
    expect = sum((p + 255) // 256 * 256 for p in parts)
    assert tm.ttt_mlp_workspace_size(d, 1) == expect


BAD_DESCS = [
    (dict(batch=0), tm.TTT_ERR_INVALID_ARGUMENT, "batch"),
    (dict(seq_len=0), tm.TTT_ERR_INVALID_ARGUMENT, "seq_len"),
    (dict(d_model=96), tm.TTT_ERR_UNSUPPORTED, "d_model"),
    (dict(d_ff=100), tm.TTT_ERR_UNSUPPORTED, "d_ff"),
    (dict(chunk=0), tm.TTT_ERR_INVALID_ARGUMENT, "chunk"),
    (dict(conv_k=0), tm.TTT_ERR_INVALID_ARGUMENT, "conv_k"),
    (dict(conv_k=9), tm.TTT_ERR_UNSUPPORTED, "conv_k"),
    (dict(eta=float("nan")), tm.TTT_ERR_INVALID_ARGUMENT, "eta"),
    (dict(eta=float("inf")), tm.TTT_ERR_INVALID_ARGUMENT, "eta"),
    (dict(dtype=7), tm.TTT_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(mode=9), tm.TTT_ERR_INVALID_ARGUMENT, "mode"),
    (dict(init_from_w0=2), tm.TTT_ERR_INVALID_ARGUMENT, "init_from_w0"),
    (dict(target=4), tm.TTT_ERR_INVALID_ARGUMENT, "target"),
    (dict(align=2), tm.TTT_ERR_INVALID_ARGUMENT, "align"),
    (dict(batch=1 << 20, seq_len=1 << 12), tm.TTT_ERR_UNSUPPORTED, "2^31"),
    # each below the d*f bound, but a 256-row tile would need offsets past 2^31
    (dict(d_ff=(1 << 20) + 64), tm.TTT_ERR_UNSUPPORTED, "d_ff must be <= 2^20"),
    (dict(d_model=1 << 24, d_ff=64), tm.TTT_ERR_UNSUPPORTED, "d_model must be <= 2^20"),
]


@pytest.mark.parametrize("kw,status,word", BAD_DESCS)
def test_bad_descriptor(lib, kw, status, word):
    d = desc(**kw)
    assert lib.ttt_mlp_workspace_size(ctypes.byref(d), 0) == 0
    assert word in tm.ttt_last_error()
    ptrs = fake_ptrs(desc())
    st = call_forward(lib, d, ptrs)
    assert st == status, tm.ttt_last_error()
    assert word in tm.ttt_last_error()


BASE = 1 << 40  # fake device addresses, never dereferenced


def fake_ptrs(d, ws_bytes=None):
    """Non-overlapping fake buffers for descriptor d."""
    es = 2 if d.dtype == tm.TTT_BF16 else 4
    B, T, dm, f, K = d.batch, d.seq_len, d.d_model, d.d_ff, d.conv_k
    sizes = dict(H=B * T * dm * es, X0=B * T * dm * es, W_gate=f * dm * es, W_up=f * dm * es,
                 W_down0=dm * f * es, taps=dm * K * es, W_target=dm * dm * es,
                 O=B * T * dm * es, W=B * dm * f * 4)
    ws = ws_bytes if ws_bytes is not None else tm.ttt_mlp_workspace_size(desc(), 0)
    sizes["ws"] = ws
    out, addr = {}, BASE
    for k, n in sizes.items():
        out[k] = addr
        addr += (n + 4095) // 4096 * 4096 + 4096
    out["ws_bytes"] = ws
    return out


def call_forward(lib, d, p, batched=False):
    fn = lib.ttt_mlp_forward_batched if batched else lib.ttt_mlp_forward
    return fn(ctypes.byref(d), p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down0"], p["taps"],
              p["W_target"], p["O"], p["W"], p["ws"], p["ws_bytes"], None)


@pytest.mark.parametrize("name", ["H", "X0", "W_gate", "W_up", "W_down0", "taps", "W_target",
                                  "O", "W", "ws"])
def test_null_pointer_rejected(lib, name):
    d = desc()
    p = fake_ptrs(d)
    p[name] = None
    assert call_forward(lib, d, p) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "NULL" in tm.ttt_last_error()


def test_w_down0_optional_without_init(lib):
    d = desc(init_from_w0=0, batch=2)
    p = fake_ptrs(d)
    p["W_down0"] = None
    p["H"] = None  # still rejected for the other pointer
    assert call_forward(lib, d, p, batched=True) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "H is NULL" in tm.ttt_last_error()


@pytest.mark.parametrize("target,unused", [("proj", "taps"), ("conv", "W_target"),
                                           ("embed", "taps"), ("embed", "W_target")])
def test_unused_target_inputs_may_be_null(lib, target, unused):
    """A target variant without the conv / projection accepts NULL taps /
    W_target: the pointer checks pass and the call fails later, on a workspace
    below the minimum."""
    d = desc(target=target)
    p = fake_ptrs(d, ws_bytes=tm.ttt_mlp_workspace_size(d, 1) - 256)
    p[unused] = None
    assert call_forward(lib, d, p) == tm.TTT_ERR_WORKSPACE_TOO_SMALL, tm.ttt_last_error()
    d = desc()  # the method itself needs both
    p = fake_ptrs(d)
    p[unused] = None
    assert call_forward(lib, d, p) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "NULL" in tm.ttt_last_error() and "H " not in tm.ttt_last_error()


@pytest.mark.parametrize("name", ["H", "O", "W", "W_target"])
def test_misaligned_pointer_rejected(lib, name):
    d = desc()
    p = fake_ptrs(d)
    p[name] += 8
    assert call_forward(lib, d, p) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "aligned" in tm.ttt_last_error()


def test_workspace_alignment_and_size(lib):
    d = desc()
    p = fake_ptrs(d)
    p["ws"] += 16
    assert call_forward(lib, d, p) == tm.TTT_ERR_INVALID_ARGUMENT
    p = fake_ptrs(d, ws_bytes=tm.ttt_mlp_workspace_size(d, 1) - 1)
    assert call_forward(lib, d, p) == tm.TTT_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("out,inp", [("O", "H"), ("W", "W_down0"), ("ws", "X0"), ("O", "W"),
                                     ("ws", "O")])
def test_overlap_rejected(lib, out, inp):
    d = desc()
    p = fake_ptrs(d)
    p[out] = p[inp] + 4096
    assert call_forward(lib, d, p) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "overlaps" in tm.ttt_last_error()


def test_forward_requires_single_sequence(lib):
    d = desc(batch=2)
    assert call_forward(lib, d, fake_ptrs(d)) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "batch" in tm.ttt_last_error()


def test_state_reset_validation(lib):
    f = lib.ttt_fastweight_state_reset
    assert f(None, BASE, tm.TTT_BF16, 1, 64, 64, None) == tm.TTT_ERR_INVALID_ARGUMENT
    assert f(BASE, BASE + (1 << 30), 5, 1, 64, 64, None) == tm.TTT_ERR_INVALID_ARGUMENT
    assert f(BASE, BASE + (1 << 30), tm.TTT_BF16, 0, 64, 64, None) == tm.TTT_ERR_INVALID_ARGUMENT
    assert f(BASE, BASE + 1024, tm.TTT_BF16, 1, 64, 64, None) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "overlaps" in tm.ttt_last_error()
    assert f(BASE + 4, BASE + (1 << 30), tm.TTT_F32, 1, 64, 64, None) == tm.TTT_ERR_INVALID_ARGUMENT


def test_last_error_is_per_thread(lib):
    d = desc(batch=0)
    call_forward(lib, d, fake_ptrs(desc()))
    seen = {}

    def other():
        seen["msg"] = tm.ttt_last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "batch" in tm.ttt_last_error()


def test_stage_names(lib):
    names = [tm.ttt_stage_name(i) for i in range(tm.TTT_NUM_STAGES)]
    assert names == ["state_reset", "weight_prep", "pad_fill", "swiglu", "target",
                     "prefix_update", "down_proj", "scan_apply", "scan_target"]
    header = open(os.path.join(ROOT, "include", "ttt_mlp.h")).read()
    assert f"#define TTT_NUM_STAGES {tm.TTT_NUM_STAGES}" in header
    assert tm.ttt_stage_name(99) == ""


def test_library_has_no_unresolved_internal_symbols():
    """Every kernel's host stub and every internal function is defined in the
    built library (an unresolved one would only fail when loaded on the GPU)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", tm.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    missing = [l.split()[-1] for l in out.splitlines() if "3ttt" in l]
    assert not missing, missing



def stream_ptrs(d, ws_bytes):
    p = fake_ptrs(d, ws_bytes=ws_bytes)
    p["carry"] = p["ws"] + (ws_bytes + 4095) // 4096 * 4096 + 4096
    return p


def call_stream(lib, d, p, pos, last):
    return lib.ttt_mlp_forward_stream(
        ctypes.byref(d), pos, last, p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down0"],
        p["taps"], p["W_target"], p["O"], p["W"], p["carry"], p["ws"], p["ws_bytes"], None)


def test_stream_sizes():
    # carry per session: C rows of H, then 7 + C rows of X0 (the conv halo
    # holds up to K - 1 <= 7 rows); for bf16 then the bf16 copies of the
    # sessions' current weights at a 256-byte boundary
    rows = 3 * (2 * 64 + 7) * 256
    assert tm.ttt_mlp_carry_size(desc(batch=3, seq_len=100, chunk=64, dtype=tm.TTT_F32)) == \
        rows * 4
    assert tm.ttt_mlp_carry_size(desc(batch=3, seq_len=100, chunk=64)) == \
        (rows * 2 + 255) // 256 * 256 + 3 * 256 * 512 * 2
    d = desc(batch=2, seq_len=300, chunk=128)
    w1 = tm.ttt_mlp_stream_workspace_size(d, 1)
    # the layer runs on sequences of up to L + C tokens
    longest = desc(batch=2, seq_len=300 + 128, chunk=128)
    rows = (2 * 428 * 256 * 2 + 255) // 256 * 256
    carry_rows = 2 * (2 * 128 + 7) * 256 * 2  # the new carry's rows, built before the copy
    assert w1 == tm.ttt_mlp_workspace_size(longest, 1) + 2 * rows + carry_rows
    assert tm.ttt_mlp_stream_workspace_size(d, 2) > w1
    assert tm.ttt_mlp_stream_workspace_size(d, 0) >= w1
    with pytest.raises(tm.TTTError, match="max_group"):
        tm.ttt_mlp_stream_workspace_size(d, -1)
    with pytest.raises(tm.TTTError, match="batch"):
        tm.ttt_mlp_carry_size(desc(batch=0))


def test_stream_validation(lib):
    d = desc(batch=2, seq_len=300, chunk=128)
    w1 = tm.ttt_mlp_stream_workspace_size(d, 1)
    p = stream_ptrs(d, w1 - 256)
    # the argument checks come first; a good call then stops at the workspace
    assert call_stream(lib, d, p, 128, 0) == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    assert "minimum %d" % w1 in tm.ttt_last_error()
    assert call_stream(lib, d, p, -1, 0) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "pos" in tm.ttt_last_error()
    assert call_stream(lib, d, p, 0, 2) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "last" in tm.ttt_last_error()
    q = dict(p, carry=None)
    for pos, last in ((0, 0), (5, 1), (5, 0)):
        assert call_stream(lib, d, q, pos, last) == tm.TTT_ERR_INVALID_ARGUMENT
        assert "carry is NULL" in tm.ttt_last_error()
    # a single closing call from the start needs no carry
    assert call_stream(lib, d, q, 0, 1) == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call_stream(lib, d, dict(p, carry=p["carry"] + 8), 5, 0) == \
        tm.TTT_ERR_INVALID_ARGUMENT
    assert "aligned" in tm.ttt_last_error()
    for other in ("H", "X0", "O", "W", "ws"):
        assert call_stream(lib, d, dict(p, carry=p[other] + 4096), 5, 0) == \
            tm.TTT_ERR_INVALID_ARGUMENT
        assert "carry overlaps" in tm.ttt_last_error()
    # W_down0 is read only on the first call of a stream
    d0 = desc(batch=2, seq_len=300, chunk=128)
    assert call_stream(lib, d0, dict(p, W_down0=None), 0, 0) == tm.TTT_ERR_INVALID_ARGUMENT
    assert call_stream(lib, d0, dict(p, W_down0=None), 256, 0) == \
        tm.TTT_ERR_WORKSPACE_TOO_SMALL


def backward_ptrs(d, ws_bytes):
    es = 2 if d.dtype == tm.TTT_BF16 else 4
    B, T, dm, f, K = d.batch, d.seq_len, d.d_model, d.d_ff, d.conv_k
    act, st = B * T * dm * es, B * dm * f * 4
    sizes = dict(H=act, X0=act, W_gate=f * dm * es, W_up=f * dm * es, W_down0=dm * f * es,
                 W_start=st, taps=dm * K * es, W_target=dm * dm * es, dO=act, dW_final=st,
                 dH=act, dX0=act, dW_gate=f * dm * 4, dW_up=f * dm * 4, dW_start=st,
                 dtaps=dm * K * 4, dW_target=dm * dm * 4, d_eta=4, ws=ws_bytes)
    out, addr = {}, BASE
    for k, n in sizes.items():
        out[k] = addr
        addr += (n + 4095) // 4096 * 4096 + 4096
    out["ws_bytes"] = ws_bytes
    return out


BACKWARD_ARGS = ("H", "X0", "W_gate", "W_up", "W_down0", "W_start", "taps", "W_target", "dO",
                 "dW_final", "dH", "dX0", "dW_gate", "dW_up", "dW_start", "dtaps", "dW_target",
                 "d_eta", "ws")


def call_backward(lib, d, p):
    return lib.ttt_mlp_backward_batched(ctypes.byref(d), *[p[k] for k in BACKWARD_ARGS],
                                        p["ws_bytes"], None)


def test_backward_workspace_and_validation(lib):
    d = desc(batch=2, seq_len=300, chunk=128)
    need = tm.ttt_mlp_backward_workspace_size(d)
    # at least the forward's workspace with one group of all chunks, plus the
    # backward's own regions (two fp32 [B*T][f] pre-activations among them)
    assert need > tm.ttt_mlp_workspace_size(d, 3) + 2 * 2 * 300 * 512 * 4
    p = backward_ptrs(d, need - 256)
    assert call_backward(lib, d, p) == tm.TTT_ERR_WORKSPACE_TOO_SMALL, tm.ttt_last_error()
    # optional inputs: W_start with init_from_w0 = 1, dW_final always
    assert call_backward(lib, d, dict(p, W_start=None, dW_final=None)) == \
        tm.TTT_ERR_WORKSPACE_TOO_SMALL
    for name in ("H", "X0", "W_gate", "W_up", "W_down0", "taps", "W_target", "dO", "dH", "dX0",
                 "dW_gate", "dW_up", "dW_start", "dtaps", "dW_target", "d_eta", "ws"):
        assert call_backward(lib, d, dict(p, **{name: None})) == tm.TTT_ERR_INVALID_ARGUMENT
        assert f"{name} is NULL" in tm.ttt_last_error()
    d0 = desc(batch=2, seq_len=300, chunk=128, init_from_w0=0)
    assert call_backward(lib, d0, dict(p, W_start=None)) == tm.TTT_ERR_INVALID_ARGUMENT
    assert call_backward(lib, d0, dict(p, W_down0=None)) == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    # a target without the conv / projection takes NULL taps, dtaps / W_target, dW_target
    de = desc(batch=2, seq_len=300, chunk=128, target="embed")
    pe = backward_ptrs(de, tm.ttt_mlp_backward_workspace_size(de) - 256)
    assert call_backward(lib, de, dict(pe, taps=None, dtaps=None, W_target=None,
                                       dW_target=None)) == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call_backward(lib, d, dict(p, dH=p["H"] + 4096)) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "overlaps" in tm.ttt_last_error()
    assert call_backward(lib, d, dict(p, dW_gate=p["dW_up"])) == tm.TTT_ERR_INVALID_ARGUMENT
    assert call_backward(lib, d, dict(p, ws=p["dO"])) == tm.TTT_ERR_INVALID_ARGUMENT
    assert call_backward(lib, d, dict(p, dH=p["dH"] + 8)) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "aligned" in tm.ttt_last_error()
    assert call_backward(lib, d, dict(p, d_eta=p["d_eta"] + 2)) == tm.TTT_ERR_INVALID_ARGUMENT


def test_stream_ragged_validation(lib):
    d = desc(batch=3, seq_len=16, chunk=64)
    w1 = tm.ttt_mlp_stream_workspace_size(d, 1)
    p = stream_ptrs(d, w1 - 256)

    def call(pos, last, q=p):
        P = (ctypes.c_int64 * 3)(*pos)
        L = (ctypes.c_int32 * 3)(*last)
        return lib.ttt_mlp_forward_stream_ragged(
            ctypes.byref(d), ctypes.cast(P, ctypes.c_void_p), ctypes.cast(L, ctypes.c_void_p),
            q["H"], q["X0"], q["W_gate"], q["W_up"], q["W_down0"], q["taps"], q["W_target"],
            q["O"], q["W"], q["carry"], q["ws"], q["ws_bytes"], None)

    assert call([0, 64, 7], [0, 1, 0]) == tm.TTT_ERR_WORKSPACE_TOO_SMALL, tm.ttt_last_error()
    assert call([0, -1, 7], [0, 0, 0]) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "session 1" in tm.ttt_last_error()
    assert call([0, 1, 7], [0, 0, 3]) == tm.TTT_ERR_INVALID_ARGUMENT
    assert "last" in tm.ttt_last_error()
    # every session closing from the start: no carry needed; W_down0 only
    # needed while some session starts at 0 with init_from_w0
    assert call([0, 0, 0], [1, 1, 1], dict(p, carry=None)) == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call([0, 5, 0], [1, 1, 1], dict(p, carry=None)) == tm.TTT_ERR_INVALID_ARGUMENT
    assert call([8, 5, 9], [0, 1, 0], dict(p, W_down0=None)) == tm.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call([8, 0, 9], [0, 1, 0], dict(p, W_down0=None)) == tm.TTT_ERR_INVALID_ARGUMENT
    assert lib.ttt_mlp_forward_stream_ragged(ctypes.byref(d), None, None, *[p[k] for k in (
        "H", "X0", "W_gate", "W_up", "W_down0", "taps", "W_target", "O", "W", "carry", "ws")],
        p["ws_bytes"], None) == tm.TTT_ERR_INVALID_ARGUMENT


# ------------------------------------------------ shares (context parallelism)
def _share_ptrs(d):
    p = fake_ptrs(d)
    es = 2 if d.dtype == tm.TTT_BF16 else 4
    top = max(v for k, v in p.items() if k != "ws_bytes") + (1 << 32)
    p["left"] = top
    p["right"] = top + (d.batch * 7 * d.d_model * es + 4095) // 4096 * 4096 + 4096
    return p


def _share_calls(lib, d, p, share, reuse=0):
    inc = lib.ttt_mlp_share_increment(ctypes.byref(d), share, p["H"], p["X0"], p["W_gate"],
                                      p["W_up"], p["taps"], p["W_target"], p["W"], p["ws"],
                                      p["ws_bytes"], None)
    msg = tm.ttt_last_error()
    fwd = lib.ttt_mlp_share_forward(ctypes.byref(d), share, reuse, p["H"], p["X0"],
                                    p["W_gate"], p["W_up"], p["taps"], p["W_target"], p["O"],
                                    p["W"], p["ws"], p["ws_bytes"], None)
    return inc, msg, fwd, tm.ttt_last_error()


def test_share_rejects_bad_arguments(lib):
    d = desc(seq_len=1000, chunk=128)  # not whole chunks
    p = _share_ptrs(d)
    # a share followed by more tokens must end on a chunk boundary
    sh = tm.ttt_share_t(p["left"], p["right"])
    inc, m1, fwd, m2 = _share_calls(lib, d, p, ctypes.byref(sh))
    assert inc == fwd == tm.TTT_ERR_INVALID_ARGUMENT and "whole chunks" in m1 and "whole chunks" in m2
    # the last share of a sequence may end on a partial chunk: the call gets
    # past validation and stops at the (too small) workspace
    p["ws_bytes"] = 1024
    sh = tm.ttt_share_t(p["left"], None)
    inc, m1, fwd, m2 = _share_calls(lib, d, p, ctypes.byref(sh))
    assert inc == fwd == tm.TTT_ERR_WORKSPACE_TOO_SMALL, (m1, m2)
    # NULL share descriptor, misaligned halo, halo overlapping an output, bad reuse
    inc, m1, fwd, m2 = _share_calls(lib, d, p, None)
    assert inc == fwd == tm.TTT_ERR_INVALID_ARGUMENT and "share is NULL" in m1
    sh = tm.ttt_share_t(p["left"] + 8, None)
    inc, m1, fwd, m2 = _share_calls(lib, d, p, ctypes.byref(sh))
    assert inc == fwd == tm.TTT_ERR_INVALID_ARGUMENT and "X0_left" in m1 and "aligned" in m1
    sh = tm.ttt_share_t(p["O"], None)  # the halo inside O: O overlaps an input
    _, _, fwd, m2 = _share_calls(lib, d, p, ctypes.byref(sh))
    assert fwd == tm.TTT_ERR_INVALID_ARGUMENT and "overlaps" in m2
    sh = tm.ttt_share_t(p["W"], None)  # the halo inside S / W_state
    inc, m1, fwd, m2 = _share_calls(lib, d, p, ctypes.byref(sh))
    assert inc == fwd == tm.TTT_ERR_INVALID_ARGUMENT and "overlaps" in m1
    _, _, fwd, m2 = _share_calls(lib, d, p, ctypes.byref(tm.ttt_share_t(None, None)), reuse=2)
    assert fwd == tm.TTT_ERR_INVALID_ARGUMENT and "reuse" in m2


def test_share_increment_needs_no_o_and_no_w_down0(lib):
    """The increment call writes no output rows and reads no starting weight:
    NULL O and W_down0 pass validation (the call stops at the workspace)."""
    d = desc(seq_len=1024, chunk=128)
    p = _share_ptrs(d)
    p["O"] = None
    p["W_down0"] = None
    p["ws_bytes"] = tm.ttt_mlp_workspace_size(d, 1) - 256
    sh = tm.ttt_share_t(p["left"], p["right"])
    st = lib.ttt_mlp_share_increment(ctypes.byref(d), ctypes.byref(sh), p["H"], p["X0"],
                                     p["W_gate"], p["W_up"], p["taps"], p["W_target"], p["W"],
                                     p["ws"], p["ws_bytes"], None)
    assert st == tm.TTT_ERR_WORKSPACE_TOO_SMALL, tm.ttt_last_error()
    p["W"] = None
    st = lib.ttt_mlp_share_increment(ctypes.byref(d), ctypes.byref(sh), p["H"], p["X0"],
                                     p["W_gate"], p["W_up"], p["taps"], p["W_target"], p["W"],
                                     p["ws"], p["ws_bytes"], None)
    assert st == tm.TTT_ERR_INVALID_ARGUMENT and "W_state is NULL" in tm.ttt_last_error()


def test_noalloc_decode_rejects_calls_it_does_not_serve():
    """Through the binding (argument count and order) with fake pointers: an
    fp32 call, a closing call and a call past the pending chunk are refused
    before anything touches the device."""
    for kw, pos, last, word in ((dict(dtype=tm.TTT_F32), 0, 0, "at most"),
                                (dict(), 0, 1, "full path"),
                                (dict(seq_len=16, chunk=16), 16, 0, "full path"),
                                (dict(seq_len=17), 0, 0, "at most")):
        base = dict(batch=2, seq_len=8, chunk=64)
        base.update(kw)
        d = desc(**base)
        p = fake_ptrs(d)
        with pytest.raises(tm.TTTError) as e:
            tm.ttt_mlp_forward_stream_decode_noalloc(
                d, [pos] * 2, [last] * 2, *[p[k] for k in (
                    "H", "X0", "W_gate", "W_up", "W_down0", "taps", "W_target", "O", "W")],
                p["ws"], stream=0)
        assert e.value.status == tm.TTT_ERR_UNSUPPORTED and word in str(e.value), str(e.value)

