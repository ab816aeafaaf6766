"""ctypes binding of libttt_mlp.so (the C ABI declared in include/ttt_mlp.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  PyTorch is used for device memory and streams; tensors are
passed as raw device pointers.  There is no fallback: if the library is not
built, or the HIP runtime is unavailable, calls raise.

The function names match the C entry points.  `forward`/`forward_batched` are
conveniences that allocate outputs and the workspace with torch and call them.
"""
from __future__ import annotations

import ctypes
import os

import torch  # must be imported before the library so both share one HIP runtime

from . import build as _build

LIB_PATH = _build.LIB

TTT_F32, TTT_BF16 = 0, 1
TTT_OK = 0
TTT_ERR_INVALID_ARGUMENT = -1
TTT_ERR_UNSUPPORTED = -2
TTT_ERR_WORKSPACE_TOO_SMALL = -3
TTT_ERR_HIP = -4
TTT_MODE_AUTO, TTT_MODE_SEQUENTIAL, TTT_MODE_CHUNK_PARALLEL = 0, 1, 2
TTT_TARGET_CONV_PROJ, TTT_TARGET_PROJ, TTT_TARGET_CONV, TTT_TARGET_EMBED = 0, 1, 2, 3
TTT_NUM_STAGES = 9

_MODES = {"auto": TTT_MODE_AUTO, "sequential": TTT_MODE_SEQUENTIAL,
          "chunk_parallel": TTT_MODE_CHUNK_PARALLEL}
_TARGETS = {"conv_proj": TTT_TARGET_CONV_PROJ, "proj": TTT_TARGET_PROJ,
            "conv": TTT_TARGET_CONV, "embed": TTT_TARGET_EMBED}
TTT_ALIGN_NEXT, TTT_ALIGN_SELF = 0, 1
_ALIGNS = {"next": TTT_ALIGN_NEXT, "self": TTT_ALIGN_SELF}


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class ttt_mlp_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("d_model", ctypes.c_int64),
        ("d_ff", ctypes.c_int64),
        ("chunk", ctypes.c_int32),
        ("conv_k", ctypes.c_int32),
        ("eta", ctypes.c_float),
        ("dtype", ctypes.c_int),
        ("mode", ctypes.c_int),
        ("init_from_w0", ctypes.c_int32),
        ("target", ctypes.c_int),
        ("align", ctypes.c_int),
    ]


class ttt_share_t(ctypes.Structure):
    _fields_ = [
        ("X0_left", ctypes.c_void_p),
        ("X0_right", ctypes.c_void_p),
    ]


EXPORTS = (
    "ttt_mlp_workspace_size", "ttt_mlp_group_size", "ttt_mlp_forward",
    "ttt_mlp_forward_batched", "ttt_fastweight_state_reset", "ttt_last_error",
    "ttt_profile_enable", "ttt_profile_read", "ttt_stage_name",
    "ttt_mlp_carry_size", "ttt_mlp_stream_workspace_size", "ttt_mlp_forward_stream",
    "ttt_mlp_forward_stream_ragged",
    "ttt_mlp_backward_workspace_size", "ttt_mlp_backward_batched",
    "ttt_mlp_share_increment", "ttt_mlp_share_forward",
    "ttt_mlp_forward_stream_decode_noalloc",
)

_lib = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as fh:
            return sorted({ln.split()[-1] for ln in fh if "libamdhip64" in ln})
    except OSError:
        return []


def load(path: str | None = None):
    """Load the built library (raises if it is missing; never builds)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run chunk_wise_weight_chunked_amd.build.build()")
    lib = ctypes.CDLL(p)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"more than one HIP runtime mapped: {runtimes}")
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    dp = ctypes.POINTER(ttt_mlp_desc_t)
    lib.ttt_mlp_workspace_size.argtypes = [dp, i64]
    lib.ttt_mlp_workspace_size.restype = sz
    lib.ttt_mlp_group_size.argtypes = [dp, sz]
    lib.ttt_mlp_group_size.restype = i64
    lib.ttt_mlp_forward.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
    lib.ttt_mlp_forward.restype = ctypes.c_int
    lib.ttt_mlp_forward_batched.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
    lib.ttt_mlp_forward_batched.restype = ctypes.c_int
    lib.ttt_mlp_carry_size.argtypes = [dp]
    lib.ttt_mlp_carry_size.restype = sz
    lib.ttt_mlp_stream_workspace_size.argtypes = [dp, i64]
    lib.ttt_mlp_stream_workspace_size.restype = sz
    lib.ttt_mlp_forward_stream.argtypes = [dp, i64, ctypes.c_int32] + [vp] * 11 + [sz, vp]
    lib.ttt_mlp_forward_stream.restype = ctypes.c_int
    lib.ttt_mlp_forward_stream_ragged.argtypes = [dp, vp, vp] + [vp] * 11 + [sz, vp]
    lib.ttt_mlp_forward_stream_ragged.restype = ctypes.c_int
    lib.ttt_mlp_backward_workspace_size.argtypes = [dp]
    lib.ttt_mlp_backward_workspace_size.restype = sz
    lib.ttt_mlp_backward_batched.argtypes = [dp] + [vp] * 18 + [vp, sz, vp]
    lib.ttt_mlp_backward_batched.restype = ctypes.c_int
    lib.ttt_mlp_forward_stream_decode_noalloc.argtypes = [dp, vp, vp] + [vp] * 10 + [vp]
    lib.ttt_mlp_forward_stream_decode_noalloc.restype = ctypes.c_int
    shp = ctypes.POINTER(ttt_share_t)
    lib.ttt_mlp_share_increment.argtypes = [dp, shp] + [vp] * 7 + [vp, sz, vp]
    lib.ttt_mlp_share_increment.restype = ctypes.c_int
    lib.ttt_mlp_share_forward.argtypes = [dp, shp, ctypes.c_int32] + [vp] * 8 + [vp, sz, vp]
    lib.ttt_mlp_share_forward.restype = ctypes.c_int
    lib.ttt_fastweight_state_reset.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp]
    lib.ttt_fastweight_state_reset.restype = ctypes.c_int
    lib.ttt_last_error.restype = ctypes.c_char_p
    lib.ttt_profile_enable.argtypes = [ctypes.c_int]
    lib.ttt_profile_enable.restype = ctypes.c_int
    lib.ttt_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    lib.ttt_profile_read.restype = ctypes.c_int
    lib.ttt_stage_name.argtypes = [ctypes.c_int]
    lib.ttt_stage_name.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def ttt_last_error() -> str:
    return load().ttt_last_error().decode()


def _check(status: int):
    if status != TTT_OK:
        raise TTTError(status, ttt_last_error())


def make_desc(batch, seq_len, d_model, d_ff, chunk, conv_k, eta, dtype, mode="auto",
              init_from_w0=1, target="conv_proj", align="next") -> ttt_mlp_desc_t:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: TTT_F32, torch.bfloat16: TTT_BF16}[dtype]
    if isinstance(mode, str):
        mode = _MODES[mode]
    if isinstance(target, str):
        target = _TARGETS[target]
    if isinstance(align, str):
        align = _ALIGNS[align]
    return ttt_mlp_desc_t(int(batch), int(seq_len), int(d_model), int(d_ff), int(chunk),
                          int(conv_k), float(eta), int(dtype), int(mode), int(init_from_w0),
                          int(target), int(align))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must be device (cuda) tensors")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def ttt_mlp_workspace_size(desc: ttt_mlp_desc_t, max_group: int = 0) -> int:
    n = load().ttt_mlp_workspace_size(ctypes.byref(desc), int(max_group))
    if n == 0:
        raise TTTError(TTT_ERR_INVALID_ARGUMENT, ttt_last_error())
    return int(n)


def ttt_mlp_group_size(desc: ttt_mlp_desc_t, ws_bytes: int) -> int:
    g = load().ttt_mlp_group_size(ctypes.byref(desc), int(ws_bytes))
    if g < 0:
        raise TTTError(int(g), ttt_last_error())
    return int(g)


def ttt_mlp_forward(desc, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O, W_down_final,
                    ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().ttt_mlp_forward(
        ctypes.byref(desc), _ptr(H), _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0),
        _ptr(conv_taps), _ptr(W_target), _ptr(O), _ptr(W_down_final), _ptr(ws), int(ws_bytes),
        _stream(stream)))


def ttt_mlp_forward_batched(desc, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O, W_state,
                            ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().ttt_mlp_forward_batched(
        ctypes.byref(desc), _ptr(H), _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0),
        _ptr(conv_taps), _ptr(W_target), _ptr(O), _ptr(W_state), _ptr(ws), int(ws_bytes),
        _stream(stream)))


def ttt_mlp_carry_size(desc: ttt_mlp_desc_t) -> int:
    n = load().ttt_mlp_carry_size(ctypes.byref(desc))
    if n == 0:
        raise TTTError(TTT_ERR_INVALID_ARGUMENT, ttt_last_error())
    return int(n)


def ttt_mlp_stream_workspace_size(desc: ttt_mlp_desc_t, max_group: int = 0) -> int:
    n = load().ttt_mlp_stream_workspace_size(ctypes.byref(desc), int(max_group))
    if n == 0:
        raise TTTError(TTT_ERR_INVALID_ARGUMENT, ttt_last_error())
    return int(n)


def ttt_mlp_forward_stream(desc, pos, last, H, X0, W_gate, W_up, W_down0, conv_taps, W_target,
                           O, W_state, carry, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().ttt_mlp_forward_stream(
        ctypes.byref(desc), int(pos), int(last), _ptr(H), _ptr(X0), _ptr(W_gate), _ptr(W_up),
        _ptr(W_down0), _ptr(conv_taps), _ptr(W_target), _ptr(O), _ptr(W_state), _ptr(carry),
        _ptr(ws), int(ws_bytes), _stream(stream)))


def make_share(X0_left=None, X0_right=None) -> ttt_share_t:
    """The halo rows of a share: X0_left [B][7][d] (the 7 X0 rows before the
    share) and X0_right [B][d] (the row after it), device tensors or None."""
    return ttt_share_t(_ptr(X0_left), _ptr(X0_right))


def ttt_mlp_share_increment(desc, share, H, X0, W_gate, W_up, conv_taps, W_target, S, ws,
                            ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().ttt_mlp_share_increment(
        ctypes.byref(desc), ctypes.byref(share), _ptr(H), _ptr(X0), _ptr(W_gate), _ptr(W_up),
        _ptr(conv_taps), _ptr(W_target), _ptr(S), _ptr(ws), int(ws_bytes), _stream(stream)))


def ttt_mlp_share_forward(desc, share, reuse, H, X0, W_gate, W_up, conv_taps, W_target, O,
                          W_state, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().ttt_mlp_share_forward(
        ctypes.byref(desc), ctypes.byref(share), int(reuse), _ptr(H), _ptr(X0), _ptr(W_gate),
        _ptr(W_up), _ptr(conv_taps), _ptr(W_target), _ptr(O), _ptr(W_state), _ptr(ws),
        int(ws_bytes), _stream(stream)))


def ttt_fastweight_state_reset(W_state, W_down0, w0_dtype, batch, d_model, d_ff,
                               stream=None) -> None:
    if isinstance(w0_dtype, torch.dtype):
        w0_dtype = {torch.float32: TTT_F32, torch.bfloat16: TTT_BF16}[w0_dtype]
    _check(load().ttt_fastweight_state_reset(_ptr(W_state), _ptr(W_down0), int(w0_dtype),
                                             int(batch), int(d_model), int(d_ff),
                                             _stream(stream)))


def ttt_profile_enable(enable: bool) -> None:
    _check(load().ttt_profile_enable(1 if enable else 0))


def ttt_profile_read() -> dict:
    """Per-stage totals since the last read: {name: (ms, launches)}."""
    ms = (ctypes.c_double * TTT_NUM_STAGES)()
    cnt = (ctypes.c_int64 * TTT_NUM_STAGES)()
    n = load().ttt_profile_read(ms, cnt, TTT_NUM_STAGES)
    if n < 0:
        raise TTTError(n, ttt_last_error())
    return {ttt_stage_name(i): (ms[i], cnt[i]) for i in range(n)}


def ttt_stage_name(i: int) -> str:
    return load().ttt_stage_name(int(i)).decode()


# ---------------------------------------------------------------- conveniences
def alloc_workspace(desc: ttt_mlp_desc_t, max_group: int = 0, device="cuda") -> torch.Tensor:
    n = ttt_mlp_workspace_size(desc, max_group)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _conv_k(conv_taps, conv_k):
    if conv_taps is not None:
        return conv_taps.shape[1]
    return 1 if conv_k is None else conv_k


def forward(H, X0, W_gate, W_up, W_down0, conv_taps, W_target, eta, chunk, mode="auto",
            max_group=0, ws=None, stream=None, target="conv_proj", conv_k=None, align="next"):
    """One sequence: H, X0 [T][d] (or [1][T][d]) device tensors.  Returns
    (O like H, W_down_final [d][f] fp32).  conv_taps / W_target may be None
    when `target` leaves the conv / projection out."""
    T, d = H.shape[-2], H.shape[-1]
    f = W_gate.shape[0]
    desc = make_desc(1, T, d, f, chunk, _conv_k(conv_taps, conv_k), eta, H.dtype, mode,
                     target=target, align=align)
    if ws is None:
        ws = alloc_workspace(desc, max_group, H.device)
    O = torch.empty_like(H)
    W = torch.empty((d, f), dtype=torch.float32, device=H.device)
    ttt_mlp_forward(desc, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O, W, ws,
                    stream=stream)
    return O, W


def forward_batched(H, X0, W_gate, W_up, W_down0, conv_taps, W_target, eta, chunk, W_state=None,
                    mode="auto", max_group=0, ws=None, stream=None, target="conv_proj",
                    conv_k=None, align="next"):
    """B sequences: H, X0 [B][T][d].  If W_state ([B][d][f] fp32) is None it is
    allocated and initialised from W_down0; otherwise it is used (and updated)
    in place as each sequence's starting weight.  Returns (O, W_state)."""
    B, T, d = H.shape
    f = W_gate.shape[0]
    init = W_state is None
    if init:
        W_state = torch.empty((B, d, f), dtype=torch.float32, device=H.device)
    desc = make_desc(B, T, d, f, chunk, _conv_k(conv_taps, conv_k), eta, H.dtype, mode,
                     init_from_w0=1 if init else 0, target=target, align=align)
    if ws is None:
        ws = alloc_workspace(desc, max_group, H.device)
    O = torch.empty_like(H)
    ttt_mlp_forward_batched(desc, H, X0, W_gate, W_up, W_down0 if init else None, conv_taps,
                            W_target, O, W_state, ws, stream=stream)
    return O, W_state


def ttt_mlp_forward_stream_ragged(desc, pos, last, H, X0, W_gate, W_up, W_down0, conv_taps,
                                  W_target, O, W_state, carry, ws, ws_bytes=None,
                                  stream=None) -> None:
    """pos, last: sequences of B ints (each session's position and closing flag)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    B = desc.batch
    if len(pos) != B or len(last) != B:
        raise ValueError(f"pos and last need {B} entries")
    p = (ctypes.c_int64 * B)(*[int(x) for x in pos])
    l_ = (ctypes.c_int32 * B)(*[int(x) for x in last])
    _check(load().ttt_mlp_forward_stream_ragged(
        ctypes.byref(desc), ctypes.cast(p, ctypes.c_void_p), ctypes.cast(l_, ctypes.c_void_p),
        _ptr(H), _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0), _ptr(conv_taps),
        _ptr(W_target), _ptr(O), _ptr(W_state), _ptr(carry), _ptr(ws), int(ws_bytes),
        _stream(stream)))


def ttt_mlp_forward_stream_decode_noalloc(desc, pos, last, H, X0, W_gate, W_up, W_down0,
                                          conv_taps, W_target, O, W_state, carry,
                                          stream=None) -> None:
    """The allocation-free decode call (no workspace); pos, last: B ints."""
    B = desc.batch
    if len(pos) != B or len(last) != B:
        raise ValueError(f"pos and last need {B} entries")
    p = (ctypes.c_int64 * B)(*[int(x) for x in pos])
    l_ = (ctypes.c_int32 * B)(*[int(x) for x in last])
    _check(load().ttt_mlp_forward_stream_decode_noalloc(
        ctypes.byref(desc), ctypes.cast(p, ctypes.c_void_p), ctypes.cast(l_, ctypes.c_void_p),
        _ptr(H), _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0), _ptr(conv_taps),
        _ptr(W_target), _ptr(O), _ptr(W_state), _ptr(carry), _stream(stream)))


def ttt_mlp_backward_workspace_size(desc: ttt_mlp_desc_t) -> int:
    n = load().ttt_mlp_backward_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise TTTError(TTT_ERR_INVALID_ARGUMENT, ttt_last_error())
    return n


def ttt_mlp_backward_batched(desc, H, X0, W_gate, W_up, W_down0, W_start, conv_taps, W_target,
                             dO, dW_final, dH, dX0, dW_gate, dW_up, dW_start, dtaps, dW_target,
                             d_eta, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().ttt_mlp_backward_batched(
        ctypes.byref(desc), *[_ptr(t) for t in (H, X0, W_gate, W_up, W_down0, W_start, conv_taps,
                                                 W_target, dO, dW_final, dH, dX0, dW_gate, dW_up,
                                                 dW_start, dtaps, dW_target, d_eta, ws)],
        int(ws_bytes), _stream(stream)))


def backward_batched(H, X0, W_gate, W_up, W_down0, conv_taps, W_target, eta, chunk, dO,
                     dW_final=None, W_start=None, target="conv_proj", align="next", conv_k=None,
                     ws=None, stream=None) -> dict:
    """Gradients of <dO, O> + <dW_final, W_final> for the layer run on H, X0
    [B][T][d] from W_down0 (or from W_start [B][d][f] fp32 per sequence).
    Returns a dict of device tensors: H, X0 (activation dtype); W_gate, W_up,
    W_start ([B][d][f]), taps, W_target (fp32; None where the target has no
    conv / projection) and eta (a 1-element fp32 tensor)."""
    B, T, d = H.shape
    f = W_gate.shape[0]
    K = _conv_k(conv_taps, conv_k)
    init = W_start is None
    desc = make_desc(B, T, d, f, chunk, K, eta, H.dtype, init_from_w0=1 if init else 0,
                     target=target, align=align)
    if ws is None:
        ws = torch.empty(ttt_mlp_backward_workspace_size(desc), dtype=torch.uint8,
                         device=H.device)
    dev, f32 = H.device, torch.float32
    conv = target in ("conv_proj", "conv")
    proj = target in ("conv_proj", "proj")
    g = {"H": torch.empty_like(H), "X0": torch.empty_like(X0),
         "W_gate": torch.empty((f, d), dtype=f32, device=dev),
         "W_up": torch.empty((f, d), dtype=f32, device=dev),
         "W_start": torch.empty((B, d, f), dtype=f32, device=dev),
         "taps": torch.empty((d, K), dtype=f32, device=dev) if conv else None,
         "W_target": torch.empty((d, d), dtype=f32, device=dev) if proj else None,
         "eta": torch.empty(1, dtype=f32, device=dev)}
    ttt_mlp_backward_batched(desc, H, X0, W_gate, W_up, W_down0 if init else None, W_start,
                             conv_taps, W_target, dO, dW_final, g["H"], g["X0"], g["W_gate"],
                             g["W_up"], g["W_start"], g["taps"], g["W_target"], g["eta"], ws,
                             stream=stream)
    return g


class Stream:
    """B sessions fed over consecutive calls (ttt_mlp_forward_stream): owns the
    fp32 states and the carry.  step(H, X0) takes the next [B][L][d] tokens and
    returns their O; the call with last=True closes the streams, after which
    `state` holds the final weights."""

    def __init__(self, W_gate, W_up, W_down0, conv_taps, W_target, eta, chunk, batch,
                 mode="auto", target="conv_proj", conv_k=None, device="cuda", align="next"):
        self.w = (W_gate, W_up, W_down0, conv_taps, W_target)
        self.eta, self.chunk, self.batch = float(eta), int(chunk), int(batch)
        self.mode, self.target, self.align = mode, target, align
        self.conv_k = _conv_k(conv_taps, conv_k)
        d, f = W_gate.shape[1], W_gate.shape[0]
        self.dtype = W_gate.dtype
        self.state = torch.empty((self.batch, d, f), dtype=torch.float32, device=device)
        desc = self._desc(1)
        self.carry = torch.empty(ttt_mlp_carry_size(desc), dtype=torch.uint8, device=device)
        self.pos = 0
        self.closed = False

    def _desc(self, L):
        d, f = self.w[0].shape[1], self.w[0].shape[0]
        return make_desc(self.batch, L, d, f, self.chunk, self.conv_k, self.eta, self.dtype,
                         self.mode, init_from_w0=1, target=self.target, align=self.align)

    def step(self, H, X0, last=False, stream=None):
        if self.closed:
            raise RuntimeError("stream already closed")
        B, L, d = H.shape
        desc = self._desc(L)
        ws = torch.empty(ttt_mlp_stream_workspace_size(desc), dtype=torch.uint8, device=H.device)
        O = torch.empty_like(H)
        Wg, Wu, W0, taps, Wt = self.w
        ttt_mlp_forward_stream(desc, self.pos, 1 if last else 0, H, X0, Wg, Wu, W0, taps, Wt, O,
                               self.state, self.carry, ws, stream=stream)
        self.pos += L
        self.closed = bool(last)
        return O

