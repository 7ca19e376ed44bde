"""ctypes binding of libtitans_mem.so (include/titans_mem.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs/workspace are allocated with torch when the caller does
not pass them, and the C entry points run on torch's current HIP stream.
Every step of the memory's computation happens in the library's kernels;
there is no Python or CPU fallback -- a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

ABI_VERSION = 1
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_ALIAS, ERR_HIP, ERR_GAVE_UP = 0, -1, -2, -3, -4, -5, -6
IO_F32, IO_BF16 = 0, 1
ACT_SILU = 0
READ_AFTER_WRITE, READ_CHUNK_START = 0, 1
FLAG_FORCE_GENERIC = 1
FLAG_CHUNK_GATES = 2
FLAG_NO_WAIT = 4
PATH_GENERIC_F32, PATH_MLP2_D64_H256, PATH_DEEP_BF16 = 0, 1, 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtitans_mem.so")

EXPORTS = ("titans_mem_abi_version", "titans_mem_param_count", "titans_mem_select_path",
           "titans_mem_workspace_bytes", "titans_mem_forward", "titans_mem_forward_noalloc",
           "titans_mem_workspace_status", "titans_mem_retrieve",
           "titans_mem_input", "titans_mem_backward", "titans_mem_backward_workspace_bytes",
           "titans_mem_status_string")


class Desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("read_mode", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class InputDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("B", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("flags", ctypes.c_uint32)]


def make_input_desc(B: int, N: int, D: int, H: int, d: int, conv_width: int = 4, flags: int = 0) -> InputDesc:
    return InputDesc(ABI_VERSION, B, N, D, H, d, conv_width, flags)


def make_desc(B: int, H: int, N: int, d: int, hidden: int, n_layers: int, io: str = "bf16",
              read_mode: int = READ_AFTER_WRITE, flags: int = 0) -> Desc:
    return Desc(ABI_VERSION, B, H, N, d, hidden if n_layers >= 2 else 0, n_layers, ACT_SILU,
                IO_BF16 if io == "bf16" else IO_F32, read_mode, flags)


_lib = None


class TitansMemError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m test_learned_neural_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i32, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    dp = ctypes.POINTER(Desc)
    lib.titans_mem_abi_version.restype = i32
    lib.titans_mem_abi_version.argtypes = []
    lib.titans_mem_param_count.restype = i64
    lib.titans_mem_param_count.argtypes = [dp]
    lib.titans_mem_select_path.restype = i32
    lib.titans_mem_select_path.argtypes = [dp, i32]
    lib.titans_mem_workspace_bytes.restype = i64
    lib.titans_mem_workspace_bytes.argtypes = [dp, i32]
    lib.titans_mem_forward.restype = ctypes.c_int
    lib.titans_mem_forward.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, i32, vp, fp, fp, vp, i64, vp]
    lib.titans_mem_forward_noalloc.restype = ctypes.c_int
    lib.titans_mem_forward_noalloc.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, i32, vp, fp, fp, vp]
    lib.titans_mem_workspace_status.restype = ctypes.c_int
    lib.titans_mem_workspace_status.argtypes = [dp, i32, vp, i64, vp]
    lib.titans_mem_retrieve.restype = ctypes.c_int
    lib.titans_mem_retrieve.argtypes = [dp, vp, fp, vp, vp]
    lib.titans_mem_backward_workspace_bytes.restype = i64
    lib.titans_mem_backward_workspace_bytes.argtypes = [dp, i32]
    lib.titans_mem_backward.restype = ctypes.c_int
    lib.titans_mem_backward.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, i32, fp, fp, fp,
                                        fp, fp, fp, fp, fp, fp, fp, fp, vp, i64, vp]
    lib.titans_mem_input.restype = ctypes.c_int
    lib.titans_mem_input.argtypes = [ctypes.POINTER(InputDesc), vp, vp, fp, vp, fp, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_float, vp, vp, vp, fp, fp, fp, vp]
    lib.titans_mem_status_string.restype = ctypes.c_char_p
    lib.titans_mem_status_string.argtypes = [ctypes.c_int]
    if lib.titans_mem_abi_version() != ABI_VERSION:
        raise ImportError("libtitans_mem.so ABI version mismatch")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().titans_mem_status_string(int(status)).decode()


def param_count(desc: Desc) -> int:
    return int(load().titans_mem_param_count(ctypes.byref(desc)))


def select_path(desc: Desc, chunk: int) -> int:
    return int(load().titans_mem_select_path(ctypes.byref(desc), int(chunk)))


def workspace_bytes(desc: Desc, chunk: int) -> int:
    return int(load().titans_mem_workspace_bytes(ctypes.byref(desc), int(chunk)))


def raw_forward(desc: Desc, k, v, q, alpha, eta, theta, W_in, S_in, chunk, y_out, W_out, S_out,
                workspace, workspace_bytes_, stream) -> int:
    """Direct call with integer device addresses (0 for NULL); returns the status."""
    return int(load().titans_mem_forward(ctypes.byref(desc), k, v, q, alpha, eta, theta, W_in, S_in,
                                         int(chunk), y_out, W_out, S_out, workspace,
                                         int(workspace_bytes_), stream))


def raw_forward_noalloc(desc: Desc, k, v, q, alpha, eta, theta, W_in, S_in, chunk, y_out, W_out, S_out,
                        stream) -> int:
    """titans_mem_forward_noalloc with integer device addresses; returns the status."""
    return int(load().titans_mem_forward_noalloc(ctypes.byref(desc), k, v, q, alpha, eta, theta, W_in, S_in,
                                                 int(chunk), y_out, W_out, S_out, stream))


def raw_workspace_status(desc: Desc, chunk: int, workspace, workspace_bytes_, stream) -> int:
    """titans_mem_workspace_status with an integer device address; returns the status."""
    return int(load().titans_mem_workspace_status(ctypes.byref(desc), int(chunk), workspace,
                                                  int(workspace_bytes_), stream))


def backward_workspace_bytes(desc: Desc, chunk: int) -> int:
    return int(load().titans_mem_backward_workspace_bytes(ctypes.byref(desc), int(chunk)))


def raw_backward(desc: Desc, k, v, q, alpha, eta, theta, W_in, S_in, chunk, dy, dW_out, dS_out, dk, dv, dq,
                 dalpha, deta, dtheta, dW_in, dS_in, workspace, workspace_bytes_, stream) -> int:
    """Direct call of titans_mem_backward with integer device addresses; returns the status."""
    return int(load().titans_mem_backward(ctypes.byref(desc), k, v, q, alpha, eta, theta, W_in, S_in, int(chunk),
                                          dy, dW_out, dS_out, dk, dv, dq, dalpha, deta, dtheta, dW_in, dS_in,
                                          workspace, int(workspace_bytes_), stream))


def raw_input(desc: InputDesc, x, w_proj, conv_w, w_gate, b_gate, scales, k_out, v_out, q_out, alpha_out,
              eta_out, theta_out, stream) -> int:
    """Direct call of titans_mem_input with integer device addresses; returns the status."""
    return int(load().titans_mem_input(ctypes.byref(desc), x, w_proj, conv_w, w_gate, b_gate, float(scales[0]),
                                       float(scales[1]), float(scales[2]), k_out, v_out, q_out, alpha_out,
                                       eta_out, theta_out, stream))


# ----------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def forward(k, v, q, alpha, eta, theta, W_in, S_in, chunk: int, *, hidden: int, n_layers: int,
            read_mode: int = READ_AFTER_WRITE, force_generic: bool = False, chunk_gates: bool = False,
            y_out=None, W_out=None, S_out=None, workspace=None, flags: int = 0) -> Tuple:
    """Run titans_mem_forward on torch tensors.

    k, v, q: [B, H, N, d] (float32 or bfloat16); alpha, eta, theta: [B, H, N]
    float32 ([B, H, ceil(N / chunk)] with chunk_gates: one value per chunk);
    W_in, S_in: [B, H, P] float32.  Returns (y, W_out, S_out).
    """
    torch = _torch()
    B, H, N, d = k.shape
    io = "bf16" if k.dtype == torch.bfloat16 else "f32"
    desc = make_desc(B, H, N, d, hidden, n_layers, io, read_mode,
                     (FLAG_FORCE_GENERIC if force_generic else 0) | (FLAG_CHUNK_GATES if chunk_gates else 0) | flags)
    P = param_count(desc)
    if P < 0:
        raise TitansMemError(P, "titans_mem_param_count")
    dev = k.device
    for name, t in (("k", k), ("v", v), ("q", q)):
        _check(t, name, (B, H, N, d), k.dtype, dev)
    n_gates = (N + chunk - 1) // chunk if chunk_gates and chunk > 0 else N
    for name, t in (("alpha", alpha), ("eta", eta), ("theta", theta)):
        _check(t, name, (B, H, n_gates), torch.float32, dev)
    for name, t in (("W_in", W_in), ("S_in", S_in)):
        _check(t, name, (B, H, P), torch.float32, dev)
    if y_out is None:
        y_out = torch.empty((B, H, N, d), dtype=k.dtype, device=dev)
    if W_out is None:
        W_out = torch.empty((B, H, P), dtype=torch.float32, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, P), dtype=torch.float32, device=dev)
    _check(y_out, "y_out", (B, H, N, d), k.dtype, dev)
    _check(W_out, "W_out", (B, H, P), torch.float32, dev)
    _check(S_out, "S_out", (B, H, P), torch.float32, dev)
    need = workspace_bytes(desc, chunk)
    if need < 0:
        raise TitansMemError(need, "titans_mem_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = raw_forward(desc, _ptr(k), _ptr(v), _ptr(q), _ptr(alpha), _ptr(eta), _ptr(theta),
                     _ptr(W_in), _ptr(S_in), chunk, _ptr(y_out), _ptr(W_out), _ptr(S_out),
                     _ptr(workspace), ws_bytes, stream)
    if rc != OK:
        raise TitansMemError(rc, "titans_mem_forward")
    return y_out, W_out, S_out


def workspace_status(k, chunk: int, workspace, *, hidden: int, n_layers: int, read_mode: int = READ_AFTER_WRITE,
                     force_generic: bool = False, chunk_gates: bool = False, flags: int = 0) -> int:
    """Outcome of the last forward() call that used ``workspace`` (same shape
    as ``k`` and the same options): waits for torch's current stream and
    returns OK or ERR_GAVE_UP."""
    torch = _torch()
    B, H, N, d = k.shape
    io = "bf16" if k.dtype == torch.bfloat16 else "f32"
    desc = make_desc(B, H, N, d, hidden, n_layers, io, read_mode,
                     (FLAG_FORCE_GENERIC if force_generic else 0) | (FLAG_CHUNK_GATES if chunk_gates else 0) | flags)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = raw_workspace_status(desc, chunk, _ptr(workspace), ws_bytes, torch.cuda.current_stream(k.device).cuda_stream)
    if rc not in (OK, ERR_GAVE_UP):
        raise TitansMemError(rc, "titans_mem_workspace_status")
    return rc


def retrieve(q, W, *, hidden: int, n_layers: int, y_out=None, force_generic: bool = False):
    """y = M*_W(q) at a fixed state.  q: [B,H,N,d]; W: [B,H,P] float32."""
    torch = _torch()
    B, H, N, d = q.shape
    io = "bf16" if q.dtype == torch.bfloat16 else "f32"
    desc = make_desc(B, H, N, d, hidden, n_layers, io, flags=FLAG_FORCE_GENERIC if force_generic else 0)
    P = param_count(desc)
    if P < 0:
        raise TitansMemError(P, "titans_mem_param_count")
    _check(q, "q", (B, H, N, d), q.dtype, q.device)
    _check(W, "W", (B, H, P), torch.float32, q.device)
    if y_out is None:
        y_out = torch.empty_like(q)
    _check(y_out, "y_out", (B, H, N, d), q.dtype, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = int(load().titans_mem_retrieve(ctypes.byref(desc), _ptr(q), _ptr(W), _ptr(y_out), stream))
    if rc != OK:
        raise TitansMemError(rc, "titans_mem_retrieve")
    return y_out


def input_side(x, w_proj, conv_w, w_gate, b_gate, gate_scale, *, H: int, d: int, out=None):
    """x -> (k, v, q, alpha, eta, theta) through titans_mem_input.

    x: [B, N, D] bfloat16; w_proj: [3, H*d, D] bfloat16; conv_w: [3, H*d, w]
    float32; w_gate: [3, H, D] bfloat16; b_gate: [3, H] float32; gate_scale:
    three floats.  Returns k, v, q as [B, H, N, d] bfloat16 and the gates as
    [B, H, N] float32 (``out`` may supply the six output tensors).
    """
    torch = _torch()
    B, N, D = x.shape
    C = H * d
    w = conv_w.shape[-1]
    dev = x.device
    _check(x, "x", (B, N, D), torch.bfloat16, dev)
    _check(w_proj, "w_proj", (3, C, D), torch.bfloat16, dev)
    _check(conv_w, "conv_w", (3, C, w), torch.float32, dev)
    _check(w_gate, "w_gate", (3, H, D), torch.bfloat16, dev)
    _check(b_gate, "b_gate", (3, H), torch.float32, dev)
    if out is None:
        out = tuple(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) for _ in range(3)) + \
              tuple(torch.empty((B, H, N), dtype=torch.float32, device=dev) for _ in range(3))
    for i, t in enumerate(out):
        _check(t, ("k", "v", "q", "alpha", "eta", "theta")[i], (B, H, N, d) if i < 3 else (B, H, N),
               torch.bfloat16 if i < 3 else torch.float32, dev)
    desc = make_input_desc(B, N, D, H, d, w)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = raw_input(desc, _ptr(x), _ptr(w_proj), _ptr(conv_w), _ptr(w_gate), _ptr(b_gate), gate_scale,
                   *[_ptr(t) for t in out], stream)
    if rc != OK:
        raise TitansMemError(rc, "titans_mem_input")
    return out


def backward(k, v, q, alpha, eta, theta, W_in, S_in, chunk: int, *, hidden: int, n_layers: int,
             dy=None, dW_out=None, dS_out=None, read_mode: int = READ_AFTER_WRITE, chunk_gates: bool = False):
    """Gradients through titans_mem_forward (titans_mem_backward).

    Same inputs as forward(); dy [B,H,N,d], dW_out / dS_out [B,H,P] are
    float32 adjoints of the outputs (None = zero).  Returns a dict of
    float32 tensors: k, v, q [B,H,N,d]; alpha, eta, theta (the gates'
    shape); W_in, S_in [B,H,P].
    """
    torch = _torch()
    B, H, N, d = k.shape
    io = "bf16" if k.dtype == torch.bfloat16 else "f32"
    desc = make_desc(B, H, N, d, hidden, n_layers, io, read_mode, FLAG_CHUNK_GATES if chunk_gates else 0)
    P = param_count(desc)
    if P < 0:
        raise TitansMemError(P, "titans_mem_param_count")
    dev = k.device
    for name, t in (("k", k), ("v", v), ("q", q)):
        _check(t, name, (B, H, N, d), k.dtype, dev)
    n_gates = (N + chunk - 1) // chunk if chunk_gates and chunk > 0 else N
    for name, t in (("alpha", alpha), ("eta", eta), ("theta", theta)):
        _check(t, name, (B, H, n_gates), torch.float32, dev)
    for name, t in (("W_in", W_in), ("S_in", S_in)):
        _check(t, name, (B, H, P), torch.float32, dev)
    if dy is not None:
        _check(dy, "dy", (B, H, N, d), torch.float32, dev)
    for name, t in (("dW_out", dW_out), ("dS_out", dS_out)):
        if t is not None:
            _check(t, name, (B, H, P), torch.float32, dev)
    g = {n: torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for n in ("k", "v", "q")}
    g.update({n: torch.empty((B, H, n_gates), dtype=torch.float32, device=dev) for n in ("alpha", "eta", "theta")})
    g.update({n: torch.empty((B, H, P), dtype=torch.float32, device=dev) for n in ("W_in", "S_in")})
    need = backward_workspace_bytes(desc, chunk)
    if need < 0:
        raise TitansMemError(need, "titans_mem_backward_workspace_bytes")
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = raw_backward(desc, _ptr(k), _ptr(v), _ptr(q), _ptr(alpha), _ptr(eta), _ptr(theta), _ptr(W_in), _ptr(S_in),
                      chunk, _ptr(dy), _ptr(dW_out), _ptr(dS_out), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["q"]),
                      _ptr(g["alpha"]), _ptr(g["eta"]), _ptr(g["theta"]), _ptr(g["W_in"]), _ptr(g["S_in"]),
                      _ptr(ws), need, stream)
    if rc != OK:
        raise TitansMemError(rc, "titans_mem_backward")
    return g
