"""MI355X (gfx950) Interdomain Attention token mixer: Python binding of libia.so.

The binding marshals arguments only: every step of the layer runs in the HIP kernels behind
the C ABI declared in ``include/ia.h``.  Functions carry the C names:

    ia_state_init(desc, state, stream=None)
    ia_prefill_workspace_bytes(desc)
    ia_check_lambda(desc, lam_host)
    ia_prefill_fwd(desc, q, k, v, lam, beta, state, o, workspace, stream=None)
    ia_prefill_fwd_strided(desc, q, k, v, lam, beta, state, o, workspace, stream=None)
    ia_prefill_fwd_noalloc(desc, q, k, v, lam, beta, state, o, stream=None)
    ia_decode_step(desc, q_t, k_t, v_t, lam, beta, state, o_t, stream=None)

Tensors are torch tensors on the GPU (PyTorch provides device memory and streams):
q, k [B,N,H,F], v and o [B,N,H,Dv] in float32 or bfloat16; lam, beta [H,M] complex64; a
state is a tuple (U [B,H,M,F], Gamma [B,H,M,Dv], eta [B,H,M]) of complex64 tensors.
``ia_prefill_fwd_strided`` also accepts q, k, v as strided views (feature axis contiguous, q
and k with equal strides), e.g. slices of one fused projection.  ``prefill``, ``decode`` and
``new_state`` are conveniences that allocate the outputs with torch and then call the same
entry points (``prefill`` passes views through the strided entry point).

Importing fails loudly when libia.so has not been built (``python
ssm_sequence_mixer_amd/build.py``): there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libia.so")

IA_F32, IA_BF16 = 0, 1
IA_FLAG_BIDIR = 1
IA_FLAG_NO_DEN = 2
IA_FLAG_IDENTITY_FEATURES = 4
IA_FLAG_SEQUENTIAL_BWD = 8
IA_FLAG_CHUNKED_BWD = 16
STATUS = ["IA_OK", "IA_ERR_NULL", "IA_ERR_SHAPE", "IA_ERR_DTYPE", "IA_ERR_ALIGN",
          "IA_ERR_ALIAS", "IA_ERR_DOMAIN", "IA_ERR_UNSUPPORTED", "IA_ERR_LAUNCH",
          "IA_ERR_WORKSPACE"]


class IADesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int),
                ("F", ctypes.c_int), ("Dv", ctypes.c_int), ("M", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("den_clamp", ctypes.c_float), ("flags", ctypes.c_uint),
                ("chunk", ctypes.c_int)]


class IAState(ctypes.Structure):
    _fields_ = [("U", ctypes.c_void_p), ("Gamma", ctypes.c_void_p), ("eta", ctypes.c_void_p)]


class IABlockParams(ctypes.Structure):
    _fields_ = [("conv_width", ctypes.c_int), ("conv_q", ctypes.c_void_p),
                ("conv_k", ctypes.c_void_p), ("conv_v", ctypes.c_void_p),
                ("rope_base", ctypes.c_float), ("pos0", ctypes.c_int),
                ("norm_gain", ctypes.c_void_p), ("norm_bias", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float)]


class IAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{where}: {name}" + (f" ({detail})" if detail else ""))


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python ssm_sequence_mixer_amd/build.py`")

# One HIP runtime per process: torch ships its own libamdhip64.so.7, so torch is loaded first
# and libia.so's dependency on that soname then binds to the copy already in the process.
# (Loading the system copy as well gives a second runtime that sees no device.)
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_D = ctypes.POINTER(IADesc)
_S = ctypes.POINTER(IAState)
lib.ia_state_init.argtypes = [_D, _S, _P]
lib.ia_state_init.restype = ctypes.c_int
lib.ia_prefill_workspace_bytes.argtypes = [_D]
lib.ia_prefill_workspace_bytes.restype = ctypes.c_size_t
lib.ia_check_lambda.argtypes = [_D, _P, ctypes.POINTER(ctypes.c_int)]
lib.ia_check_lambda.restype = ctypes.c_int
lib.ia_prefill_fwd.argtypes = [_D, _P, _P, _P, _P, _P, _S, _P, _P, ctypes.c_size_t, _P]
lib.ia_prefill_fwd.restype = ctypes.c_int
_STRIDES = (ctypes.c_longlong * 3) * 3
lib.ia_prefill_fwd_strided.argtypes = [_D, _P, _P, _P, ctypes.POINTER(_STRIDES), _P, _P, _S,
                                       _P, _P, ctypes.c_size_t, _P]
lib.ia_prefill_fwd_strided.restype = ctypes.c_int
lib.ia_prefill_fwd_noalloc.argtypes = [_D, _P, _P, _P, _P, _P, _S, _P, _P]
lib.ia_prefill_fwd_noalloc.restype = ctypes.c_int
lib.ia_decode_step.argtypes = [_D, _P, _P, _P, _P, _P, _S, _P, _P]
lib.ia_decode_step.restype = ctypes.c_int
lib.ia_prefill_fwd_profiled.argtypes = [_D, _P, _P, _P, _P, _P, _S, _P, _P, ctypes.c_size_t,
                                        _P, ctypes.POINTER(ctypes.c_void_p),
                                        ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int)]
lib.ia_prefill_fwd_profiled.restype = ctypes.c_int
lib.ia_prefill_bwd_workspace_bytes.argtypes = [_D]
lib.ia_prefill_bwd_workspace_bytes.restype = ctypes.c_size_t
lib.ia_prefill_bwd.argtypes = [_D, _P, _P, _P, _P, _P, _S, _P, _P, _P, _P, _P, _P, _S, _P,
                               ctypes.c_size_t, _P]
lib.ia_prefill_bwd.restype = ctypes.c_int
lib.ia_prefill_readout_workspace_bytes.argtypes = [_D]
lib.ia_prefill_readout_workspace_bytes.restype = ctypes.c_size_t
lib.ia_prefill_fwd_readout.argtypes = [_D, _P, _P, _P, _P, _P, _P, _S, _P, _P, ctypes.c_size_t,
                                       _P]
lib.ia_prefill_fwd_readout.restype = ctypes.c_int
lib.ia_decode_step_readout.argtypes = [_D, _P, _P, _P, _P, _P, _P, _S, _P, _P]
lib.ia_decode_step_readout.restype = ctypes.c_int
lib.ia_prefill_gated_workspace_bytes.argtypes = [_D]
lib.ia_prefill_gated_workspace_bytes.restype = ctypes.c_size_t
lib.ia_prefill_fwd_gated.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _S, _P, _P, ctypes.c_size_t,
                                     _P]
lib.ia_prefill_fwd_gated.restype = ctypes.c_int
lib.ia_decode_step_gated.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _S, _P, _P]
lib.ia_decode_step_gated.restype = ctypes.c_int
lib.ia_block_prologue.argtypes = [_D, ctypes.POINTER(IABlockParams), _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P]
lib.ia_block_prologue.restype = ctypes.c_int
lib.ia_block_gate.argtypes = [_D, _P, _P, _P, _P]
lib.ia_block_gate.restype = ctypes.c_int
lib.ia_block_decode_step.argtypes = [_D, ctypes.POINTER(IABlockParams), _P, _P, _P, _P, _P, _P,
                                     _P, _P, _S, _P, _P]
lib.ia_block_decode_step.restype = ctypes.c_int
lib.ia_status_string.argtypes = [ctypes.c_int]
lib.ia_status_string.restype = ctypes.c_char_p
lib.ia_last_launch_error.argtypes = []
lib.ia_last_launch_error.restype = ctypes.c_char_p

EXPORTS = ("ia_state_init", "ia_prefill_workspace_bytes", "ia_check_lambda", "ia_prefill_fwd",
           "ia_prefill_fwd_strided", "ia_prefill_fwd_noalloc", "ia_prefill_fwd_profiled", "ia_decode_step",
           "ia_prefill_bwd_workspace_bytes", "ia_prefill_bwd", "ia_prefill_readout_workspace_bytes",
           "ia_prefill_fwd_readout", "ia_decode_step_readout", "ia_prefill_gated_workspace_bytes",
           "ia_prefill_fwd_gated", "ia_decode_step_gated", "ia_block_prologue", "ia_block_gate",
           "ia_block_decode_step", "ia_status_string", "ia_last_launch_error")
KIND_NAMES = {0: "fill", 1: "scan", 2: "tables", 3: "summary", 4: "carry", 5: "chunk",
              6: "decode", 7: "bwd_forward", 8: "bwd_reverse", 9: "bwd_reduce", 10: "copy",
              11: "block"}


def make_desc(B, H, N, F, Dv, M, in_dtype=IA_BF16, out_dtype=IA_F32, den_clamp=1e-6,
              bidir=False, chunk=0, no_den=False, identity_features=False,
              bwd_path="auto") -> IADesc:
    """bwd_path: "auto", "chunked" or "sequential", the backward kernels ia_prefill_bwd runs."""
    if bwd_path not in ("auto", "chunked", "sequential"):
        raise ValueError(f"bwd_path {bwd_path!r}")
    flags = ((IA_FLAG_BIDIR if bidir else 0) | (IA_FLAG_NO_DEN if no_den else 0)
             | (IA_FLAG_IDENTITY_FEATURES if identity_features else 0)
             | (IA_FLAG_SEQUENTIAL_BWD if bwd_path == "sequential" else 0)
             | (IA_FLAG_CHUNKED_BWD if bwd_path == "chunked" else 0))
    return IADesc(B, H, N, F, Dv, M, in_dtype, out_dtype, den_clamp, flags, chunk)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)


def _state(state):
    if state is None:
        return None
    for t in state:
        if not t.is_contiguous():
            raise ValueError("state tensors must be contiguous")
    return ctypes.pointer(IAState(*(t.data_ptr() for t in state)))


def _dense(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libia must be contiguous")


def _keep_for(t, stream):
    """Tell torch's caching allocator that `t` (allocated on the current stream) is used by
    work enqueued on `stream`, so its memory is not reused before that work ends."""
    if t is None or stream is None:
        return
    import torch
    if isinstance(stream, torch.cuda.Stream):
        t.record_stream(stream)
    elif stream != torch.cuda.current_stream().cuda_stream:
        raise ValueError("pass a torch.cuda.Stream (or a workspace you keep alive) when "
                         "enqueuing on another stream")


def _check(status, where):
    if status != 0:
        detail = lib.ia_last_launch_error().decode() if status == 8 else ""
        raise IAError(status, where, detail)


def dtype_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return IA_F32
    if dtype == torch.bfloat16:
        return IA_BF16
    raise ValueError(f"unsupported dtype {dtype}")


# ---------------------------------------------------------------- the C entry points

def ia_state_init(desc: IADesc, state, stream=None) -> None:
    _check(lib.ia_state_init(ctypes.byref(desc), _state(state), _stream(stream)),
           "ia_state_init")


def ia_prefill_workspace_bytes(desc: IADesc) -> int:
    return int(lib.ia_prefill_workspace_bytes(ctypes.byref(desc)))


def ia_check_lambda(desc: IADesc, lam_host) -> int:
    """lam_host: numpy complex64 [H, M] in host memory.  Raises on IA_ERR_DOMAIN; returns the
    number of heads the chunked bf16 prefill runs on its fp32 route."""
    import numpy as np
    arr = np.ascontiguousarray(lam_host, dtype=np.complex64)
    n = ctypes.c_int(-1)
    _check(lib.ia_check_lambda(ctypes.byref(desc), arr.ctypes.data_as(ctypes.c_void_p),
                               ctypes.byref(n)), "ia_check_lambda")
    return n.value


def ia_prefill_fwd(desc: IADesc, q, k, v, lam, beta, state, o, workspace, stream=None):
    _dense(q, k, v, lam, beta, o, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ia_prefill_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                              _ptr(beta), _state(state), _ptr(o), _ptr(workspace), ws_bytes,
                              _stream(stream)), "ia_prefill_fwd")


def ia_prefill_fwd_strided(desc: IADesc, q, k, v, lam, beta, state, o, workspace, stream=None):
    """ia_prefill_fwd for q, k, v of any element strides along (b, n, h) with the last axis
    contiguous (the strides are the tensors' own); the other tensors dense."""
    _dense(lam, beta, o, workspace)
    st = _STRIDES()
    for i, t in enumerate((q, k, v)):
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("q, k, v need 4 axes with the last one contiguous")
        for j in range(3):
            st[i][j] = t.stride(j)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ia_prefill_fwd_strided(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                      ctypes.byref(st), _ptr(lam), _ptr(beta), _state(state),
                                      _ptr(o), _ptr(workspace), ws_bytes, _stream(stream)),
           "ia_prefill_fwd_strided")


NOALLOC_SCRATCH_BYTES = 32 << 20


def ia_prefill_fwd_noalloc(desc: IADesc, q, k, v, lam, beta, state, o, stream=None):
    """ia_prefill_fwd with the library's own fixed workspace (no workspace argument, nothing
    allocated)."""
    _dense(q, k, v, lam, beta, o)
    _check(lib.ia_prefill_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                      _ptr(beta), _state(state), _ptr(o), _stream(stream)),
           "ia_prefill_fwd_noalloc")


def ia_prefill_fwd_profiled(desc: IADesc, q, k, v, lam, beta, state, o, workspace, events,
                            stream=None):
    """As ia_prefill_fwd; `events` is a list of 2*n raw hipEvent_t handles.  Returns the kind
    codes of the launches recorded (events[2i], events[2i+1] bracket launch i)."""
    _dense(q, k, v, lam, beta, o, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    n = len(events) // 2
    ev = (ctypes.c_void_p * (2 * n))(*events)
    kinds = (ctypes.c_int * max(n, 1))()
    used = ctypes.c_int(0)
    _check(lib.ia_prefill_fwd_profiled(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                       _ptr(beta), _state(state), _ptr(o), _ptr(workspace),
                                       ws_bytes, _stream(stream), ev, kinds, n,
                                       ctypes.byref(used)), "ia_prefill_fwd_profiled")
    return [kinds[i] for i in range(used.value)]


def ia_prefill_bwd_workspace_bytes(desc: IADesc) -> int:
    return int(lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(desc)))


def ia_prefill_bwd(desc: IADesc, q, k, v, lam, beta, state0, dO, dq, dk, dv, dlam, dbeta,
                   dstate0, workspace, stream=None):
    _dense(q, k, v, lam, beta, dO, dq, dk, dv, dlam, dbeta, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ia_prefill_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                              _ptr(beta), _state(state0), _ptr(dO), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(dlam), _ptr(dbeta), _state(dstate0),
                              _ptr(workspace), ws_bytes, _stream(stream)), "ia_prefill_bwd")


def ia_prefill_readout_workspace_bytes(desc: IADesc) -> int:
    return int(lib.ia_prefill_readout_workspace_bytes(ctypes.byref(desc)))


def ia_prefill_fwd_readout(desc: IADesc, q, k, v, lam, beta, readout, state, o, workspace,
                           stream=None):
    _dense(q, k, v, lam, beta, readout, o, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ia_prefill_fwd_readout(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                      _ptr(beta), _ptr(readout), _state(state), _ptr(o),
                                      _ptr(workspace), ws_bytes, _stream(stream)),
           "ia_prefill_fwd_readout")


def ia_decode_step_readout(desc: IADesc, q_t, k_t, v_t, lam, beta, readout, state, o_t,
                           stream=None):
    _dense(q_t, k_t, v_t, lam, beta, readout, o_t)
    _check(lib.ia_decode_step_readout(ctypes.byref(desc), _ptr(q_t), _ptr(k_t), _ptr(v_t),
                                      _ptr(lam), _ptr(beta), _ptr(readout), _state(state),
                                      _ptr(o_t), _stream(stream)), "ia_decode_step_readout")


def ia_prefill_gated_workspace_bytes(desc: IADesc) -> int:
    return int(lib.ia_prefill_gated_workspace_bytes(ctypes.byref(desc)))


def ia_prefill_fwd_gated(desc: IADesc, q, k, v, wgate, dgate, lam, beta, state, o, workspace,
                         stream=None):
    _dense(q, k, v, wgate, dgate, lam, beta, o, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ia_prefill_fwd_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(wgate),
                                    _ptr(dgate), _ptr(lam), _ptr(beta), _state(state), _ptr(o),
                                    _ptr(workspace), ws_bytes, _stream(stream)),
           "ia_prefill_fwd_gated")


def ia_decode_step_gated(desc: IADesc, q_t, k_t, v_t, wgate, dgate, lam, beta, state, o_t,
                         stream=None):
    _dense(q_t, k_t, v_t, wgate, dgate, lam, beta, o_t)
    _check(lib.ia_decode_step_gated(ctypes.byref(desc), _ptr(q_t), _ptr(k_t), _ptr(v_t),
                                    _ptr(wgate), _ptr(dgate), _ptr(lam), _ptr(beta),
                                    _state(state), _ptr(o_t), _stream(stream)),
           "ia_decode_step_gated")


def ia_decode_step(desc: IADesc, q_t, k_t, v_t, lam, beta, state, o_t, stream=None):
    _dense(q_t, k_t, v_t, lam, beta, o_t)
    _check(lib.ia_decode_step(ctypes.byref(desc), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(lam),
                              _ptr(beta), _state(state), _ptr(o_t), _stream(stream)),
           "ia_decode_step")


def block_params(conv=None, rope_base=0.0, pos0=0, norm=None, eps=1e-6) -> IABlockParams:
    """conv: (wq [H,F,W], wk [H,F,W], wv [H,Dv,W]) float32 device tensors or None; norm:
    (gain [H,F+Dv], bias [H,F+Dv]) float32 device tensors or None.  The structure holds their
    addresses only: the caller keeps the tensors alive while it is in use."""
    if conv is not None:
        _dense(*conv)
    if norm is not None:
        _dense(*norm)
    W = 0 if conv is None else int(conv[0].shape[2])
    return IABlockParams(W, *(None if conv is None else c.data_ptr() for c in
                              (conv or (None,) * 3)), float(rope_base), int(pos0),
                         *(None if norm is None else t.data_ptr() for t in (norm or (None,) * 2)),
                         float(eps))


def ia_block_prologue(desc: IADesc, params: IABlockParams, q, k, v, state_in, state_out, fq, fk,
                      vo, stream=None):
    _dense(q, k, v, state_in, state_out, fq, fk, vo)
    _check(lib.ia_block_prologue(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(state_in), _ptr(state_out), _ptr(fq), _ptr(fk),
                                 _ptr(vo), _stream(stream)), "ia_block_prologue")


def ia_block_gate(desc: IADesc, o, gate, out, stream=None):
    _dense(o, gate, out)
    _check(lib.ia_block_gate(ctypes.byref(desc), _ptr(o), _ptr(gate), _ptr(out),
                             _stream(stream)), "ia_block_gate")


def ia_block_decode_step(desc: IADesc, params: IABlockParams, q_t, k_t, v_t, state_in,
                         state_out, gate_t, lam, beta, state, out_t, stream=None):
    _dense(q_t, k_t, v_t, state_in, state_out, gate_t, lam, beta, out_t)
    _check(lib.ia_block_decode_step(ctypes.byref(desc), ctypes.byref(params), _ptr(q_t),
                                    _ptr(k_t), _ptr(v_t), _ptr(state_in), _ptr(state_out),
                                    _ptr(gate_t), _ptr(lam), _ptr(beta), _state(state),
                                    _ptr(out_t), _stream(stream)), "ia_block_decode_step")


# ---------------------------------------------------------------- conveniences (torch alloc)

def new_state(B, H, M, F, Dv, device="cuda", stream=None, zero=True):
    import torch
    st = (torch.empty((B, H, M, F), dtype=torch.complex64, device=device),
          torch.empty((B, H, M, Dv), dtype=torch.complex64, device=device),
          torch.empty((B, H, M), dtype=torch.complex64, device=device))
    if zero:
        ia_state_init(make_desc(B, H, 1, F, Dv, M), st, stream)
    return st


def prefill(q, k, v, lam, beta, state=None, out_dtype=None, bidir=False, chunk=0,
            den_clamp=1e-6, want_output=True, stream=None, workspace=None, no_den=False,
            identity_features=False, readout=None, gates=None):
    """Allocate o (and the workspace) with torch and run ia_prefill_fwd (or, for strided
    views q, k, v, ia_prefill_fwd_strided; with gates=(wgate, dgate) [B,N,H] float32,
    ia_prefill_fwd_gated); returns o."""
    import torch
    B, N, H, F = q.shape
    Dv, M = v.shape[3], lam.shape[1]
    out_dtype = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, N, F, Dv, M, dtype_code(q.dtype), dtype_code(out_dtype), den_clamp,
                     bidir, chunk, no_den, identity_features)
    o = torch.empty((B, N, H, Dv), dtype=out_dtype, device=q.device) if want_output else None
    if gates is not None:
        own_ws = workspace is None
        if own_ws:
            nb = ia_prefill_gated_workspace_bytes(desc)
            workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
        ia_prefill_fwd_gated(desc, q, k, v, gates[0], gates[1], lam, beta, state, o, workspace,
                             stream)
        if own_ws:
            _keep_for(workspace, stream)
        return o
    if readout is not None:
        own_ws = workspace is None
        if own_ws:
            nb = ia_prefill_readout_workspace_bytes(desc)
            workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
        ia_prefill_fwd_readout(desc, q, k, v, lam, beta, readout, state, o, workspace, stream)
        if own_ws:
            _keep_for(workspace, stream)
        return o
    own_ws = workspace is None
    if own_ws:
        nb = ia_prefill_workspace_bytes(desc)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device) if nb else None
    if all(t.is_contiguous() for t in (q, k, v)):
        ia_prefill_fwd(desc, q, k, v, lam, beta, state, o, workspace, stream)
    else:
        ia_prefill_fwd_strided(desc, q, k, v, lam, beta, state, o, workspace, stream)
    if own_ws:
        _keep_for(workspace, stream)
    return o


def decode(q_t, k_t, v_t, lam, beta, state, out_dtype=None,
           den_clamp=1e-6, stream=None, o_t=None, no_den=False, identity_features=False,
           readout=None, gates=None):
    """One decode step for every (b,h) (with gates=(wgate, dgate) [B,H] float32,
    ia_decode_step_gated); allocates o_t unless given; returns o_t."""
    import torch
    B, H, F = q_t.shape
    Dv, M = v_t.shape[2], lam.shape[1]
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    desc = make_desc(B, H, 1, F, Dv, M, dtype_code(q_t.dtype), dtype_code(out_dtype), den_clamp,
                     no_den=no_den, identity_features=identity_features)
    if o_t is None:
        o_t = torch.empty((B, H, Dv), dtype=out_dtype, device=q_t.device)
    if gates is not None:
        ia_decode_step_gated(desc, q_t, k_t, v_t, gates[0], gates[1], lam, beta, state, o_t,
                             stream)
    elif readout is not None:
        ia_decode_step_readout(desc, q_t, k_t, v_t, lam, beta, readout, state, o_t, stream)
    else:
        ia_decode_step(desc, q_t, k_t, v_t, lam, beta, state, o_t, stream)
    return o_t


def block_prologue(q, k, v, conv=None, state=None, rope_base=0.0, pos0=0, norm=None, eps=1e-6,
                   M=16, stream=None):
    """Run ia_block_prologue on raw q, k [B,N,H,F], v [B,N,H,Dv] (bf16 or float32); returns
    (phi(q'), phi(k') and v' after the normalisation, the new convolution state or None), the
    inputs of the layer with identity_features=True.  state: [B,H,W-1,2F+Dv] float32."""
    import torch
    B, N, H, F = q.shape
    Dv = v.shape[3]
    desc = make_desc(B, H, N, F, Dv, M, dtype_code(q.dtype), dtype_code(q.dtype))
    p = block_params(conv, rope_base, pos0, norm, eps)
    fq, fk, vo = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st_out = None
    if conv is not None and p.conv_width > 1:
        st_out = torch.empty((B, H, p.conv_width - 1, 2 * F + Dv), dtype=torch.float32,
                             device=q.device)
    ia_block_prologue(desc, p, q, k, v, state, st_out, fq, fk, vo, stream)
    return fq, fk, vo, st_out


def block_gate(o, gate, out=None, stream=None):
    """out = o * SiLU(gate) (ia_block_gate); o, gate [B,N,H,Dv] (or [B,H,Dv]) of one dtype."""
    import torch
    if o.dim() == 3:
        B, H, Dv = o.shape
        N = 1
    else:
        B, N, H, Dv = o.shape
    desc = make_desc(B, H, N, 16, Dv, 16, dtype_code(o.dtype), dtype_code(o.dtype))
    out = torch.empty_like(o) if out is None else out
    ia_block_gate(desc, o, gate, out, stream)
    return out


def prefill_bwd(q, k, v, lam, beta, dO, state0=None, den_clamp=1e-6, no_den=False,
                identity_features=False, want_state_grad=False, stream=None, workspace=None,
                bidir=False, path="auto"):
    """Gradients of the layer (causal, or bidirectional with bidir=True) for dL/do = dO:
    allocates the outputs (and the workspace) with torch and runs ia_prefill_bwd (path:
    "auto", "chunked" or "sequential", its kernels).  Returns (dq, dk, dv, dlam, dbeta,
    dstate0 or None)."""
    import torch
    B, N, H, F = q.shape
    Dv, M = v.shape[3], lam.shape[1]
    desc = make_desc(B, H, N, F, Dv, M, dtype_code(q.dtype), dtype_code(dO.dtype), den_clamp,
                     bidir=bidir, no_den=no_den, identity_features=identity_features,
                     bwd_path=path)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dlam = torch.empty((H, M), dtype=torch.complex64, device=q.device)
    dbeta = torch.empty_like(dlam)
    dst = new_state(B, H, M, F, Dv, device=q.device, zero=False) if want_state_grad else None
    own_ws = workspace is None
    if own_ws:
        workspace = torch.empty(max(ia_prefill_bwd_workspace_bytes(desc), 16), dtype=torch.uint8,
                                device=q.device)
    ia_prefill_bwd(desc, q, k, v, lam, beta, state0, dO, dq, dk, dv, dlam, dbeta, dst, workspace,
                   stream)
    if own_ws:
        _keep_for(workspace, stream)
    return dq, dk, dv, dlam, dbeta, dst
