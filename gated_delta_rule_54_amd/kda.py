"""Python binding of the KDA C ABI (include/kda.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the operator runs in the HIP kernels of
libkda.so.  There is no fallback: if the library cannot be loaded, every
call raises.

    o, final_state, ckpt = kda_chunk_fwd(q, k, v, g, beta, init_state, cu_seqlens)
    o = kda_decode_step(q, k, v, g, beta, state)      # state updated in place
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_HIP = 4
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

# Names every build of the library must export (the declarations of kda.h).
EXPORTED = ("kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_chunk_fwd_noalloc",
            "kda_chunk_fwd_conv",
            "kda_chunk_bwd_workspace_bytes",
            "kda_chunk_bwd", "kda_decode_step",
            "kda_output_gate_norm", "kda_short_conv_swish", "kda_status_string",
            "kda_last_error", "kda_abi_version")


class KdaDesc(ctypes.Structure):
    """Mirror of kda_desc_t."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("seqlen", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("qk_l2norm", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("gate_per_head", ctypes.c_int32),
        ("ckpt_every", ctypes.c_int64),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: Optional[str] = None):
    """Load libkda.so (raises if it is missing; there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"KDA HIP library not built: {p} is missing "
                          "(run `python -m gated_delta_rule_54_amd.build`)")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(KdaDesc)
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [dp]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_chunk_fwd_conv.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, sz, vp]
    lib.kda_chunk_fwd_conv.restype = i32
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [dp]
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd.argtypes = [dp] + [vp] * 17 + [sz, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_decode_step.restype = i32
    lib.kda_output_gate_norm.argtypes = [ctypes.c_int64, i32, i32, vp, vp, vp, ctypes.c_float,
                                         vp, vp]
    lib.kda_output_gate_norm.restype = i32
    lib.kda_short_conv_swish.argtypes = [i32, ctypes.c_int64, i32, i32, i32, i32, vp, vp, vp, vp,
                                         vp, vp, vp, vp]
    lib.kda_short_conv_swish.restype = i32
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int, what: str):
    if status != KDA_OK:
        name = lib.kda_status_string(status).decode()
        raise KdaError(status, f"{what}: {name}: {lib.kda_last_error().decode()}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_DTYPE_F32
    if t == torch.bfloat16:
        return KDA_DTYPE_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _on(stream):
    """Allocation context for a call launched on `stream`: tensors the
    binding allocates (outputs, workspace) come from that stream's pool, so
    the caching allocator hands a freed block (the workspace, once the call
    returns) only to later work on the same stream, which the stream orders
    after the kernels that still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _stream_scoped(fn):
    """Run a binding call with its allocations on the call's stream (_on)."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kwargs):
        with _on(stream):
            return fn(*args, stream=stream, **kwargs)
    return wrapped


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def make_desc(*, batch, num_seqs, seqlen, heads, dk, dv, dtype, qk_l2norm=True, scale=1.0,
              ckpt_every=0, chunk=64, gate_per_head=False) -> KdaDesc:
    return KdaDesc(batch=batch, num_seqs=num_seqs, seqlen=seqlen, heads=heads, dk=dk, dv=dv,
                   dtype=_dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype),
                   chunk=chunk, qk_l2norm=int(bool(qk_l2norm)), scale=float(scale),
                   gate_per_head=int(gate_per_head), ckpt_every=int(ckpt_every))


def chunk_fwd_workspace_bytes(desc: KdaDesc) -> int:
    lib = load_library()
    return int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc)))


@_stream_scoped
def kda_chunk_fwd(q, k, v, g, beta, init_state=None, cu_seqlens=None, *, qk_l2norm=True,
                  scale=1.0, ckpt_every=0, out=None, final_state=None, want_final=True,
                  state_ckpt=None, workspace=None, stream=None, noalloc=False):
    """Chunkwise KDA prefill through the C ABI.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (float32 or bfloat16); g: [B, T, H, dk]
    fp32 (per-channel gates, KDA) or [B, T, H] (one gate per token and head,
    Gated DeltaNet); beta: [B, T, H] fp32; init_state: [N, H, dk, dv] fp32 or None;
    cu_seqlens: int32 [N + 1] device tensor (B must be 1) or None.
    Returns (o, final_state, state_ckpt); final_state may be passed in (it may
    be the init_state tensor itself).  noalloc=True calls kda_chunk_fwd_noalloc
    (no workspace; the library's fixed per-device scratch); pass out,
    final_state and state_ckpt to keep the whole call free of allocations.
    """
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _need(q, "q", dt, (B, T, H, dk))
    _need(k, "k", dt, (B, T, H, dk))
    _need(v, "v", dt, (B, T, H, dv))
    per_head = g.dim() == 3
    _need(g, "g", torch.float32, (B, T, H) if per_head else (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (N, H, dk, dv))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(out, "out", dt, (B, T, H, dv))
    if final_state is None and want_final:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    if ckpt_every and state_ckpt is None:
        state_ckpt = torch.empty((B, T // ckpt_every, H, dk, dv), dtype=torch.float32, device=dev)
    desc = make_desc(batch=B, num_seqs=N, seqlen=T, heads=H, dk=dk, dv=dv, dtype=dt,
                     qk_l2norm=qk_l2norm, scale=scale, ckpt_every=ckpt_every,
                     gate_per_head=per_head)
    if noalloc:
        st = lib.kda_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(init_state), _ptr(cu_seqlens), _ptr(out),
                                       _ptr(final_state), _ptr(state_ckpt),
                                       _stream_handle(stream, dev))
        _check(lib, st, "kda_chunk_fwd_noalloc")
        return out, final_state, state_ckpt
    ws_bytes = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc)))
    if ws_bytes == 0 and lib.kda_last_error():
        _check(lib, KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_workspace_bytes")
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.kda_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(init_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
                           _ptr(state_ckpt), _ptr(workspace),
                           0 if workspace is None else workspace.numel() * workspace.element_size(),
                           _stream_handle(stream, dev))
    _check(lib, st, "kda_chunk_fwd")
    return out, final_state, state_ckpt


def _ptr3(ts):
    """Three optional tensors as a C array of three pointers (None: NULL array)."""
    if ts is None:
        return None
    return (ctypes.c_void_p * 3)(*[None if t is None else t.data_ptr() for t in ts])


@_stream_scoped
def kda_chunk_fwd_conv(xq, xk, xv, conv_w, g, beta, init_state=None, cu_seqlens=None, *,
                       conv_bias=None, conv_state=None, conv_state_out=None,
                       want_conv_state=True, qk_l2norm=True, scale=1.0, ckpt_every=0, out=None,
                       final_state=None, want_final=True, state_ckpt=None, workspace=None,
                       stream=None):
    """Prefill with the ShortConv + Swish prologue (width 4) fused into the
    operator, through the C ABI (kda_chunk_fwd_conv).

    xq, xk, xv: the prologue's inputs, shaped as q, k, v of kda_chunk_fwd;
    conv_w: three [H*dk, 4] fp32 filters (q, k, v); conv_bias: None or three
    [H*dk] fp32 tensors or Nones; conv_state: None or three [N, H*dk, 3] fp32
    carried-in inputs or Nones (zeros); conv_state_out: None or three tensors
    (each may be the matching conv_state).  Other arguments as for
    kda_chunk_fwd.  Returns (o, final_state, state_ckpt, conv_state_out),
    conv_state_out a list of three [N, H*dk, 3] tensors (None when
    want_conv_state is False and none were passed).
    """
    lib = load_library()
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    dt = xq.dtype
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    C = H * dk
    _need(xq, "xq", dt, (B, T, H, dk))
    _need(xk, "xk", dt, (B, T, H, dk))
    _need(xv, "xv", dt, (B, T, H, dv))
    per_head = g.dim() == 3
    _need(g, "g", torch.float32, (B, T, H) if per_head else (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    if len(conv_w) != 3:
        raise ValueError("conv_w: one filter tensor per q, k, v")
    for i, w in enumerate(conv_w):
        _need(w, f"conv_w[{i}]", torch.float32, (C, 4))
    if conv_bias is not None:
        for i, b in enumerate(conv_bias):
            if b is not None:
                _need(b, f"conv_bias[{i}]", torch.float32, (C,))
    if conv_state is not None:
        for i, st in enumerate(conv_state):
            if st is not None:
                _need(st, f"conv_state[{i}]", torch.float32, (N, C, 3))
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (N, H, dk, dv))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    dev = xq.device
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(out, "out", dt, (B, T, H, dv))
    if final_state is None and want_final:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    if ckpt_every and state_ckpt is None:
        state_ckpt = torch.empty((B, T // ckpt_every, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_state_out is None and want_conv_state:
        conv_state_out = [torch.empty((N, C, 3), dtype=torch.float32, device=dev)
                          for _ in range(3)]
    if conv_state_out is not None:
        for i, st in enumerate(conv_state_out):
            if st is not None:
                _need(st, f"conv_state_out[{i}]", torch.float32, (N, C, 3))
    desc = make_desc(batch=B, num_seqs=N, seqlen=T, heads=H, dk=dk, dv=dv, dtype=dt,
                     qk_l2norm=qk_l2norm, scale=scale, ckpt_every=ckpt_every,
                     gate_per_head=per_head)
    ws_bytes = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc)))
    if ws_bytes == 0 and lib.kda_last_error():
        _check(lib, KDA_ERR_INVALID_ARGUMENT, "kda_chunk_fwd_workspace_bytes")
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.kda_chunk_fwd_conv(ctypes.byref(desc), _ptr(xq), _ptr(xk), _ptr(xv),
                                _ptr3(conv_w), _ptr3(conv_bias), _ptr3(conv_state),
                                _ptr3(conv_state_out), _ptr(g), _ptr(beta), _ptr(init_state),
                                _ptr(cu_seqlens), _ptr(out), _ptr(final_state), _ptr(state_ckpt),
                                _ptr(workspace),
                                0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream_handle(stream, dev))
    _check(lib, st, "kda_chunk_fwd_conv")
    return out, final_state, state_ckpt, conv_state_out


def chunk_bwd_workspace_bytes(desc: KdaDesc) -> int:
    """Workspace bytes kda_chunk_bwd needs for `desc` (0 if unsupported)."""
    return int(load_library().kda_chunk_bwd_workspace_bytes(ctypes.byref(desc)))


@_stream_scoped
def kda_chunk_bwd(q, k, v, g, beta, do, init_state=None, dfinal=None, cu_seqlens=None, *,
                  qk_l2norm=True, scale=1.0, want_dinit=True, range_flag=None, workspace=None,
                  stream=None):
    """Gradients of the chunkwise KDA prefill through the C ABI.

    Inputs as kda_chunk_fwd, plus do: [B, T, H, dv] (q's dtype), the gradient
    of o, and dfinal: [N, H, dk, dv] fp32 or None (zero), the gradient of the
    final state.  Returns (dq, dk, dv, dg, dbeta, dinit): dq, dk, dv in q's
    dtype, dg fp32 shaped like g, dbeta [B, T, H] fp32, dinit [N, H, dk, dv]
    fp32 (None unless want_dinit).  range_flag: None, or a one-element int32
    tensor on q's device, set to 1 by the call when some chunk decays beyond
    the fast kernels' exponent range (that chunk's gradients then come from
    the slow exact kernel); the caller clears it.
    """
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    for t, name, shape in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)),
                           (v, "v", (B, T, H, dv)), (do, "do", (B, T, H, dv))):
        _need(t, name, dt, shape)
    per_head = g.dim() == 3
    _need(g, "g", torch.float32, (B, T, H) if per_head else (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    for t, name in ((init_state, "init_state"), (dfinal, "dfinal")):
        if t is not None:
            _need(t, name, torch.float32, (N, H, dk, dv))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if range_flag is not None:
        _need(range_flag, "range_flag", torch.int32, (1,))
    dev = q.device
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dg = torch.empty_like(g)
    db = torch.empty_like(beta)
    dinit = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dinit else None
    desc = make_desc(batch=B, num_seqs=N, seqlen=T, heads=H, dk=dk, dv=dv, dtype=dt,
                     qk_l2norm=qk_l2norm, scale=scale, gate_per_head=per_head)
    ws_bytes = int(lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(desc)))
    if ws_bytes == 0:
        _check(lib, KDA_ERR_UNSUPPORTED if lib.kda_last_error() else KDA_ERR_INVALID_ARGUMENT,
               "kda_chunk_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.kda_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(init_state), _ptr(cu_seqlens), _ptr(do), _ptr(dfinal), _ptr(dq),
                           _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dinit),
                           _ptr(range_flag), _ptr(workspace),
                           workspace.numel() * workspace.element_size(),
                           _stream_handle(stream, dev))
    _check(lib, st, "kda_chunk_bwd")
    return dq, dkk, dvv, dg, db, dinit


@_stream_scoped
def kda_decode_step(q, k, v, g, beta, state, *, qk_l2norm=True, scale=1.0, out=None,
                    stream=None):
    """One KDA decode step through the C ABI; `state` [N, H, dk, dv] fp32 is
    updated in place.  q, k: [N, H, dk]; g: [N, H, dk] (per-channel) or
    [N, H] (per head, Gated DeltaNet); v: [N, H, dv]; beta: [N, H]."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q", dt, (N, H, dk))
    _need(k, "k", dt, (N, H, dk))
    _need(v, "v", dt, (N, H, dv))
    per_head = g.dim() == 2
    _need(g, "g", torch.float32, (N, H) if per_head else (N, H, dk))
    _need(beta, "beta", torch.float32, (N, H))
    _need(state, "state", torch.float32, (N, H, dk, dv))
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=q.device)
    _need(out, "out", dt, (N, H, dv))
    desc = make_desc(batch=max(N, 1), num_seqs=N, seqlen=1, heads=H, dk=dk, dv=dv, dtype=dt,
                     qk_l2norm=qk_l2norm, scale=scale, gate_per_head=per_head)
    st = lib.kda_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(state), _ptr(out), _stream_handle(stream, q.device))
    _check(lib, st, "kda_decode_step")
    return out


@_stream_scoped
def kda_output_gate_norm(o, z, w=None, *, eps=1e-6, out=None, stream=None):
    """Output epilogue through the C ABI: head-wise RMSNorm of o times
    sigmoid(z).  o, z: [..., dv] (same dtype and shape, contiguous); w: [dv]
    fp32 or None.  out may be o itself (in place).  Returns out."""
    lib = load_library()
    dt = o.dtype
    dv = o.shape[-1]
    _need(o, "o", dt, tuple(o.shape))
    _need(z, "z", dt, tuple(o.shape))
    if w is not None:
        _need(w, "w", torch.float32, (dv,))
    if out is None:
        out = torch.empty_like(o)
    _need(out, "out", dt, tuple(o.shape))
    rows = o.numel() // dv if dv else 0
    st = lib.kda_output_gate_norm(rows, dv, _dtype_code(dt), _ptr(o), _ptr(z), _ptr(w),
                                  float(eps), _ptr(out), _stream_handle(stream, o.device))
    _check(lib, st, "kda_output_gate_norm")
    return out


@_stream_scoped
def kda_short_conv_swish(x, w, bias=None, state=None, cu_seqlens=None, *, want_state=True,
                         state_out=None, out=None, stream=None):
    """ShortConv + Swish through the C ABI.  x: [B, T, C] (float32 or
    bfloat16, contiguous); w: [C, W] fp32; bias: [C] fp32 or None; state:
    [N, C, W-1] fp32 carried-in inputs or None (zeros); cu_seqlens: int32
    [N + 1] (B must be 1) or None.  Returns (y, state_out); state_out may be
    passed as `state` itself for decode-sized calls (T <= 32, dense)."""
    lib = load_library()
    B, T, C = x.shape
    W = w.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dt = x.dtype
    _need(x, "x", dt, (B, T, C))
    _need(w, "w", torch.float32, (C, W))
    if bias is not None:
        _need(bias, "bias", torch.float32, (C,))
    if state is not None:
        _need(state, "state", torch.float32, (N, C, W - 1))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", dt, (B, T, C))
    if state_out is None and want_state and W > 1:
        state_out = torch.empty((N, C, W - 1), dtype=torch.float32, device=x.device)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (N, C, W - 1))
    st = lib.kda_short_conv_swish(B, T, N, C, W, _dtype_code(dt), _ptr(x), _ptr(w), _ptr(bias),
                                  _ptr(state), _ptr(cu_seqlens), _ptr(out), _ptr(state_out),
                                  _stream_handle(stream, x.device))
    _check(lib, st, "kda_short_conv_swish")
    return out, state_out
