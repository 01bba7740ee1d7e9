"""CPU fp64 oracle for the KDA operator -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product library never does.

This is a thin ctypes wrapper over ``oracle/kda_oracle.c`` (plain C, fp64,
one pthread per (sequence, head) chain).  See that file for the recurrence
and the page citations; this wrapper only moves host tensors into it.

Inputs are CPU torch tensors (or numpy arrays): q, k, v in float32 or
bfloat16 (bf16 is passed as raw 16-bit patterns and widened exactly inside
the C code), g and beta in float32, states in float32.  Outputs are numpy
float64 arrays.  Every function takes an optional ``lib`` (a library opened
with :func:`open_library`), which the planted-mistake tests use to run the
pins against deliberately broken copies of the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_default = None


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source with the host C compiler (gcc)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", tmp, src, "-lpthread", "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle/kda_oracle.c into oracle/liboracle.so if it is stale."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def open_library(path: str):
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    i64, vp, dp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.kda_oracle_fwd_f64.argtypes = [i64, i64, i64, i64, i64, i64, ip,
                                       vp, vp, vp, vp, vp, vp, vp, ip, dp, i64,
                                       vp, vp, vp, ip]
    lib.kda_oracle_fwd_f64.restype = ip
    lib.kda_oracle_decode_f64.argtypes = [i64, i64, i64, i64, i64, ip,
                                          vp, vp, vp, vp, vp, vp, ip, dp, vp, vp, ip]
    lib.kda_oracle_decode_f64.restype = ip
    lib.kda_oracle_gate_norm_f64.argtypes = [i64, i64, ip, vp, vp, vp, dp, vp]
    lib.kda_oracle_gate_norm_f64.restype = ip
    lib.kda_oracle_short_conv_f64.argtypes = [i64, i64, i64, i64, i64, ip, vp, vp, vp, vp, vp,
                                              vp, vp]
    lib.kda_oracle_short_conv_f64.restype = ip
    lib.kda_oracle_bwd_f64.argtypes = [i64, i64, i64, i64, i64, i64, ip,
                                       vp, vp, vp, vp, vp, vp, vp, ip, dp,
                                       vp, vp, vp, vp, vp, vp, vp, vp, ip]
    lib.kda_oracle_bwd_f64.restype = ip
    return lib


def _load(lib=None):
    global _default
    if lib is not None:
        return lib
    if _default is None:
        build()
        _default = open_library(_LIB)
    return _default


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as_np(x, what):
    """Return (contiguous numpy array, dtype code) for an input tensor."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                raise ValueError(f"{what}: oracle inputs must be host tensors")
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), 1
            x = x.contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    if x.dtype != np.float32:
        raise ValueError(f"{what}: expected float32 or bfloat16, got {x.dtype}")
    return np.ascontiguousarray(x), 0


def _f32(x, what):
    if x is None:
        return None
    a, code = _as_np(x, what)
    if code != 0:
        raise ValueError(f"{what}: must be float32")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kda_fwd(q, k, v, g, beta, init_state=None, cu_seqlens=None, *, qk_l2norm=True,
            scale=1.0, ckpt_every=0, want_final=True, nthreads=None, lib=None):
    """Sequential fp64 KDA prefill.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; g: [B, T, H, dk]; beta: [B, T, H];
    init_state: [N, H, dk, dv] or None; cu_seqlens: int32 [N+1] (B must be 1).
    Returns (o [B,T,H,dv], final_state [N,H,dk,dv] or None, ckpt or None).
    """
    qa, dt = _as_np(q, "q")
    ka, dt2 = _as_np(k, "k")
    va, dt3 = _as_np(v, "v")
    if not (dt == dt2 == dt3):
        raise ValueError("q, k, v must share a dtype")
    ga = _f32(g, "g")
    ba = _f32(beta, "beta")
    sa = _f32(init_state, "init_state")
    B, T, H, dk = qa.shape
    dv = va.shape[-1]
    if ka.shape != (B, T, H, dk) or va.shape != (B, T, H, dv) or ga.shape != (B, T, H, dk) \
            or ba.shape != (B, T, H):
        raise ValueError("shape mismatch")
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        N = B
    if sa is not None and sa.shape != (N, H, dk, dv):
        raise ValueError("init_state shape mismatch")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    fs = np.zeros((N, H, dk, dv), dtype=np.float64) if want_final else None
    ck = None
    if ckpt_every:
        ck = np.zeros((B, T // ckpt_every, H, dk, dv), dtype=np.float64)
    rc = _load(lib).kda_oracle_fwd_f64(B, T, N, H, dk, dv, dt, _ptr(qa), _ptr(ka), _ptr(va),
                                    _ptr(ga), _ptr(ba), _ptr(sa), _ptr(cu), int(bool(qk_l2norm)),
                                    float(scale), int(ckpt_every), _ptr(o), _ptr(fs), _ptr(ck),
                                    int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd_f64 failed with code {rc}")
    return o, fs, ck


def kda_bwd(q, k, v, g, beta, do, init_state=None, dfinal=None, cu_seqlens=None, *,
            qk_l2norm=True, scale=1.0, nthreads=None, lib=None):
    """fp64 gradients of the KDA prefill (reverse sweep of the token recurrence).

    q, k, v, g, beta, init_state, cu_seqlens as :func:`kda_fwd`; do: [B, T, H, dv]
    with q's dtype; dfinal: [N, H, dk, dv] float32 or None (zero).
    Returns (dq, dk, dv, dg, dbeta, dinit) as float64 arrays of the inputs'
    shapes (dinit [N, H, dk, dv]).
    """
    qa, dt = _as_np(q, "q")
    ka, dt2 = _as_np(k, "k")
    va, dt3 = _as_np(v, "v")
    da, dt4 = _as_np(do, "do")
    if not (dt == dt2 == dt3 == dt4):
        raise ValueError("q, k, v, do must share a dtype")
    ga = _f32(g, "g")
    ba = _f32(beta, "beta")
    sa = _f32(init_state, "init_state")
    fa = _f32(dfinal, "dfinal")
    B, T, H, dk = qa.shape
    dv = va.shape[-1]
    if ka.shape != (B, T, H, dk) or va.shape != (B, T, H, dv) or ga.shape != (B, T, H, dk) \
            or ba.shape != (B, T, H) or da.shape != (B, T, H, dv):
        raise ValueError("shape mismatch")
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        N = B
    for a, what in ((sa, "init_state"), (fa, "dfinal")):
        if a is not None and a.shape != (N, H, dk, dv):
            raise ValueError(f"{what} shape mismatch")
    dq = np.zeros((B, T, H, dk), dtype=np.float64)
    dkk = np.zeros((B, T, H, dk), dtype=np.float64)
    dvv = np.zeros((B, T, H, dv), dtype=np.float64)
    dg = np.zeros((B, T, H, dk), dtype=np.float64)
    db = np.zeros((B, T, H), dtype=np.float64)
    ds0 = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load(lib).kda_oracle_bwd_f64(B, T, N, H, dk, dv, dt, _ptr(qa), _ptr(ka), _ptr(va),
                                    _ptr(ga), _ptr(ba), _ptr(sa), _ptr(cu), int(bool(qk_l2norm)),
                                    float(scale), _ptr(da), _ptr(fa), _ptr(dq), _ptr(dkk),
                                    _ptr(dvv), _ptr(dg), _ptr(db), _ptr(ds0),
                                    int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd_f64 failed with code {rc}")
    return dq, dkk, dvv, dg, db, ds0


def kda_decode(q, k, v, g, beta, state, *, qk_l2norm=True, scale=1.0, nthreads=None,
               lib=None):
    """fp64 KDA decode over `steps` tokens per chain.

    q, k, g: [steps, N, H, dk]; v: [steps, N, H, dv]; beta: [steps, N, H];
    state: [N, H, dk, dv] fp32 (None = zeros).
    Returns (o [steps, N, H, dv], state_out [N, H, dk, dv]) as float64.
    """
    qa, dt = _as_np(q, "q")
    ka, _ = _as_np(k, "k")
    va, _ = _as_np(v, "v")
    ga = _f32(g, "g")
    ba = _f32(beta, "beta")
    sa = _f32(state, "state")
    steps, N, H, dk = qa.shape
    dv = va.shape[-1]
    o = np.zeros((steps, N, H, dv), dtype=np.float64)
    so = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load(lib).kda_oracle_decode_f64(steps, N, H, dk, dv, dt, _ptr(qa), _ptr(ka), _ptr(va),
                                       _ptr(ga), _ptr(ba), _ptr(sa), int(bool(qk_l2norm)),
                                       float(scale), _ptr(o), _ptr(so),
                                       int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_f64 failed with code {rc}")
    return o, so


def gate_norm(o, z, w=None, *, eps=1e-6, lib=None):
    """fp64 output epilogue: head-wise RMSNorm of o times sigmoid(z).

    o, z: [..., dv] (same dtype, fp32 or bf16); w: [dv] fp32 or None.
    Returns y with o's shape as float64.
    """
    oa, dt = _as_np(o, "o")
    za, dt2 = _as_np(z, "z")
    if dt != dt2 or oa.shape != za.shape:
        raise ValueError("o and z must have the same dtype and shape")
    wa = _f32(w, "w")
    dv = oa.shape[-1]
    rows = int(np.prod(oa.shape[:-1])) if oa.ndim > 1 else 1
    if wa is not None and wa.shape != (dv,):
        raise ValueError("w must have shape [dv]")
    y = np.zeros(oa.shape, dtype=np.float64)
    rc = _load(lib).kda_oracle_gate_norm_f64(rows, dv, dt, _ptr(oa), _ptr(za), _ptr(wa),
                                            float(eps), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_gate_norm_f64 failed with code {rc}")
    return y


def short_conv(x, w, bias=None, state=None, cu_seqlens=None, *, want_state=True, lib=None):
    """fp64 ShortConv + Swish: causal depthwise convolution of width W then
    x * sigmoid(x).  x: [B, T, C] (fp32 or bf16); w: [C, W] fp32; bias: [C]
    or None; state: [N, C, W-1] fp32 carried inputs (oldest first) or None for
    zeros; cu_seqlens: int32 [N+1] (B must be 1) or None.
    Returns (y [B, T, C], state_out [N, C, W-1] or None) as float64."""
    xa, dt = _as_np(x, "x")
    wa = _f32(w, "w")
    ba = _f32(bias, "bias")
    sa = _f32(state, "state")
    B, T, C = xa.shape
    W = wa.shape[1]
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.size - 1
    else:
        N = B
    y = np.zeros((B, T, C), dtype=np.float64)
    so = np.zeros((N, C, W - 1), dtype=np.float64) if want_state else None
    rc = _load(lib).kda_oracle_short_conv_f64(B, T, N, C, W, dt, _ptr(xa), _ptr(wa), _ptr(ba),
                                             _ptr(sa), _ptr(cu), _ptr(y), _ptr(so))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_short_conv_f64 failed with code {rc}")
    return y, so
