"""The C ABI without a GPU: the library loads, exports exactly what
include/kda.h declares, and rejects invalid calls on the host (before any
launch) with the documented status."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_54_amd as K
from gated_delta_rule_54_amd import kda as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    out = subprocess.check_output(["nm", "-D", "--defined-only", B.LIB_PATH], text=True)
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == _declared(), (exported, _declared())
    assert sorted(B.EXPORTED) == _declared()


def test_abi_version_and_strings():
    lib = K.load_library()
    assert lib.kda_abi_version() == 7
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(3) == b"KDA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.kda_status_string(99) == b"KDA_STATUS_UNKNOWN"


FAKE = 0x10000  # an aligned non-null address: validation fails before it is touched


def _desc(**kw):
    base = dict(batch=1, num_seqs=1, seqlen=128, heads=2, dk=64, dv=64, dtype=0)
    base.update(kw)
    return K.make_desc(**base)


def _call_chunk(desc, *, q=FAKE, o=FAKE + 0x100, ws=None, ws_bytes=None, cu=None, ckpt=None,
                misalign=None, shift=4):
    """Every call here must fail validation: the fake addresses are never
    dereferenced because nothing is launched."""
    lib = K.load_library()
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc))
    ptrs = dict(q=q, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=o)
    if misalign:
        ptrs[misalign] += shift
    wsp = FAKE if ws is None else ws
    wsb = need if ws_bytes is None else ws_bytes
    return lib.kda_chunk_fwd(ctypes.byref(desc), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"],
                             ptrs["beta"], None, cu, ptrs["o"], None, ckpt, wsp, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96, dv=96), B.KDA_ERR_UNSUPPORTED),
    (dict(dk=64, dv=128), B.KDA_ERR_UNSUPPORTED),
    (dict(chunk=32), B.KDA_ERR_UNSUPPORTED),
    (dict(heads=0), B.KDA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.KDA_ERR_INVALID_ARGUMENT),
    (dict(seqlen=-1), B.KDA_ERR_INVALID_ARGUMENT),
    (dict(batch=2, num_seqs=1), B.KDA_ERR_INVALID_ARGUMENT),
    (dict(ckpt_every=100), B.KDA_ERR_INVALID_ARGUMENT),
    (dict(ckpt_every=96), B.KDA_ERR_INVALID_ARGUMENT),
    (dict(gate_per_head=2), B.KDA_ERR_INVALID_ARGUMENT),
])
def test_chunk_desc_errors(kw, status):
    lib = K.load_library()
    st = _call_chunk(_desc(**kw))
    assert st == status, lib.kda_last_error()
    assert lib.kda_last_error() != b""


def test_chunk_pointer_errors():
    lib = K.load_library()
    assert _call_chunk(_desc(), q=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert b"q is NULL" in lib.kda_last_error()
    assert _call_chunk(_desc(), misalign="q") == B.KDA_ERR_INVALID_ARGUMENT
    assert b"q is not 16-byte aligned" in lib.kda_last_error()
    assert _call_chunk(_desc(), misalign="g", shift=8) == B.KDA_ERR_INVALID_ARGUMENT
    assert b"g is not 16-byte aligned" in lib.kda_last_error()
    assert _call_chunk(_desc(), misalign="beta", shift=2) == B.KDA_ERR_INVALID_ARGUMENT
    assert b"beta is not 4-byte aligned" in lib.kda_last_error()
    assert _call_chunk(_desc(), o=FAKE) == B.KDA_ERR_INVALID_ARGUMENT  # o aliases q
    assert _call_chunk(_desc(), ws_bytes=16) == B.KDA_ERR_WORKSPACE_TOO_SMALL
    assert _call_chunk(_desc(ckpt_every=64)) == B.KDA_ERR_INVALID_ARGUMENT  # ckpt buffer missing
    assert _call_chunk(_desc(), ckpt=FAKE) == B.KDA_ERR_INVALID_ARGUMENT    # ckpt without every
    # varlen needs batch == 1 and no checkpoints
    assert _call_chunk(_desc(batch=2, num_seqs=3), cu=FAKE) == B.KDA_ERR_INVALID_ARGUMENT
    assert _call_chunk(_desc(num_seqs=3, ckpt_every=64), cu=FAKE, ckpt=FAKE) == \
        B.KDA_ERR_INVALID_ARGUMENT


def test_chunk_fwd_conv_errors():
    """The fused prologue entry point: the prefill's checks, then its own."""
    lib = K.load_library()
    desc = _desc()
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(desc))
    arr = lambda *a: (ctypes.c_void_p * 3)(*a)
    w_ok = arr(FAKE, FAKE + 0x40, FAKE + 0x80)

    def call(*, x=FAKE, w=w_ok, bias=None, sin=None, sout=None, o=FAKE + 0x100, ws_bytes=need,
             d=desc):
        return lib.kda_chunk_fwd_conv(ctypes.byref(d), x, FAKE, FAKE, w, bias, sin, sout, FAKE,
                                      FAKE, None, None, o, None, None, FAKE, ws_bytes, None)

    assert call(x=None) == B.KDA_ERR_INVALID_ARGUMENT                       # xq NULL
    assert call(o=FAKE) == B.KDA_ERR_INVALID_ARGUMENT                       # o aliases xq
    assert call(d=_desc(dk=96, dv=96)) == B.KDA_ERR_UNSUPPORTED
    assert call(w=None) == B.KDA_ERR_INVALID_ARGUMENT                       # no filter array
    assert call(w=arr(FAKE, None, FAKE)) == B.KDA_ERR_INVALID_ARGUMENT      # k's filter NULL
    assert call(w=arr(FAKE, FAKE + 8, FAKE)) == B.KDA_ERR_INVALID_ARGUMENT  # not 16-byte aligned
    assert call(bias=arr(None, FAKE + 2, None)) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(sin=arr(FAKE + 1, None, None)) == B.KDA_ERR_INVALID_ARGUMENT
    # carried-out inputs overlapping the carried-in ones without being them
    assert call(sin=arr(FAKE, None, None), sout=arr(FAKE + 4, None, None)) == \
        B.KDA_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=16) == B.KDA_ERR_WORKSPACE_TOO_SMALL


def test_workspace_sizes():
    lib = K.load_library()
    ws = lambda **kw: lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(**kw)))
    assert ws(dk=96, dv=96) == 0 and b"supported" in lib.kda_last_error()
    small, big = ws(seqlen=64), ws(seqlen=8192)
    assert 0 < small < big
    # a long dense problem is processed in segments of bounded size: the
    # workspace stops growing with T (records of one segment + carried states)
    w1m = ws(seqlen=1 << 20, dk=128, dv=128, dtype=1, heads=32)
    assert w1m == ws(seqlen=1 << 16, dk=128, dv=128, dtype=1, heads=32)
    assert 32 * 128 * 128 * 4 < w1m <= (160 << 20) + 32 * 128 * 128 * 4
    # the varlen bound leaves room for one partial chunk per sequence:
    # 640 packed tokens in 10 sequences need up to (640 + 63*10)/64 = 19 slots
    assert ws(seqlen=640, num_seqs=10) > ws(seqlen=640, num_seqs=1)


def test_decode_errors():
    lib = K.load_library()

    def call(desc, **ptrs):
        p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, o=FAKE + 0x100)
        p.update(ptrs)
        return lib.kda_decode_step(ctypes.byref(desc), p["q"], p["k"], p["v"], p["g"],
                                   p["beta"], p["state"], p["o"], None)

    assert call(_desc(dk=32, dv=32)) == B.KDA_ERR_UNSUPPORTED
    assert call(_desc(), state=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(_desc(), o=FAKE) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(_desc(), beta=FAKE + 2) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(_desc(), state=FAKE + 8) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(_desc(num_seqs=-1)) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(_desc(num_seqs=0)) == B.KDA_OK  # nothing to do, nothing launched


def test_gate_norm_errors():
    """Every invalid epilogue call fails on the host; the fake pointers are
    never dereferenced because nothing is launched."""
    lib = K.load_library()
    Z, Y = FAKE + 0x100000, FAKE + 0x200000  # disjoint 16-byte-aligned regions

    def call(rows=4, dv=128, dtype=1, o=FAKE, z=Z, w=None, eps=1e-6, y=Y):
        return lib.kda_output_gate_norm(rows, dv, dtype, o, z, w, eps, y, None)

    assert call(rows=-1) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(dtype=7) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(dv=96) == B.KDA_ERR_UNSUPPORTED
    assert call(eps=-1.0) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(eps=float("nan")) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(o=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(z=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(y=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(o=FAKE + 8) == B.KDA_ERR_INVALID_ARGUMENT        # not 16-byte aligned
    assert call(w=FAKE + 2) == B.KDA_ERR_INVALID_ARGUMENT        # w not 4-byte aligned
    assert call(y=Z) == B.KDA_ERR_INVALID_ARGUMENT               # y overlaps z
    assert call(y=FAKE + 256) == B.KDA_ERR_INVALID_ARGUMENT      # partial overlap with o
    assert call(rows=0, o=None, z=None, y=None) == B.KDA_OK      # nothing to do


def test_short_conv_errors():
    """Every invalid ShortConv call fails on the host (nothing is launched)."""
    lib = K.load_library()
    X, Y, S = FAKE, FAKE + 0x100000, FAKE + 0x200000

    def call(batch=1, seqlen=64, num_seqs=1, channels=64, width=4, dtype=1, x=X, w=FAKE,
             bias=None, si=None, cu=None, y=Y, so=None):
        return lib.kda_short_conv_swish(batch, seqlen, num_seqs, channels, width, dtype, x, w,
                                        bias, si, cu, y, so, None)

    assert call(dtype=7) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(width=0) == B.KDA_ERR_UNSUPPORTED
    assert call(width=5) == B.KDA_ERR_UNSUPPORTED
    assert call(channels=12) == B.KDA_ERR_UNSUPPORTED          # bf16 needs a multiple of 8
    # a token row may hold at most 2^25 bytes (the kernel's 32-bit offsets)
    assert call(channels=(1 << 24) + 8, seqlen=1) == B.KDA_ERR_UNSUPPORTED
    assert call(channels=(1 << 23) + 4, seqlen=1, dtype=0) == B.KDA_ERR_UNSUPPORTED
    assert call(batch=0) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(seqlen=-1) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(num_seqs=2) == B.KDA_ERR_INVALID_ARGUMENT      # dense: num_seqs == batch
    assert call(batch=2, num_seqs=3, cu=FAKE) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(w=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(x=None) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(x=X + 8) == B.KDA_ERR_INVALID_ARGUMENT          # not 16-byte aligned
    assert call(bias=FAKE + 2) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(y=X + 1024) == B.KDA_ERR_INVALID_ARGUMENT      # y overlaps x
    assert call(si=S, so=S) == B.KDA_ERR_INVALID_ARGUMENT      # in place needs seqlen <= 32
    assert call(seqlen=8, si=S, so=S, cu=FAKE, num_seqs=1) == B.KDA_ERR_INVALID_ARGUMENT
    assert call(seqlen=8, si=S, so=S + 16) == B.KDA_ERR_INVALID_ARGUMENT  # partial overlap
    assert call(num_seqs=0, cu=FAKE) == B.KDA_OK                # nothing to do


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        B.load_library(str(tmp_path / "missing.so"))


def _call_bwd(desc, *, ws=None, ws_bytes=None, nulls=(), misalign=None, alias=None):
    """Backward calls that must fail host validation (nothing launched)."""
    lib = K.load_library()
    need = lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(desc))
    names = ("q", "k", "v", "g", "beta", "d_o", "dq", "dk", "dv", "dg", "dbeta", "range_flag")
    ptrs = {n: FAKE + 0x1000 * i for i, n in enumerate(names)}
    for n in nulls:
        ptrs[n] = None
    if misalign:
        ptrs[misalign] += 2 if misalign == "range_flag" else 4  # its alignment is 4
    if alias:
        ptrs[alias[0]] = ptrs[alias[1]]
    wsp = FAKE + 0x100000 if ws is None else ws
    wsb = need if ws_bytes is None else ws_bytes
    return lib.kda_chunk_bwd(ctypes.byref(desc), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"],
                             ptrs["beta"], None, None, ptrs["d_o"], None, ptrs["dq"], ptrs["dk"],
                             ptrs["dv"], ptrs["dg"], ptrs["dbeta"], None, ptrs["range_flag"], wsp,
                             wsb, None)


def test_bwd_workspace_and_support():
    lib = K.load_library()
    # fp32 operands at d = 128 are not supported by the backward
    d = _desc(dk=128, dv=128, dtype=0)
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(d)) == 0
    assert _call_bwd(d) == B.KDA_ERR_UNSUPPORTED
    for dt, dk in ((0, 64), (1, 64), (1, 128)):
        d = _desc(dk=dk, dv=dk, dtype=dt)
        need = lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(d))
        # at least the entering states and their gradients (in the element
        # type) for every chunk slot
        esz = 4 if dt == 0 else 2
        assert need >= 2 * 2 * 2 * dk * dk * esz
    d = _desc(dk=64, dv=64, dtype=1)
    assert _call_bwd(d, ws_bytes=1) == B.KDA_ERR_WORKSPACE_TOO_SMALL
    assert _call_bwd(d, ws=0) == B.KDA_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("case", [
    dict(nulls=("d_o",)), dict(nulls=("dg",)), dict(nulls=("dbeta",)),
    dict(misalign="dq"), dict(misalign="d_o"), dict(alias=("dq", "q")),
    dict(alias=("dv", "d_o")), dict(misalign="range_flag"), dict(alias=("range_flag", "dg")),
])
def test_bwd_pointer_errors(case):
    lib = K.load_library()
    st = _call_bwd(_desc(dk=64, dv=64, dtype=1), **case)
    assert st == B.KDA_ERR_INVALID_ARGUMENT, lib.kda_last_error()


def test_noalloc_rejects_descriptors_beyond_its_scratch():
    """kda_chunk_fwd_noalloc checks its fixed scratch on the host: carried
    states of 2048 sequences x 32 heads (d = 128) need 4 GiB, far beyond the
    64 MiB array, so it returns KDA_ERR_WORKSPACE_TOO_SMALL before any launch;
    invalid arguments are rejected as kda_chunk_fwd rejects them."""
    lib = K.load_library()
    d = K.make_desc(batch=1, num_seqs=2048, seqlen=2048 * 1024, heads=32, dk=128, dv=128,
                    dtype=1)
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   FAKE, FAKE + 0x100, None, None, None)
    assert st == B.KDA_ERR_WORKSPACE_TOO_SMALL
    assert b"kda_chunk_fwd_noalloc holds" in lib.kda_last_error()
    d2 = _desc()
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(d2), FAKE + 4, FAKE, FAKE, FAKE, FAKE, None,
                                   None, FAKE + 0x100, None, None, None)
    assert st == B.KDA_ERR_INVALID_ARGUMENT
    assert b"q is not 16-byte aligned" in lib.kda_last_error()
