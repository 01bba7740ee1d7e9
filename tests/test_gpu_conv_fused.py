"""The ShortConv + Swish prologue fused into the prefill (kda_chunk_fwd_conv)
on the GPU.  Against the two-step path (kda_short_conv_swish on each of q, k,
v, then kda_chunk_fwd): bitwise, since both take the same arithmetic in the
same order; against the fp64 oracle's prologue followed by its operator: to
the prefill's tolerance.  Dense and varlen layouts (empty sequences and
sequences shorter than the filter), carried conv states (also updated in
place), biases or none, per-head gates, fp32 and bf16, and the full 8K x
32-head workload.  Inputs are seeded and synthetic."""
import numpy as np
import pytest
import torch

from gated_delta_rule_54_amd import kda_chunk_fwd, kda_chunk_fwd_conv, kda_short_conv_swish
from gated_delta_rule_54_amd import workloads as W
from oracle import oracle as O
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _conv_params(C, N, seed, bias=True, state=True):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    w = [0.5 * torch.randn(C, 4, generator=gen, device=DEV) for _ in range(3)]
    b = [0.1 * torch.randn(C, generator=gen, device=DEV) for _ in range(3)] if bias else None
    s = [torch.randn(N, C, 3, generator=gen, device=DEV) for _ in range(3)] if state else None
    return w, b, s


def _two_step(inp, w, b, s, ckpt_every=0):
    """kda_short_conv_swish on q, k, v, then kda_chunk_fwd."""
    B, T, H, d = inp["q"].shape
    cu = inp["cu_seqlens"]
    ys, souts = [], []
    for i, name in enumerate(("q", "k", "v")):
        y, so = kda_short_conv_swish(inp[name].reshape(B, T, H * d), w[i],
                                     None if b is None else b[i], None if s is None else s[i],
                                     cu)
        ys.append(y.reshape(B, T, H, d))
        souts.append(so)
    o, fs, ck = kda_chunk_fwd(ys[0], ys[1], ys[2], inp["g"], inp["beta"], inp["init_state"], cu,
                              ckpt_every=ckpt_every)
    return o, fs, ck, souts


def _fused(inp, w, b, s, **kw):
    return kda_chunk_fwd_conv(inp["q"], inp["k"], inp["v"], w, inp["g"], inp["beta"],
                              inp["init_state"], inp["cu_seqlens"], conv_bias=b, conv_state=s,
                              **kw)


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _assert_same(name, a, b):
    assert a.shape == b.shape and a.dtype == b.dtype, (name, a.shape, b.shape)
    same = torch.equal(_bits(a), _bits(b))  # the same bits, NaN patterns included
    if not same:
        diff = (a.float() - b.float()).abs().max().item()
        raise AssertionError(f"{name}: not bitwise equal to the two-step path (max diff {diff})")
    print(f"  {name}: bitwise equal", flush=True)


CASES = [
    # id, dtype, d, dense (B, T) or varlen lengths, gate_per_head, bias, state
    ("bf16-d128-dense-ragged", torch.bfloat16, 128, (2, 300), False, True, True),
    ("bf16-d64-dense-noconvstate", torch.bfloat16, 64, (1, 130), False, False, False),
    ("f32-d64-dense", torch.float32, 64, (1, 200), False, True, True),
    ("bf16-d128-varlen-short", torch.bfloat16, 128, [0, 2, 70, 1, 64, 3, 200], False, True, True),
    ("bf16-d64-pergate-varlen", torch.bfloat16, 64, [5, 0, 129], True, True, False),
    ("f32-d128-dense", torch.float32, 128, (1, 100), False, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_two_steps(case):
    name, dt, d, shape, per_head, bias, state = case
    H = 4
    print(f"fused prologue {name}", flush=True)
    if isinstance(shape, list):
        inp = W.prefill_inputs(batch=1, seqlen=0, heads=H, dk=d, dv=d, dtype=dt, device=DEV,
                               seed=760, init="normal", lengths=shape, gate_per_head=per_head)
        N = len(shape)
    else:
        B, T = shape
        inp = W.prefill_inputs(batch=B, seqlen=T, heads=H, dk=d, dv=d, dtype=dt, device=DEV,
                               seed=761, init="normal", gate_per_head=per_head)
        N = B
    w, b, s = _conv_params(H * d, N, 762, bias, state)
    o2, fs2, _, so2 = _two_step(inp, w, b, s)
    o1, fs1, _, so1 = _fused(inp, w, b, s)
    torch.cuda.synchronize()
    _assert_same("o", o1, o2)
    _assert_same("final_state", fs1, fs2)
    for i in range(3):
        _assert_same(f"conv_state_out[{'qkv'[i]}]", so1[i], so2[i])


@pytest.mark.parametrize("shift", [-1.0, -30.0], ids=["mid-reference", "exact"])
def test_fused_strong_gates(shift):
    """Fast-forgetting gates send chunks down the intra-chunk kernel's other
    exponent paths (the mid reference; the exact path past it), which stage
    the convolved rows and load v on their own."""
    H, d, T = 2, 128, 200
    inp = W.prefill_inputs(batch=1, seqlen=T, heads=H, dk=d, dv=d, dtype=torch.bfloat16,
                           device=DEV, seed=770, init="normal", gate_shift=shift)
    w, b, s = _conv_params(H * d, 1, 771)
    o2, fs2, _, so2 = _two_step(inp, w, b, s)
    o1, fs1, _, so1 = _fused(inp, w, b, s)
    torch.cuda.synchronize()
    _assert_same("o", o1, o2)
    _assert_same("final_state", fs1, fs2)


def test_fused_without_norm_with_scale():
    """qk_l2norm off and a query scale: the same options reach both paths.
    Small filters keep the unnormalised keys short (|k| < 1), so the
    recurrence stays bounded."""
    H, d, T = 2, 64, 150
    inp = W.prefill_inputs(batch=1, seqlen=T, heads=H, dk=d, dv=d, dtype=torch.bfloat16,
                           device=DEV, seed=768, init="normal")
    w, b, s = _conv_params(H * d, 1, 769)
    w = [0.1 * t for t in w]
    b = [0.1 * t for t in b]
    ys = []
    for i, name in enumerate(("q", "k", "v")):
        y, _ = kda_short_conv_swish(inp[name].reshape(1, T, H * d), w[i], b[i], s[i])
        ys.append(y.reshape(1, T, H, d))
    o2, fs2, _ = kda_chunk_fwd(ys[0], ys[1], ys[2], inp["g"], inp["beta"], inp["init_state"],
                               qk_l2norm=False, scale=0.5)
    o1, fs1, _, _ = _fused(inp, w, b, s, qk_l2norm=False, scale=0.5)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o2).all()), "the recurrence diverged: inputs too large"
    _assert_same("o", o1, o2)
    _assert_same("final_state", fs1, fs2)


def test_fused_conv_state_in_place_and_checkpoints():
    """conv_state_out given as conv_state itself (decode continues from it),
    with state checkpoints."""
    H, d, T = 2, 128, 256
    inp = W.prefill_inputs(batch=2, seqlen=T, heads=H, dk=d, dv=d, dtype=torch.bfloat16,
                           device=DEV, seed=763, init="normal")
    w, b, s = _conv_params(H * d, 2, 764)
    o2, fs2, ck2, so2 = _two_step(inp, w, b, s, ckpt_every=128)
    s_inplace = [t.clone() for t in s]
    o1, fs1, ck1, so1 = _fused(inp, w, b, s_inplace, conv_state_out=s_inplace, ckpt_every=128)
    torch.cuda.synchronize()
    _assert_same("o", o1, o2)
    _assert_same("final_state", fs1, fs2)
    _assert_same("state_ckpt", ck1, ck2)
    for i in range(3):
        assert so1[i] is s_inplace[i]
        _assert_same(f"conv_state_out[{'qkv'[i]}] (in place)", so1[i], so2[i])


def test_fused_against_oracle_chain():
    """The oracle's prologue (fp64, its output rounded to the input dtype as
    the GPU path stores it) followed by the oracle's operator."""
    B, T, H, d = 1, 300, 4, 128
    inp = W.prefill_inputs(batch=B, seqlen=T, heads=H, dk=d, dv=d, dtype=torch.bfloat16,
                           device=DEV, seed=765, init="normal")
    w, b, s = _conv_params(H * d, B, 766)
    o, fs, _, so = _fused(inp, w, b, s)
    torch.cuda.synchronize()
    ref, ref_state = {}, []
    for i, name in enumerate(("q", "k", "v")):
        x = inp[name].reshape(B, T, H * d).cpu()
        yr, sr = O.short_conv(x, w[i].cpu(), b[i].cpu(), s[i].cpu())
        ref[name] = torch.from_numpy(yr.astype(np.float32)).reshape(B, T, H, d).bfloat16()
        ref_state.append(sr)
    o_ref, fs_ref, _ = O.kda_fwd(ref["q"], ref["k"], ref["v"], inp["g"].cpu(), inp["beta"].cpu(),
                                 inp["init_state"].cpu())
    assert_close("o", o, o_ref, TOL[torch.bfloat16])
    assert_close("final_state", fs, fs_ref, TOL[torch.bfloat16])
    for i in range(3):
        # carried-out inputs are copies of inputs: exact
        assert np.array_equal(so[i].cpu().double().numpy(), ref_state[i]), "qkv"[i]


def test_fused_full_size():
    """The 8K x 32-head prefill workload: bitwise against the two-step path."""
    w8 = W.PREFILL_8K
    inp = W.prefill_inputs(batch=1, seqlen=8192, heads=32, dk=128, dv=128, dtype=w8.dtype,
                           device=DEV, seed=w8.seed, init="normal")
    w, b, s = _conv_params(32 * 128, 1, 767)
    print("fused prologue, 8K x 32 heads", flush=True)
    o2, fs2, _, so2 = _two_step(inp, w, b, s)
    o1, fs1, _, so1 = _fused(inp, w, b, s)
    torch.cuda.synchronize()
    _assert_same("o", o1, o2)
    _assert_same("final_state", fs1, fs2)
    for i in range(3):
        _assert_same(f"conv_state_out[{'qkv'[i]}]", so1[i], so2[i])
