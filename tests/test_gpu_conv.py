"""ShortConv + Swish prologue on the GPU against the fp64 oracle: seeded
synthetic x, filters, biases and carried states (none from the HIP path),
dense and varlen layouts, decode-sized steps in place, the full 8K-token
q-projection size, and the prologue followed by the operator."""
import numpy as np
import pytest
import torch

from gated_delta_rule_54_amd import kda_chunk_fwd, kda_short_conv_swish
from gated_delta_rule_54_amd import workloads as W
from oracle import oracle as O
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(B, T, C, Wd, dtype, seed, N=None, bias=True, state=True):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(B, T, C, generator=gen, device=DEV).to(dtype)
    w = 0.5 * torch.randn(C, Wd, generator=gen, device=DEV)
    b = 0.1 * torch.randn(C, generator=gen, device=DEV) if bias else None
    n = B if N is None else N
    s = torch.randn(n, C, Wd - 1, generator=gen, device=DEV) if (state and Wd > 1) else None
    return x, w, b, s


def _host(t):
    return None if t is None else t.cpu()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 33, 100])
@pytest.mark.parametrize("Wd", [1, 2, 4])
@pytest.mark.parametrize("with_state", [False, True], ids=["zeros", "state"])
def test_conv_dense(dtype, T, Wd, with_state):
    x, w, b, s = _draw(2, T, 64, Wd, dtype, seed=700 + T + Wd, state=with_state)
    y, so = kda_short_conv_swish(x, w, b, s)
    torch.cuda.synchronize()
    y_ref, s_ref = O.short_conv(x.cpu(), w.cpu(), _host(b), _host(s))
    print(f"conv dense T={T} W={Wd} state={with_state} {dtype}", flush=True)
    assert_close("y", y, y_ref, TOL[dtype])
    if Wd > 1:
        assert_close("state_out", so, s_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_conv_varlen(dtype):
    lens = [70, 0, 1, 2, 33, 200, 0, 31]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    x, w, b, s = _draw(1, int(cu[-1]), 128, 4, dtype, seed=720, N=len(lens))
    y, so = kda_short_conv_swish(x, w, b, s, cu)
    torch.cuda.synchronize()
    y_ref, s_ref = O.short_conv(x.cpu(), w.cpu(), b.cpu(), s.cpu(), cu.cpu().numpy())
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("state_out (incl. empty sequences)", so, s_ref, TOL[dtype])
    # no carried state: zeros before every sequence, zeros carried by empty ones
    y2, so2 = kda_short_conv_swish(x, w, b, None, cu)
    torch.cuda.synchronize()
    y2_ref, s2_ref = O.short_conv(x.cpu(), w.cpu(), b.cpu(), None, cu.cpu().numpy())
    assert_close("y (zero state)", y2, y2_ref, TOL[dtype])
    assert_close("state_out (zero state)", so2, s2_ref, TOL[dtype])


def test_conv_decode_steps_in_place():
    """Decode-sized calls (T = 1, N sequences) updating the state in place."""
    N, C, steps = 16, 4096, 6
    x, w, b, s = _draw(N, steps, C, 4, torch.bfloat16, seed=730)
    s_host = s.cpu().clone()
    ys = []
    for t in range(steps):
        xt = x[:, t:t + 1].contiguous()
        yt, so = kda_short_conv_swish(xt, w, b, s, state_out=s)
        assert so.data_ptr() == s.data_ptr()
        ys.append(yt)
    torch.cuda.synchronize()
    y_ref, s_ref = O.short_conv(x.cpu(), w.cpu(), b.cpu(), s_host)
    assert_close("decode steps", torch.cat(ys, dim=1), y_ref, TOL[torch.bfloat16])
    assert_close("state after steps", s, s_ref, TOL[torch.bfloat16])


def test_conv_full_size():
    """One q projection of the 8K-token, 32-head workload: [1, 8192, 4096] bf16."""
    x, w, b, s = _draw(1, 8192, 4096, 4, torch.bfloat16, seed=740)
    y, so = kda_short_conv_swish(x, w, b, s)
    torch.cuda.synchronize()
    y_ref, s_ref = O.short_conv(x.cpu(), w.cpu(), b.cpu(), s.cpu())
    assert_close("y", y, y_ref, TOL[torch.bfloat16])
    assert_close("state_out", so, s_ref, TOL[torch.bfloat16])


def test_prologue_then_operator():
    """ShortConv + Swish on q, k, v, then the operator (which L2-normalises q
    and k), against the oracle's prologue followed by the oracle's operator."""
    B, T, H, d = 1, 300, 4, 128
    inp = W.prefill_inputs(batch=B, seqlen=T, heads=H, dk=d, dv=d, dtype=torch.bfloat16,
                           device=DEV, seed=750, init="normal")
    gen = torch.Generator(device=DEV).manual_seed(751)
    conv = {}
    ref = {}
    for name in ("q", "k", "v"):
        w = 0.5 * torch.randn(H * d, 4, generator=gen, device=DEV)
        x = inp[name].reshape(B, T, H * d)
        y, _ = kda_short_conv_swish(x, w)
        conv[name] = y.reshape(B, T, H, d)
        yr, _ = O.short_conv(x.cpu(), w.cpu(), want_state=False)
        # the oracle operator takes its own prologue output rounded to the
        # input dtype, as the GPU operator does
        ref[name] = torch.from_numpy(yr.astype(np.float32)).reshape(B, T, H, d).bfloat16()
    o, fs, _ = kda_chunk_fwd(conv["q"], conv["k"], conv["v"], inp["g"], inp["beta"],
                             inp["init_state"])
    torch.cuda.synchronize()
    o_ref, fs_ref, _ = O.kda_fwd(ref["q"], ref["k"], ref["v"], inp["g"].cpu(), inp["beta"].cpu(),
                                 inp["init_state"].cpu())
    assert_close("o", o, o_ref, TOL[torch.bfloat16])
    assert_close("final_state", fs, fs_ref, TOL[torch.bfloat16])
