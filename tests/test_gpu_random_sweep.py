"""Randomised parity sweep on the GPU: forward and backward against the fp64
oracle over configurations drawn from a fixed seed per case -- batch, length
(ragged, varlen with empty and single-token sequences), head count, head
width, element type, gate mode (per channel or per head), gate strength
(slow, normal, mid-reference and exact-path decay), initial state, final-state gradient,
norm and scale.  Each case names its configuration in its output."""
import random

import pytest
import torch

from gated_delta_rule_54_amd import kda_chunk_bwd, kda_chunk_fwd
from gated_delta_rule_54_amd import workloads as W
from oracle import oracle as O
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(x):
    return None if x is None else x.cpu()


def _config(seed):
    rng = random.Random(7919 * seed + 13)
    c = dict(d=rng.choice([64, 128]), dtype=rng.choice([torch.bfloat16, torch.bfloat16, torch.float32]),
             H=rng.choice([1, 2, 3, 4, 5]), gs=rng.random() < 0.25,
             init=rng.choice(["zeros", "normal"]), shift=rng.choice([3.0, 3.0, 1.0, 8.0, -1.0]),
             qk_l2norm=rng.random() < 0.8, scale=rng.choice([1.0, 0.5]), final=rng.random() < 0.7)
    if rng.random() < 0.4:
        c["lengths"] = [rng.choice([0, 1, 5, 63, 64, 65, 100, 130, 200])
                        for _ in range(rng.randint(1, 5))]
    else:
        c["B"], c["T"] = rng.randint(1, 3), rng.choice([1, 17, 64, 65, 127, 128, 129, 300])
    if rng.random() < 0.25:  # beyond the mid reference: the exact kernels
        c["shift"] = -4.0
    return c


@pytest.mark.parametrize("seed", range(24))
def test_random_config(seed):
    c = _config(seed)
    d, dtype, H = c["d"], c["dtype"], c["H"]
    print(f"case {seed}: {c}", flush=True)
    kw = dict(heads=H, dk=d, dv=d, dtype=dtype, device=DEV, seed=9000 + seed, init=c["init"],
              gate_shift=c["shift"], gate_per_head=c["gs"])
    if "lengths" in c:
        inp = W.prefill_inputs(batch=1, seqlen=0, lengths=c["lengths"], **kw)
    else:
        inp = W.prefill_inputs(batch=c["B"], seqlen=c["T"], **kw)
    if not c["qk_l2norm"]:  # keys normalised on the host so the recurrence stays bounded
        kf = inp["k"].float()
        inp["k"] = (kf / kf.norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(dtype)
    B, T, _, _ = inp["q"].shape
    cu = inp["cu_seqlens"]
    cu_np = None if cu is None else cu.cpu().numpy()
    # the oracle takes a per-head gate broadcast over the channels
    g_ref = inp["g"].unsqueeze(-1).expand(B, T, H, d).contiguous() if c["gs"] else inp["g"]
    opts = dict(qk_l2norm=c["qk_l2norm"], scale=c["scale"])
    tol = TOL[dtype]

    o, fs, _ = kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             inp["init_state"], cu, **opts)
    torch.cuda.synchronize()
    o_ref, fs_ref, _ = O.kda_fwd(*(_host(inp[k]) for k in ("q", "k", "v")), _host(g_ref),
                                 _host(inp["beta"]), _host(inp["init_state"]), cu_np, **opts)
    assert_close("o", o, o_ref, tol)
    assert_close("final_state", fs, fs_ref, tol)

    # the backward: bf16 at d = 64 or 128, fp32 at d = 64 (every gate strength:
    # the strong ones take the mid-reference products, the strongest the
    # exact kernel)
    if dtype == torch.float32 and d == 128:
        return
    N = B if cu is None else cu.numel() - 1
    up = W.upstream_grads(batch=B, seqlen=T, heads=H, dk=d, dv=d, num_seqs=N, dtype=dtype,
                          device=DEV, seed=9500 + seed, final=c["final"])
    got = kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], up["do"],
                        inp["init_state"], up["dfinal"], cu, **opts)
    torch.cuda.synchronize()
    ref = list(O.kda_bwd(*(_host(inp[k]) for k in ("q", "k", "v")), _host(g_ref),
                         _host(inp["beta"]), _host(up["do"]), _host(inp["init_state"]),
                         _host(up["dfinal"]), cu_np, **opts))
    if c["gs"]:
        ref[3] = ref[3].sum(axis=-1)  # one gate per (token, head): the channel sum
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dinit"), got, ref):
        assert torch.isfinite(a).all(), name
        assert_close(name, a, b, tol)
