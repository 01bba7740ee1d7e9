"""Gated DeltaNet mode (one forget gate per token and head, broadcast over the
key channels) on the GPU against the fp64 oracle run with that gate copied to
every channel -- the reduction the oracle's GDN pin fixes ([XT §3])."""
import pytest
import torch

from gated_delta_rule_54_amd import kda_chunk_fwd, kda_decode_step
from gated_delta_rule_54_amd import workloads as W
from oracle import oracle as O
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _broadcast(g, dk):
    return g.unsqueeze(-1).expand(*g.shape, dk).contiguous()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_gdn_prefill(dtype, d, T):
    inp = W.prefill_inputs(batch=2, seqlen=T, heads=3, dk=d, dv=d, dtype=dtype, device=DEV,
                           seed=500 + T + d, init="normal", gate_per_head=True)
    assert inp["g"].shape == (2, T, 3)
    o, fs, _ = kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             inp["init_state"])
    torch.cuda.synchronize()
    host = [inp[x].cpu() for x in ("q", "k", "v")]
    o_ref, fs_ref, _ = O.kda_fwd(*host, _broadcast(inp["g"], d).cpu(), inp["beta"].cpu(),
                                 inp["init_state"].cpu())
    print(f"gdn prefill T={T} d={d} {dtype}", flush=True)
    assert_close("o", o, o_ref, TOL[dtype])
    assert_close("final_state", fs, fs_ref, TOL[dtype])


def test_gdn_prefill_long_varlen():
    inp = W.prefill_inputs(batch=1, seqlen=0, heads=4, dk=128, dv=128, dtype=torch.bfloat16,
                           device=DEV, seed=520, init="normal", lengths=[700, 1, 2100, 64],
                           gate_per_head=True)
    o, fs, _ = kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             inp["init_state"], inp["cu_seqlens"])
    torch.cuda.synchronize()
    host = [inp[x].cpu() for x in ("q", "k", "v")]
    o_ref, fs_ref, _ = O.kda_fwd(*host, _broadcast(inp["g"], 128).cpu(), inp["beta"].cpu(),
                                 inp["init_state"].cpu(), inp["cu_seqlens"].cpu().numpy())
    assert_close("o", o, o_ref, TOL[torch.bfloat16])
    assert_close("final_state", fs, fs_ref, TOL[torch.bfloat16])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gdn_decode(dtype):
    gen = W.make_generator(530, DEV)
    N, H, d, steps = 6, 4, 128, 5
    state = W.decode_initial_state(num_seqs=N, heads=H, dk=d, dv=d, gen=gen, device=DEV)
    s0 = state.cpu().clone()
    xs = [W.decode_step_inputs(num_seqs=N, heads=H, dk=d, dv=d, dtype=dtype, gen=gen,
                               device=DEV, gate_per_head=True) for _ in range(steps)]
    outs = [kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state) for x in xs]
    torch.cuda.synchronize()
    stack = lambda key: torch.stack([x[key].cpu() for x in xs])
    o_ref, s_ref = O.kda_decode(stack("q"), stack("k"), stack("v"),
                                _broadcast(stack("g"), d), stack("beta"), s0)
    assert_close("o", torch.stack(outs), o_ref, TOL[dtype])
    assert_close("state", state, s_ref, TOL[dtype])
