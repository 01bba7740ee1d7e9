"""kda_chunk_fwd_noalloc (no workspace, no allocation: the library's fixed
per-device scratch) against kda_chunk_fwd on the same inputs, through the C
ABI: two calls in a row, the second with a smaller input, each bitwise equal
to the workspace entry point (same kernels; only the segment length differs,
and the state crosses segment boundaries in fp32 unchanged) and so within
the tolerance against the oracle too.  Outputs are preallocated, so the
calls themselves allocate nothing."""
import pytest
import torch

from gated_delta_rule_54_amd import kda_chunk_fwd
from gated_delta_rule_54_amd import workloads as W
from oracle import oracle as O
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(inp, **kw):
    o_ref, fs_ref, ck_ref = kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                          inp["init_state"], inp["cu_seqlens"], **kw)
    o = torch.full_like(o_ref, float("nan"))
    fs = torch.full_like(fs_ref, float("nan"))
    ck = None if ck_ref is None else torch.full_like(ck_ref, float("nan"))
    kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["init_state"],
                  inp["cu_seqlens"], out=o, final_state=fs, state_ckpt=ck, noalloc=True, **kw)
    torch.cuda.synchronize()
    return (o, fs, ck), (o_ref, fs_ref, ck_ref)


def test_noalloc_two_calls_match_workspace_entry():
    # 1: the 8K x 32-head bf16 workload (24-slot segments in the 64 MiB array
    #    instead of 64-slot ones); 2: a smaller varlen fp32 input with an empty
    #    sequence and a ragged tail, which leaves the first call's contents in
    #    the array
    w = W.PREFILL_8K
    first = W.workload_inputs(w, DEV)
    second = W.prefill_inputs(batch=1, seqlen=0, heads=3, dk=64, dv=64, dtype=torch.float32,
                              device=DEV, seed=91, init="normal", lengths=[130, 0, 700, 65])
    for name, inp, dtype in (("8K x 32 heads bf16", first, w.dtype),
                             ("varlen fp32 d64", second, torch.float32)):
        print(f"no-alloc prefill: {name}", flush=True)
        (o, fs, _), (o_ref, fs_ref, _) = _both(inp)
        assert torch.equal(o, o_ref), f"{name}: o differs from kda_chunk_fwd"
        assert torch.equal(fs, fs_ref), f"{name}: final state differs from kda_chunk_fwd"
        if inp["q"].shape[1] <= 1024:
            ref = O.kda_fwd(*(inp[k].cpu() for k in ("q", "k", "v", "g", "beta")),
                            inp["init_state"].cpu(), inp["cu_seqlens"].cpu().numpy())
            assert_close("o vs oracle", o, ref[0], TOL[dtype])
            assert_close("final state vs oracle", fs, ref[1], TOL[dtype])


def test_noalloc_checkpoints():
    inp = W.prefill_inputs(batch=2, seqlen=4096, heads=4, dk=128, dv=128, dtype=torch.bfloat16,
                           device=DEV, seed=92, init="normal")
    print("no-alloc prefill with checkpoints", flush=True)
    (o, fs, ck), (o_ref, fs_ref, ck_ref) = _both(inp, ckpt_every=1024)
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref) and torch.equal(ck, ck_ref)
