"""NaN inputs propagate through the GPU path and stay inside their chain.

Each test poisons one input value in three different (sequence, head)
chains -- a query, a gate and a beta -- and checks, against the fp64 oracle
run on the same inputs:
  * every clean chain is finite and matches the oracle;
  * a NaN query at token t makes that chain's output at t non-finite and
    leaves every other output and the state of that chain exact (the query
    only reads the state);
  * a NaN gate or beta at token t makes the chain's state non-finite from t
    on: every output from t on and the final state are non-finite, and every
    output before t's chunk (prefill) or step (decode) matches the oracle.
    Inside the poisoned chunk the chunkwise products mix rows, so outputs of
    that chunk before t may be NaN too; they are not checked.
No kernel waits on data, so none of this can hang.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_54_amd import kda_chunk_fwd, kda_decode_step
from gated_delta_rule_54_amd import workloads as W
from oracle import oracle as O
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _all_nonfinite(x):
    return bool((~torch.isfinite(x.float())).all())


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)],
                         ids=["bf16-d128", "f32-d64"])
def test_prefill_nan_stays_in_its_chain(dtype, d):
    B, T, H = 2, 300, 4
    inp = W.prefill_inputs(batch=B, seqlen=T, heads=H, dk=d, dv=d, dtype=dtype, device=DEV,
                           seed=77, init="normal")
    nan = float("nan")
    # (sequence, head, token) of each poisoned value
    pq, pg, pb = (0, 1, 100), (1, 2, 150), (1, 0, 200)
    inp["q"][pq[0], pq[2], pq[1], 5] = nan
    inp["g"][pg[0], pg[2], pg[1], 7] = nan
    inp["beta"][pb[0], pb[2], pb[1]] = nan
    print(f"prefill NaN propagation {dtype} d={d}: q at {pq}, g at {pg}, beta at {pb}", flush=True)
    o, fs, _ = kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             inp["init_state"])
    torch.cuda.synchronize()
    o_ref, fs_ref, _ = O.kda_fwd(*(inp[k].cpu() for k in ("q", "k", "v", "g", "beta")),
                                 inp["init_state"].cpu())
    tol = TOL[dtype]
    poisoned = {(pg[0], pg[1]): pg[2], (pb[0], pb[1]): pb[2]}
    for n in range(B):
        for h in range(H):
            if (n, h) in poisoned:
                t = poisoned[(n, h)]
                c0 = (t // 64) * 64
                assert np.all(np.isfinite(o_ref[n, :t, h])) and not np.isfinite(fs_ref[n, h]).any()
                assert_close(f"chain ({n},{h}) before its poisoned chunk", o[n, :c0, h],
                             o_ref[n, :c0, h], tol)
                assert _all_nonfinite(o[n, t:, h]), f"chain ({n},{h}): outputs from {t} on"
                assert _all_nonfinite(fs[n, h]), f"chain ({n},{h}): final state"
            elif (n, h) == (pq[0], pq[1]):
                t = pq[2]
                assert _all_nonfinite(o[n, t, h]), "the poisoned query's output"
                keep = [i for i in range(T) if i != t]
                assert_close(f"chain ({n},{h}) other outputs", o[n, keep, h], o_ref[n, keep, h],
                             tol)
                assert_close(f"chain ({n},{h}) final state", fs[n, h], fs_ref[n, h], tol)
            else:
                assert_close(f"clean chain ({n},{h})", o[n, :, h], o_ref[n, :, h], tol)
                assert_close(f"clean chain ({n},{h}) final state", fs[n, h], fs_ref[n, h], tol)


def test_decode_nan_stays_in_its_chain():
    N, H, d, steps, dtype = 4, 2, 128, 5, torch.bfloat16
    gen = W.make_generator(78, DEV)
    s0 = W.decode_initial_state(num_seqs=N, heads=H, dk=d, dv=d, gen=gen, device=DEV)
    xs = [W.decode_step_inputs(num_seqs=N, heads=H, dk=d, dv=d, dtype=dtype, gen=gen, device=DEV)
          for _ in range(steps)]
    nan = float("nan")
    t = 2
    xs[t]["q"][2, 0, 3] = nan       # chain (2, 0): only its output at step t
    xs[t]["g"][0, 1, 9] = nan       # chain (0, 1): state from step t on
    xs[t]["beta"][3, 1] = nan       # chain (3, 1): state from step t on
    print("decode NaN propagation: q at (2,0), g at (0,1), beta at (3,1), step 2", flush=True)
    state = s0.clone()
    outs = []
    for x in xs:
        outs.append(kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state).clone())
    torch.cuda.synchronize()
    o = torch.stack(outs)
    st = lambda key: torch.stack([x[key] for x in xs]).cpu()
    o_ref, s_ref = O.kda_decode(st("q"), st("k"), st("v"), st("g"), st("beta"), s0.cpu())
    tol = TOL[dtype]
    for n in range(N):
        for h in range(H):
            if (n, h) in ((0, 1), (3, 1)):
                assert_close(f"chain ({n},{h}) before step {t}", o[:t, n, h], o_ref[:t, n, h], tol)
                assert _all_nonfinite(o[t:, n, h]) and _all_nonfinite(state[n, h])
            elif (n, h) == (2, 0):
                assert _all_nonfinite(o[t, n, h])
                keep = [i for i in range(steps) if i != t]
                assert_close(f"chain ({n},{h}) other steps", o[keep, n, h], o_ref[keep, n, h], tol)
                assert_close(f"chain ({n},{h}) state", state[n, h], s_ref[n, h], tol / 10)
            else:
                assert_close(f"clean chain ({n},{h})", o[:, n, h], o_ref[:, n, h], tol)
                assert_close(f"clean chain ({n},{h}) state", state[n, h], s_ref[n, h], tol / 10)
