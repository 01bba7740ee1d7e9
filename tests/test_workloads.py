"""Host logic of the seeded input generators (CPU)."""
import torch

from gated_delta_rule_54_amd import workloads as W


def test_seeded_and_distributed():
    a = W.prefill_inputs(batch=1, seqlen=512, heads=4, dk=64, dv=64, dtype=torch.bfloat16,
                         device="cpu", seed=5, init="normal")
    b = W.prefill_inputs(batch=1, seqlen=512, heads=4, dk=64, dv=64, dtype=torch.bfloat16,
                         device="cpu", seed=5, init="normal")
    for key in ("q", "k", "v", "g", "beta", "init_state"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.bfloat16 and a["g"].dtype == torch.float32
    assert (a["g"] < 0).all() and (a["beta"] > 0).all() and (a["beta"] < 1).all()
    alpha = a["g"].exp().mean().item()
    assert 0.9 < alpha < 0.96   # logsigmoid(N(0,1)+3): mean alpha ~ 0.93
    assert abs(a["init_state"].std().item() - 0.02) < 0.002


def test_varlen_lengths_drawn_first():
    w = W.VARLEN_16
    x = W.prefill_inputs(batch=1, seqlen=0, heads=2, dk=64, dv=64, dtype=torch.bfloat16,
                         device="cpu", seed=w.seed, num_seqs=w.num_seqs, len_range=w.len_range,
                         init=w.init)
    cu = x["cu_seqlens"]
    lens = cu[1:] - cu[:-1]
    assert cu.dtype == torch.int32 and cu[0] == 0 and int(cu[-1]) == x["q"].shape[1]
    assert (lens >= 1024).all() and (lens <= 32768).all()
    assert x["init_state"].shape == (w.num_seqs, 2, 64, 64)


def test_workload_table():
    assert set(W.ALL) == {W.FP32_SMALL.name, W.PREFILL_8K.name, W.DECODE_256.name,
                          W.VARLEN_16.name, W.PREFILL_1M.name}
    assert W.PREFILL_1M.seqlen == 1 << 20 and W.PREFILL_1M.ckpt_every == 65536


def test_chunk_exponent_mode_shares():
    """The benchmark's count of chunks per exponent mode: constant gates put
    the chunk decay and the half decays at known values (g = -1: gamma = -64,
    fast; g = -2: halves -64, mid; one channel at g = -3: halves -96, exact)."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    g = torch.full((1, 192, 2, 4), -1.0)
    g[:, 64:128] = -2.0
    g[:, 128:192, 1, 3] = -3.0
    m = bench.chunk_exponent_modes(g)
    assert m == {"fast": 3 / 6, "mid": 2 / 6, "exact": 1 / 6}
