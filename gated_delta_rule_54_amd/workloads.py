"""Seeded synthetic inputs for the KDA operator.

This module draws random inputs and nothing else: it holds none of the
operator's arithmetic, so the HIP path and the CPU oracle can both be fed
from it.  Inputs follow the distributions the workloads below are specified
with: q, k, v ~ N(0, 1) (q and k left raw; the operator normalises them),
the per-channel log-gate g = logsigmoid(N(0, 1) + 3) with shape [B, T, H, dk],
beta = sigmoid(N(0, 1)), and initial states either zero or N(0, 0.02^2).

Draw order (fixed, so a seed names one input set): [varlen lengths], q, k, v,
g, beta, [init_state].  Random q, k, v are drawn in fp32 and rounded to the
workload dtype (round-to-nearest-even).  A torch.Generator on the target
device is used, so GPU-drawn and CPU-drawn inputs differ; every comparison
copies the very tensors the GPU used to the host.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode" | "varlen"
    batch: int
    heads: int
    seqlen: int          # prefill: tokens per sequence; varlen: 0 (drawn)
    dk: int
    dv: int
    dtype: torch.dtype
    init: str            # "zeros" | "normal"
    seed: int
    steps: int = 0       # decode: number of sequential single-token steps
    num_seqs: int = 0    # decode / varlen: number of sequences
    len_range: tuple = (0, 0)  # varlen: inclusive length range
    ckpt_every: int = 0

    def describe(self) -> str:
        dt = "fp32" if self.dtype == torch.float32 else "bf16"
        if self.kind == "decode":
            return (f"decode N={self.num_seqs} H={self.heads} d={self.dk} {dt} "
                    f"steps={self.steps}")
        if self.kind == "varlen":
            return (f"varlen N={self.num_seqs} len~U{list(self.len_range)} H={self.heads} "
                    f"d={self.dk} {dt}")
        s = f"prefill B={self.batch} H={self.heads} T={self.seqlen} d={self.dk} {dt}"
        if self.ckpt_every:
            s += f" ckpt_every={self.ckpt_every}"
        return s


# The five workloads the operator is specified and measured on.
FP32_SMALL = Workload("fp32_B1_H2_T256_d64", "prefill", 1, 2, 256, 64, 64, torch.float32,
                      "zeros", 1000)
PREFILL_8K = Workload("bf16_B1_H32_T8192_d128", "prefill", 1, 32, 8192, 128, 128,
                      torch.bfloat16, "zeros", 1001)
DECODE_256 = Workload("decode_N256_H32_d128_x1024", "decode", 256, 32, 0, 128, 128,
                      torch.bfloat16, "normal", 1002, steps=1024, num_seqs=256)
VARLEN_16 = Workload("varlen_N16_len1K-32K_H32_d128", "varlen", 1, 32, 0, 128, 128,
                     torch.bfloat16, "normal", 1003, num_seqs=16, len_range=(1024, 32768))
PREFILL_1M = Workload("bf16_B1_H32_T1M_d128_ckpt64K", "prefill", 1, 32, 1 << 20, 128, 128,
                      torch.bfloat16, "zeros", 1004, ckpt_every=65536)

ALL = {w.name: w for w in (FP32_SMALL, PREFILL_8K, DECODE_256, VARLEN_16, PREFILL_1M)}


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def draw_gate(shape, gen, device, shift: float = 3.0):
    """Per-channel log forget gate, logsigmoid(N(0,1) + shift) (always < 0)."""
    return F.logsigmoid(_randn(shape, gen, device) + shift)


def draw_beta(shape, gen, device):
    return torch.sigmoid(_randn(shape, gen, device))


def draw_lengths(num_seqs: int, lo: int, hi: int, gen, device) -> torch.Tensor:
    """Varlen lengths, uniform integers in [lo, hi]; drawn first."""
    return torch.randint(lo, hi + 1, (num_seqs,), generator=gen, device=device)


def cu_from_lengths(lengths: torch.Tensor) -> torch.Tensor:
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64, device=lengths.device)
    cu[1:] = torch.cumsum(lengths.to(torch.int64), 0)
    return cu.to(torch.int32)


def prefill_inputs(*, batch: int, seqlen: int, heads: int, dk: int, dv: int,
                   dtype: torch.dtype, device, seed: int, init: str = "zeros",
                   num_seqs: Optional[int] = None, lengths: Optional[list] = None,
                   len_range: Optional[tuple] = None, gate_shift: float = 3.0,
                   gate_per_head: bool = False) -> dict:
    """Draw one prefill input set.  gate_per_head draws one log-gate per
    (token, head), [B, T, H] (Gated DeltaNet), instead of one per channel.

    Dense: [batch, seqlen, H, d].  Varlen: pass `len_range` (lengths drawn
    from the generator first) or explicit `lengths`; inputs are packed as
    [1, sum(lengths), H, d] with int32 cu_seqlens.
    """
    gen = make_generator(seed, device)
    cu = None
    if len_range is not None or lengths is not None:
        if lengths is None:
            lens = draw_lengths(num_seqs, len_range[0], len_range[1], gen, device)
        else:
            lens = torch.tensor(lengths, dtype=torch.int64, device=device)
        cu = cu_from_lengths(lens)
        batch, seqlen = 1, int(cu[-1].item())
        n = lens.numel()
    else:
        n = batch
    shp_k = (batch, seqlen, heads, dk)
    shp_v = (batch, seqlen, heads, dv)
    q = _randn(shp_k, gen, device).to(dtype)
    k = _randn(shp_k, gen, device).to(dtype)
    v = _randn(shp_v, gen, device).to(dtype)
    g = draw_gate((batch, seqlen, heads) if gate_per_head else shp_k, gen, device, gate_shift)
    beta = draw_beta((batch, seqlen, heads), gen, device)
    if init == "zeros":
        s0 = None
    elif init == "normal":
        s0 = 0.02 * _randn((n, heads, dk, dv), gen, device)
    else:
        raise ValueError(init)
    return dict(q=q, k=k, v=v, g=g, beta=beta, init_state=s0, cu_seqlens=cu)


def upstream_grads(*, batch: int, seqlen: int, heads: int, dk: int, dv: int, num_seqs: int,
                   dtype: torch.dtype, device, seed: int, final: bool = True) -> dict:
    """Upstream gradients for the backward: do ~ N(0,1) [B, T, H, dv] in the
    operand dtype and d_final ~ N(0,1) [N, H, dk, dv] fp32 (None unless final)."""
    gen = make_generator(seed, device)
    do = _randn((batch, seqlen, heads, dv), gen, device).to(dtype)
    dfin = _randn((num_seqs, heads, dk, dv), gen, device) if final else None
    return dict(do=do, dfinal=dfin)


def decode_step_inputs(*, num_seqs: int, heads: int, dk: int, dv: int, dtype: torch.dtype,
                       gen: torch.Generator, device, gate_per_head: bool = False) -> dict:
    """One decode step's fresh q, k, v, g, beta ([N, H, d] / [N, H]); g is
    [N, H] with gate_per_head."""
    q = _randn((num_seqs, heads, dk), gen, device).to(dtype)
    k = _randn((num_seqs, heads, dk), gen, device).to(dtype)
    v = _randn((num_seqs, heads, dv), gen, device).to(dtype)
    g = draw_gate((num_seqs, heads) if gate_per_head else (num_seqs, heads, dk), gen, device)
    beta = draw_beta((num_seqs, heads), gen, device)
    return dict(q=q, k=k, v=v, g=g, beta=beta)


def decode_initial_state(*, num_seqs: int, heads: int, dk: int, dv: int,
                         gen: torch.Generator, device) -> torch.Tensor:
    return 0.02 * _randn((num_seqs, heads, dk, dv), gen, device)


def workload_inputs(w: Workload, device) -> dict:
    """Prefill/varlen input set of a named workload."""
    if w.kind == "prefill":
        return prefill_inputs(batch=w.batch, seqlen=w.seqlen, heads=w.heads, dk=w.dk, dv=w.dv,
                              dtype=w.dtype, device=device, seed=w.seed, init=w.init)
    if w.kind == "varlen":
        return prefill_inputs(batch=1, seqlen=0, heads=w.heads, dk=w.dk, dv=w.dv,
                              dtype=w.dtype, device=device, seed=w.seed, init=w.init,
                              num_seqs=w.num_seqs, len_range=w.len_range)
    raise ValueError(f"{w.name} is not a prefill workload")
