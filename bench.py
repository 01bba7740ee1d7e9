"""Benchmark of the KDA operator on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

One step is one chunkwise prefill (kda_chunk_fwd: q/k L2 norm, in-chunk
gate prefix sum, intra-chunk UT transform, inter-chunk state pass) over the
B=1, H=32, T=8192, d=128 bf16 workload.  The step is timed with HIP events on
the stream the library launches on, K steps back to back between two device
synchronisations; inputs are resident in HBM before timing starts.  The
decode workload (256 sequences x 32 heads, d=128, 1024 sequential steps) is
timed the same way and reported in the "decode" object; the output epilogue,
the ShortConv prologue, the gate-mode sweep and the backward (gradients of
the same prefill workload) in objects of their own.  The CPU oracle is timed
on a bounded sample of the same prefill workload on this host's cores.

Prints ONE JSON line.

    python bench.py --probe

runs, for hardware-counter passes (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE),
one 1 GiB device-to-device copy (the calibration kernel: 1 GiB read, 1 GiB
written), then 2 prefill calls, 2 decode steps, 2 epilogue, 2 prologue and
2 backward calls, and prints nothing.

    python bench.py --write-traffic FETCH_CSV WRITE_CSV

turns the two passes' counter_collection.csv files into per-call bytes
(scaled by the copy's counters) and records them in
profiles/kda_hbm_traffic.json together with a hash of the kernel sources; the
benchmark reports them as the roofline "traffic" only while the sources still
match.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_delta_rule_54_amd import (chunk_bwd_workspace_bytes,  # noqa: E402
                                     chunk_fwd_workspace_bytes, kda_chunk_bwd, kda_chunk_fwd,
                                     kda_decode_step, kda_output_gate_norm,
                                     kda_short_conv_swish, make_desc)
from gated_delta_rule_54_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

# Algorithmic (compulsory) bytes and flops per token-head, d = 128:
#   prefill: q, k, v bf16 (3 x 256) + g fp32 (512) + beta (4) + o bf16 (256)
#   decode:  prefill I/O + the fp32 state read and written (2 x 65536)
#   prefill flops: 6 d^2 + 3 C d + C^2 per token-head at C = 64 (the
#   chunkwise FLOP model of the pages; the dense count of the kernels'
#   products is 6 d^2 + 10 C d + C^2 / 3)
PREFILL_BYTES_PER_TH = 3 * 256 + 512 + 4 + 256
#   backward: reads q, k, v, do bf16 (4 x 256), g (512), beta (4); writes dq,
#   dk, dv bf16 (3 x 256), dg (512), dbeta (4).  The per-sequence states
#   (init_state, d_final, d_init: 3 x 64 KiB per head) are left out, as the
#   prefill figure leaves out init and final states.
BACKWARD_BYTES_PER_TH = 4 * 256 + 512 + 4 + 3 * 256 + 512 + 4
DECODE_BYTES_PER_TH = PREFILL_BYTES_PER_TH + 2 * 128 * 128 * 4
PREFILL_FLOPS_PER_TH = 6 * 128 ** 2 + 3 * 64 * 128 + 64 ** 2
DECODE_FLOPS_PER_TH = 7 * 128 ** 2


KERNEL_SOURCES = ("gated_delta_rule_54_amd/csrc/kda_chunk_common.h",
                  "gated_delta_rule_54_amd/csrc/kda_chunk.hip",
                  "gated_delta_rule_54_amd/csrc/kda_chunk_bwd.hip",
                  "gated_delta_rule_54_amd/csrc/kda_decode.hip",
                  "gated_delta_rule_54_amd/csrc/kda_epilogue.hip",
                  "gated_delta_rule_54_amd/csrc/kda_conv.hip")
# prologue bytes per element (bf16): x read + y written (the state is negligible)
PROLOGUE_BYTES_PER_EL = 2 + 2
# output epilogue bytes per element (bf16): o read + gate read + y written
EPILOGUE_BYTES_PER_EL = 2 + 2 + 2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_hbm_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per prefill call / decode step / epilogue call from the
    committed counter passes, or None when the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None, None, None, None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None, None, None, None, None
    return (t.get("prefill_call_bytes"), t.get("decode_step_bytes"), t.get("epilogue_call_bytes"),
            t.get("prologue_call_bytes"), t.get("backward_call_bytes"))


def probe():
    """Kernels for the counter passes: calibration copy, prefill, decode."""
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = W.PREFILL_8K
    inp = W.workload_inputs(w, "cuda")
    for _ in range(2):
        kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["init_state"])
    torch.cuda.synchronize()
    del inp
    dw = W.DECODE_256
    gen = W.make_generator(dw.seed, "cuda")
    state = W.decode_initial_state(num_seqs=dw.num_seqs, heads=dw.heads, dk=dw.dk, dv=dw.dv,
                                   gen=gen, device="cuda")
    for _ in range(2):
        x = W.decode_step_inputs(num_seqs=dw.num_seqs, heads=dw.heads, dk=dw.dk, dv=dw.dv,
                                 dtype=dw.dtype, gen=gen, device="cuda")
        kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state)
    torch.cuda.synchronize()
    del state
    o, z, w = epilogue_inputs()
    for _ in range(2):
        kda_output_gate_norm(o, z, w)
    torch.cuda.synchronize()
    del o, z, w
    x, w, b, s = prologue_inputs()
    for _ in range(2):
        kda_short_conv_swish(x, w, b, s)
    torch.cuda.synchronize()
    del x, w, b, s
    inp, up = backward_inputs()
    for _ in range(2):
        kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], up["do"],
                      inp["init_state"], up["dfinal"])
    torch.cuda.synchronize()


# kernel-name fragment -> (key in the traffic file, calls the probe makes).
# The backward runs the forward's kernels too: those dispatched after the
# last prologue dispatch belong to the backward.
_PROBE_KERNELS = (("kda_intra_chunk", "prefill", 2), ("kda_state_pass", "prefill", 2),
                  ("decode_step_kernel", "decode", 2), ("gate_norm_kernel", "epilogue", 2),
                  ("short_conv_kernel", "prologue", 2), ("kda_bwd_prep", "backward", 2),
                  ("kda_bwd_state_pass", "backward", 2), ("kda_bwd_intra", "backward", 2))


def _probe_key(name: str, after_prologue: bool):
    for frag, key, _ in _PROBE_KERNELS:
        if frag in name:
            if key == "prefill" and after_prologue:
                return f"backward_fwd_{frag}", "backward"
            return frag, key
    return None, None


def write_traffic(fetch_csv: str, write_csv: str, out: str = TRAFFIC_FILE) -> dict:
    """Turn the two counter passes over `--probe` (rocprofv3 --pmc FETCH_SIZE,
    then WRITE_SIZE; csv output) into HBM bytes per call.  Each counter reads
    KiB per dispatch; it is scaled by what it reads for the 1 GiB copy."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if len(copy) != 1:
            raise SystemExit(f"{path}: expected one calibration copy, found {len(copy)}")
        last_pro = max((i for i, r in enumerate(rows) if "short_conv_kernel" in r["Kernel_Name"]),
                       default=len(rows))
        sums, parts = {}, {}
        for i, r in enumerate(rows):
            part, key = _probe_key(r["Kernel_Name"], i > last_pro)
            if key is not None:
                sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
                parts[part] = parts.get(part, 0.0) + float(r["Counter_Value"])
        return copy[0], sums, parts

    gib = 1 << 30
    f_copy, f_sum, f_parts = per_kernel(fetch_csv, "FETCH_SIZE")
    w_copy, w_sum, w_parts = per_kernel(write_csv, "WRITE_SIZE")
    fs, wsc = gib / (f_copy * 1024), gib / (w_copy * 1024)
    calls = {key: n for _, key, n in _PROBE_KERNELS}
    t = {"what": "HBM-side bytes (TCC FETCH_SIZE + WRITE_SIZE, each scaled by what it reads "
                 "for a 1 GiB device copy) per prefill call (B1 H32 T8192 d128 bf16), per "
                 "decode step (256 x 32 heads, d128), per epilogue call (262144 x 128 bf16), "
                 "per prologue call ([1, 8192, 4096] bf16, width 4) and per backward call "
                 "(B1 H32 T8192 d128 bf16, its forward recompute included)",
         "kernel_source_sha256": kernel_source_hash(),
         "calibration": {"copy_bytes": gib, "fetch_kib_read": f_copy, "write_kib_read": w_copy,
                         "fetch_scale": fs, "write_scale": wsc}}
    for key in calls:
        if key not in f_sum or key not in w_sum:
            raise SystemExit(f"no {key} dispatches in the counter files")
        unit = "step" if key == "decode" else "call"
        t[f"{key}_{unit}_bytes"] = (f_sum[key] * fs + w_sum[key] * wsc) * 1024 / calls[key]
    t["breakdown_bytes_per_call"] = {
        f"{part}_{kind}": parts[part] * scale * 1024 / 2
        for part in sorted(f_parts)
        for kind, parts, scale in (("fetch", f_parts, fs), ("write", w_parts, wsc))}
    with open(out, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    return t


def epilogue_inputs():
    """Synthetic epilogue operands at the prefill output's size."""
    gen = torch.Generator(device="cuda").manual_seed(1005)
    rows, dv = 8192 * 32, 128
    o = torch.randn(rows, dv, generator=gen, device="cuda").bfloat16()
    z = (2.0 * torch.randn(rows, dv, generator=gen, device="cuda")).bfloat16()
    w = 0.5 + torch.rand(dv, generator=gen, device="cuda")
    return o, z, w


def bench_epilogue(steps: int, warmup: int):
    o, z, w = epilogue_inputs()
    y = torch.empty_like(o)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        kda_output_gate_norm(o, z, w, out=y, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        kda_output_gate_norm(o, z, w, out=y, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = o.numel() * EPILOGUE_BYTES_PER_EL + w.numel() * 4
    return dict(ms=ms, rows=o.shape[0], achieved_gbs=nbytes / (ms * 1e-3) / 1e9, nbytes=nbytes)


def prologue_inputs():
    """Synthetic ShortConv + Swish operands at one projection of the prefill
    workload: [1, 8192, 32 heads x 128] bf16, width 4."""
    gen = torch.Generator(device="cuda").manual_seed(1007)
    C = 32 * 128
    x = torch.randn(1, 8192, C, generator=gen, device="cuda").bfloat16()
    w = 0.5 * torch.randn(C, 4, generator=gen, device="cuda")
    b = 0.1 * torch.randn(C, generator=gen, device="cuda")
    s = torch.randn(1, C, 3, generator=gen, device="cuda")
    return x, w, b, s


def bench_prologue(steps: int, warmup: int):
    x, w, b, s = prologue_inputs()
    y = torch.empty_like(x)
    so = torch.empty_like(s)
    stream = torch.cuda.current_stream()
    run = lambda: kda_short_conv_swish(x, w, b, s, state_out=so, out=y, stream=stream)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = x.numel() * PROLOGUE_BYTES_PER_EL
    return dict(ms=ms, achieved_gbs=nbytes / (ms * 1e-3) / 1e9)


def backward_inputs():
    """The prefill workload (B1 H32 T8192 d128 bf16, nonzero initial state)
    with seeded upstream gradients do and d_final."""
    w = W.PREFILL_8K
    inp = W.prefill_inputs(batch=w.batch, seqlen=w.seqlen, heads=w.heads, dk=w.dk, dv=w.dv,
                           dtype=w.dtype, device="cuda", seed=w.seed, init="normal")
    up = W.upstream_grads(batch=w.batch, seqlen=w.seqlen, heads=w.heads, dk=w.dk, dv=w.dv,
                          num_seqs=w.batch, dtype=w.dtype, device="cuda", seed=w.seed + 7)
    return inp, up


def bench_backward(steps: int, warmup: int):
    inp, up = backward_inputs()
    B, T, H, d = inp["q"].shape
    desc = make_desc(batch=B, num_seqs=B, seqlen=T, heads=H, dk=d, dv=d, dtype=inp["q"].dtype)
    ws = torch.empty(chunk_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], up["do"],
                                inp["init_state"], up["dfinal"], workspace=ws, stream=stream)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    th = B * T * H
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), ws_bytes=ws.numel(),
                achieved_gbs=BACKWARD_BYTES_PER_TH * th / (ms * 1e-3) / 1e9)


def bench_gate_modes(reps: int = 5):
    """Prefill at the shape of the pages' kernel comparison (batch 1, 16
    heads, 2K..64K tokens), d = 128 bf16: per-channel gates (KDA) against one
    gate per token and head (Gated DeltaNet), microseconds per call."""
    rows = []
    stream = torch.cuda.current_stream()
    for T in (2048, 4096, 8192, 16384, 32768, 65536):
        row = {"T": T}
        for mode, per_head in (("kda_us", False), ("gdn_us", True)):
            inp = W.prefill_inputs(batch=1, seqlen=T, heads=16, dk=128, dv=128,
                                   dtype=torch.bfloat16, device="cuda", seed=1006 + T,
                                   gate_per_head=per_head)
            o = torch.empty_like(inp["v"])
            fs = torch.empty((1, 16, 128, 128), dtype=torch.float32, device="cuda")
            run = lambda: kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                        out=o, final_state=fs, stream=stream)
            for _ in range(2):
                run()
            torch.cuda.synchronize()
            e0, e1 = _events()
            e0.record(stream)
            for _ in range(reps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            row[mode] = e0.elapsed_time(e1) / reps * 1e3
            del inp, o, fs
        row["kda_over_gdn"] = row["kda_us"] / row["gdn_us"]
        rows.append(row)
    return rows


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_prefill(steps: int, warmup: int):
    w = W.PREFILL_8K
    inp = W.workload_inputs(w, "cuda")
    B, T, H, d = inp["q"].shape
    o = torch.empty_like(inp["v"])
    fs = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    desc = make_desc(batch=B, num_seqs=B, seqlen=T, heads=H, dk=d, dv=d, dtype=w.dtype)
    ws = torch.empty(chunk_fwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["init_state"],
                      out=o, final_state=fs, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = _events()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    th = B * T * H
    sec = ms * 1e-3
    achieved_gbs = PREFILL_BYTES_PER_TH * th / sec / 1e9
    achieved_tf = PREFILL_FLOPS_PER_TH * th / sec / 1e12
    return dict(w=w, inp=inp, ms=ms, wall=wall, tokens=B * T, token_heads=th,
                achieved_gbs=achieved_gbs, achieved_tflops=achieved_tf,
                ws_bytes=ws.numel())


def bench_decode(warmup: int):
    w = W.DECODE_256
    N, H, d = w.num_seqs, w.heads, w.dk
    gen = W.make_generator(w.seed, "cuda")
    state = W.decode_initial_state(num_seqs=N, heads=H, dk=d, dv=d, gen=gen, device="cuda")
    xs = [W.decode_step_inputs(num_seqs=N, heads=H, dk=d, dv=d, dtype=w.dtype, gen=gen,
                               device="cuda") for _ in range(w.steps)]
    o = torch.empty((N, H, d), dtype=w.dtype, device="cuda")
    stream = torch.cuda.current_stream()
    scratch = state.clone()  # warm-up runs on a copy; the timed run starts from the real state
    for i in range(warmup):
        x = xs[i]
        kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], scratch, out=o, stream=stream)
    del scratch
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record(stream)
    for x in xs:
        kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, out=o, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    sec_step = ms_total * 1e-3 / w.steps
    th = N * H
    achieved_gbs = DECODE_BYTES_PER_TH * th / sec_step / 1e9
    return dict(w=w, ms_step=sec_step * 1e3, tokens_per_s=N * w.steps / (ms_total * 1e-3),
                achieved_gbs=achieved_gbs,
                achieved_tflops=DECODE_FLOPS_PER_TH * th / sec_step / 1e12)


def cpu_baseline(inp, heads_sample: int, min_seconds: float = 10.0):
    """Time the fp64 oracle on the prefill workload: all T tokens of the
    first `heads_sample` heads (one thread per head), repeated until at least
    `min_seconds` of wall time have passed, so the rate is a stable average."""
    from oracle import oracle as O
    O.build()
    sl = lambda x: x[:, :, :heads_sample].contiguous().cpu()
    q, k, v, g, b = (sl(inp[key]) for key in ("q", "k", "v", "g", "beta"))
    threads = min(O.default_threads(), heads_sample)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.kda_fwd(q, k, v, g, b, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    B, T, H, _ = q.shape
    # tokens/s of the whole problem (all heads) at this per-head rate
    full_heads = inp["q"].shape[2]
    return dict(value=reps * B * T * heads_sample / full_heads / dt, unit="tokens/s",
                cores=threads, kind="oracle",
                sample=f"all {T} tokens of {heads_sample} of {full_heads} heads, {reps} repetitions "
                       f"(fp64, {dt:.1f} s wall on {threads} threads); value scaled to all heads")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 50 untimed calls (~13 ms of prefill) bring the GPU to its steady clocks;
    # measured right after a few calls, the same kernels run ~15 % slower
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--probe", action="store_true",
                    help="run the kernels for hardware-counter passes and exit")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic file from the two counter passes over --probe")
    args = ap.parse_args()
    if args.write_traffic:
        t = write_traffic(*args.write_traffic)
        print(json.dumps({k: v for k, v in t.items() if k.endswith("_bytes")}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are "
                                   "not supported by this benchmark (--gpus must be 1)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)

    if args.probe:
        probe()
        return
    pf = bench_prefill(args.steps, args.warmup)
    tr_prefill, tr_decode, tr_epi, tr_pro, tr_bwd = measured_traffic()
    dc = bench_decode(min(args.warmup, 8))
    ep = bench_epilogue(args.steps, args.warmup)
    gm = bench_gate_modes()
    pl = bench_prologue(args.steps, args.warmup)
    bw = bench_backward(max(1, args.steps // 2), min(args.warmup, 2))
    w = pf["w"]
    value = pf["tokens"] / (pf["ms"] * 1e-3)
    line = {
        "metric": "KDA prefill tokens/s (H32,d128) + decode tok/s; % of MFMA/HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k,v ~ N(0,1) bf16, g = logsigmoid(N(0,1)+3), "
                "beta = sigmoid(N(0,1)))",
        "config": {"workload": "prefill B=1 H=32 T=8192 d_k=d_v=128 bf16 q/k/v, fp32 g/beta/"
                               "state, chunk 64", "global_batch": 1, "seq_len": 8192,
                   "heads": 32, "head_dim": 128, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": pf["achieved_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": pf["achieved_gbs"] / HBM_PEAK_GBS,
                     "traffic": (tr_prefill / (pf["ms"] * 1e-3) / 1e9) if tr_prefill else None,
                     "traffic_bytes_per_call": tr_prefill,
                     "kernel": "kda_chunk_fwd (intra-chunk + state-pass launches of one call)",
                     "bytes_per_token_head": PREFILL_BYTES_PER_TH,
                     "mfma_tflops": pf["achieved_tflops"],
                     "mfma_frac": pf["achieved_tflops"] / MFMA_BF16_PEAK_TFLOPS},
        "decode": {"workload": dc["w"].describe(), "value": dc["tokens_per_s"],
                   "unit": "tokens/s", "ms_per_step": dc["ms_step"],
                   "roofline": {"bound": "hbm", "achieved": dc["achieved_gbs"],
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dc["achieved_gbs"] / HBM_PEAK_GBS,
                                "traffic": (tr_decode / (dc["ms_step"] * 1e-3) / 1e9)
                                if tr_decode else None,
                                "traffic_bytes_per_step": tr_decode,
                                "kernel": "decode_step_kernel<bf16,128>",
                                "bytes_per_token_head": DECODE_BYTES_PER_TH}},
        "epilogue": {"workload": "head-wise RMSNorm x sigmoid gate on the prefill output: "
                                 "262144 rows (8192 tokens x 32 heads) x 128, bf16",
                     "us_per_call": ep["ms"] * 1e3,
                     "roofline": {"bound": "hbm", "achieved": ep["achieved_gbs"],
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": ep["achieved_gbs"] / HBM_PEAK_GBS,
                                  "traffic": (tr_epi / (ep["ms"] * 1e-3) / 1e9) if tr_epi else None,
                                  "kernel": "gate_norm_kernel<bf16,128>",
                                  "bytes_per_element": EPILOGUE_BYTES_PER_EL}},
        "prologue": {"workload": "ShortConv (width 4) + Swish on one projection of the prefill "
                                 "workload: [1, 8192, 4096] bf16, carried state in and out",
                     "us_per_call": pl["ms"] * 1e3,
                     "roofline": {"bound": "hbm", "achieved": pl["achieved_gbs"],
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": pl["achieved_gbs"] / HBM_PEAK_GBS,
                                  "traffic": (tr_pro / (pl["ms"] * 1e-3) / 1e9) if tr_pro else None,
                                  "kernel": "short_conv_kernel<bf16,4>",
                                  "bytes_per_element": PROLOGUE_BYTES_PER_EL}},
        "backward": {"workload": "gradients of the prefill workload (B=1 H=32 T=8192 "
                                 "d=128 bf16, nonzero initial state, seeded do and d_final): "
                                 "dq, dk, dv, dg, dbeta, d_init",
                     "us_per_call": bw["ms"] * 1e3, "value": bw["tokens_per_s"],
                     "unit": "tokens/s",
                     "roofline": {"bound": "hbm", "achieved": bw["achieved_gbs"],
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": bw["achieved_gbs"] / HBM_PEAK_GBS,
                                  "traffic": (tr_bwd / (bw["ms"] * 1e-3) / 1e9) if tr_bwd else None,
                                  "traffic_bytes_per_call": tr_bwd,
                                  "kernel": "kda_chunk_bwd (forward recompute + kda_bwd_prep + "
                                            "kda_bwd_state_pass + kda_bwd_intra)",
                                  "bytes_per_token_head": BACKWARD_BYTES_PER_TH}},
        "gate_modes": {"workload": "prefill B=1 H=16 d=128 bf16, T = 2K..64K: per-channel "
                                   "gates (KDA) vs one gate per token and head (GDN)",
                       "rows": gm},
        "wall_s_prefill_loop": pf["wall"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pf["inp"], args.cpu_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
