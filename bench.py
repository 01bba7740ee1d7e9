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
                                     kda_chunk_fwd_conv, kda_decode_step, kda_output_gate_norm,
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
                  ("kda_bwd_state_pass", "backward", 2), ("kda_bwd_intra", "backward", 2),
                  ("kda_bwd_exact", "backward", 2))


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


# Counter passes over --probe for the compute-side profile (at most 8 SQ and
# 2 GRBM counters fit one pass).
COUNTER_PASSES = (
    ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVES", "SQ_INSTS_VALU",
     "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM", "GRBM_GUI_ACTIVE"),
    ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
     "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
)
MI355X_SIMDS = 256 * 4
MI355X_XCDS = 8
COUNTER_FILE = os.path.join(ROOT, "profiles", "kda_compute_counters.md")
# token-heads of one probe call of each workload (prefill and backward: 8192 x 32)
_PROBE_TOKEN_HEADS = {"prefill": 8192 * 32, "backward": 8192 * 32, "decode": 256 * 32}


def write_counters(csvs, out: str = COUNTER_FILE, command: str = "") -> str:
    """Per-kernel compute counters from the passes of COUNTER_PASSES over
    `--probe` (rocprofv3 --pmc ... --output-format csv): MFMA FLOPs per call
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) and per token-head, MFMA busy share
    (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs)), instructions per
    wave, LDS bank-conflict cycles per LDS-active cycle."""
    import csv
    per = {}   # part -> counter -> summed value
    disp = {}  # part -> dispatches
    keys = {}  # part -> workload
    for path in csvs:
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        ids = sorted({int(r["Dispatch_Id"]) for r in rows})
        names = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in rows}
        last_pro = max((i for i in ids if "short_conv_kernel" in names[i]), default=ids[-1] + 1)
        seen = set()
        for r in rows:
            i = int(r["Dispatch_Id"])
            part, key = _probe_key(r["Kernel_Name"], i > last_pro)
            if key is None:
                continue
            keys[part] = key
            c = per.setdefault(part, {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if path == csvs[0] and i not in seen:
                seen.add(i)
                disp[part] = disp.get(part, 0) + 1
    calls = {key: n for _, key, n in _PROBE_KERNELS}
    lines = ["# Compute-side counters per kernel", "",
             "Two `rocprofv3 --pmc` passes over `python3 bench.py --probe` (each kernel",
             "dispatched for two calls of its workload; counters serialize the dispatches).",
             "Prefill and backward: B=1 T=8192 H=32 d=128 bf16 (262,144 token-heads per call).",
             "MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; busy = SQ_VALU_MFMA_BUSY_CYCLES /",
             f"(GRBM_GUI_ACTIVE / {MI355X_XCDS} x {MI355X_SIMDS} SIMDs; the csv's GRBM_GUI_ACTIVE is the",
             "sum over the XCDs' GRBM instances, each counting the dispatch: 2.98 M for a 151 us",
             "fill kernel); LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; VALU active",
             "and LDS wait = SQ_ACTIVE_INST_VALU, SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES;",
             "per-wave figures divide by SQ_WAVES.", ""]
    if not command:  # the passes' commands, from the csv paths (-d DIR -o pmc)
        rel = lambda x: os.path.relpath(x, ROOT)
        command = "\n".join(
            ["cd /tmp && export TMPDIR=/tmp && cd /root/repo"]
            + [f"rocprofv3 --pmc {' '.join(pas)} --output-format csv "
               f"-d {rel(os.path.dirname(os.path.abspath(path)))} -o pmc -- python3 bench.py --probe"
               for pas, path in zip(COUNTER_PASSES, csvs)]
            + ["python3 bench.py --write-counters " + " ".join(rel(x) for x in csvs)])
    lines += ["Commands:", "", "```", command, "```", ""]
    lines += ["| kernel | dispatches | MFMA GFLOP per call | MFMA FLOP per token-head | "
              "MFMA busy | VALU instr / wave | MFMA instr / wave | LDS instr / wave | "
              "SALU instr / wave | VMEM instr / wave | LDS bank conflict | VALU active | "
              "LDS wait share |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for part in sorted(per):
        c = per[part]
        key = keys[part]
        n = calls[key]
        g = lambda k: c.get(k, float("nan"))
        waves = g("SQ_WAVES")
        flop = g("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / n
        th = _PROBE_TOKEN_HEADS.get(key)
        # GRBM_GUI_ACTIVE appears in both passes, each the sum over the XCDs'
        # GRBM instances (one per XCD, each counting the whole dispatch)
        gui = g("GRBM_GUI_ACTIVE") / 2 / MI355X_XCDS
        ratio = lambda a, b: 100 * a / b if b else float("nan")
        lines.append(
            f"| {part} | {disp.get(part, 0)} | {flop / 1e9:.2f} | "
            f"{(flop / th) if th else float('nan'):,.0f} | "
            f"{ratio(g('SQ_VALU_MFMA_BUSY_CYCLES'), gui * MI355X_SIMDS):.1f} % | "
            f"{g('SQ_INSTS_VALU') / waves:,.0f} | {g('SQ_INSTS_MFMA') / waves:,.0f} | "
            f"{g('SQ_INSTS_LDS') / waves:,.0f} | {g('SQ_INSTS_SALU') / waves:,.0f} | "
            f"{g('SQ_INSTS_VMEM') / waves:,.0f} | "
            f"{ratio(g('SQ_LDS_BANK_CONFLICT'), g('SQ_LDS_IDX_ACTIVE')):.1f} % | "
            f"{ratio(g('SQ_ACTIVE_INST_VALU'), g('SQ_WAVE_CYCLES')):.1f} % | "
            f"{ratio(g('SQ_WAIT_INST_LDS'), g('SQ_WAVE_CYCLES')):.1f} % |")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


KERNEL_STATS_FILE = os.path.join(ROOT, "profiles", "kda_prefill_8k_decode_256x32_kernel_stats.md")
# (kernel-name fragment, template arguments shown, workload, from the trace?)
_STATS_ROWS = (
    ("kda_intra_chunk<__hip_bfloat16, 128, false, false>", "kda_intra_chunk<bf16, 128, false, false>",
     "prefill 8K, 20 timed calls (trace)", "prefill"),
    ("kda_state_pass<__hip_bfloat16, 128, 16, true>", "kda_state_pass<bf16, 128, 16, true>",
     "prefill 8K, 20 timed calls (trace)", "prefill"),
    ("decode_step_kernel<__hip_bfloat16, 128>", "decode_step_kernel<bf16, 128>", "decode (stats)", False),
    ("gate_norm_kernel<__hip_bfloat16, 128>", "gate_norm_kernel<bf16, 128>", "epilogue (stats)", False),
    ("short_conv_kernel<__hip_bfloat16, 4>", "short_conv_kernel<bf16, 4>", "prologue (stats)", False),
    ("kda_intra_chunk<__hip_bfloat16, 128, false, true>", "kda_intra_chunk<bf16, 128, false, true>",
     "prefill with the prologue fused, per segment (stats)", False),
    ("conv_state_out_kernel<__hip_bfloat16>", "conv_state_out_kernel<bf16>",
     "prefill with the prologue fused, carried-out inputs (stats)", False),
    ("kda_bwd_prep<__hip_bfloat16, 128, false>", "kda_bwd_prep<bf16, 128, false>",
     "backward, 10 timed calls, per segment (trace)", "backward"),
    ("kda_state_pass<__hip_bfloat16, 128, 16, false>", "kda_state_pass<bf16, 128, 16, false>",
     "backward's forward, 10 timed calls, per segment (trace)", "backward"),
    ("kda_bwd_state_pass<__hip_bfloat16, 128>", "kda_bwd_state_pass<bf16, 128>",
     "backward, 10 timed calls (trace)", "backward"),
    ("kda_bwd_intra<__hip_bfloat16, 128, false>", "kda_bwd_intra<bf16, 128, false>",
     "backward, 10 timed calls (trace)", "backward"),
    ("kda_bwd_exact<__hip_bfloat16, 128, false>", "kda_bwd_exact<bf16, 128, false>",
     "backward, 10 timed calls (trace; no chunk beyond the mid reference)", "backward"),
)


def write_kernel_stats(trace_csv: str, stats_csv: str, out: str = KERNEL_STATS_FILE,
                       warmup: int = 50, steps: int = 20) -> str:
    """Kernel durations from `rocprofv3 --kernel-trace --stats --output-format
    csv -- python3 bench.py --no-cpu-baseline`: the prefill kernels from the
    trace (the dispatches of the timed calls: 2 segments per call, after
    `warmup` warm-up calls), everything else pooled from the stats file."""
    bwd_warmup, bwd_steps = min(warmup, 5), max(1, steps // 2)  # as main() runs the backward
    import csv
    trace = list(csv.DictReader(open(trace_csv)))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    stats = {r["Name"]: r for r in csv.DictReader(open(stats_csv))}

    def short(name):
        return name.replace("void kda::(anonymous namespace)::", "").split("(")[0]

    # the commands that produced the two files (rocprofv3 names them after
    # the -o prefix inside the -d directory)
    out_dir = os.path.relpath(os.path.dirname(os.path.abspath(trace_csv)), ROOT)
    lines = ["# rocprofv3 kernel stats: prefill 8K x 32 heads, decode 256 x 32 heads, "
             "epilogue, prologue, backward", "",
             "Command (run from the repository root on one MI355X), then the summary:", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d {out_dir} "
             "-o bench -- python3 bench.py --no-cpu-baseline",
             f"    python3 bench.py --write-kernel-stats {os.path.relpath(trace_csv, ROOT)} "
             f"{os.path.relpath(stats_csv, ROOT)}", "",
             f"Kernel durations (ns). Prefill rows: the dispatches of the {steps} timed calls "
             f"(after {warmup} warm-up calls, two segments per call) from the trace. Backward "
             f"rows: the dispatches of the backward section's {bwd_steps} timed calls (after "
             f"{bwd_warmup} warm-up calls; the window between the ends of their neighbouring "
             "calls' last kernels) from the trace. The other rows pool every call of the "
             "kernel in the run (stats file).", "",
             "| Kernel | Workload | Calls | Average | Min | Max |", "|---|---|---|---|---|---|"]
    # the backward section's timed calls: each call ends with one kda_bwd_exact
    # dispatch, and the section runs the first backward calls of the run
    bwd_end = [int(r["End_Timestamp"]) for r in trace
               if short(r["Kernel_Name"]) == "kda_bwd_exact<__hip_bfloat16, 128, false>"]
    bwd_window = None
    if len(bwd_end) >= bwd_warmup + bwd_steps and bwd_warmup >= 1:
        bwd_window = (bwd_end[bwd_warmup - 1], bwd_end[bwd_warmup + bwd_steps - 1])
    for frag, label, workload, from_trace in _STATS_ROWS:
        if from_trace == "backward":
            if bwd_window is None:
                continue
            d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace
                 if short(r["Kernel_Name"]) == frag
                 and bwd_window[0] < int(r["Start_Timestamp"]) <= bwd_window[1]]
            if not d:
                continue
            lines.append(f"| `{label}` | {workload} | {len(d)} | {sum(d) / len(d):,.0f} | "
                         f"{min(d):,} | {max(d):,} |")
        elif from_trace:
            d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                 for r in trace if short(r["Kernel_Name"]) == frag]
            # the prefill section's zero-token setup call launches the state
            # pass once (over no chunks) before the warm-up calls
            lead = 1 if frag.startswith("kda_state_pass") else 0
            d = d[lead + 2 * warmup: lead + 2 * (warmup + steps)]
            if not d:
                continue
            lines.append(f"| `{label}` | {workload} | {len(d)} | {sum(d) / len(d):,.0f} | "
                         f"{min(d):,} | {max(d):,} |")
        else:
            r = next((v for k, v in stats.items() if short(k) == frag), None)
            if r is None:
                continue
            lines.append(f"| `{label}` | {workload} | {int(r['Calls'])} | "
                         f"{float(r['AverageNs']):,.0f} | {int(float(r['MinNs'])):,} | "
                         f"{int(float(r['MaxNs'])):,} |")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


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


def bench_prologue_fused(inp, steps: int, warmup: int, rounds: int = 3):
    """The prologue -> operator chain on the 8K x 32-head prefill workload
    (its q, k, v taken as the prologue's inputs; seeded width-4 filters,
    biases and carried states): kda_short_conv_swish on each of q, k, v then
    kda_chunk_fwd, against kda_chunk_fwd_conv, rounds alternating; best
    round of each, microseconds per call."""
    B, T, H, d = inp["q"].shape
    C = H * d
    gen = torch.Generator(device="cuda").manual_seed(1011)
    w = [0.5 * torch.randn(C, 4, generator=gen, device="cuda") for _ in range(3)]
    b = [0.1 * torch.randn(C, generator=gen, device="cuda") for _ in range(3)]
    s = [torch.randn(B, C, 3, generator=gen, device="cuda") for _ in range(3)]
    so = [torch.empty_like(t) for t in s]
    ys = [torch.empty(B, T, C, dtype=inp["q"].dtype, device="cuda") for _ in range(3)]
    o = torch.empty_like(inp["v"])
    fs = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    desc = make_desc(batch=B, num_seqs=B, seqlen=T, heads=H, dk=d, dv=d, dtype=inp["q"].dtype)
    ws = torch.empty(chunk_fwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def two_step():
        for i, n in enumerate(("q", "k", "v")):
            kda_short_conv_swish(inp[n].reshape(B, T, C), w[i], b[i], s[i], state_out=so[i],
                                 out=ys[i], stream=stream)
        kda_chunk_fwd(ys[0].reshape(B, T, H, d), ys[1].reshape(B, T, H, d),
                      ys[2].reshape(B, T, H, d), inp["g"], inp["beta"], inp["init_state"],
                      out=o, final_state=fs, workspace=ws, stream=stream)

    def fused():
        kda_chunk_fwd_conv(inp["q"], inp["k"], inp["v"], w, inp["g"], inp["beta"],
                           inp["init_state"], conv_bias=b, conv_state=s, conv_state_out=so,
                           out=o, final_state=fs, workspace=ws, stream=stream)

    best = {"two_step": float("inf"), "fused": float("inf")}
    for _ in range(rounds):
        for name, run in (("two_step", two_step), ("fused", fused)):
            for _ in range(warmup):
                run()
            torch.cuda.synchronize()
            e0, e1 = _events()
            e0.record(stream)
            for _ in range(steps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            best[name] = min(best[name], e0.elapsed_time(e1) / steps * 1e3)
    return best


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


def chunk_exponent_modes(g: torch.Tensor, chunk: int = 64, bound: float = -80.0) -> dict:
    """Share of (chunk, head) pairs in each exponent mode of the chunk form,
    from the per-channel log-gates [B, T, H, d] (T a multiple of the chunk):
    fast while every channel's chunk decay is >= bound, mid while each 32-token
    half decays by at most -bound, exact beyond."""
    B, T, H, d = g.shape
    x = g.float().reshape(B, T // chunk, chunk, H, d)
    half = chunk // 2
    gam = x.sum(2).amin(-1)
    h1 = x[:, :, :half].sum(2).amin(-1)
    h2 = x[:, :, half:].sum(2).amin(-1)
    fast = gam >= bound
    mid = ~fast & (h1 >= bound) & (h2 >= bound)
    n = gam.numel()
    return {"fast": fast.sum().item() / n, "mid": mid.sum().item() / n,
            "exact": (n - fast.sum().item() - mid.sum().item()) / n}


def bench_strong_gates(steps: int, warmup: int, shift: float = -1.0):
    """The prefill workload's shapes with fast-forgetting gates,
    g = logsigmoid(N(0,1) + shift) per channel: shift -1 (mean about -1.3 per
    token, so most chunks decay far beyond -80 and take the mid-chunk
    reference) or -4 (about -4 per token: every chunk beyond the mid
    reference's range, on the exact paths): prefill and backward per call."""
    w = W.PREFILL_8K
    inp = W.prefill_inputs(batch=w.batch, seqlen=w.seqlen, heads=w.heads, dk=w.dk, dv=w.dv,
                           dtype=w.dtype, device="cuda", seed=w.seed, init="normal",
                           gate_shift=shift)
    up = W.upstream_grads(batch=w.batch, seqlen=w.seqlen, heads=w.heads, dk=w.dk, dv=w.dv,
                          num_seqs=w.batch, dtype=w.dtype, device="cuda", seed=w.seed + 7)
    B, T, H, d = inp["q"].shape
    o = torch.empty_like(inp["v"])
    fs = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fwd = lambda: kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                inp["init_state"], out=o, final_state=fs, stream=stream)
    bwd = lambda: kda_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], up["do"],
                                inp["init_state"], up["dfinal"], stream=stream)
    res = {}
    for name, run, n in (("prefill", fwd, steps), ("backward", bwd, max(1, steps // 2))):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record(stream)
        for _ in range(n):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n * 1e3
    finite = bool(torch.isfinite(o).all().item())
    return {"workload": "prefill B=1 H=32 T=8192 d=128 bf16 as above, gates g = "
                        f"logsigmoid(N(0,1) {shift:+g}) per channel, nonzero initial state",
            "prefill_us_per_call": res["prefill"],
            "prefill_tokens_per_s": B * T / (res["prefill"] * 1e-6),
            "backward_us_per_call": res["backward"],
            "chunk_modes": chunk_exponent_modes(inp["g"]),
            "output_finite": finite}


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def device_warm_up(seconds: float = 0.2):
    """Bring the GPU to steady clocks with none of the benchmarked kernels:
    plain 1 GiB device-to-device copies back to back for `seconds` of wall
    time, then bf16 8192 x 8192 matrix products (torch) for as long.  From
    idle, the first calls run at lower clocks: the 8K prefill timed after 5
    warm-up calls measured ~13 % slower than after 50 with no load before
    them, 234-239 us per call after the copies alone and 229 us (twice, one
    process each) after copies and products, against ~228 us after 50
    warm-up calls."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    dst = torch.empty_like(src)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
    del src, dst
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn_like(a)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            c = a @ b
        torch.cuda.synchronize()
    del a, b, c


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

    # Setup before the warm-up calls: a zero-token call loads the library's
    # code object (it computes nothing; otherwise the first warm-up call loads
    # it while the GPU idles and its clocks fall back), then the device is
    # brought to steady clocks by neutral copies (device_warm_up).
    empty = lambda t: t[:, :0].contiguous()
    kda_chunk_fwd(empty(inp["q"]), empty(inp["k"]), empty(inp["v"]), empty(inp["g"]),
                  empty(inp["beta"]), stream=stream)
    torch.cuda.synchronize()
    device_warm_up()
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
                cores=threads, kind="oracle", cpu_model=_cpu_model(),
                sample=f"all {T} tokens of {heads_sample} of {full_heads} heads, {reps} repetitions "
                       f"(fp64, {dt:.1f} s wall on {threads} threads); value scaled to all heads")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _rocm_version() -> str:
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            continue
    return getattr(torch.version, "hip", None) or "unknown"


def _git_sha():
    import subprocess
    try:
        return subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        return None


def _source_sha256() -> str:
    """SHA-256 over the library sources, the binding and this file (the box
    that runs the benchmark has no git metadata)."""
    import glob
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_54_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "gated_delta_rule_54_amd", "*.py")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")) + [os.path.abspath(__file__)])
    for path in files:
        with open(path, "rb") as f:
            h.update(os.path.relpath(path, ROOT).encode())
            h.update(f.read())
    return h.hexdigest()


def _tensor_sha256(t: torch.Tensor) -> str:
    b = t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes()
    return hashlib.sha256(b).hexdigest()


def reproducibility(inputs_sha: dict) -> dict:
    props = torch.cuda.get_device_properties(0)
    return {"device": torch.cuda.get_device_name(0), "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "cpu_model": _cpu_model(),
            "host_threads": len(os.sched_getaffinity(0)), "rocm": _rocm_version(),
            "torch": torch.__version__, "git_sha": _git_sha(), "source_sha256": _source_sha256(),
            "inputs_sha256": inputs_sha}


def _flush(buf: torch.Tensor):
    """Overwrite a scratch buffer larger than the last-level cache (256 MB)."""
    buf.fill_(1)


def bench_prefill_flushed(inp, steps: int, flush_mb: int = 512):
    """The prefill call timed one at a time with HIP events, a 512 MB scratch
    write between calls (outside the events), so no input is served from the
    last-level cache by an earlier call."""
    B, T, H, d = inp["q"].shape
    o = torch.empty_like(inp["v"])
    fs = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    desc = make_desc(batch=B, num_seqs=B, seqlen=T, heads=H, dk=d, dv=d, dtype=inp["q"].dtype)
    ws = torch.empty(chunk_fwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    scratch = torch.empty(flush_mb << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    evs = [_events() for _ in range(steps)]
    for e0, e1 in evs:
        _flush(scratch)
        e0.record(stream)
        kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["init_state"],
                      out=o, final_state=fs, workspace=ws, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    return ms


def bench_varlen(steps: int, warmup: int):
    """The varlen workload: 16 packed sequences, lengths U[1024, 32768],
    32 heads, nonzero initial states; calls back to back."""
    w = W.VARLEN_16
    inp = W.workload_inputs(w, "cuda")
    cu = inp["cu_seqlens"]
    total = int(cu[-1].item())
    o = torch.empty_like(inp["v"])
    fs = torch.empty_like(inp["init_state"])
    desc = make_desc(batch=1, num_seqs=w.num_seqs, seqlen=total, heads=w.heads, dk=w.dk,
                     dv=w.dv, dtype=w.dtype)
    ws = torch.empty(chunk_fwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                inp["init_state"], cu, out=o, final_state=fs, workspace=ws,
                                stream=stream)
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
    th = total * w.heads
    sha = {k: _tensor_sha256(inp[k]) for k in ("q", "k", "v", "g", "beta", "init_state",
                                                 "cu_seqlens")}
    gbs = PREFILL_BYTES_PER_TH * th / (ms * 1e-3) / 1e9
    return {"workload": w.describe() + " (nonzero initial states)", "tokens": total,
            "lengths": torch.diff(cu).tolist(), "us_per_call": ms * 1e3,
            "value": total / (ms * 1e-3), "unit": "tokens/s",
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_token_head": PREFILL_BYTES_PER_TH,
                         "hbm_floor_us": PREFILL_BYTES_PER_TH * th / (HBM_PEAK_GBS * 1e9) * 1e6}}, sha


def bench_prefill_1m(steps: int = 3):
    """The 1,048,576-token workload (32 heads, checkpoints every 65,536
    tokens): one warm-up call, then `steps` calls back to back."""
    w = W.PREFILL_1M
    inp = W.workload_inputs(w, "cuda")
    B, T, H, d = inp["q"].shape
    o = torch.empty_like(inp["v"])
    fs = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    ck = torch.empty((B, T // w.ckpt_every, H, d, d), dtype=torch.float32, device="cuda")
    desc = make_desc(batch=B, num_seqs=B, seqlen=T, heads=H, dk=d, dv=d, dtype=w.dtype,
                     ckpt_every=w.ckpt_every)
    ws = torch.empty(chunk_fwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                ckpt_every=w.ckpt_every, out=o, final_state=fs, state_ckpt=ck,
                                workspace=ws, stream=stream)
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
    gbs = PREFILL_BYTES_PER_TH * th / (ms * 1e-3) / 1e9
    # inputs hashed over their first 65,536 tokens (hashing 40 GB would take minutes)
    sha = {k: _tensor_sha256(inp[k][:, :65536]) for k in ("q", "k", "v", "g", "beta")}
    del inp
    return {"workload": w.describe() + ", checkpoints written", "tokens": B * T,
            "us_per_call": ms * 1e3, "value": B * T / (ms * 1e-3), "unit": "tokens/s",
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_token_head": PREFILL_BYTES_PER_TH,
                         "hbm_floor_us": PREFILL_BYTES_PER_TH * th / (HBM_PEAK_GBS * 1e9) * 1e6}}, sha


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
    ap.add_argument("--write-counters", nargs="+", metavar="PASS_CSV",
                    help="write the compute-counter summary from the passes of "
                         "COUNTER_PASSES over --probe")
    ap.add_argument("--write-kernel-stats", nargs=2, metavar=("TRACE_CSV", "STATS_CSV"),
                    help="write the kernel-duration summary from a kernel-trace run of this "
                         "benchmark")
    ap.add_argument("--counter-command", default="",
                    help="the commands that made the passes, quoted in the summary")
    args = ap.parse_args()
    if args.write_traffic:
        t = write_traffic(*args.write_traffic)
        print(json.dumps({k: v for k, v in t.items() if k.endswith("_bytes")}))
        return
    if args.write_counters:
        print(write_counters(args.write_counters, command=args.counter_command))
        return
    if args.write_kernel_stats:
        print(write_kernel_stats(*args.write_kernel_stats, warmup=args.warmup, steps=args.steps))
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
    def progress(what):  # one stderr line per finished section
        print(f"[bench] {what} done", file=sys.stderr, flush=True)

    pf = bench_prefill(args.steps, args.warmup)
    progress("prefill")
    pf_cold_ms = bench_prefill_flushed(pf["inp"], args.steps)
    inputs_sha = {"prefill_8k": {k: _tensor_sha256(pf["inp"][k])
                                 for k in ("q", "k", "v", "g", "beta")}}
    tr_prefill, tr_decode, tr_epi, tr_pro, tr_bwd = measured_traffic()
    dc = bench_decode(min(args.warmup, 8))
    progress("decode")
    ep = bench_epilogue(args.steps, args.warmup)
    gm = bench_gate_modes()
    pl = bench_prologue(args.steps, args.warmup)
    pfu = bench_prologue_fused(pf["inp"], args.steps, min(args.warmup, 10))
    progress("epilogue, gate modes, prologue")
    bw = bench_backward(max(1, args.steps // 2), min(args.warmup, 5))
    progress("backward")
    vl, inputs_sha["varlen"] = bench_varlen(max(1, args.steps // 2), 2)
    m1, inputs_sha["prefill_1m_first_65536_tokens"] = bench_prefill_1m()
    progress("varlen, 1M tokens")
    sg = bench_strong_gates(max(2, args.steps // 2), 3)
    xg = bench_strong_gates(2, 1, shift=-4.0)
    progress("strong gates")
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
                     "mfma_frac": pf["achieved_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                     "us_per_call": pf["ms"] * 1e3,
                     "hbm_floor_us": PREFILL_BYTES_PER_TH * pf["token_heads"] / (HBM_PEAK_GBS * 1e9) * 1e6,
                     "flushed_us_per_call": pf_cold_ms * 1e3,
                     "flushed_frac": PREFILL_BYTES_PER_TH * pf["token_heads"] / (pf_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
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
        "prologue_fused": {"workload": "ShortConv (width 4) + Swish on q, k, v, then the "
                                       "prefill (B=1 H=32 T=8192 d=128 bf16): three prologue "
                                       "calls and kda_chunk_fwd, against kda_chunk_fwd_conv",
                           "two_step_us_per_call": pfu["two_step"],
                           "fused_us_per_call": pfu["fused"],
                           "fused_tokens_per_s": pf["tokens"] / (pfu["fused"] * 1e-6)},
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
                                  "kernel": "kda_chunk_bwd (kda_bwd_prep + forward state pass "
                                            "+ kda_bwd_state_pass + kda_bwd_intra)",
                                  "bytes_per_token_head": BACKWARD_BYTES_PER_TH}},
        "gate_modes": {"workload": "prefill B=1 H=16 d=128 bf16, T = 2K..64K: per-channel "
                                   "gates (KDA) vs one gate per token and head (GDN)",
                       "rows": gm},
        "varlen": vl,
        "prefill_1m": m1,
        "strong_gates": sg,
        "exact_gates": xg,
        "wall_s_prefill_loop": pf["wall"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pf["inp"], args.cpu_heads)
        progress("cpu baseline")
    line["reproducibility"] = reproducibility(inputs_sha)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
