"""Benchmark of the FP8 rollout hot path on one MI355X.

One step = one Qwen3-8B-like attention block at 4096 tokens through every hot-path
call, inputs resident in HBM:
  weight sync of q/k/v/o (128x128 blockwise quantization, one batched call)
  -> 1x128 quantization of the block input X [4096, 4096]
  -> block-scaled W8A8 GEMMs q (4096x4096) and kv (k and v, 1024x4096 each, stored as one
     2048x4096 weight and run as one GEMM)
  -> FP8 KV-cache write of the k/v outputs (8 heads x 128) with scale recalibration
  -> 1x128 quantization of the attention output stand-in [4096, 4096]
  -> o GEMM (4096x4096).
`value` is the step's GEMM FLOPs divided by the measured step time (TFLOP/s).
Side legs (not in `value`) time the full 36-layer weight sync, one MoE layer's
grouped GEMMs (128 experts, Zipf top-8 routing of 4096 tokens) and one layer of the
20,000-token x 64-sequence FP8 KV step.  The CPU oracle is timed on a bounded sample
of the same step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-legs] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
TOKENS = 4096
HIDDEN = 4096
KV_DIM = 1024
DOM_ROUNDS = 5          # alternating rounds of step graphs with and without the q and o GEMMs
DOM_BURST = 20          # back-to-back launches of it: a short burst ...
DOM_SUSTAINED = 100     # ... and sustained load


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-legs", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-full", action="store_true",
                   help="time the oracle on the whole step (about 150 s) instead of the 512-token sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only copy 1 GiB device-to-device 3 times (reference for HBM byte counters)")
    p.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                   help="no GPU: turn four rocprofv3 --pmc output directories (FETCH_SIZE and WRITE_SIZE of a "
                        "bench run, then of a --calibrate-copy run) into the traffic summaries under profiles/")
    p.add_argument("--summarize-mfma", metavar="PMC_DIR",
                   help="no GPU: matrix-core utilisation of the GEMM kernels from a rocprofv3 --pmc run of "
                        "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_MFMA "
                        "SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS GRBM_GUI_ACTIVE")
    p.add_argument("--vendor-reference", action="store_true",
                   help="only time the vendor library's plain per-tensor-scaled FP8 GEMM (torch._scaled_mm) and "
                        "the bf16 matmul at the dense GEMM shapes, as context for the block-scaled GEMM's rate")
    p.add_argument("--profile-gemms", action="store_true",
                   help="only launch each GEMM workload of the side legs 8 times (a target for counter passes)")
    p.add_argument("--profile-quantizers", action="store_true",
                   help="only run the large quantizer workloads 3 times each: the 36-layer weight sync, one MoE "
                        "layer's expert weights, one 64 x 20,000-token KV layer (a target for counter passes)")
    p.add_argument("--summarize-quantizer-counters", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                   help="write profiles/quantizers_large_traffic.md from FETCH_SIZE / WRITE_SIZE passes over "
                        "--profile-quantizers and the 1 GiB copy calibration")
    p.add_argument("--summarize-gemm-counters", nargs=5,
                   metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE", "MFMA"),
                   help="write profiles/gemm_workloads_counters.md from counter passes over --profile-gemms")
    p.add_argument("--summarize-lds-counters", metavar="LDS_DIR",
                   help="write profiles/gemm_lds_counters.md from an LDS counter pass over --profile-gemms")
    p.add_argument("--summarize-legs-trace", metavar="TRACE_DIR",
                   help="write profiles/bench_legs_kernel_trace.md from a rocprofv3 --stats run of the full bench")
    p.add_argument("--summarize-trace", nargs="+", metavar="TRACE_DIR [BENCH_JSON]",
                   help="no GPU: per-kernel table from a rocprofv3 --kernel-trace --stats output directory "
                        "(optionally with the JSON line of a bench.py run of the same source)")
    return p.parse_args()


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_block_scaled_weight_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_tag: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on
    the current source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_rows(d):
    """(kernel name, counter, value) of every row of the rocprofv3 counter CSVs under d."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_launch(rows, counter, match):
    v = [x for k, c, x in rows if c.startswith(counter) and match(k)]
    return (sum(v) / len(v), len(v)) if v else (None, 0)


def summarize_counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """Write profiles/gemm_w8a8_4096_traffic.txt and profiles/quantizers_traffic.md from
    FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch), each scaled by what the same counter
    reads for a plain 1 GiB device copy."""
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    cf, cw = _counter_rows(cal_fetch_dir), _counter_rows(cal_write_dir)
    kib = (1 << 30) / 1024
    cal_f = max(x for _, c, x in cf if c.startswith("FETCH_SIZE"))
    cal_w = max(x for _, c, x in cw if c.startswith("WRITE_SIZE"))
    fs, ws = kib / cal_f, kib / cal_w
    dom = lambda k: "GemmCfg<256, 256" in k and "gemm_w8a8_kernel" in k
    f_raw, nf = _per_launch(fr, "FETCH_SIZE", dom)
    w_raw, nw = _per_launch(wr, "WRITE_SIZE", dom)
    fb, wb = f_raw * 1024 * fs, w_raw * 1024 * ws
    alg = TOKENS * HIDDEN + HIDDEN * HIDDEN + 2 * TOKENS * HIDDEN + 4 * (HIDDEN // 128) * TOKENS \
        + 4 * (HIDDEN // 128) ** 2
    cmd = "rocprofv3 --pmc {c} --output-format csv -d <out>/{d} -o {o} -- python3 bench.py {a}"
    lines = [
        "# HBM traffic of the dominant kernel (M=N=K=4096 block-scaled GEMM, 256x256 tiles)",
        "#",
        "# Counters, one pass each, on one MI355X from the repository root:",
        "#   " + cmd.format(c="FETCH_SIZE", d="pmc_FETCH_SIZE", o="bench", a="--steps 5 --warmup 2 --no-legs --no-cpu"),
        "#   " + cmd.format(c="WRITE_SIZE", d="pmc_WRITE_SIZE", o="bench", a="--steps 5 --warmup 2 --no-legs --no-cpu"),
        "# Calibration with a plain device copy of 1 GiB (torch copy_, 3 times):",
        "#   " + cmd.format(c="FETCH_SIZE", d="cal_FETCH_SIZE", o="cal", a="--calibrate-copy"),
        "#   " + cmd.format(c="WRITE_SIZE", d="cal_WRITE_SIZE", o="cal", a="--calibrate-copy"),
        "# Summary written by:",
        "#   python3 bench.py --summarize-counters <out>/pmc_FETCH_SIZE <out>/pmc_WRITE_SIZE "
        "<out>/cal_FETCH_SIZE <out>/cal_WRITE_SIZE",
        f"# The copy reads and writes {kib:.0f} KiB; the counters report {cal_f:.0f} KiB fetched and "
        f"{cal_w:.0f} KiB written, so FETCH_SIZE is scaled by {fs:.4f} and WRITE_SIZE by {ws:.4f}.",
        f"# Averages over every launch of the kernel in the run ({nf} and {nw} dispatches; KiB per dispatch).",
        "# bench.py uses hbm_bytes_per_launch only while source_digest matches gemm.hip.",
        f"source_digest: {source_digest('gemm.hip')}",
        f"fetch_kib_per_launch_raw: {f_raw:.1f}",
        f"write_kib_per_launch_raw: {w_raw:.1f}",
        f"fetch_scale: {fs:.4f}",
        f"write_scale: {ws:.4f}",
        f"fetch_bytes_per_launch: {fb:.0f}",
        f"write_bytes_per_launch: {wb:.0f}",
        f"hbm_bytes_per_launch: {fb + wb:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"# fetched / algorithmic operand bytes (A, B, scales): {fb / (alg - 2 * TOKENS * HIDDEN):.2f}x; "
        f"written / output bytes: {wb / (2 * TOKENS * HIDDEN):.2f}x",
    ]
    with open(os.path.join(ROOT, "profiles", "gemm_w8a8_4096_traffic.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    w_el = 2 * HIDDEN * HIDDEN + 2 * KV_DIM * HIDDEN
    quant = [("quant_weight_blk128_kernel", 2 * w_el, w_el + 4 * w_el // 16384),
             ("quant_act_g128_kernel", 2 * TOKENS * HIDDEN, TOKENS * HIDDEN + 4 * TOKENS * HIDDEN // 128),
             ("kv_amax_kernel", 2 * 2 * TOKENS * KV_DIM, 0),
             ("kv_write_kernel", 2 * 2 * TOKENS * KV_DIM + 8 * TOKENS, 2 * TOKENS * KV_DIM)]
    md = ["# HBM traffic of the quantizers in the benchmark step", "",
          f"Same counter runs and calibration as `gemm_w8a8_4096_traffic.txt` (FETCH_SIZE x{fs:.4f}, "
          f"WRITE_SIZE x{ws:.4f}), summarized by the same `bench.py --summarize-counters` command.", "",
          "| kernel | fetched (MB) | algorithmic read (MB) | written (MB) | algorithmic write (MB) |",
          "|---|---|---|---|---|"]
    for name, rd, wrt in quant:
        f_, _ = _per_launch(fr, "FETCH_SIZE", lambda k, n=name: n in k)
        w_, _ = _per_launch(wr, "WRITE_SIZE", lambda k, n=name: n in k)
        if f_ is None or w_ is None:
            continue
        md.append(f"| `{name}` | {f_ * 1024 * fs / 1e6:.2f} | {rd / 1e6:.2f} | {w_ * 1024 * ws / 1e6:.2f} | "
                  f"{wrt / 1e6:.2f} |")
    md += ["", "Figures are per launch (`quant_act_g128_kernel` runs twice per step, for the block input and",
           "the attention output; the KV write also reads each token's 8-byte slot)."]
    with open(os.path.join(ROOT, "profiles", "quantizers_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(lines))


# GEMM workloads of the side legs, as targets for counter passes: (label, kind, m, n, k);
# grouped workloads run the MoE layer's routing (128 experts, 4096 tokens top-8 = 32768 rows).
_GEMM_WORKLOADS = [
    ("dense 4096x4096x4096 (q, o)", "dense", 4096, 4096, 4096),
    ("dense 4096x2048x4096 (k and v stacked)", "dense", 4096, 2048, 4096),
    ("dense 512x4096x4096", "dense", 512, 4096, 4096),
    ("dense 512x1024x4096", "dense", 512, 1024, 4096),
    ("dense 4096x12288x4096 (gate/up)", "dense", 4096, 12288, 4096),
    ("dense 64x4096x4096 (q, o at 64 tokens)", "dense", 64, 4096, 4096),
    ("dense 64x12288x4096 (gate/up at 64 tokens)", "dense", 64, 12288, 4096),
    ("dense UE8M0 4096x4096x4096 (q, o; power-of-two scales)", "ue8m0", 4096, 4096, 4096),
    ("grouped MoE fc1 (128 experts, 32768 rows, 1536x2048)", "grouped", 32768, 1536, 2048),
    ("grouped MoE fc2 (128 experts, 32768 rows, 2048x768)", "grouped", 32768, 2048, 768),
]
_MOE_EXPERTS = 128


def _gemm_work(kind, m, n, k):
    """FLOPs and algorithmic bytes (operands, bf16 output, scales) of one workload."""
    g = _MOE_EXPERTS if kind == "grouped" else 1
    flops = 2 * m * n * k
    by = m * k + g * n * k + 2 * m * n + 4 * (k // 128) * m + 4 * g * (n // 128) * (k // 128)
    return flops, by


def profile_gemms():
    """Launch each GEMM workload 8 times, eagerly (a target for counter passes)."""
    import torch
    import fp8_block_scaled_weight_amd as fq
    from fp8_block_scaled_weight_amd import synth
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    _, off, _ = synth.moe_routing(0)
    offs = torch.from_numpy(off).to(dev)
    for label, kind, m, n, k in _GEMM_WORKLOADS:
        e = _MOE_EXPERTS if kind == "grouped" else 1
        a = torch.randint(0, 0x77, (m, k), dtype=torch.uint8, device=dev, generator=gen)
        asc = torch.rand((k // 128, m), device=dev, generator=gen)
        b = torch.randint(0, 0x77, (e * n, k), dtype=torch.uint8, device=dev, generator=gen)
        bsc = torch.rand((e * n // 128, k // 128), device=dev, generator=gen)
        if kind == "ue8m0":
            asc, bsc = torch.exp2(torch.round(torch.log2(asc))), torch.exp2(torch.round(torch.log2(bsc)))
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        for _ in range(8):
            if kind == "grouped":
                fq.fp8q_grouped_gemm_w8a8(a, asc, b.view(e, n, k), bsc.view(e, n // 128, k // 128), offs, y)
            elif kind == "ue8m0":
                fq.fp8q_gemm_w8a8_ue8m0(a, asc, b, bsc, y)
            else:
                fq.fp8q_gemm_w8a8_blkscaled(a, asc, b, bsc, y)
        torch.cuda.synchronize()
        log(f"profiled: {label}")


_SYNC_SHAPES = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (12288, 4096), (12288, 4096), (4096, 12288)]
_MOE_WEIGHT_SHAPES = [(128 * 2 * 768, 2048), (128 * 2048, 768)]
_QUANT_CALLS = 3


def profile_quantizers():
    """The large quantizer workloads, _QUANT_CALLS calls each, eagerly: the 36-layer weight sync
    (one batched call), one MoE layer's expert weights, one 64 x 20,000-token KV layer with
    recalibration, then FP8 decode attention over that cache (a target for counter passes)."""
    import torch
    import fp8_block_scaled_weight_amd as fq
    from fp8_block_scaled_weight_amd import synth
    dev = torch.device("cuda:0")
    for label, shapes in (("36-layer sync", _SYNC_SHAPES * 36), ("MoE expert weights", _MOE_WEIGHT_SHAPES)):
        descs = [(synth.device_normal_bf16((n, k), 0.02, dev, 3, i, 0, outlier_p=1e-3, outlier_mult=20.0),
                  torch.empty((n, k), dtype=torch.uint8, device=dev),
                  torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev)) for i, (n, k) in enumerate(shapes)]
        for _ in range(_QUANT_CALLS):
            fq.fp8q_quant_weight_blk128(descs)
        torch.cuda.synchronize()
        log(f"profiled: {label}")
        del descs
        torch.cuda.empty_cache()
    slots_np, pages = synth.kv_slot_mapping()
    t = len(slots_np)
    k = synth.device_kv(t, dev, 5, 0, 0)
    v = synth.device_kv(t, dev, 5, 0, 1)
    sl = torch.from_numpy(slots_np).to(dev)
    kc = torch.empty((pages, 16, 8, 128), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    ks, vs = torch.ones(1, device=dev), torch.ones(1, device=dev)
    for _ in range(_QUANT_CALLS):
        fq.fp8q_kv_quant(k, v, sl, kc, vc, ks, vs, 448.0, recalibrate=True)
    torch.cuda.synchronize()
    log("profiled: KV layer")
    # FP8 decode attention over the cache just written (the bench leg's shape, stored query scale)
    import numpy as np
    seqs, hq = 64, 32
    bt = torch.from_numpy((slots_np.reshape(seqs, -1)[:, ::16] // 16).astype(np.int32)).to(dev)
    lens = torch.full((seqs,), t // seqs, dtype=torch.int32, device=dev)
    qd = synth.device_activation(seqs, hq * 128, dev, 5, 0, 50).view(seqs, hq, 128)
    od = torch.empty((seqs, hq, 128), dtype=torch.bfloat16, device=dev)
    qsc = torch.full((1,), 0.01, device=dev)
    for _ in range(_QUANT_CALLS):
        fq.fp8q_paged_decode_attention(qd, kc, vc, bt, lens, qsc, ks, vs, 128 ** -0.5, od)
    torch.cuda.synchronize()
    log("profiled: decode attention")


def summarize_quantizer_counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """HBM bytes per call of the --profile-quantizers workloads (FETCH_SIZE / WRITE_SIZE scaled by
    the 1 GiB copy calibration) against their algorithmic bytes.  Writes
    profiles/quantizers_large_traffic.md."""
    import csv
    import glob

    def dispatches(d):
        per = {}
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                if "fp8q" not in r["Kernel_Name"]:
                    continue
                e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"].split("(")[0]})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [per[k] for k in sorted(per)]

    cf, cw = _counter_rows(cal_fetch_dir), _counter_rows(cal_write_dir)
    kib = (1 << 30) / 1024
    fs = kib / max(x for _, c, x in cf if c.startswith("FETCH_SIZE"))
    ws = kib / max(x for _, c, x in cw if c.startswith("WRITE_SIZE"))
    fd, wd = dispatches(fetch_dir), dispatches(write_dir)
    from fp8_block_scaled_weight_amd import synth
    t = len(synth.kv_slot_mapping()[0])
    row = 8 * 128
    sync_el = sum(n * k for n, k in _SYNC_SHAPES) * 36
    moe_el = sum(n * k for n, k in _MOE_WEIGHT_SHAPES)
    # (label, launches per call, algorithmic read and write bytes per call)
    work = [("36-layer weight sync (252 tensors, one call)", -(-252 // 64), 2 * sync_el, sync_el + 4 * sync_el / 16384),
            ("MoE expert weights of one layer (2 tensors)", 1, 2 * moe_el, moe_el + 4 * moe_el / 16384),
            ("KV layer, 64 x 20,000 tokens, recalibrate + write", 3, 2 * (2 * 2 * t * row) + 2 * 8 * t,
             2 * t * row),
            ("FP8 decode attention over that cache (64 sequences, 32 query heads)", 1,
             2 * t * row + 2 * 64 * 32 * 128 + 4 * (t // 16) + 4 * 64, 2 * 64 * 32 * 128)]
    md = ["# HBM traffic of the large quantizer workloads and the decode attention", "",
          "Counter passes over `python3 bench.py --profile-quantizers` (each workload called "
          f"{_QUANT_CALLS} times, eagerly), one MI355X, repository root, TMPDIR=/tmp:", "",
          "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/q_fetch -o q -- python3 bench.py --profile-quantizers",
          "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/q_write -o q -- python3 bench.py --profile-quantizers",
          "    python3 bench.py --summarize-quantizer-counters <out>/q_fetch <out>/q_write <out>/cal_FETCH_SIZE "
          "<out>/cal_WRITE_SIZE", "",
          f"FETCH_SIZE x{fs:.4f} and WRITE_SIZE x{ws:.4f} (the 1 GiB copy calibration of "
          "`gemm_w8a8_4096_traffic.txt`).  Bytes per call, averaged over the calls after the first.", "",
          "| workload | kernels | fetched GB | algorithmic read GB | written GB | algorithmic write GB |",
          "|---|---|---|---|---|---|"]
    pos = 0
    for label, launches, alg_r, alg_w in work:
        n = launches * _QUANT_CALLS
        f_, w_ = fd[pos:pos + n], wd[pos:pos + n]
        pos += n
        if len(f_) < n or len(w_) < n:
            continue
        per_call = lambda lst, c: sum(x.get(c, 0.0) for x in lst[launches:]) / (_QUANT_CALLS - 1)
        fb = per_call(f_, "FETCH_SIZE") * 1024 * fs
        wb = per_call(w_, "WRITE_SIZE") * 1024 * ws
        names = sorted({x["name"].replace("void fp8q::", "").replace("fp8q::", "") for x in f_})
        md.append(f"| {label} | {', '.join('`' + x + '`' for x in names)} | {fb / 1e9:.3f} | {alg_r / 1e9:.3f} | "
                  f"{wb / 1e9:.3f} | {alg_w / 1e9:.3f} |")
    md += ["", "Source digests: " + ", ".join(f"{n} {source_digest(n)}" for n in ("quant.hip", "kv_quant.hip",
                                                                                   "attention.hip"))]
    with open(os.path.join(ROOT, "profiles", "quantizers_large_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def _gemm_dispatches(d):
    """The GEMM dispatches of a rocprofv3 --pmc output directory in launch order: kernel
    name, duration and the summed value of each counter."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if "fp8q" not in r["Kernel_Name"] or "gemm" not in r["Kernel_Name"]:
                continue
            e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"].split("(")[0],
                                                       "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def summarize_lds_counters(lds_dir):
    """Per GEMM workload of --profile-gemms: LDS bank- and address-conflict cycles against
    the cycles the LDS serves indexed operations, the share of cycles its data FIFO was
    full, and LDS instructions per CU.  Writes profiles/gemm_lds_counters.md."""
    rows = _gemm_dispatches(lds_dir)
    md = ["# LDS counters of the GEMM workloads", "",
          "One counter pass over `python3 bench.py --profile-gemms` (each workload launched 8 times,",
          "eagerly), one MI355X, repository root, TMPDIR=/tmp:", "",
          "    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_ADDR_CONFLICT SQ_LDS_DATA_FIFO_FULL "
          "SQ_WAIT_INST_LDS SQ_INSTS_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE "
          "--output-format csv -d <out>/lds_pmc -o g -- python3 bench.py --profile-gemms",
          "    python3 bench.py --summarize-lds-counters <out>/lds_pmc", "",
          "Averages over dispatches 3-8 of each workload.  Columns: kernel duration; cycles the LDS is",
          "stalled by bank conflicts, and by address conflicts, as a share of the cycles it serves",
          "indexed operations (SQ_LDS_BANK_CONFLICT, SQ_LDS_ADDR_CONFLICT over SQ_LDS_IDX_ACTIVE); cycles",
          "its data FIFO was full (SQ_LDS_DATA_FIFO_FULL over SQ_LDS_IDX_ACTIVE); LDS instructions per CU",
          "(SQ_INSTS_LDS / 256).", "",
          "| workload | kernel | us | bank-conflict share | address-conflict share | FIFO-full share | "
          "LDS instructions per CU (thousands) |",
          "|---|---|---|---|---|---|---|"]
    for i, (label, _kind, _m, _n, _k) in enumerate(_GEMM_WORKLOADS):
        d = rows[8 * i + 2: 8 * i + 8]
        if not d:
            continue
        avg = lambda c: sum(x.get(c, 0.0) for x in d) / len(d)
        act = max(avg("SQ_LDS_IDX_ACTIVE"), 1.0)
        md.append(f"| {label} | `{d[0]['name'].replace('void ', '').replace('fp8q::', '')}` | {avg('ns') / 1e3:.1f} | "
                  f"{avg('SQ_LDS_BANK_CONFLICT') / act:.3f} | {avg('SQ_LDS_ADDR_CONFLICT') / act:.3f} | "
                  f"{avg('SQ_LDS_DATA_FIFO_FULL') / act:.3f} | {avg('SQ_INSTS_LDS') / 256 / 1e3:.2f} |")
    md += ["", "The fragment reads of the tile kernels are conflict-free by construction (16 distinct bank",
           "groups per 16-lane group); their conflict cycles come from the other LDS accesses.", "",
           f"gemm.hip source_digest: {source_digest('gemm.hip')}"]
    with open(os.path.join(ROOT, "profiles", "gemm_lds_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def summarize_gemm_counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, mfma_dir):
    """Per GEMM workload of --profile-gemms (matched by launch order, 8 dispatches each):
    average duration, HBM bytes fetched and written (FETCH_SIZE / WRITE_SIZE scaled by the
    1 GiB copy calibration) against the algorithmic bytes, and the matrix-core busy share.
    Writes profiles/gemm_workloads_counters.md."""
    dispatches = _gemm_dispatches
    cf, cw = _counter_rows(cal_fetch_dir), _counter_rows(cal_write_dir)
    kib = (1 << 30) / 1024
    fs = kib / max(x for _, c, x in cf if c.startswith("FETCH_SIZE"))
    ws = kib / max(x for _, c, x in cw if c.startswith("WRITE_SIZE"))
    fd, wd, md_ = dispatches(fetch_dir), dispatches(write_dir), dispatches(mfma_dir)
    md = ["# HBM traffic and matrix-core use of the GEMM workloads", "",
          "Counter passes over `python3 bench.py --profile-gemms` (each workload launched 8 times, eagerly),",
          "one MI355X, repository root, TMPDIR=/tmp:", "",
          "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/g_fetch -o g -- python3 bench.py --profile-gemms",
          "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/g_write -o g -- python3 bench.py --profile-gemms",
          "    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d <out>/g_mfma -o g -- "
          "python3 bench.py --profile-gemms",
          "    python3 bench.py --summarize-gemm-counters <out>/g_fetch <out>/g_write <out>/cal_FETCH_SIZE "
          "<out>/cal_WRITE_SIZE <out>/g_mfma", "",
          f"FETCH_SIZE x{fs:.4f} and WRITE_SIZE x{ws:.4f} (the 1 GiB copy calibration of "
          "`gemm_w8a8_4096_traffic.txt`).  Averages over dispatches 3-8 of each workload.  Matrix core busy:",
          "SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x the kernel duration x 2.4 GHz (the clock of the 5.0 PF peak).", "",
          "| workload | kernel | us | TFLOP/s | fetched MB | written MB | algorithmic MB | HBM / algorithmic | "
          "matrix core busy |",
          "|---|---|---|---|---|---|---|---|---|"]
    for i, (label, kind, m, n, k) in enumerate(_GEMM_WORKLOADS):
        flops, alg = _gemm_work(kind, m, n, k)
        sl = lambda lst: lst[8 * i + 2: 8 * i + 8]
        f_, w_, m_ = sl(fd), sl(wd), sl(md_)
        if not f_ or not w_ or not m_:
            continue
        avg = lambda lst, c: sum(x.get(c, 0.0) for x in lst) / len(lst)
        ns = avg(m_, "ns")
        fb = avg(f_, "FETCH_SIZE") * 1024 * fs
        wb = avg(w_, "WRITE_SIZE") * 1024 * ws
        busy = avg(m_, "SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * ns * 2.4)
        md.append(f"| {label} | `{m_[0]['name'].replace('void fp8q::', '')}` | {ns / 1e3:.1f} | "
                  f"{flops / ns / 1e3:.0f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {alg / 1e6:.1f} | "
                  f"{(fb + wb) / alg:.2f} | {busy:.3f} |")
    md += ["", f"gemm.hip source_digest: {source_digest('gemm.hip')}"]
    with open(os.path.join(ROOT, "profiles", "gemm_workloads_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def summarize_mfma(d):
    """Per GEMM instantiation: dispatches, average duration, matrix-core busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES summed over the 1024 SIMDs, against the kernel duration at
    the nominal 2.4 GHz and against GRBM_GUI_ACTIVE / 8 cycles per XCD) and the fraction
    of wave time spent waiting on counters (s_waitcnt).  Writes
    profiles/gemm_mfma_utilisation.txt."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            if "gemm_w8a8_kernel" not in k:
                continue
            key = k.split("(")[0].replace("void fp8q::", "")
            e = per.setdefault(key, {})
            disp = e.setdefault(r["Dispatch_Id"], {"ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            disp[r["Counter_Name"]] = disp.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = [
        "# Matrix-core utilisation of the block-scaled GEMMs in the benchmark step",
        "#",
        "# One counter pass on one MI355X from the repository root (TMPDIR=/tmp):",
        "#   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_MFMA "
        "SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS GRBM_GUI_ACTIVE --output-format csv -d <out>/pmc_mfma -o bench -- "
        "python3 bench.py --steps 5 --warmup 2 --no-legs --no-cpu",
        "# Summary written by:",
        "#   python3 bench.py --summarize-mfma <out>/pmc_mfma",
        "# Averages per dispatch (the first two dispatches of each kernel skipped).  Each",
        "# v_mfma_f32_32x32x64_f8f6f4 counts 64 busy cycles: 131072 FLOP per 64 cycles per SIMD is the FP8",
        "# dense peak rate.  SQ_WAVE_CYCLES and SQ_WAIT_INST_ANY count in the same unit, so their ratio is",
        "# the share of wave time spent in s_waitcnt (mostly the wait for a step's global-to-LDS copies).",
        "# GRBM_GUI_ACTIVE / 8 over the duration gives the mean shader clock of the run.",
        f"# gemm.hip source_digest: {source_digest('gemm.hip')}",
        "",
    ]
    for key, disps in per.items():
        ds = list(disps.values())[2:] or list(disps.values())
        avg = lambda c: sum(x.get(c, 0.0) for x in ds) / len(ds)
        ns = avg("ns")
        gpu_cycles = avg("GRBM_GUI_ACTIVE") / 8
        util = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (gpu_cycles * 1024) if gpu_cycles else float("nan")
        wait = avg("SQ_WAIT_INST_ANY") / avg("SQ_WAVE_CYCLES") if avg("SQ_WAVE_CYCLES") else float("nan")
        nominal = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * ns * 2.4)
        out += [
            f"[{key}]",
            f"dispatches: {len(ds)}",
            f"duration_us: {ns / 1e3:.2f}",
            f"grbm_gui_active_per_xcd: {gpu_cycles:.0f}",
            f"mean_clock_GHz: {gpu_cycles / ns:.2f}",
            f"mfma_instructions: {avg('SQ_INSTS_MFMA'):.0f}",
            f"mfma_busy_cycles_total: {avg('SQ_VALU_MFMA_BUSY_CYCLES'):.0f}",
            f"mfma_utilisation_at_2.4GHz: {nominal:.3f}   (busy cycles / (1024 SIMDs x duration x 2.4 GHz))",
            f"mfma_utilisation_vs_grbm_cycles: {util:.3f}",
            f"wave_time_waiting_on_counters: {wait:.3f}",
            f"lds_instructions: {avg('SQ_INSTS_LDS'):.0f}",
            f"lds_bank_conflict_cycles: {avg('SQ_LDS_BANK_CONFLICT'):.0f}",
            "",
        ]
    with open(os.path.join(ROOT, "profiles", "gemm_mfma_utilisation.txt"), "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def summarize_trace(d, bench_json=None):
    """Markdown table of per-kernel statistics from a rocprofv3 --stats output directory,
    written to profiles/bench_step_kernel_trace.md (with the live HIP-event duration of
    the dominant GEMM from a bench.py JSON line of the same source, when given)."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    md = [
        "# Kernel trace of the benchmark step (Qwen3-8B-like attention block, 4096 tokens)",
        "",
        "Command (on one MI355X, from the repository root, TMPDIR=/tmp):",
        "",
        "    rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o bench -- "
        "python3 bench.py --steps 20 --no-legs --no-cpu",
        "",
        "Table written by `python3 bench.py --summarize-trace <out>/trace [<bench json line>]` from "
        "`bench_kernel_stats.csv` (all",
        "launches in the run: warm-up, graph replays, per-call timing graphs and the direct launches that time",
        "the dominant GEMM).",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if "fp8q" not in r["Name"]:
            continue
        md.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{100 * float(r['TotalDurationNs']) / total:.1f} % |")
    dom = _dominant_loop_from_trace(d)
    live = {}
    if bench_json:
        line = [l for l in open(bench_json) if l.startswith("{")][-1]
        live = json.loads(line)["roofline"]
    md += [
        "",
        "The 256x256-tile GEMM instantiation runs only the two M=N=K=4096 projections (q, o) in this command.",
        "Its launches, grouped by pattern from `bench_kernel_trace.csv`, against bench.py's live HIP-event",
        "figures in the same run:",
        "",
        "| launches | traced | traced average (us) | live (us) |",
        "|---|---|---|---|",
    ]
    if dom:
        for key, what, lkey in (("step", "single launches between other kernels: the q and o GEMMs inside steps "
                                 "(eager and graph-replayed)", "avg_us"),
                                ("burst", f"a burst of {DOM_BURST} back to back (the last {DOM_BURST} of a run "
                                 f"of {DOM_BURST + 3})", "burst_avg_us"),
                                ("sustained", f"{DOM_SUSTAINED} back to back (the last {DOM_SUSTAINED} of a run "
                                 f"of {DOM_SUSTAINED + 3})", "sustained_avg_us"),
                                ("other", "other runs (per-call timing graphs)", None),
                                ("all", "all launches", None)):
            g = dom.get(key)
            if not g:
                continue
            lv = live.get(lkey, "") if lkey else ""
            md.append(f"| {what} | {g['n']} | {g['avg']:.2f} (min {g['min']:.2f}, max {g['max']:.2f}) | {lv} |")
        st = dom.get("step")
        if st:
            md += ["", f"`roofline.avg_us` is the in-step figure; from the trace: 2*4096^3 FLOP / {st['avg']:.2f} us "
                       f"/ 5.0 PF = {2 * 4096 ** 3 / (st['avg'] * 1e-6) / 5e15:.4f} of the FP8 peak."]
    md += [f"gemm.hip source_digest: {source_digest('gemm.hip')}"]
    with open(os.path.join(ROOT, "profiles", "bench_step_kernel_trace.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def _dominant_loop_from_trace(d):
    """Durations of the 256x256 FP32-scale GEMM's launches in a rocprofv3 kernel trace,
    grouped by launch pattern: single launches between other kernels (inside steps), the
    timed part of the burst and sustained runs of consecutive launches, other runs, all."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        return None
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    tag = "GemmCfg<256, 256, 2, 4, 2, 1>, false>"
    is_dom = [tag in r["Kernel_Name"] for r in rows]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    groups = {"step": [], "burst": [], "sustained": [], "other": [], "all": []}
    i = 0
    while i < len(rows):
        if not is_dom[i]:
            i += 1
            continue
        j = i
        while j < len(rows) and is_dom[j]:
            j += 1
        run = dur[i:j]
        groups["all"] += run
        if j - i == 1:
            groups["step"] += run
        elif j - i == DOM_BURST + 3:
            groups["burst"] += run[3:]
        elif j - i == DOM_SUSTAINED + 3:
            groups["sustained"] += run[3:]
        else:
            groups["other"] += run
        i = j
    return {k: {"n": len(v), "avg": sum(v) / len(v), "min": min(v), "max": max(v)} for k, v in groups.items() if v}


def summarize_legs_trace(d):
    """Markdown table of every libfp8q kernel in a rocprofv3 --stats run of the full bench
    (step and side legs), written to profiles/bench_legs_kernel_trace.md."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = [r for r in csv.DictReader(open(files[0])) if "fp8q" in r["Name"]]
    md = [
        "# Kernel trace of the full benchmark (step and side legs)",
        "",
        "Command (on one MI355X, from the repository root, TMPDIR=/tmp):",
        "",
        "    rocprofv3 --kernel-trace --stats --output-format csv -d <out>/legs -o legs -- "
        "python3 bench.py --steps 5 --warmup 2 --no-cpu",
        "",
        "Table written by `python3 bench.py --summarize-legs-trace <out>/legs` from `legs_kernel_stats.csv`.",
        "Every launch of the run is counted: warm-ups, graph replays and the per-call timing graphs.  A kernel",
        "that several legs run at different shapes (the few-token GEMM, the quantizers, the KV passes) mixes",
        "those shapes in its average; min and max bound them.  Kernels run by one leg at one shape: the",
        "attention kernels (64 sequences x 20,000 tokens; q_scale_kernel with recalibration), the MoE kernels",
        "(4096 tokens top-8 of 128 experts: route, gather, SwiGLU-quant, combine, fc1 and fc2 grouped GEMMs,",
        "the fused fc1 + SwiGLU-quant kernel).",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) |",
        "|---|---|---|---|---|",
    ]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0].replace("void ", "").replace("fp8q::", "")
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    md += ["", "Source digests: " + ", ".join(f"{f} {source_digest(f)}" for f in
                                             ("gemm.hip", "moe.hip", "attention.hip", "kv_quant.hip", "quant.hip"))]
    with open(os.path.join(ROOT, "profiles", "bench_legs_kernel_trace.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def vendor_reference():
    """Context only: the vendor library's plain FP8 GEMM (one scale per tensor, no blocks,
    no promotion) and the bf16 matmul at the dense shapes, timed like the legs."""
    import torch

    dev = torch.device("cuda:0")
    res = {}
    for m, n, k in ((4096, 4096, 4096), (4096, 1024, 4096), (4096, 12288, 4096), (4096, 4096, 16384)):
        x = torch.randn(m, k, device=dev).to(torch.float8_e4m3fn)
        w = torch.randn(n, k, device=dev).to(torch.float8_e4m3fn)
        one = torch.tensor(1.0, device=dev)
        ms8 = _time(torch, lambda: torch._scaled_mm(x, w.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 20)
        xb = torch.randn(m, k, device=dev, dtype=torch.bfloat16)
        wb = torch.randn(n, k, device=dev, dtype=torch.bfloat16)
        msb = _time(torch, lambda: xb @ wb.t(), 20)
        f = 2 * m * n * k
        res[f"{m}x{n}x{k}"] = {"fp8_per_tensor_us": round(ms8 * 1e3, 1),
                               "fp8_per_tensor_TFLOPs": round(f / (ms8 * 1e-3) / 1e12, 1),
                               "bf16_us": round(msb * 1e3, 1), "bf16_TFLOPs": round(f / (msb * 1e-3) / 1e12, 1)}
    print(json.dumps({"vendor_reference": res}))


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_legs_trace:
        summarize_legs_trace(args.summarize_legs_trace)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.vendor_reference:
        vendor_reference()
        return
    if args.summarize_gemm_counters:
        summarize_gemm_counters(*args.summarize_gemm_counters)
        return
    if args.summarize_lds_counters:
        summarize_lds_counters(args.summarize_lds_counters)
        return
    if args.profile_gemms:
        profile_gemms()
        return
    if args.profile_quantizers:
        profile_quantizers()
        return
    if args.summarize_quantizer_counters:
        summarize_quantizer_counters(*args.summarize_quantizer_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (single-GPU hot path; see the sharding notes)")
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_block_scaled_weight_amd as fq
    from fp8_block_scaled_weight_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (libfp8q runs on gfx950 only)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fq.lib()
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "copies": 3}))
        return

    # ------------------------------------------------------------------ inputs
    log("generating inputs")
    W = {
        "q": synth.device_normal_bf16((HIDDEN, HIDDEN), 0.02, dev, 2, 0, 0, outlier_p=1e-3, outlier_mult=20.0),
        "k": synth.device_normal_bf16((KV_DIM, HIDDEN), 0.02, dev, 2, 0, 1, outlier_p=1e-3, outlier_mult=20.0),
        "v": synth.device_normal_bf16((KV_DIM, HIDDEN), 0.02, dev, 2, 0, 2, outlier_p=1e-3, outlier_mult=20.0),
        "o": synth.device_normal_bf16((HIDDEN, HIDDEN), 0.02, dev, 2, 0, 3, outlier_p=1e-3, outlier_mult=20.0),
    }
    WQ = {n: torch.empty(w.shape, dtype=torch.uint8, device=dev) for n, w in W.items()}
    WS = {n: torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.float32, device=dev)
          for n, w in W.items()}
    # The k and v projections are one 2048x4096 weight, as serving engines store them: k's
    # and v's quantized rows and scale rows are row blocks of one buffer (their 128-row
    # scale blocks never straddle the two), and one GEMM writes both outputs as column
    # slices of one [tokens, 2048] result: 512 128x128 tiles, two workgroups per CU, where
    # two 1024-column GEMMs run 256 tiles each.
    WQ["kv"] = torch.empty((2 * KV_DIM, HIDDEN), dtype=torch.uint8, device=dev)
    WS["kv"] = torch.empty((2 * KV_DIM // 128, HIDDEN // 128), dtype=torch.float32, device=dev)
    WQ["k"], WQ["v"] = WQ["kv"][:KV_DIM], WQ["kv"][KV_DIM:]
    WS["k"], WS["v"] = WS["kv"][:KV_DIM // 128], WS["kv"][KV_DIM // 128:]
    X = synth.device_activation(TOKENS, HIDDEN, dev, 2, 0, 10)
    O_in = synth.device_activation(TOKENS, HIDDEN, dev, 2, 0, 11)
    Xq = torch.empty((TOKENS, HIDDEN), dtype=torch.uint8, device=dev)
    Xs = torch.empty((HIDDEN // 128, TOKENS), dtype=torch.float32, device=dev)
    Oq = torch.empty_like(Xq)
    Os = torch.empty_like(Xs)
    Y = {n: torch.empty((TOKENS, W[n].shape[0]), dtype=torch.bfloat16, device=dev) for n in ("q", "o")}
    Y["kv"] = torch.empty((TOKENS, 2 * KV_DIM), dtype=torch.bfloat16, device=dev)
    Y["k"], Y["v"] = Y["kv"][:, :KV_DIM], Y["kv"][:, KV_DIM:]
    slots_np, pages = synth.kv_slot_mapping(2, 0, seqs=64, seq_len=TOKENS // 64)
    slots = torch.from_numpy(slots_np).to(dev)
    Kc = torch.empty((pages, 16, 8, 128), dtype=torch.uint8, device=dev)
    Vc = torch.empty_like(Kc)
    ks = torch.ones(1, dtype=torch.float32, device=dev)
    vs = torch.ones(1, dtype=torch.float32, device=dev)
    descs = [(W[n], WQ[n], WS[n]) for n in ("q", "k", "v", "o")]

    calls = [
        ("a1_weight_sync_qkvo", lambda: fq.fp8q_quant_weight_blk128(descs)),
        ("a2_act_quant_x", lambda: fq.fp8q_quant_act_g128(X, Xq, Xs)),
        ("a3_gemm_q", lambda: fq.fp8q_gemm_w8a8_blkscaled(Xq, Xs, WQ["q"], WS["q"], Y["q"])),
        ("a3_gemm_kv", lambda: fq.fp8q_gemm_w8a8_blkscaled(Xq, Xs, WQ["kv"], WS["kv"], Y["kv"])),
        ("a5a6_kv_recal_write", lambda: fq.fp8q_kv_quant(Y["k"].view(TOKENS, 8, 128), Y["v"].view(TOKENS, 8, 128),
                                                          slots, Kc, Vc, ks, vs, 448.0, recalibrate=True)),
        ("a2_act_quant_o", lambda: fq.fp8q_quant_act_g128(O_in, Oq, Os)),
        ("a3_gemm_o", lambda: fq.fp8q_gemm_w8a8_blkscaled(Oq, Os, WQ["o"], WS["o"], Y["o"])),
    ]
    outputs = [WQ[n] for n in ("q", "kv", "o")] + [WS[n] for n in ("q", "kv", "o")]
    outputs += [Xq, Xs, Oq, Os, Y["q"], Y["kv"], Y["o"], Kc, Vc, ks, vs]

    def step():
        for _, fn in calls:
            fn()

    log(f"warmup {args.warmup} eager steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]

    # The step is captured once into a HIP graph and replayed: the timed region then
    # measures the GPU, not Python's launch overhead.  A replay must reproduce the
    # eager step byte for byte (every call is deterministic).
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for t in outputs:
        t.zero_()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs, eager):
            if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
                raise SystemExit("graph replay differs from the eager step")

    # untimed replays first: the shader clock settles over the first few tens of steps
    for _ in range(max(args.steps, 20)):
        graph.replay()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    gemm_flops = 2 * TOKENS * HIDDEN * (HIDDEN + 2 * KV_DIM + HIDDEN)
    value = gemm_flops / (ms_step * 1e-3) / 1e12

    # Per-call times: each call captured REPS times into one graph (so the graph launch
    # is amortized) and replayed back to back.
    per_call_ms = {}
    for name, fn in calls:
        per_call_ms[name] = _time(torch, fn, 5, reps=20)
    # The quantizer calls again with their operands outside the caches (the step's working
    # set, about 130 MB, is otherwise served by the 256 MB last-level cache on back-to-back
    # calls): each call on its own buffer set, rotated over >= 1 GB.  These cold times are
    # the calls' HBM rates.
    log("cold quantizer timing (buffer rotation over >= 1 GB)")
    cold_ms = {}
    per_set = 3 * sum(w.numel() for w in W.values())
    fns = []
    for _ in range(_rotation_sets(per_set)):
        d = [(W[n].clone(), torch.empty_like(WQ[n]), torch.empty_like(WS[n])) for n in ("q", "k", "v", "o")]
        fns.append(lambda d=d: fq.fp8q_quant_weight_blk128(d))
    cold_ms["a1_weight_sync_qkvo"] = _time_rotated(torch, fns)
    for name, src in (("a2_act_quant_x", X), ("a2_act_quant_o", O_in)):
        fns = []
        for _ in range(_rotation_sets(3 * src.numel())):
            xc, qc, sc = src.clone(), torch.empty_like(Xq), torch.empty_like(Xs)
            fns.append(lambda xc=xc, qc=qc, sc=sc: fq.fp8q_quant_act_g128(xc, qc, sc))
        cold_ms[name] = _time_rotated(torch, fns)
    fns = []
    for _ in range(_rotation_sets(2 * Y["kv"].numel() + 2 * Kc.numel())):
        ykv, kc_, vc_ = Y["kv"].clone(), torch.empty_like(Kc), torch.empty_like(Vc)
        ks_, vs_ = torch.ones_like(ks), torch.ones_like(vs)
        fns.append(lambda ykv=ykv, kc_=kc_, vc_=vc_, ks_=ks_, vs_=vs_: fq.fp8q_kv_quant(
            ykv[:, :KV_DIM].view(TOKENS, 8, 128), ykv[:, KV_DIM:].view(TOKENS, 8, 128), slots, kc_, vc_, ks_, vs_,
            448.0, recalibrate=True))
    cold_ms["a5a6_kv_recal_write"] = _time_rotated(torch, fns)
    del fns, d, xc, qc, sc, ykv, kc_, vc_, ks_, vs_
    torch.cuda.empty_cache()
    # The step's GEMMs the same way, for context: each call on its own operands and output,
    # rotated over >= 1 GB (in the step their operands were just written by a quantizer and
    # are read warm, which the per-call GEMM rates and `roofline` report)
    log("cold GEMM timing (operands rotated over >= 1 GB)")
    for name, (a_, as_, b_, bs_, y_) in (("a3_gemm_q", (Xq, Xs, WQ["q"], WS["q"], Y["q"])),
                                         ("a3_gemm_kv", (Xq, Xs, WQ["kv"], WS["kv"], Y["kv"])),
                                         ("a3_gemm_o", (Oq, Os, WQ["o"], WS["o"], Y["o"]))):
        per = a_.numel() + 4 * as_.numel() + b_.numel() + 4 * bs_.numel() + 2 * y_.numel()
        fns = []
        for _ in range(_rotation_sets(per)):
            t = (a_.clone(), as_.clone(), b_.clone(), bs_.clone(), torch.empty_like(y_))
            fns.append(lambda t=t: fq.fp8q_gemm_w8a8_blkscaled(*t))
        cold_ms[name] = _time_rotated(torch, fns)
        del fns, t
        torch.cuda.empty_cache()

    # The dominant kernel (the q and o GEMMs) inside steps: the step graph against the same
    # step captured without those two GEMMs, replayed alternately (medians of DOM_ROUNDS
    # rounds of `steps` replays each); half the difference per step is the average duration
    # of one in-step launch, with no event between kernels.  For context, the same kernel in
    # a short burst (20 launches back to back) and sustained (100 back to back).  Each group
    # is a distinct launch pattern in a kernel trace of the same command (single launches
    # between other kernels, and runs of 23 and 103 consecutive launches of which the last
    # 20 / 100 are timed).
    dom_names = ("a3_gemm_q", "a3_gemm_o")
    graph_wo = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph_wo, stream=side):
            for name, fn in calls:
                if name not in dom_names:
                    fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    full, wo = [], []
    for _ in range(DOM_ROUNDS):
        full.append(_time_graph(torch, graph, args.steps))
        wo.append(_time_graph(torch, graph_wo, args.steps))
    med = lambda v: sorted(v)[len(v) // 2]
    dom_avg_ms = (med(full) - med(wo)) / 2
    n_dom = 2 * args.steps * DOM_ROUNDS
    dom_fn = calls[2][1]

    def back_to_back(n):
        for _ in range(3):
            dom_fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            dom_fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    burst_ms = back_to_back(DOM_BURST)
    fill = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    fill.fill_(0)  # a different kernel between the two runs
    sustained_ms = back_to_back(DOM_SUSTAINED)
    del fill

    # algorithmic bytes / flops per call
    w_elems = sum(w.numel() for w in W.values())
    bytes_of = {
        "a1_weight_sync_qkvo": 3 * w_elems + 4 * w_elems / 16384,
        "a2_act_quant_x": 3 * TOKENS * HIDDEN + 4 * TOKENS * HIDDEN / 128,
        "a2_act_quant_o": 3 * TOKENS * HIDDEN + 4 * TOKENS * HIDDEN / 128,
        "a5a6_kv_recal_write": 5 * 2 * TOKENS * KV_DIM + 8 * TOKENS,
    }
    flops_of = {"a3_gemm_q": 2 * TOKENS * HIDDEN * HIDDEN, "a3_gemm_kv": 2 * TOKENS * 2 * KV_DIM * HIDDEN,
                "a3_gemm_o": 2 * TOKENS * HIDDEN * HIDDEN}
    call_info = {}
    for name, ms in per_call_ms.items():
        d = {"avg_us": round(ms * 1e3, 2)}
        if name in bytes_of:
            # quantizers: the cold (rotated-buffer) time is the rate; the warm time is context
            d = {"avg_us": round(cold_ms[name] * 1e3, 2), "warm_us": round(ms * 1e3, 2)}
            gbs = bytes_of[name] / (cold_ms[name] * 1e-3) / 1e9
            d.update(GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBPS, 4))
        if name in flops_of:
            tf = flops_of[name] / (ms * 1e-3) / 1e12
            d.update(TFLOPs=round(tf, 1), frac_fp8_peak=round(tf / FP8_PEAK_TFLOPS, 4),
                     cold_us=round(cold_ms[name] * 1e3, 2))
        call_info[name] = d
    q_bytes = sum(bytes_of.values())
    q_ms = sum(cold_ms[n] for n in bytes_of)
    g_ms = sum(per_call_ms[n] for n in flops_of)

    dom_flops = 2 * TOKENS * HIDDEN * HIDDEN
    achieved = dom_flops / (dom_avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                "traffic": traffic_from_profile("gemm_w8a8_4096", source_digest("gemm.hip")),
                "kernel": "gemm_w8a8_kernel<GemmCfg<256,256,2,4,2>> M=N=K=4096 (q/o projection)",
                "avg_us": round(dom_avg_ms * 1e3, 2), "launches_timed": n_dom,
                "timed_as": f"inside the step: (step graph - step graph without the q and o GEMMs) / 2, "
                            f"medians of {DOM_ROUNDS} alternating rounds of {args.steps} replays",
                "step_ms_with": round(med(full), 4), "step_ms_without": round(med(wo), 4),
                "burst_avg_us": round(burst_ms * 1e3, 2), "burst_launches": DOM_BURST,
                "sustained_avg_us": round(sustained_ms * 1e3, 2), "sustained_launches": DOM_SUSTAINED}

    out = {
        "metric": "W8A8 block-scaled GEMM TFLOP/s (% FP8 peak) + quantizer GB/s (% HBM) at 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-in/fp32-acc/bf16-out",
        "data": "synthetic (seeded; Qwen3-8B-like shapes, N(0,0.02) weights with 0.1% x20 outliers, "
                "N(0,1) activations with 4 outlier channels x50)",
        "config": {"workload": "attention block, Qwen3-8B-like: hidden 4096, q/o 4096x4096, k/v 1024x4096 "
                               "(stored as one 2048x4096 kv weight), 4096 tokens; weight sync + act quant + "
                               "W8A8 GEMMs for q, kv, o + FP8 KV write",
                   "tokens": TOKENS, "hidden": HIDDEN, "kv_heads": 8, "head_dim": 128, "parallelism": "none"},
        "gemm_TFLOPs": round(gemm_flops / (g_ms * 1e-3) / 1e12, 1),
        "gemm_frac_fp8_peak": round(gemm_flops / (g_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
        "quantizer_timing": "cold: each call on its own buffers, rotated over >= 1 GB (4x the last-level cache)",
        "quantizer_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "quantizer_frac_hbm": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "calls": call_info,
        "roofline": roofline,
    }

    if not args.no_legs:
        out["legs"] = legs(torch, fq, synth, dev)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(torch, np, X, O_in, W, slots_np, value, gemm_flops,
                                           rows=TOKENS if args.cpu_full else 512)

    print(json.dumps(out), flush=True)


def _time_graph(torch, g, iters):
    """Average time of a captured graph replayed `iters` times back to back."""
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def _time_cold(torch, fn, iters=10):
    """Median time of one call of `fn` after a 512 MB fill has evicted the last-level cache
    (HIP events around the call alone)."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    fn()
    ts = []
    for _ in range(iters):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del flush
    return sorted(ts)[len(ts) // 2]


ROTATE_BYTES = 1 << 30   # buffer rotation footprint: 4x the 256 MB last-level cache


def _time_rotated(torch, fns, iters=5):
    """Average time of one call when every call finds its operands outside the caches:
    `fns` are the same call on distinct buffer sets whose total footprint is at least
    ROTATE_BYTES, captured in order into one graph and replayed `iters` times, so each
    call's buffers were last touched a whole rotation (>= 1 GB of traffic) earlier."""
    for f in fns[:2]:
        f()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for f in fns:
                f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return _time_graph(torch, g, iters) / len(fns)


def _rotation_sets(set_bytes):
    """Buffer sets needed for a ROTATE_BYTES rotation of sets of `set_bytes` each."""
    return max(2, -(-ROTATE_BYTES // int(set_bytes)))


def _time(torch, fn, iters, warm=2, reps=10):
    """Average time of one call of `fn`: `reps` calls captured into one graph, the graph
    replayed `iters` times back to back."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(reps):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return _time_graph(torch, g, iters) / reps


def legs(torch, fq, synth, dev):
    """Side measurements of the other hot-path workloads (not part of `value`)."""
    import numpy as np

    res = {}
    # full weight sync: 36 layers x {q, k, v, o, gate, up, down}
    log("leg: 36-layer weight sync")
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (12288, 4096), (12288, 4096), (4096, 12288)]
    ws, qs, ss = [], [], []
    for layer in range(36):
        for t, (n, k) in enumerate(shapes):
            ws.append(synth.device_normal_bf16((n, k), 0.02, dev, 3, layer, t, outlier_p=1e-3, outlier_mult=20.0))
            qs.append(torch.empty((n, k), dtype=torch.uint8, device=dev))
            ss.append(torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev))
    descs = list(zip(ws, qs, ss))
    el = sum(w.numel() for w in ws)
    ms = _time(torch, lambda: fq.fp8q_quant_weight_blk128(descs), 5, 1)
    gb = (3 * el + 4 * el / 16384) / 1e9
    res["a1_sync_36_layers"] = {"tensors": len(ws), "params": el, "ms": round(ms, 3),
                                "GBps": round(gb / ms * 1e3, 1), "frac_hbm": round(gb / ms * 1e3 / HBM_PEAK_GBPS, 4)}
    del ws, qs, ss, descs
    torch.cuda.empty_cache()

    # MoE layer: expert weight quantization + grouped fc1 / fc2
    log("leg: MoE layer")
    E, H, I = 128, 2048, 768
    row_token, off, _ = synth.moe_routing(0)
    mrows = int(off[-1])
    fc1 = synth.device_normal_bf16((E * 2 * I, H), 0.02, dev, 4, 0, 0)
    fc2 = synth.device_normal_bf16((E * H, I), 0.02, dev, 4, 0, 1)
    fc1q = torch.empty(fc1.shape, dtype=torch.uint8, device=dev)
    fc2q = torch.empty(fc2.shape, dtype=torch.uint8, device=dev)
    fc1s = torch.empty((E * 2 * I // 128, H // 128), dtype=torch.float32, device=dev)
    fc2s = torch.empty((E * H // 128, I // 128), dtype=torch.float32, device=dev)
    edescs = [(fc1, fc1q, fc1s), (fc2, fc2q, fc2s)]
    el = fc1.numel() + fc2.numel()
    ms = _time(torch, lambda: fq.fp8q_quant_weight_blk128(edescs), 5)
    gb = (3 * el + 4 * el / 16384) / 1e9
    res["a1_moe_expert_weights_layer"] = {"params": el, "ms": round(ms, 3), "GBps": round(gb / ms * 1e3, 1),
                                          "frac_hbm": round(gb / ms * 1e3 / HBM_PEAK_GBPS, 4)}
    x = synth.device_activation(4096, H, dev, 4, 0, 5)
    xs_rows = x[torch.from_numpy(row_token).to(dev)]
    a1q = torch.empty((mrows, H), dtype=torch.uint8, device=dev)
    a1s = torch.empty((H // 128, mrows), dtype=torch.float32, device=dev)
    fq.fp8q_quant_act_g128(xs_rows, a1q, a1s)
    a2 = synth.device_activation(mrows, I, dev, 4, 0, 6, outlier_channels=0)
    a2q = torch.empty((mrows, I), dtype=torch.uint8, device=dev)
    a2s = torch.empty((I // 128, mrows), dtype=torch.float32, device=dev)
    fns = []
    for _ in range(_rotation_sets(3 * a2.numel())):
        xc, qc, sc = a2.clone(), torch.empty_like(a2q), torch.empty_like(a2s)
        fns.append(lambda xc=xc, qc=qc, sc=sc: fq.fp8q_quant_act_g128(xc, qc, sc))
    ms_aq = _time_rotated(torch, fns)
    del fns, xc, qc, sc
    offs = torch.from_numpy(off).to(dev)
    y1 = torch.empty((mrows, 2 * I), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((mrows, H), dtype=torch.bfloat16, device=dev)
    b1 = fc1q.view(E, 2 * I, H)
    b1s = fc1s.view(E, 2 * I // 128, H // 128)
    b2 = fc2q.view(E, H, I)
    b2s = fc2s.view(E, H // 128, I // 128)
    ms1 = _time(torch, lambda: fq.fp8q_grouped_gemm_w8a8(a1q, a1s, b1, b1s, offs, y1), 10)
    ms2 = _time(torch, lambda: fq.fp8q_grouped_gemm_w8a8(a2q, a2s, b2, b2s, offs, y2), 10)
    f1 = 2 * mrows * 2 * I * H
    f2 = 2 * mrows * H * I
    by1 = mrows * H + b1.numel() + 2 * mrows * 2 * I
    by2 = mrows * I + b2.numel() + 2 * mrows * H
    for name, f, by, ms_ in (("a4_moe_fc1", f1, by1, ms1), ("a4_moe_fc2", f2, by2, ms2)):
        tf = f / (ms_ * 1e-3) / 1e12
        ceil = min(FP8_PEAK_TFLOPS, f / by * HBM_PEAK_GBPS / 1e3)
        res[name] = {"rows": mrows, "us": round(ms_ * 1e3, 1), "TFLOPs": round(tf, 1),
                     "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4), "frac_roofline": round(tf / ceil, 4),
                     "roofline_TFLOPs": round(ceil, 1)}
    gbs = (3 * a2.numel() + 4 * a2.numel() / 128) / (ms_aq * 1e-3) / 1e9
    res["a2_moe_fc2_act_quant"] = {"us": round(ms_aq * 1e3, 1), "GBps": round(gbs, 1),
                                   "frac_hbm": round(gbs / HBM_PEAK_GBPS, 4), "timing": "cold (1 GB rotation)"}

    # the layer's data movement around the grouped GEMMs: dispatch of the quantized tokens
    # by their recorded top-8 expert ids, SwiGLU + 1x128 quantization of fc1's output,
    # weighted combine of fc2's output; then the whole layer as one sequence
    log("leg: MoE dispatch / SwiGLU-quant / combine")
    ids_np, rw_np = synth.moe_topk(0)
    T, topk = ids_np.shape
    n = T * topk
    ids = torch.from_numpy(ids_np).to(dev)
    rw = torch.from_numpy(rw_np).to(dev)
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xsc = torch.empty((H // 128, T), dtype=torch.float32, device=dev)
    fq.fp8q_quant_act_g128(x, xq, xsc)
    dq = torch.empty((n, H), dtype=torch.uint8, device=dev)
    dsc = torch.empty((H // 128, n), dtype=torch.float32, device=dev)
    doff = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, topk), dtype=torch.int32, device=dev)
    q2 = torch.empty((n, I), dtype=torch.uint8, device=dev)
    s2 = torch.empty((I // 128, n), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    f_d = lambda: fq.fp8q_moe_dispatch(xq, xsc, ids, E, dq, dsc, doff, row_of)
    f_sw = lambda: fq.fp8q_swiglu_quant_g128(y1, q2, s2)
    f_c = lambda: fq.fp8q_moe_combine(y2, row_of, rw, out)
    ms_d, ms_sw, ms_c = _time(torch, f_d, 10), _time(torch, f_sw, 10), _time(torch, f_c, 10)
    # their inputs (75-150 MB) fit the 256 MB last-level cache, so back-to-back calls run
    # partly from it; the cold figure evicts it (a 512 MB fill) before each single call
    cold = {k: _time_cold(torch, f_) for k, f_ in (("d", f_d), ("sw", f_sw), ("c", f_c))}

    def layer():
        fq.fp8q_moe_dispatch(xq, xsc, ids, E, dq, dsc, doff, row_of)
        fq.fp8q_grouped_gemm_w8a8(dq, dsc, b1, b1s, doff, y1)
        fq.fp8q_swiglu_quant_g128(y1, q2, s2)
        fq.fp8q_grouped_gemm_w8a8(q2, s2, b2, b2s, doff, y2)
        fq.fp8q_moe_combine(y2, row_of, rw, out)

    ms_l = _time(torch, layer, 5, reps=2)

    # fc1 with SwiGLU and fc2's input quantization fused into its epilogue (no bf16 fc1
    # output): alone, and in the layer in place of fc1 + SwiGLU-quant
    q2f = torch.empty((n, I), dtype=torch.uint8, device=dev)
    s2f = torch.empty((I // 128, n), dtype=torch.float32, device=dev)
    ms_f1f = _time(torch, lambda: fq.fp8q_grouped_gemm_swiglu_quant(dq, dsc, b1, b1s, doff, q2f, s2f), 10)
    # and reading the token rows through the routing's row -> token map (no dispatch copy)
    rtok = torch.empty(n, dtype=torch.int32, device=dev)
    fq.fp8q_moe_route(ids, E, doff, row_of, rtok)
    ms_f1t = _time(torch, lambda: fq.fp8q_grouped_gemm_swiglu_quant(xq, xsc, b1, b1s, doff, q2f, s2f,
                                                                    row_token=rtok), 10)
    ms_rt = _time(torch, lambda: fq.fp8q_moe_route(ids, E, doff, row_of, rtok), 10)

    def layer_fused():
        fq.fp8q_moe_route(ids, E, doff, row_of, rtok)
        fq.fp8q_grouped_gemm_swiglu_quant(xq, xsc, b1, b1s, doff, q2f, s2f, row_token=rtok)
        fq.fp8q_grouped_gemm_w8a8(q2f, s2f, b2, b2s, doff, y2)
        fq.fp8q_moe_combine(y2, row_of, rw, out)

    ms_lf = _time(torch, layer_fused, 5, reps=2)
    by_d = T * H + 4 * T * H / 128 + 2 * n + n * H + 4 * n * H / 128 + 4 * n + 4 * (E + 1)
    by_sw = n * 2 * I * 2 + n * I + 4 * n * I / 128
    by_c = n * H * 2 + 8 * n + T * H * 2
    for name, by, ms_, key in (("f1_moe_dispatch", by_d, ms_d, "d"), ("f1_swiglu_quant", by_sw, ms_sw, "sw"),
                               ("f1_moe_combine", by_c, ms_c, "c")):
        res[name] = {"us": round(ms_ * 1e3, 1), "GBps": round(by / (ms_ * 1e-3) / 1e9, 1),
                     "frac_hbm": round(by / (ms_ * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "cold_us": round(cold[key] * 1e3, 1),
                     "cold_GBps": round(by / (cold[key] * 1e-3) / 1e9, 1)}
    res["f1_moe_layer"] = {"tokens": T, "rows": n, "us": round(ms_l * 1e3, 1),
                           "TFLOPs": round((f1 + f2) / (ms_l * 1e-3) / 1e12, 1),
                           "steps": "dispatch, fc1, swiglu-quant, fc2, combine"}
    res["a4_moe_fc1_swiglu_fused"] = {"rows": n, "us": round(ms_f1f * 1e3, 1),
                                      "TFLOPs": round(f1 / (ms_f1f * 1e-3) / 1e12, 1),
                                      "token_rows_us": round(ms_f1t * 1e3, 1),
                                      "unfused_fc1_plus_swiglu_us": round((ms1 + ms_sw) * 1e3, 1)}
    res["f1_moe_route"] = {"us": round(ms_rt * 1e3, 1)}
    res["f1_moe_layer_fused"] = {"tokens": T, "rows": n, "us": round(ms_lf * 1e3, 1),
                                 "TFLOPs": round((f1 + f2) / (ms_lf * 1e-3) / 1e12, 1),
                                 "steps": "route, fc1 + swiglu-quant fused reading the token rows, fc2, combine"}

    # the same fused layer with power-of-two (UE8M0) scales throughout: expert weights, tokens
    # and fc2's input (the fc1 epilogue's quantization) all take the UE8M0 rule
    fc1u, fc2u = torch.empty_like(fc1q), torch.empty_like(fc2q)
    fc1us, fc2us = torch.empty_like(fc1s), torch.empty_like(fc2s)
    fq.fp8q_quant_weight_blk128_ue8m0([(fc1, fc1u, fc1us), (fc2, fc2u, fc2us)])
    b1u, b1us = fc1u.view(E, 2 * I, H), fc1us.view(E, 2 * I // 128, H // 128)
    b2u, b2us = fc2u.view(E, H, I), fc2us.view(E, H // 128, I // 128)
    xqu, xscu = torch.empty_like(xq), torch.empty_like(xsc)
    fq.fp8q_quant_act_g128_ue8m0(x, xqu, xscu)
    ms_swu = _time(torch, lambda: fq.fp8q_swiglu_quant_g128_ue8m0(y1, q2, s2), 10)
    ms_f1u = _time(torch, lambda: fq.fp8q_grouped_gemm_swiglu_quant_ue8m0(xqu, xscu, b1u, b1us, doff, q2f, s2f,
                                                                          row_token=rtok), 10)

    def layer_fused_ue8m0():
        fq.fp8q_moe_route(ids, E, doff, row_of, rtok)
        fq.fp8q_grouped_gemm_swiglu_quant_ue8m0(xqu, xscu, b1u, b1us, doff, q2f, s2f, row_token=rtok)
        fq.fp8q_grouped_gemm_w8a8_ue8m0(q2f, s2f, b2u, b2us, doff, y2)
        fq.fp8q_moe_combine(y2, row_of, rw, out)

    ms_lfu = _time(torch, layer_fused_ue8m0, 5, reps=2)
    res["f2_ue8m0_moe_layer_fused"] = {"tokens": T, "rows": n, "us": round(ms_lfu * 1e3, 1),
                                       "TFLOPs": round((f1 + f2) / (ms_lfu * 1e-3) / 1e12, 1),
                                       "fc1_swiglu_fused_token_rows_us": round(ms_f1u * 1e3, 1),
                                       "swiglu_quant_us": round(ms_swu * 1e3, 1),
                                       "steps": "route, UE8M0 fc1 + swiglu-quant fused reading the token rows, "
                                                "UE8M0 fc2, combine"}
    del fc1u, fc2u, fc1us, fc2us, xqu, xscu
    del xq, dq, q2, out, q2f, s2f, rtok
    del fc1, fc2, fc1q, fc2q, x, xs_rows, a1q, a2, a2q, y1, y2
    torch.cuda.empty_cache()

    # KV: one layer of 64 sequences x 20,000 tokens, recalibrate + write; then a decode write
    log("leg: KV layer")
    slots_np, pages = synth.kv_slot_mapping()
    T = len(slots_np)
    k = synth.device_kv(T, dev, 5, 0, 0)
    v = synth.device_kv(T, dev, 5, 0, 1)
    sl = torch.from_numpy(slots_np).to(dev)
    kc = torch.empty((pages, 16, 8, 128), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.ones(1, device=dev)
    vs = torch.ones(1, device=dev)
    ms = _time(torch, lambda: fq.fp8q_kv_quant(k, v, sl, kc, vc, ks, vs, 448.0, recalibrate=True), 5)
    gb = (5 * 2 * T * 1024 + 8 * T) / 1e9
    res["a5a6_kv_layer_recal_write"] = {"tokens": T, "ms": round(ms, 3), "GBps": round(gb / ms * 1e3, 1),
                                        "frac_hbm": round(gb / ms * 1e3 / HBM_PEAK_GBPS, 4),
                                        "step_36_layers_ms_est": round(36 * ms, 2)}
    dec_idx = torch.arange(64, device=dev) * 20000 + 19999
    kd, vd, sd = k[dec_idx].contiguous(), v[dec_idx].contiguous(), sl[dec_idx].contiguous()
    ms = _time(torch, lambda: fq.fp8q_kv_quant(kd, vd, sd, kc, vc, ks, vs, 448.0, recalibrate=False), 20)
    res["a6_kv_decode_write_64_tokens"] = {"us": round(ms * 1e3, 2)}

    # FP8 decode attention over the layer's cache just written: 64 sequences x 20,000
    # tokens, 32 query heads on 8 KV heads, one query per sequence; with and without the
    # query-scale recalibration
    log("leg: FP8 paged decode attention")
    hq = 32
    seqs = 64
    bt = torch.from_numpy((slots_np.reshape(seqs, -1)[:, ::16] // 16).astype(np.int32)).to(dev)
    lens = torch.full((seqs,), T // seqs, dtype=torch.int32, device=dev)
    qd = synth.device_activation(seqs, hq * 128, dev, 5, 0, 50).view(seqs, hq, 128)
    od = torch.empty((seqs, hq, 128), dtype=torch.bfloat16, device=dev)
    qsc = torch.ones(1, device=dev)
    att = lambda recal: fq.fp8q_paged_decode_attention(qd, kc, vc, bt, lens, qsc, ks, vs, 128 ** -0.5, od,
                                                       recalibrate_q=recal)
    ms_r = _time(torch, lambda: att(True), 10)
    ms_s = _time(torch, lambda: att(False), 10)
    by = 2 * T * 8 * 128 + 2 * 2 * seqs * hq * 128 + 4 * bt.numel() + 4 * seqs
    res["f3_decode_attention_layer"] = {
        "seqs": seqs, "context": T // seqs, "q_heads": hq, "kv_heads": 8,
        "us": round(ms_s * 1e3, 1), "us_with_q_recalibration": round(ms_r * 1e3, 1),
        "GBps": round(by / (ms_s * 1e-3) / 1e9, 1), "frac_hbm": round(by / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del k, v, kc, vc, qd, od
    torch.cuda.empty_cache()

    # power-of-two (UE8M0) scale variant of the attention block's calls: quantizers and
    # the GEMMs whose block scales the matrix core applies
    log("leg: UE8M0 variant")
    X = synth.device_activation(TOKENS, HIDDEN, dev, 2, 0, 10)
    Wq = synth.device_normal_bf16((HIDDEN, HIDDEN), 0.02, dev, 2, 0, 0, outlier_p=1e-3, outlier_mult=20.0)
    Wk = synth.device_normal_bf16((KV_DIM, HIDDEN), 0.02, dev, 2, 0, 1, outlier_p=1e-3, outlier_mult=20.0)
    xq = torch.empty((TOKENS, HIDDEN), dtype=torch.uint8, device=dev)
    xs = torch.empty((HIDDEN // 128, TOKENS), dtype=torch.float32, device=dev)
    wq = {n: torch.empty(w.shape, dtype=torch.uint8, device=dev) for n, w in (("q", Wq), ("k", Wk))}
    wsc = {n: torch.empty((w.shape[0] // 128, HIDDEN // 128), dtype=torch.float32, device=dev)
           for n, w in (("q", Wq), ("k", Wk))}
    wd = [(Wq, wq["q"], wsc["q"]), (Wk, wq["k"], wsc["k"])]
    ms_w = _time(torch, lambda: fq.fp8q_quant_weight_blk128_ue8m0(wd), 10)
    ms_a = _time(torch, lambda: fq.fp8q_quant_act_g128_ue8m0(X, xq, xs), 10)
    yq = torch.empty((TOKENS, HIDDEN), dtype=torch.bfloat16, device=dev)
    yk = torch.empty((TOKENS, KV_DIM), dtype=torch.bfloat16, device=dev)
    ms_q = _time(torch, lambda: fq.fp8q_gemm_w8a8_ue8m0(xq, xs, wq["q"], wsc["q"], yq), 10)
    ms_k = _time(torch, lambda: fq.fp8q_gemm_w8a8_ue8m0(xq, xs, wq["k"], wsc["k"], yk), 10)
    fq_, fk_ = 2 * TOKENS * HIDDEN * HIDDEN, 2 * TOKENS * KV_DIM * HIDDEN
    el = Wq.numel() + Wk.numel()
    res["f2_ue8m0"] = {
        "weight_quant_qk_us": round(ms_w * 1e3, 2),
        "weight_quant_GBps": round((3 * el + 4 * el / 16384) / (ms_w * 1e-3) / 1e9, 1),
        "act_quant_x_us": round(ms_a * 1e3, 2),
        "gemm_q_us": round(ms_q * 1e3, 2), "gemm_q_TFLOPs": round(fq_ / (ms_q * 1e-3) / 1e12, 1),
        "gemm_q_frac_fp8_peak": round(fq_ / (ms_q * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
        "gemm_k_us": round(ms_k * 1e3, 2), "gemm_k_TFLOPs": round(fk_ / (ms_k * 1e-3) / 1e12, 1),
    }
    del X, Wq, Wk, xq, wq, yq, yk
    torch.cuda.empty_cache()

    # small-M GEMMs (decode / short prefill shapes)
    log("leg: small-M GEMMs")
    for m in (1, 64, 512):
        for n in (4096, 1024):
            a = torch.randint(0, 0x77, (m, 4096), dtype=torch.uint8, device=dev)
            b = torch.randint(0, 0x77, (n, 4096), dtype=torch.uint8, device=dev)
            asc = torch.rand((32, m), device=dev)
            bsc = torch.rand((n // 128, 32), device=dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ms = _time(torch, lambda: fq.fp8q_gemm_w8a8_blkscaled(a, asc, b, bsc, y), 20)
            f = 2 * m * n * 4096
            by = m * 4096 + n * 4096 + 2 * m * n
            ceil = min(FP8_PEAK_TFLOPS, f / by * HBM_PEAK_GBPS / 1e3)
            tf = f / (ms * 1e-3) / 1e12
            res[f"a3_gemm_m{m}_n{n}"] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 2),
                                         "frac_roofline": round(tf / ceil, 4)}

    # 1x128 activation quantization at the dense model's other shapes: 4096 tokens of the
    # MLP's down-projection input (K = 12288) and 64 tokens at K = 4096 and 12288, cold
    log("leg: activation quantization shapes")
    for m, k in ((4096, 12288), (64, 4096), (64, 12288)):
        x = synth.device_activation(m, k, dev, 3, 0, 20 + k // 4096)
        fns = []
        for _ in range(_rotation_sets(3 * x.numel())):
            xc = x.clone()
            qc = torch.empty((m, k), dtype=torch.uint8, device=dev)
            sc = torch.empty((k // 128, m), dtype=torch.float32, device=dev)
            fns.append(lambda xc=xc, qc=qc, sc=sc: fq.fp8q_quant_act_g128(xc, qc, sc))
        ms = _time_rotated(torch, fns, iters=5 if m > 64 else 2)
        gbs = (3 * m * k + 4 * m * k / 128) / (ms * 1e-3) / 1e9
        res[f"a2_act_quant_m{m}_k{k}"] = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
                                          "frac_hbm": round(gbs / HBM_PEAK_GBPS, 4), "timing": "cold (1 GB rotation)"}
        del fns, xc, qc, sc, x
    torch.cuda.empty_cache()

    # dense MLP GEMMs: gate/up (4096 -> 12288) and down (12288 -> 4096) at 64 and 4096 tokens
    log("leg: MLP GEMMs")
    for name, n, k in (("gate_up", 12288, 4096), ("down", 4096, 12288)):
        b = torch.randint(0, 0x77, (n, k), dtype=torch.uint8, device=dev)
        bsc = torch.rand((n // 128, k // 128), device=dev)
        for m in (64, 4096):
            a = torch.randint(0, 0x77, (m, k), dtype=torch.uint8, device=dev)
            asc = torch.rand((k // 128, m), device=dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ms = _time(torch, lambda: fq.fp8q_gemm_w8a8_blkscaled(a, asc, b, bsc, y), 10)
            f = 2 * m * n * k
            by = m * k + n * k + 2 * m * n
            ceil = min(FP8_PEAK_TFLOPS, f / by * HBM_PEAK_GBPS / 1e3)
            tf = f / (ms * 1e-3) / 1e12
            res[f"a3_mlp_{name}_m{m}"] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1),
                                          "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                                          "frac_roofline": round(tf / ceil, 4)}

    # few tokens: activation quantization fused into the GEMM's operand load, against the
    # activation quantizer followed by the GEMM (both as one graph of calls)
    log("leg: fused activation quantization (few tokens)")
    for m in (1, 4, 16, 64):
        for n in (4096, 1024):
            x = synth.device_activation(m, 4096, dev, 2, 9, m)
            b = torch.randint(0, 0x77, (n, 4096), dtype=torch.uint8, device=dev)
            bsc = torch.rand((n // 128, 32), device=dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            xq = torch.empty((m, 4096), dtype=torch.uint8, device=dev)
            xs = torch.empty((32, m), dtype=torch.float32, device=dev)
            ms_f = _time(torch, lambda: fq.fp8q_gemm_w8a8_bf16act(x, b, bsc, y), 20)

            def two():
                fq.fp8q_quant_act_g128(x, xq, xs)
                fq.fp8q_gemm_w8a8_blkscaled(xq, xs, b, bsc, y)

            ms_2 = _time(torch, two, 20)
            by = 2 * m * 4096 + n * 4096 + 2 * m * n
            res[f"f4_fused_m{m}_n{n}"] = {"us": round(ms_f * 1e3, 2), "quant_then_gemm_us": round(ms_2 * 1e3, 2),
                                          "frac_hbm_roofline": round(by / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    return res


def cpu_baseline(torch, np, X, O_in, W, slots_np, gpu_value, gemm_flops, rows=512):
    """The oracle, as it stands, on a bounded sample of the step: every weight of q/k/v/o
    through blockwise quantization (the whole sync of the step), and `rows` of the 4096
    tokens through act-quant, the q/k/v/o GEMMs (fp64), the KV write and the o input's
    act-quant; the token part is scaled by 4096/rows to a full step, and the step's GEMM
    FLOPs are divided by the estimated step time (TFLOP/s, like `value`).  rows = 4096 runs
    the whole step unsampled (about 150 s of 16 host threads)."""
    import oracle

    tok_scale = TOKENS / rows
    h = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    xb, ob = h(X[:rows]), h(O_in[:rows])
    wfull = {n: h(W[n]) for n in W}
    log(f"cpu baseline: oracle on the q/k/v/o weights and {rows} of {TOKENS} tokens "
        f"({oracle.num_threads()} threads, {os.cpu_count()} logical CPUs on the host)")

    t0 = time.perf_counter()
    wq = {n: oracle.quant_weight_blk128(wfull[n]) for n in wfull}
    t_w = time.perf_counter() - t0

    t1 = time.perf_counter()
    xq, xs = oracle.quant_act_g128(xb)
    oracle.gemm_w8a8(xq, xs, *wq["q"])
    yk = oracle.gemm_w8a8(xq, xs, *wq["k"])
    yv = oracle.gemm_w8a8(xq, xs, *wq["v"])
    t_gemm_kv_in = time.perf_counter() - t1
    bf = lambda y: torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16).reshape(rows, 8, 128)
    kb, vb = bf(yk), bf(yv)
    kcache = np.zeros((int(slots_np[:rows].max()) // 16 + 1, 16, 8, 128), np.uint8)
    vcache = kcache.copy()
    t2 = time.perf_counter()
    oracle.kv_quant(kb, vb, slots_np[:rows], kcache, vcache, 16)
    oq, os_ = oracle.quant_act_g128(ob)
    oracle.gemm_w8a8(oq, os_, *wq["o"])
    t_rest = time.perf_counter() - t2

    t_tok = t_gemm_kv_in + t_rest
    sample_s = t_w + t_tok
    est_step_s = t_w + t_tok * tok_scale
    value = gemm_flops / est_step_s / 1e12
    what = ("the whole step (unsampled)" if rows == TOKENS else
            f"all q/k/v/o weights (blockwise quantization, unscaled) and {rows} of {TOKENS} tokens "
            f"(act quant, q/k/v/o GEMMs in fp64, KV write; scaled x{tok_scale:g})")
    return {"value": value, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{what}; {sample_s:.1f} s measured, {est_step_s:.1f} s per step",
            "host_logical_cpus": os.cpu_count(), "threads": oracle.num_threads(),
            "sample_seconds": round(sample_s, 2), "est_step_seconds": round(est_step_s, 1),
            "weight_sync_seconds": round(t_w, 2), "token_part_seconds": round(t_tok, 2),
            "gpu_over_cpu": round(gpu_value / value, 1)}


if __name__ == "__main__":
    main()
