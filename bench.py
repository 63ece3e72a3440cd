#!/usr/bin/env python3
"""Benchmark: one step = the three NVFP4 projections of an H3 block at
37,810 tokens, each producer + GEMM on one stream:

  QKV  modulation producer (x [37810,5376], 2 segments) -> GEMM N=21504, K=5376
  FC1  modulation producer (same x, own shift/scale)    -> GEMM N=14336, K=5376
  FC2  SwiGLU producer (gate/up [37810, 2*14336])       -> GEMM N=5376,  K=14336

Inputs are seeded synthetic tensors resident in HBM before timing starts;
weights are prepacked to NVFP4 (untimed).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Profile summaries (no GPU needed): ``--summarize-trace DIR`` prints the
kernel table of a ``rocprofv3 --kernel-trace --stats --output-format csv`` run
of this script; ``--summarize-traffic FETCH_DIR WRITE_DIR`` reads two
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs made with
``--copy-calibration``, prints the per-dispatch table and writes
``profiles/traffic.json`` for the current GEMM source.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "producer GB/s (% HBM peak) + NVFP4 GEMM TFLOP/s at M=37810 QKV/FC1/FC2"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-attn-out", action="store_true",
                   help="skip the separately timed attention-output projection")
    p.add_argument("--two-pass", action="store_true",
                   help="run every producer as its two passes (absmax, pack: separate calls, per-pass times) instead of one call")
    p.add_argument("--cpu-rows", type=int, default=16,
                   help="checked rows per projection for the CPU-baseline GEMM (x 8 rows of the SwiGLU producer)")
    p.add_argument("--no-ring", action="store_true",
                   help="skip the separately timed QKV projection through the packed-tile ring")
    p.add_argument("--no-hash", action="store_true", help="skip the SHA-256 of the step's outputs")
    p.add_argument("--no-standalone", action="store_true",
                   help="skip the standalone cold/warm producer timings (profiling runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="before timing, copy 1 GiB once (a plain copy kernel of known size, for scaling "
                        "rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    p.add_argument("--summarize-trace", metavar="DIR", help="print the kernel table of a rocprofv3 trace run")
    p.add_argument("--skip-steps", type=int, default=0,
                   help="summaries: leave out the first N steps' calls (the run's warm-up steps)")
    p.add_argument("--bench-json", metavar="FILE",
                   help="summaries: a bench.py output line from the same node, set beside the profiled times")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarize FETCH_SIZE/WRITE_SIZE runs and write profiles/traffic.json")
    p.add_argument("--summarize-counters", metavar="DIR",
                   help="per-kernel means of the counters of a rocprofv3 --pmc run of this script, and VALU lane-ops "
                        "per element for the producer kernels (SQ_INSTS_VALU x 64 / elements)")
    p.add_argument("--summarize-mfma", metavar="DIR",
                   help="MFMA busy and clock per GEMM launch from a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                        "SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE run")
    return p.parse_args()


_TOKEN = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_only(text: str) -> str:
    """C/C++ source without its comments and with every run of whitespace
    made one space: a comment edit leaves the code, and so this text, as it
    was (string and character literals are kept as written)."""
    text = _TOKEN.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    return " ".join(text.split())


def src_hash(*names):
    """Hash of the code (comments and layout aside) of the named sources,
    which identifies the kernels that counter readings were taken on."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_activation_quantization_segment_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def modulation_bytes(M: int, M_pad: int, K: int) -> int:
    """Algorithmic bytes of the modulation producer: two reads of x [M, K] bf16,
    QDATA [M_pad, K/2] and SFA [M_pad, K/16] written (padding rows included)."""
    return 2 * M * K * 2 + M_pad * (K // 2 + K // 16)


def swiglu_bytes(M: int, M_pad: int, F: int) -> int:
    """Algorithmic bytes of the SwiGLU producer: two reads of gate/up [M, 2F]
    bf16, QDATA and SFA of h [M_pad, F] written."""
    return 2 * M * 2 * F * 2 + M_pad * (F // 2 + F // 16)


def one_read_bytes(M: int, M_pad: int, in_cols: int, K: int) -> int:
    """What any producer must move: the bf16 input [M, in_cols] read once,
    QDATA and SFA of [M_pad, K] written."""
    return M * in_cols * 2 + M_pad * (K // 2 + K // 16)


def gemm_flop(M: int, N: int, K: int) -> float:
    """Algorithmic flops of the [M, K] x [N, K]^T product over the logical rows."""
    return 2.0 * M * N * K


def traffic_entry(kernel: str, source_hash: str):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain-copy calibration), if they were taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        e = data.get(kernel)
        if not e or e.get("source_hash") != source_hash:
            return None
        return float(e["bytes_per_launch"])
    except Exception:
        return None


def producer_counter_bytes(kind: str):
    """FETCH_SIZE + WRITE_SIZE bytes per launch of the single-launch producer
    (the rows held on chip are not read twice, so fewer than the algorithmic
    bytes), if measured on the current producer source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        e = json.load(open(path)).get("producer_single_launch")
        if not e or e.get("source_hash") != src_hash("producer.hip", "nvfp4_device.h", "internal.h"):
            return None
        b = e["per_launch_bytes"].get(kind)
        return None if b is None else {"fetch": b["fetch"], "write": b["write"], "total": b["fetch"] + b["write"]}
    except Exception:
        return None


def main():
    args = parse()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.skip_steps, args.bench_json))
        return
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma, args.skip_steps))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(a multi-GPU step would shard rows and all-reduce one 4-byte maximum; it is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_activation_quantization_segment_amd as nv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    t_setup = time.time()
    wq, wf1, wf2 = synth.workload("qkv"), synth.workload("fc1"), synth.workload("fc2")
    M = wq.M
    M_pad = wq.m_pad
    # SHA-256 of every generated input (the same as tests/golden/synth_sha256.json)
    input_sha = {}

    def sha(a):
        return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()

    x_h = wq.x()
    input_sha["x (qkv, fc1)"] = sha(x_h)
    x = up(x_h)
    segs = {}
    for w in (wq, wf1):
        rs, sh, sc = w.segments()
        input_sha[f"{w.name} shift"], input_sha[f"{w.name} scale"] = sha(sh), sha(sc)
        segs[w.name] = (rs, up(sh), up(sc))
    gu_h = wf2.gate_up()
    input_sha["fc2 gate_up"] = sha(gu_h)
    gu = up(gu_h)
    weights = {}
    for w in (wq, wf1, wf2):
        wt_h = w.weight()
        input_sha[f"{w.name} weight"] = sha(wt_h)
        wt = up(wt_h)
        with torch.cuda.stream(stream):
            weights[w.name] = nv.quantize_weight(wt, stream=stream)
        stream.synchronize()
        del wt, wt_h
    # outputs and per-projection scratch, allocated once
    bufs = {}
    for w in (wq, wf1, wf2):
        K = w.K
        bufs[w.name] = dict(
            q=torch.empty((M_pad, K // 2), dtype=torch.uint8, device=dev),
            s=torch.empty((M_pad, K // 16), dtype=torch.uint8, device=dev),
            ts=torch.empty(1, dtype=torch.float32, device=dev),
            amax=torch.empty(1, dtype=torch.float32, device=dev),
            out=torch.empty((M, w.N), dtype=torch.bfloat16, device=dev),
            ws=torch.zeros(int(nv.lib.nvfp4_absmax_workspace_bytes()), dtype=torch.uint8, device=dev),
            gws_bytes=nv.nvfp4_gemm_workspace_bytes(M, w.N, K),
        )
        b = bufs[w.name]
        b["gws"] = torch.empty(max(b["gws_bytes"], 16), dtype=torch.uint8, device=dev)
    seg_structs = {n: nv.make_segments(*segs[n]) for n in segs}
    F = wf2.K
    gate_ptr, up_ptr = gu.data_ptr(), gu.data_ptr() + 2 * F
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    # kernel sequence of one step: (label, kind, fn)
    def launches():
        seq = []
        for w in (wq, wf1):
            b = bufs[w.name]
            seg = seg_structs[w.name][0]
            qw, sfw, tw = weights[w.name]
            if args.two_pass:
                seq.append((f"{w.name}.absmax", "mod_absmax",
                            lambda b=b, seg=seg, w=w: nv.nvfp4_modulate_absmax(x, M, w.K, w.K, seg, b["ws"], b["ts"],
                                                                               b["amax"], stream)))
                seq.append((f"{w.name}.pack", "mod_pack",
                            lambda b=b, seg=seg, w=w: nv.nvfp4_modulate_pack(x, M, w.K, w.K, seg, b["ts"], b["q"],
                                                                             b["s"], M_pad, stream)))
            else:
                seq.append((f"{w.name}.quantize", "mod_quantize",
                            lambda b=b, seg=seg, w=w: nv.nvfp4_modulate_quantize(
                                x, M, w.K, w.K, seg, b["ws"], b["ts"], b["amax"], b["q"], b["s"], M_pad, stream)))
            seq.append((f"{w.name}.gemm", "gemm",
                        lambda b=b, w=w, qw=qw, sfw=sfw, tw=tw: nv.nvfp4_gemm_ws(
                            b["q"], b["s"], b["ts"], M, M_pad, qw, sfw, tw, w.N, w.K, b["out"], w.N, b["gws"],
                            b["gws_bytes"], stream)))
        b = bufs["fc2"]
        qw, sfw, tw = weights["fc2"]
        if args.two_pass:
            seq.append(("fc2.absmax", "swiglu_absmax",
                        lambda: nv.nvfp4_swiglu_absmax(gate_ptr, up_ptr, M, F, 2 * F, b["ws"], b["ts"], b["amax"],
                                                       stream)))
            seq.append(("fc2.pack", "swiglu_pack",
                        lambda: nv.nvfp4_swiglu_pack(gate_ptr, up_ptr, M, F, 2 * F, b["ts"], b["q"], b["s"], M_pad,
                                                     stream)))
        else:
            seq.append(("fc2.quantize", "swiglu_quantize",
                        lambda: nv.nvfp4_swiglu_quantize(gate_ptr, up_ptr, M, F, 2 * F, b["ws"], b["ts"], b["amax"],
                                                         b["q"], b["s"], M_pad, stream)))
        seq.append(("fc2.gemm", "gemm",
                    lambda: nv.nvfp4_gemm_ws(b["q"], b["s"], b["ts"], M, M_pad, qw, sfw, tw, wf2.N, wf2.K, b["out"],
                                             wf2.N, b["gws"], b["gws_bytes"], stream)))
        return seq

    seq = launches()
    n = len(seq)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            src.fill_(1)
            dst.copy_(src)
        stream.synchronize()
        del src, dst

    def run_step(events=None):
        for i, (_, _, fn) in enumerate(seq):
            if events is not None:
                events[i].record(stream)
            fn()
        if events is not None:
            events[n].record(stream)

    for _ in range(args.warmup):
        run_step()
    stream.synchronize()

    # timed region: K steps, events between launches on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(args.steps):
        run_step(evs[k])
    end.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    per = {label: [] for label, _, _ in seq}
    for k in range(args.steps):
        for i, (label, _, _) in enumerate(seq):
            per[label].append(evs[k][i].elapsed_time(evs[k][i + 1]))
    med = {label: float(np.median(v)) for label, v in per.items()}
    launch_pct = {label: {"p50": round(float(np.percentile(v, 50)), 4), "p95": round(float(np.percentile(v, 95)), 4)}
                  for label, v in per.items()}
    hashes = {} if args.no_hash else output_hashes(bufs)
    standalone = {} if args.no_standalone else standalone_producers(seq, stream, dev, reps=20)

    # algorithmic work
    flops = {w.name: gemm_flop(M, w.N, w.K) for w in (wq, wf1, wf2)}
    prod_bytes = {"qkv": modulation_bytes(M, M_pad, wq.K), "fc1": modulation_bytes(M, M_pad, wf1.K),
                  "fc2": swiglu_bytes(M, M_pad, F)}
    prod_one_read = {"qkv": one_read_bytes(M, M_pad, wq.K, wq.K), "fc1": one_read_bytes(M, M_pad, wf1.K, wf1.K),
                     "fc2": one_read_bytes(M, M_pad, 2 * F, F)}
    total_flops = sum(flops.values())
    gemm_ms = {nme: med[f"{nme}.gemm"] for nme in flops}
    def prod_parts(nme):
        return [k for k in (f"{nme}.quantize", f"{nme}.absmax", f"{nme}.pack") if k in med]

    prod_ms = {nme: sum(med[k] for k in prod_parts(nme)) for nme in flops}
    gemm_avg_ms = float(np.mean([np.mean(per[f"{nme}.gemm"]) for nme in flops]))
    gemm_achieved = (total_flops / 3) / (gemm_avg_ms * 1e-3) / 1e12

    value = total_flops / (ms_per_step * 1e-3) / 1e12
    gemm_hash = src_hash("gemm.hip", "nvfp4_device.h", "internal.h")
    traffic = traffic_entry("gemm_kernel", gemm_hash)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_detail": "NVFP4 (e2m1 values, e4m3 block scales) operands decoded exactly to f16 for the MFMA, "
                        "fp32 accumulation, bf16 output; producers in binary32 with bf16 roundings",
        "data": "synthetic (seeded; shapes of the H3 block at 37,810 tokens)",
        "config": {
            "workload": "H3 block NVFP4 projections QKV+FC1+FC2, M=37810 (padded 37824): modulation producer "
                        "K=5376 -> GEMM N=21504 and N=14336; SwiGLU producer F=14336 -> GEMM N=5376",
            "M": M, "M_pad": M_pad,
            "value_definition": "total GEMM flop of the three projections / whole step time (producers included)",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "nvfp4_gemm_ws: gemm_kernel per projection (QKV, FC1, FC2; FC2 adds a K-split launch for its "
                      "last partial wave and a finalize launch); achieved = per-projection call time",
            "achieved": round(gemm_achieved, 1),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_achieved / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(gemm_avg_ms, 4),
            "flop_per_launch_avg": total_flops / 3,
        },
        "producer": {
            nme: {"ms": round(prod_ms[nme], 4), "launches": {k.split(".")[1]: round(med[k], 4) for k in prod_parts(nme)},
                  "bytes": prod_bytes[nme],
                  "bytes_definition": "algorithmic: two reads of the input, QDATA and SFA written (padding rows "
                                      "included); GBps and frac_hbm divide these by the time",
                  "counter_bytes": producer_counter_bytes("swiglu" if nme == "fc2" else "modulate"),
                  "GBps": round(prod_bytes[nme] / (prod_ms[nme] * 1e-3) / 1e9, 1),
                  "frac_hbm": round(prod_bytes[nme] / (prod_ms[nme] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "one_read_bytes": prod_one_read[nme],
                  "frac_hbm_one_read": round(prod_one_read[nme] / (prod_ms[nme] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            for nme in flops
        },
        "gemm": {
            nme: {"ms": round(gemm_ms[nme], 4), "flop": flops[nme],
                  "TFLOPs": round(flops[nme] / (gemm_ms[nme] * 1e-3) / 1e12, 1),
                  "frac_peak": round(flops[nme] / (gemm_ms[nme] * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
            for nme in flops
        },
        "timing": {"wall_ms_timed_region": round(wall_ms, 2), "event_ms_timed_region": round(total_ms, 2),
                   "setup_s": round(setup_s, 1), "kernel_source_hash": gemm_hash,
                   "launch_ms_in_step": launch_pct},
        "input_sha256": input_sha,
        "output_sha256": hashes,
        "producer_standalone": {
            nme: dict(v, bytes=prod_bytes[nme],
                      frac_hbm_cold_p50=round(prod_bytes[nme] / (v["cold_p50_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
            for nme, v in standalone.items()
        },
        "context": "pages' numbers (GB10/DGX Spark): fused producer 6.02 ms for the block-24 QKV input vs "
                   "10.47/10.60 ms unfused modulation; CUTLASS 1024^3 block-scaled GEMM 126.57 TFLOP/s",
        "cpu_baseline": None,
    }

    if not args.no_attn_out:
        result["attn_out"] = attn_out_projection(nv, synth, dev, stream, args.steps)
    if not args.no_ring:
        result["ring"] = ring_projection(nv, x, seg_structs["qkv"][0], weights["qkv"], bufs["qkv"], M, M_pad, wq,
                                         dev, stream, reps=max(5, args.steps))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, x_h, segs, gu_h, (wq, wf1, wf2))
    print(json.dumps(result), flush=True)


def ring_projection(nv, x, seg, weight, b, M, M_pad, w, dev, stream, reps):
    """The QKV projection through the packed-tile ring (nvfp4_modulate_gemm_ring)
    timed next to the chained path (single-launch producer + GEMM) on the same
    stream, alternating, after the step; not part of value."""
    import numpy as np
    import torch

    qw, sfw, tw = weight
    K, N = w.K, w.N
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    variants = {}
    for chunk, slots in ((2048, 3), (2304, 3), (4096, 3)):
        ring = torch.empty(slots * nv.nvfp4_ring_slot_bytes(chunk, K), dtype=torch.uint8, device=dev)
        gws_bytes = nv.nvfp4_ring_gemm_workspace_bytes(M, chunk, N, K)
        gws = torch.empty(max(gws_bytes, 16), dtype=torch.uint8, device=dev)
        variants[f"ring_{chunk}x{slots}"] = (
            lambda ring=ring, gws=gws, gws_bytes=gws_bytes, chunk=chunk, slots=slots: nv.nvfp4_modulate_gemm_ring(
                x, M, K, K, seg, b["ws"], b["ts"], b["amax"], ring, slots, chunk, qw, sfw, tw, N, out, N, gws,
                gws_bytes, stream))

    def chained():
        nv.nvfp4_modulate_quantize(x, M, K, K, seg, b["ws"], b["ts"], b["amax"], b["q"], b["s"], M_pad, stream)
        nv.nvfp4_gemm_ws(b["q"], b["s"], b["ts"], M, M_pad, qw, sfw, tw, N, K, b["out"], N, b["gws"], b["gws_bytes"],
                         stream)

    runs = {"chained": chained, **variants}
    times = {k: [] for k in runs}
    for fn in runs.values():  # warm-up
        fn()
    stream.synchronize()
    for _ in range(reps):
        for k, fn in runs.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            times[k].append((e0, e1))
    stream.synchronize()
    ms = {k: float(np.median([a.elapsed_time(z) for a, z in v])) for k, v in times.items()}
    full_rows = (M // 2304) * 2304  # rows of the full 2304-row chunks (no K-split tiles in either path there)
    same = bool(torch.equal(out[:full_rows].view(torch.int16), b["out"][:full_rows].view(torch.int16)))
    flop = 2.0 * M * N * K
    return {
        "workload": "QKV projection M=37810 K=5376 N=21504: pass 1 over all rows, then chunks packed into a ring of "
                    "slots and multiplied (packs and odd/even chunk GEMMs on three streams); timed after the step, "
                    "alternating with the chained path; not part of value",
        "ms_p50": {k: round(v, 4) for k, v in ms.items()},
        "TFLOPs": {k: round(flop / (v * 1e-3) / 1e12, 1) for k, v in ms.items()},
        "vs_chained": {k: round(ms["chained"] / v, 4) for k, v in ms.items() if k != "chained"},
        "outputs_equal_chained_full_chunks": same,
    }


def output_hashes(bufs):
    """SHA-256 of each projection's outputs after the timed steps: tensor scale
    (its 4 bytes), QDATA and SFA (padding rows included) and the bf16 GEMM
    output.  Every kernel sums in a fixed order, so these are the same on every
    run and every device."""
    import hashlib

    import torch

    def sha(t):
        flat = t.contiguous().view(torch.uint8).view(-1)
        h = hashlib.sha256()
        step = 1 << 28
        for i in range(0, flat.numel(), step):
            h.update(flat[i:i + step].cpu().numpy().tobytes())
        return h.hexdigest()

    torch.cuda.synchronize()
    return {name: {k: sha(b[k]) for k in ("ts", "q", "s", "out")} for name, b in bufs.items()}


def standalone_producers(seq, stream, dev, reps):
    """Each producer of the step timed on its own (after the timed steps):
    cold = right after a 1 GiB read of another buffer, which evicts the input
    from every cache level (a read, not a write: written lines would still be
    dirty in the memory-side cache and their write-back would be timed with the
    producer), warm = run again straight after itself.  HIP events on the launch
    stream; p50 and p95 over `reps`."""
    import numpy as np
    import torch

    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    parts = {}
    for label, _, fn in seq:
        nme, part = label.split(".")
        if part != "gemm":
            parts.setdefault(nme, []).append(fn)
    out = {}
    for nme, fns in parts.items():
        cold, warm = [], []
        for k in range(reps + 1):  # the first rep is a warm-up
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            with torch.cuda.stream(stream):
                flush.max()
            ev[0].record(stream)
            for fn in fns:
                fn()
            ev[1].record(stream)
            ev[2].record(stream)
            for fn in fns:
                fn()
            ev[3].record(stream)
            stream.synchronize()
            if k:
                cold.append(ev[0].elapsed_time(ev[1]))
                warm.append(ev[2].elapsed_time(ev[3]))
        out[nme] = {"cold_p50_ms": round(float(np.percentile(cold, 50)), 4),
                    "cold_p95_ms": round(float(np.percentile(cold, 95)), 4),
                    "warm_p50_ms": round(float(np.percentile(warm, 50)), 4),
                    "warm_p95_ms": round(float(np.percentile(warm, 95)), 4)}
    del flush
    return out


def attn_out_projection(nv, synth, dev, stream, reps):
    """The attention-output projection, timed on its own after the step (not
    part of `value`): the plain quantizer on the attention values [37810, 7168]
    and the GEMM to the model width 5376 with the residual epilogue
    out = bf16(residual + bf16(gate * o)) written in place into the residual."""
    import numpy as np
    import torch

    w = synth.workload("attn_out")
    M, K, N, M_pad = w.M, w.K, w.N, w.m_pad

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x = up(w.x())
    wt = up(w.weight())
    rs, gate = w.gates()
    residual0 = up(w.residual())
    residual = residual0.clone()
    gates, keep = nv.make_row_gates(rs, up(gate))
    with torch.cuda.stream(stream):
        qw, sfw, tw = nv.quantize_weight(wt, stream=stream)
    q = torch.empty((M_pad, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M_pad, K // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.zeros(int(nv.lib.nvfp4_absmax_workspace_bytes()), dtype=torch.uint8, device=dev)
    need = nv.nvfp4_gemm_workspace_bytes(M, N, K)
    gws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 1)]
    for k in range(reps + 1):  # the first is a warm-up
        ev[k][0].record(stream)
        nv.nvfp4_quantize(x, M, K, K, ws, ts, None, q, s, M_pad, stream)
        ev[k][1].record(stream)
        nv.nvfp4_gemm_gate_residual(q, s, ts, M, M_pad, qw, sfw, tw, N, K, gates, residual, N, residual, N, gws,
                                    need, stream)
        ev[k][2].record(stream)
    stream.synchronize()
    pq = float(np.median([e[0].elapsed_time(e[1]) for e in ev[1:]]))
    pg = float(np.median([e[1].elapsed_time(e[2]) for e in ev[1:]]))
    pbytes = 2 * M * K * 2 + M_pad * (K // 2 + K // 16)
    flop = 2.0 * M * N * K
    del keep
    return {
        "workload": "plain quantizer on [37810, 7168] -> NVFP4 GEMM N=5376 with the residual epilogue (2 gate "
                    "segments, residual updated in place); timed on its own, not part of value",
        "producer_ms": round(pq, 4), "producer_GBps": round(pbytes / (pq * 1e-3) / 1e9, 1),
        "producer_frac_hbm": round(pbytes / (pq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "gemm_ms": round(pg, 4), "gemm_TFLOPs": round(flop / (pg * 1e-3) / 1e12, 1),
        "gemm_frac_peak": round(flop / (pg * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
    }


def _oracle_weight(oracle, wt):
    """NVFP4 weight bytes from the oracle quantizer (untimed preparation; row
    ranges on several host threads, the maximum over ranges is exact)."""
    import concurrent.futures as cf

    import numpy as np

    N = wt.shape[0]
    nthr = max(1, min(16, len(os.sched_getaffinity(0))))
    step = (N + 4 * nthr - 1) // (4 * nthr)
    ranges = [(a, min(N, a + step)) for a in range(0, N, step)]
    with cf.ThreadPoolExecutor(nthr) as ex:
        amax = max(ex.map(lambda r: oracle.bf16_amax(wt[r[0]:r[1]]), ranges))
        sw = oracle.tensor_scale(amax)
        parts = list(ex.map(lambda r: oracle.bf16_pack_rows(wt, sw, *r), ranges))
    return sw, np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _pool_map(ex, fn, items):
    return list(ex.map(fn, items)) if ex is not None else [fn(i) for i in items]


def _ranges(n, parts):
    return [r for r in ((a * n // parts, (a + 1) * n // parts) for a in range(parts)) if r[1] > r[0]]


def _oracle_modulation_producer(oracle, x_h, seg, M, M_pad, ex, parts):
    """The whole modulation producer through the oracle: pass 1 over every row,
    then pass 2 over every padded row (row ranges; maxima merged exactly)."""
    s_g = oracle.tensor_scale(_max_bits(_pool_map(ex, lambda r: oracle.modulate_amax_rows(x_h, seg, *r),
                                                  _ranges(M, parts))))
    _pool_map(ex, lambda r: oracle.modulate_pack_rows(x_h, seg, s_g, *r), _ranges(M_pad, parts))
    return s_g


def _max_bits(vals):
    """Maximum of binary32 maxima as the producers define it: over the bit
    patterns of the magnitudes (NaN above Inf above every finite value)."""
    import numpy as np

    bits = np.array(vals, np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)
    return float(np.array([bits.max()], np.uint32).view(np.float32)[0])


def cpu_baseline(args, x_h, segs, gu_h, works):
    """The oracle as it stands, timed in the same run on this host.

    - The whole producer of the 37,810 x 5,376 modulation workload (pass 1 over
      every row, pass 2 over every padded row), once single-threaded and once
      on all host cores (row ranges on a thread pool, maxima merged exactly).
    - The SwiGLU producer on its first `cpu_rows` * 8 rows (single-threaded),
      extrapolated to all rows.
    - The FP64 GEMM reference on `cpu_rows` sampled rows of each projection
      with all N (single-threaded), as seconds per row, extrapolated to all
      37,810 rows.
    `value` is the whole step at the oracle's single-threaded rates: GEMM flop
    of the three projections / (measured modulation producer x 2 + the
    extrapolated SwiGLU producer and GEMMs); `extrapolated` says which parts are
    extrapolated.  Weight prepacking is not part of the step and is not timed."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    oracle.lib()
    rows = args.cpu_rows
    cores = len(os.sched_getaffinity(0))
    wq = works[0]
    M, M_pad, K = wq.M, wq.m_pad, wq.K
    rs, sh, sc = wq.segments()
    seg = oracle.Segments(rs, sh, sc)
    mod_bytes = modulation_bytes(M, M_pad, K)

    t0 = time.perf_counter()
    _oracle_modulation_producer(oracle, x_h, seg, M, M_pad, None, 1)
    t_mod1 = time.perf_counter() - t0
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        _oracle_modulation_producer(oracle, x_h, seg, M, M_pad, ex, 4 * cores)
        t_modn = time.perf_counter() - t0

    # SwiGLU producer on a row prefix, single-threaded
    w2 = works[2]
    sr = min(M, 8 * rows)
    t0 = time.perf_counter()
    a = oracle.swiglu_amax_rows(gu_h, 0, sr)
    oracle.swiglu_pack_rows(gu_h, oracle.tensor_scale(a), 0, sr)
    t_sw_rows = time.perf_counter() - t0
    t_sw = t_sw_rows * M_pad / sr

    # GEMM reference per checked row, single-threaded, on oracle-packed operands
    gemm = {}
    t_gemm_total = 0.0
    flop_total = 0.0
    for w in works:
        # untimed preparation on the thread pool: oracle weight bytes, the
        # activation's tensor scale and the checked rows' packed bytes
        wts = w.weight()
        sw, qw, sfw = _oracle_weight(oracle, wts)
        del wts
        chk = w.check_rows(rows)
        with cf.ThreadPoolExecutor(max_workers=cores) as ex:
            if w.kind == "modulate":
                rs_w, sh_w, sc_w = w.segments()
                seg_w = oracle.Segments(rs_w, sh_w, sc_w)
                s_a = oracle.tensor_scale(_max_bits(_pool_map(
                    ex, lambda r: oracle.modulate_amax_rows(x_h, seg_w, *r), _ranges(M, 4 * cores))))
                packed = [oracle.modulate_pack_rows(x_h, seg_w, s_a, int(r), int(r) + 1) for r in chk]
            else:
                s_a = oracle.tensor_scale(_max_bits(_pool_map(
                    ex, lambda r: oracle.swiglu_amax_rows(gu_h, *r), _ranges(M, 4 * cores))))
                packed = [oracle.swiglu_pack_rows(gu_h, s_a, int(r), int(r) + 1) for r in chk]
        qa = np.concatenate([p[0] for p in packed])
        sfa = np.concatenate([p[1] for p in packed])
        # the reference decodes the whole weight once per call: timed alone
        # (no rows), then with the checked rows; the difference per row
        # scales to all rows
        t0 = time.perf_counter()
        oracle.gemm_rows(qa, sfa, s_a, qw, sfw, sw, np.arange(0))
        t_dec = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm_rows(qa, sfa, s_a, qw, sfw, sw, np.arange(chk.size))
        t = time.perf_counter() - t0
        per_row = max(t - t_dec, 1e-9) / chk.size
        gemm[w.name] = {"rows_timed": int(chk.size), "s_weight_decode": round(t_dec, 3),
                        "s_per_row": round(per_row, 4), "GFLOPs_per_row": round(2.0 * w.N * w.K / per_row / 1e9, 3),
                        "extrapolated_s_all_rows": round(t_dec + per_row * M, 1)}
        t_gemm_total += t_dec + per_row * M
        flop_total += 2.0 * M * w.N * w.K
    step_s = 2 * t_mod1 + t_sw + t_gemm_total
    return {
        "value": round(flop_total / step_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"whole 37,810 x 5,376 modulation producer measured ({t_mod1:.1f} s, 1 thread), counted for QKV "
                   f"and FC1; SwiGLU producer timed on {sr} rows and FP64 GEMM reference on {rows} checked rows per "
                   f"projection (all N), both extrapolated to 37,810 rows"),
        "extrapolated": ["swiglu producer", "gemm"],
        "step_s_extrapolated": round(step_s, 1),
        "producer_full": {"workload": "modulation producer [37810, 5376], both passes, every row",
                          "bytes": mod_bytes,
                          "one_core": {"s": round(t_mod1, 2), "GBps": round(mod_bytes / t_mod1 / 1e9, 4)},
                          "all_cores": {"cores": cores, "s": round(t_modn, 2),
                                        "GBps": round(mod_bytes / t_modn / 1e9, 4)}},
        "swiglu_producer": {"rows_timed": sr, "s": round(t_sw_rows, 2), "extrapolated_s_all_rows": round(t_sw, 1)},
        "gemm": gemm,
        "host_cores_available": cores,
    }


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------
PROJ = ("qkv", "fc1", "fc2")  # GEMM launch order within a step
SHAPES = {"qkv": (37810, 21504, 5376), "fc1": (37810, 14336, 5376), "fc2": (37810, 5376, 14336)}


def _gemm_role(name):
    """'main', 'split' or 'finalize' for the GEMM kernels, else None."""
    if "gemm_finalize_kernel" in name:
        return "finalize"
    if "gemm_kernel" not in name:
        return None
    args = name.split("gemm_kernel<", 1)[1].split(">", 1)[0].split(",") if "gemm_kernel<" in name else []
    return "split" if len(args) > 1 and args[1].strip() == "true" else "main"


def _gemm_calls(items):
    """Group GEMM dispatches (in dispatch order) into calls: a main launch
    starts a call, split and finalize launches belong to the call before them.
    items: (dispatch_id, kernel_name, grid, payload).  The step's calls cycle
    through QKV, FC1, FC2, each with its own main-launch grid; the grids are
    taken from the first three calls and the grouping stops at the first call
    that breaks the cycle (the attention-output projection timed after the
    steps).  Returns [(projection, [payloads])]."""
    calls = []
    for _, name, grid, payload in sorted(items, key=lambda t: t[0]):
        role = _gemm_role(name)
        if role is None:
            continue
        if role == "main" or not calls:
            calls.append((grid, []))
        calls[-1][1].append(payload)
    out = []
    for i, (grid, c) in enumerate(calls):
        if i >= 3 and grid != calls[i % 3][0]:
            break
        out.append((PROJ[i % 3], c))
    return out


def _csv_rows(d, suffix):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    return name.split("(")[0].replace("void ", "")


def _bench_line(path):
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def summarize_trace(d, skip=0, bench_json=None):
    import numpy as np

    stats = _csv_rows(d, "kernel_stats.csv")
    trace = _csv_rows(d, "kernel_trace.csv")
    out = ["| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats:
        if "nvfp4::" not in r["Name"]:
            continue
        out.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    calls = _gemm_calls([(int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size_X"]),
                          (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in trace])
    per = {p: [] for p in PROJ}
    for p, c in calls:
        per[p].append(sum(c))
    per = {p: v[skip:] for p, v in per.items()}
    gem = [u for p in PROJ for u in per[p]]
    out += ["", "GEMM calls (main launch plus, for FC2, the K-split launch and the finalize launch)"
            + (f", the {skip} warm-up steps left out" if skip else "") + ":", "",
            "| GEMM call | M, N, K | calls | mean us | TFLOP/s | % of 2516.6 |", "|---|---|---|---|---|---|"]
    tot_f = tot_us = 0.0
    for p in PROJ:
        if not per[p]:
            continue
        M, N, K = SHAPES[p]
        us = float(np.mean(per[p]))
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        tot_f += 2.0 * M * N * K * len(per[p])
        tot_us += sum(per[p])
        out.append(f"| {p} | {M}, {N}, {K} | {len(per[p])} | {us:.1f} | {tf:.1f} | {100 * tf / MFMA_F16_PEAK_TFLOPS:.1f} |")
    if tot_us:
        tf = tot_f / (tot_us * 1e-6) / 1e12
        out.append(f"| all | | {len(gem)} | {tot_us / len(gem):.1f} | {tf:.1f} | {100 * tf / MFMA_F16_PEAK_TFLOPS:.1f} |")
    # the step's producer launches, in dispatch order: modulation (QKV, FC1) and SwiGLU (FC2)
    tr = sorted(trace, key=lambda r: int(r["Dispatch_Id"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # noqa: E731
    mod = [dur(r) for r in tr if "modulate_quantize_kernel<false>" in r["Kernel_Name"]]
    fill = [dur(r) for r in tr if "silu_lut_fill_kernel" in r["Kernel_Name"]]
    sw = [dur(r) for r in tr if "swiglu_quantize_kernel" in r["Kernel_Name"]]
    # the FC2 producer call is the silu table fill and the single launch
    prod = {"qkv": mod[0::2][skip:], "fc1": mod[1::2][skip:],
            "fc2": [a + b for a, b in zip(fill, sw)][skip:]}
    bench = _bench_line(bench_json) if bench_json else None
    out += ["", "The step's launches, median over the profiled steps" + (f" after the {skip} warm-up steps" if skip
                                                                        else "")
            + (", beside the bench line of the same node (HIP events on the launch stream, p50)" if bench else "")
            + ":", "",
            "| launch | profiled steps | median us | bench p50 us | profiled / bench |", "|---|---|---|---|---|"]
    for p in PROJ:
        for kind, vals in (("quantize", prod[p]), ("gemm", per[p])):
            if not vals:
                continue
            med = float(np.median(vals))
            b = bench["timing"]["launch_ms_in_step"].get(f"{p}.{kind}", {}).get("p50") if bench else None
            bcol = f"{b * 1e3:.1f} | {med / (b * 1e3):.4f}" if b else " | "
            out.append(f"| {p}.{kind} | {len(vals)} | {med:.1f} | {bcol} |")
    if bench:
        out += ["", f"Bench line of the same node: {bench['ms_per_step']} ms per step, value {bench['value']} "
                    f"{bench['unit']}, roofline frac {bench['roofline']['frac']} "
                    f"(achieved {bench['roofline']['achieved']} of {bench['roofline']['peak']} TFLOP/s)."]
    return "\n".join(out)


def _counter_by_dispatch(d):
    rows = _csv_rows(d, "counter_collection.csv")
    by = {}
    for r in rows:
        k = int(r["Dispatch_Id"])
        e = by.setdefault(k, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "v": 0.0})
        e["v"] += float(r["Counter_Value"])
    return by


def summarize_traffic(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the GEMM launches, each
    scaled by what the same counter reads for the 1 GiB calibration copy."""
    import numpy as np

    f = _counter_by_dispatch(fetch_dir)
    w = _counter_by_dispatch(write_dir)
    gib_kib = float(1 << 20)

    def calib(by):
        """Scale factor and dispatch id of the 1 GiB calibration copy, which
        runs after the untimed weight prepacks and before the first step."""
        cps = [(e["v"], k) for k, e in by.items() if "copy" in e["name"].lower() and e["v"] > gib_kib / 4]
        if not cps:
            raise SystemExit("no 1 GiB calibration copy found (run bench.py with --copy-calibration)")
        v, k = max(cps)
        return gib_kib / v, k

    (fs, f0), (ws, w0) = calib(f), calib(w)
    f = {k: e for k, e in f.items() if k > f0}
    w = {k: e for k, e in w.items() if k > w0}

    per = {p: {"fetch": [], "write": []} for p in PROJ}
    for p, c in _gemm_calls([(k, e["name"], e["grid"], e["v"]) for k, e in f.items()]):
        per[p]["fetch"].append(sum(c) * fs * 1024)
    for p, c in _gemm_calls([(k, e["name"], e["grid"], e["v"]) for k, e in w.items()]):
        per[p]["write"].append(sum(c) * ws * 1024)
    shapes = {}
    for p in PROJ:
        M, N, K = SHAPES[p]
        Mp = (M + 63) // 64 * 64
        alg = Mp * (K // 2 + K // 16) + N * (K // 2 + K // 16) + M * N * 2
        shapes[p] = {"fetch": int(np.mean(per[p]["fetch"])), "write": int(np.mean(per[p]["write"])),
                     "algorithmic_operand_and_output_bytes": alg}
    bpl = float(np.mean([shapes[p]["fetch"] + shapes[p]["write"] for p in PROJ]))
    entry = {
        "bytes_per_launch": int(bpl),
        "source_hash": src_hash("gemm.hip", "nvfp4_device.h", "internal.h"),
        "fetch_scale": round(fs, 4),
        "write_scale": round(ws, 4),
        "per_shape_bytes": shapes,
        "note": "FETCH_SIZE and WRITE_SIZE (KiB/dispatch, rocprofv3 --pmc, one counter per run) scaled by the "
                "readings of a 1 GiB plain copy in the same run; mean over the QKV, FC1 and FC2 launches",
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data["gemm_kernel"] = entry
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1)
    out = [f"Calibration: 1 GiB copy -> fetch x{fs:.3f}, write x{ws:.3f}.", "",
           "| kernel | launch | fetch (scaled, MB) | write (scaled, MB) | algorithmic bytes (MB) |",
           "|---|---|---|---|---|"]
    for p in PROJ:
        e = shapes[p]
        out.append(f"| gemm_kernel | {p} | {e['fetch'] / 1e6:.1f} | {e['write'] / 1e6:.1f} | "
                   f"{e['algorithmic_operand_and_output_bytes'] / 1e6:.1f} |")
    prod = {}
    for k in sorted(f):
        e = f[k]
        n = _short(e["name"])
        if "nvfp4::" in n and "gemm" not in n:
            prod.setdefault((n, e["grid"]), {"fetch": [], "write": []})["fetch"].append(e["v"] * fs * 1024)
    for k in sorted(w):
        e = w[k]
        n = _short(e["name"])
        if (n, e["grid"]) in prod:
            prod[(n, e["grid"])]["write"].append(e["v"] * ws * 1024)
    prod_entry = {}
    for (n, g), e in prod.items():
        fm = float(np.mean(e["fetch"])) if e["fetch"] else 0.0
        wm = float(np.mean(e["write"])) if e["write"] else 0.0
        out.append(f"| {n.replace('nvfp4::', '')} | grid {g} | {fm / 1e6:.1f} | {wm / 1e6:.1f} | |")
        # the step's producer launches (256 workgroups of 1024 or 896 threads)
        if "modulate_quantize_kernel<false>" in n and g == 256 * 1024:
            prod_entry["modulate"] = {"fetch": int(fm), "write": int(wm)}
        elif "swiglu_quantize_kernel" in n and g == 256 * 896:
            prod_entry["swiglu"] = {"fetch": int(fm), "write": int(wm)}
    if prod_entry:
        data["producer_single_launch"] = {
            "source_hash": src_hash("producer.hip", "nvfp4_device.h", "internal.h"), "per_launch_bytes": prod_entry,
            "note": "FETCH_SIZE / WRITE_SIZE of the step's single-launch producers, scaled like the GEMM's"}
        with open(path, "w") as fh:
            json.dump(data, fh, indent=1)
    out.append("")
    out.append(f"profiles/traffic.json: gemm_kernel bytes_per_launch {int(bpl)} (source hash {entry['source_hash']})")
    return "\n".join(out)


def summarize_counters(d):
    """Mean of each counter per kernel (dispatches grouped by kernel name and
    grid), with the elements one launch covers for the producer kernels of the
    step: modulation [37810, 5376], SwiGLU output [37810, 14336], and for the
    plain quantizer of the attention-output projection [37810, 7168]."""
    import numpy as np

    rows = _csv_rows(d, "counter_collection.csv")
    by = {}
    for r in rows:
        k = int(r["Dispatch_Id"])
        e = by.setdefault(k, {"name": _short(r["Kernel_Name"]), "grid": int(r["Grid_Size"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    groups = {}
    for e in by.values():
        if "nvfp4::" in e["name"]:
            groups.setdefault((e["name"].replace("nvfp4::", ""), e["grid"]), []).append(e)
    names = sorted({c for e in by.values() for c in e if c not in ("name", "grid")})
    elems = {"modulate": 37810 * 5376, "plain": 37810 * 7168, "swiglu": 37810 * 14336}
    out = ["| kernel | grid | dispatches | " + " | ".join(names) + " | VALU lane-ops / element |",
           "|---|---|---|" + "---|" * len(names) + "---|"]
    for (n, g), es in sorted(groups.items(), key=lambda t: -len(t[1])):
        means = [float(np.mean([e.get(c, 0.0) for e in es])) for c in names]
        # the step's producer launches: 256 workgroups of 1024 (modulation) or 896 (SwiGLU) threads
        kind = ("modulate" if "modulate_quantize_kernel<false>" in n and g == 256 * 1024 else
                "plain" if "modulate_quantize_kernel<true>" in n and g == 256 * 1024 else
                "swiglu" if "swiglu" in n and "fill" not in n and g == 256 * 896 else None)
        per = ""
        if kind and "SQ_INSTS_VALU" in names:
            per = f"{means[names.index('SQ_INSTS_VALU')] * 64 / elems[kind]:.2f}"
        out.append(f"| {n} | {g} | {len(es)} | " + " | ".join(f"{m:.4g}" for m in means) + f" | {per} |")
    return "\n".join(out)


def summarize_mfma(d, skip=0):
    """Per GEMM launch: mean engine clock (GRBM_GUI_ACTIVE summed over the 8
    XCDs / duration) and MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES summed over the
    1024 SIMDs / 1024 / active cycles).  A v_mfma_f32_32x32x16_f16 keeps a
    SIMD's matrix core busy 32 cycles, so busy x clock x 1024 SIMDs x 1024
    flop/cycle is the MFMA rate the counters imply."""
    import numpy as np

    rows = _csv_rows(d, "counter_collection.csv")
    by = {}
    for r in rows:
        if _gemm_role(r["Kernel_Name"]) is None:
            continue
        e = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                 "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = {p: [] for p in PROJ}
    for p, c in _gemm_calls([(k, e["name"], e["grid"], e) for k, e in by.items()]):
        tot = {"us": sum(x["us"] for x in c)}
        for key in ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES"):
            tot[key] = sum(x.get(key, 0.0) for x in c)
        per[p].append(tot)
    per = {p: v[skip:] for p, v in per.items()}
    out = ["| GEMM call | calls | mean us (profiled) | clock GHz | MFMA busy | implied TFLOP/s | measured TFLOP/s |",
           "|---|---|---|---|---|---|---|"]
    for p in PROJ:
        if not per[p]:
            continue
        M, N, K = SHAPES[p]
        us = float(np.mean([e["us"] for e in per[p]]))
        act = float(np.mean([e["GRBM_GUI_ACTIVE"] / 8 for e in per[p]]))
        busy = float(np.mean([e["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (e["GRBM_GUI_ACTIVE"] / 8) for e in per[p]]))
        clk = act / (us * 1e3)
        implied = busy * clk * 1e9 * 1024 * 1024 / 1e12
        meas = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out.append(f"| {p} | {len(per[p])} | {us:.1f} | {clk:.3f} | {busy:.3f} | {implied:.1f} | {meas:.1f} |")
    return "\n".join(out)


if __name__ == "__main__":
    main()
