#!/usr/bin/env python3
"""Throughput of the ConvRot INT4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--M M]

One "step" is one pass of the whole layer over one batch, the w4_linear call: rotate +
quantize the activations and the integer GEMM with the fused dequant epilogue (two
launches, or one fused launch for a single token); for the 20-block workload a step is all 80 linears
of the 20 blocks with the rotation cache and the low-rank branches.  Weights are packed
once before timing (an offline step).  Inputs are resident in HBM; the timed loop
cycles through enough distinct input copies (> 256 MB) that reads come from HBM, not
from the 256 MB Infinity Cache.

The K timed steps run as one HIP graph holding their launches in order (captured once
before timing, then replayed once; ``--eager`` times plain launches instead).

Prints ONE JSON line.  ``roofline`` describes the dominant kernel, timed live with HIP
events on the stream it runs on around K back-to-back launches of it (before the timed
replays); ``cpu_baseline`` is the CPU oracle timed on this host's cores on a bounded sample
of the same workload.

Workloads (sizes of FLUX / Z-Image style DiT blocks and text-encoder linears):
  attn_proj    (default) W4A8 g=256, X [4096, 3072] -> 3072           metric: TOPS
  mlp_up       W4A4 g=256, X [4096, 3072] -> 12288                   metric: TOPS
  mlp_down     W4A4 g=256, X [4096, 12288] -> 3072                   metric: TOPS
  small_m      asym W4A8 g=256, M in {1,4,16,64}, K/N 4096/12288     metric: weight GB/s
  double_block 20 blocks x {QKV, out, up, down} at M=4608, cached    metric: TOPS
  tiny         W4A8 g=64, 16 x 256 -> 256                            metric: TOPS
  attn_proj_grouped  attn_proj shape, fp16 weight scales per row and --gw inputs (W4A8)
  attn_proj_w4a16    attn_proj shape, W4A16 (no rotation, bf16 activations, grouped scales)
  small_m_w4a16      small_m shapes (symmetric codes) as W4A16                metric: weight GB/s
The default run also times the small-M text-encoder linear at M = 1 and 16 (K = 12288) and
reports them under "detail" (--no-small-m-detail skips that).
  mfma_peak    the int8 MFMA rate probe (libw4probe.so, not a layer): the chip's sustained
               dense int8 rate with random and with constant operands
  hbm_peak     the streaming-read probe (libw4probe.so): the HBM read rate a plain kernel
               reaches on 25 MB, the practical ceiling of the small-M kernels
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A8/W4A4 linear TOPS at M=4096; weight GB/s at M≤16; % of roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, 5.0 POPS
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="attn_proj",
                    choices=["attn_proj", "mlp_up", "mlp_down", "small_m", "double_block", "tiny", "mfma_peak",
                             "attn_proj_grouped", "attn_proj_w4a16", "small_m_w4a16", "hbm_peak"])
    ap.add_argument("--probe-mb", type=int, default=25, help="hbm_peak: buffer size in MB")
    ap.add_argument("--gw", type=int, default=128, help="grouped-scale workloads: inputs per weight scale")
    ap.add_argument("--lowrank", type=int, default=0, metavar="R",
                    help="single-linear workloads: add a rank-R low-rank branch (x . L1 computed once, untimed, "
                         "and added in the GEMM epilogue)")
    ap.add_argument("--no-small-m-detail", action="store_true",
                    help="attn_proj: skip timing the two small-M text-encoder shapes reported in detail")
    ap.add_argument("--summarize-trace", metavar="TRACE", default=None,
                    help="no GPU: per-kernel statistics of a rocprofv3 kernel trace (kernel_trace.csv or the "
                         "results .db), plus each kernel's mean duration over its timed back-to-back launches")
    ap.add_argument("--M", type=int, default=None, help="tokens (small_m: 1, 4, 16 or 64)")
    ap.add_argument("--K", type=int, default=12288, help="small_m: input features (4096 or 12288)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--cpu-rows", type=int, default=None, help="token rows in the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed loop, run two plain 512 MiB device copies (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU: read two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script with "
                         "--copy-calibration and record the dominant kernel's HBM bytes in profiles/traffic.json")
    return ap.parse_args()


# --------------------------------------------------------------------------- workloads
class Linear:
    """One quantized linear with its inputs on the GPU (weights packed once, untimed).

    gw > 0: the grouped-scale format (fp16 scales [N, K/gw], symmetric codes); bits 16 with
    g = 0 is W4A16."""

    def __init__(self, X, W, bias, g, bits, asym, lowrank=None, gw=0):
        import int4_weight_quantized_block_amd as w4
        self.g, self.bits, self.asym, self.gw = g, bits, asym, gw
        self.M, self.K = X.shape
        self.N = W.shape[0]
        self.X = X
        self.bias = bias
        if gw:
            self.packed, self.s_w = w4.w4_pack_weights_grouped(W, g, gw)
            self.zp = None
        else:
            self.packed, self.s_w, self.zp = w4.w4_pack_weights(W, g, asym)
        self.lowrank = lowrank

    def ops(self):
        return 2.0 * self.M * self.N * self.K

    def gemm_bytes(self):
        """Algorithmic HBM bytes of one GEMM launch (codes or bf16 X, weights, scales, bias, output)."""
        M, N, K = self.M, self.N, self.K
        a = {8: M * K, 4: M * K // 2, 16: 2 * M * K}[self.bits]
        return a + self.weight_bytes() + (0 if self.bits == 16 else 8 * M) + 2 * N + 2 * M * N

    def weight_bytes(self):
        if self.gw:
            return self.N * self.K // 2 + 2 * self.N * (self.K // self.gw)
        return self.N * self.K // 2 + 4 * self.N + (self.N if self.asym else 0)

    def fused_bytes(self):
        """Algorithmic HBM bytes of the fused single-token launch (bf16 X instead of codes)."""
        M, N, K = self.M, self.N, self.K
        return 2 * M * K + self.weight_bytes() + 2 * N + 2 * M * N

    def rotquant_bytes(self):
        M, K = self.M, self.K
        return 2 * M * K + (M * K if self.bits == 8 else M * K // 2) + 8 * M


def build_workload(args, dev):
    import torch
    import synth
    name = args.workload
    if name == "attn_proj":
        M = args.M or 4096
        d = synth.attn_proj(M=M)
        return [[("attn_proj", d["X"], d["W"], d["bias"], 256, 8, False)]], {
            "workload": "attn_proj", "M": M, "K": 3072, "N": 3072, "g": 256, "act_bits": 8,
            "weights": "sym int4 per-row"}
    if name in ("mlp_up", "mlp_down"):
        M = args.M or 4096
        up = synth.mlp_up(M=M)
        if name == "mlp_up":
            return [[("mlp_up", up["X"], up["W"], up["bias"], 256, 4, False)]], {
                "workload": "mlp_up", "M": M, "K": 3072, "N": 12288, "g": 256, "act_bits": 4,
                "weights": "sym int4 per-row"}
        dn = synth.mlp_down_weights()
        # the down-projection input has the shape of GELU(up); drawn as GELU of a scaled normal
        h = torch.nn.functional.gelu(torch.randn((M, 12288), generator=torch.Generator().manual_seed(2010)) * 0.6)
        return [[("mlp_down", h.to(torch.bfloat16), dn["W"], dn["bias"], 256, 4, False)]], {
            "workload": "mlp_down", "M": M, "K": 12288, "N": 3072, "g": 256, "act_bits": 4,
            "weights": "sym int4 per-row"}
    if name == "small_m":
        M = args.M or 16
        K = args.K
        N = 12288 if K == 4096 else 4096
        d = synth.small_m(M, K, N)
        return [[("small_m", d["X"], d["W"], d["bias"], 256, 8, True)]], {
            "workload": "small_m", "M": M, "K": K, "N": N, "g": 256, "act_bits": 8,
            "weights": "asym int4 per-row + zero point"}
    if name in ("attn_proj_grouped", "attn_proj_w4a16"):
        M = args.M or 4096
        d = synth.attn_proj(M=M)
        gw = args.gw
        if name == "attn_proj_grouped":
            return [[("attn_proj", d["X"], d["W"], d["bias"], 256, 8, False, gw)]], {
                "workload": name, "M": M, "K": 3072, "N": 3072, "g": 256, "act_bits": 8,
                "weights": "sym int4, fp16 scale per row and %d inputs" % gw}
        return [[("attn_proj", d["X"], d["W"], d["bias"], 0, 16, False, gw)]], {
            "workload": name, "M": M, "K": 3072, "N": 3072, "g": 0, "act_bits": 16,
            "weights": "sym int4, fp16 scale per row and %d inputs (W4A16, no rotation)" % gw}
    if name == "small_m_w4a16":
        M = args.M or 16
        K = args.K
        N = 12288 if K == 4096 else 4096
        d = synth.small_m(M, K, N)
        return [[("small_m", d["X"], d["W"], d["bias"], 0, 16, False, args.gw)]], {
            "workload": name, "M": M, "K": K, "N": N, "g": 0, "act_bits": 16,
            "weights": "sym int4, fp16 scale per row and %d inputs (W4A16, no rotation)" % args.gw}
    if name == "tiny":
        d = synth.tiny()
        return [[("tiny", d["X"], d["W"], d["bias"], 64, 8, False)]], {
            "workload": "tiny", "M": 16, "K": 256, "N": 256, "g": 64, "act_bits": 8,
            "weights": "sym int4 per-row"}
    raise SystemExit("unknown workload")


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(layer, rows_wanted):
    """The oracle as it stands, on this host's cores, over the first ``rows_wanted`` token rows
    of the layer: rotate + quantize, int64 GEMM, fp64 epilogue (weight packing not counted).
    Returns (dict, seconds, rows)."""
    import oracle
    name, X, W, bias, g, bits, asym = layer[:7]
    gw = layer[7] if len(layer) > 7 else 0
    M = X.shape[0]
    rows = min(M, rows_wanted)
    Xs = X[:rows].cpu()
    if gw:
        pw = oracle.pack_weights_grouped(W.cpu(), g, gw)
        t1 = time.perf_counter()
        if bits == 16:
            oracle.bf16_rne(oracle.to_f64(Xs) @ oracle.dequant_grouped(pw["packed"], pw["scale"], gw).T
                            + oracle.to_f64(bias.cpu())[None, :])
        else:
            qa = oracle.rotate_quant_act(Xs, g, bits)
            accg = oracle.gemm_i64_groups(qa["q"], oracle.weight_operand(pw["packed"], None, False), gw)
            oracle.bf16_rne(oracle.epilogue_grouped(accg, qa["scale"], pw["scale"], bias.cpu()))
        sec = time.perf_counter() - t1
        return {"cores": oracle.num_threads(), "kind": "oracle",
                "sample": "%s: %d of %d token rows, one pass (%s)" % (
                    name, rows, M, "fp64 product with the dequantized weights" if bits == 16 else
                    "rotate + quantize + int64 GEMM per weight group + grouped epilogue"),
                "seconds": round(sec, 3)}, sec, rows
    pw = oracle.pack_weights(W.cpu(), g, asym)
    t1 = time.perf_counter()
    qa = oracle.rotate_quant_act(Xs, g, bits)
    oracle.linear_from_codes(qa["q"], qa["scale"], pw["packed"], pw["scale"], pw["zp"], asym, bias.cpu())
    sec = time.perf_counter() - t1
    return {"cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%s: %d of %d token rows, one pass (rotate + quantize + int64 GEMM + epilogue)"
                      % (name, rows, M), "seconds": round(sec, 3)}, sec, rows


COPY_BYTES = 512 << 20
# kernel-name prefix -> (short name, source file)
KERNEL_SOURCE = {"k_gemm<": ("k_gemm", "gemm.hip"), "k_gemv": ("k_gemv", "gemv.hip"),
                 "k_rotquant": ("k_rotquant", "rotquant.hip"), "k_gemm_grp": ("k_gemm_grp", "gemm_grp.hip"),
                 "k_grp_stream": ("k_grp_stream", "gemm_grp.hip")}


def copy_calibration(dev):
    """Two plain device-to-device copies of COPY_BYTES: the known-size reference that scales the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("bench: %d MiB calibration copies done" % (COPY_BYTES >> 20))


def traffic_workload(workload, M, K):
    """Key of a workload in profiles/traffic.json (small-M entries carry their shape)."""
    return "%s_M%d_K%d" % (workload, M, K) if workload in ("small_m", "small_m_w4a16") else workload


def ingest_counters(fetch_dir, write_dir, workload):
    """Per-dispatch FETCH_SIZE and WRITE_SIZE of the dominant kernels, each scaled by the bytes
    per counter unit that the same counter shows for the calibration copy (which reads and
    writes COPY_BYTES), recorded with the hash of the kernel's source."""
    import csv
    import glob

    def per_kernel(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return by

    out_path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(out_path)) if os.path.exists(out_path) else {}
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def copy_units(by):
        vals = [v for k, vs in by.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs
                if v * 1024 >= COPY_BYTES / 4]
        if not vals:
            raise SystemExit("no calibration copy found in the counter runs")
        return sorted(vals)[len(vals) // 2]

    f_fetch = COPY_BYTES / copy_units(fetch)
    f_write = COPY_BYTES / copy_units(write)
    for prefix, (short, src) in KERNEL_SOURCE.items():
        fk = [v for k, vs in fetch.items() if prefix in k for v in vs]
        wk = [v for k, vs in write.items() if prefix in k for v in vs]
        if not fk or not wk:
            continue
        fm, wm = sorted(fk)[len(fk) // 2], sorted(wk)[len(wk) // 2]
        path = os.path.join(ROOT, "int4_weight_quantized_block_amd", "csrc", src)
        data["%s:%s" % (short, workload)] = {
            "bytes": round(fm * f_fetch + wm * f_write), "read_bytes": round(fm * f_fetch),
            "write_bytes": round(wm * f_write), "fetch_size": fm, "write_size": wm,
            "bytes_per_fetch_unit": f_fetch, "bytes_per_write_unit": f_write, "dispatches": len(fk),
            "source": src, "sha256": hashlib.sha256(open(path, "rb").read()).hexdigest()}
        log("traffic %s:%s  read %.1f MB  write %.1f MB" % (short, workload, fm * f_fetch / 1e6, wm * f_write / 1e6))
    with open(out_path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.steps)
    if args.ingest_counters:
        return ingest_counters(args.ingest_counters[0], args.ingest_counters[1],
                               traffic_workload(args.workload, args.M or 16, args.K))
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import int4_weight_quantized_block_amd as w4

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    w4.load_library()
    log("bench: workload %s on %s" % (args.workload, torch.cuda.get_device_name(0)))

    if args.workload == "double_block":
        return bench_double_block(args, dev)
    if args.workload == "mfma_peak":
        return bench_mfma_peak(args, dev)
    if args.workload == "hbm_peak":
        return bench_hbm_peak(args, dev)

    layer_specs, cfg = build_workload(args, dev)
    if args.lowrank:
        cfg = dict(cfg, lowrank=args.lowrank)
    spec = layer_specs[0][0]
    r = time_layer(args, dev, spec)
    lin, fused, t_rq, t_mm, wall = r["lin"], r["fused"], r["t_rq"], r["t_mm"], r["wall"]
    M, bits = lin.M, lin.bits
    ms_step = wall / args.steps * 1e3
    log("bench: %.3f ms/step wall (%s)" % (ms_step, "eager" if args.eager else "graph replay"))
    if args.copy_calibration:
        copy_calibration(dev)

    small = M <= 64
    if small:
        value = lin.weight_bytes() / (wall / args.steps) / 1e9
        unit = "GB/s"
        alg = lin.fused_bytes() if fused else lin.gemm_bytes()
        roof = {"bound": "hbm", "achieved": alg / t_mm / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        value = lin.ops() / (wall / args.steps) / 1e12
        unit = "TOPS"
        peak = PEAK_BF16_TFLOPS if bits == 16 else PEAK_INT8_TOPS
        roof = {"bound": "mfma", "achieved": lin.ops() / t_mm / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = r["kernel"]
    roof["traffic"] = measured_traffic(r["kernel"], cfg)
    roof["launch_us"] = round(t_mm * 1e6, 3)
    extra = {
        "fused": fused,
        "rotquant_us": round(t_rq * 1e6, 3) if t_rq else None,
        "rotquant_hbm_gbs": round(lin.rotquant_bytes() / t_rq / 1e9, 1) if t_rq else None,
        "rotquant_hbm_frac": round(lin.rotquant_bytes() / t_rq / 1e9 / PEAK_HBM_GBS, 4) if t_rq else None,
        "gemm_tops": round(lin.ops() / t_mm / 1e12, 2),
        "gemm_weight_gbs": round(lin.weight_bytes() / t_mm / 1e9, 1),
        "gemm_alg_bytes": lin.fused_bytes() if fused else lin.gemm_bytes(),
        "timed_launch": "eager" if args.eager else "one hip graph of the K steps",
        "input_copies": r["ncopy"],
    }
    if args.workload == "attn_proj" and not args.no_small_m_detail:
        # the metric's second half: weight GB/s of the HBM-bound text-encoder linears at M <= 16
        # (asymmetric W4A8, K = 12288 -> N = 4096), whole w4_linear step and dominant kernel
        extra["small_m"] = {}
        for Ms in (1, 16):
            sub = argparse.Namespace(**vars(args))
            sub.workload, sub.M, sub.K = "small_m", Ms, 12288
            sspec = build_workload(sub, dev)[0][0][0]
            rs = time_layer(sub, dev, sspec)
            ls = rs["lin"]
            step_s = rs["wall"] / args.steps
            alg = ls.fused_bytes() if rs["fused"] else ls.gemm_bytes()
            extra["small_m"]["M%d_K12288_N4096" % Ms] = {
                "weight_gbs_per_step": round(ls.weight_bytes() / step_s / 1e9, 1),
                "us_per_step": round(step_s * 1e6, 3),
                "kernel": rs["kernel"], "kernel_us": round(rs["t_mm"] * 1e6, 3),
                "kernel_hbm_gbs": round(alg / rs["t_mm"] / 1e9, 1),
                "kernel_hbm_frac": round(alg / rs["t_mm"] / 1e9 / PEAK_HBM_GBS, 4),
                "rotquant_us": round(rs["t_rq"] * 1e6, 3) if rs["t_rq"] else None}
            log("bench: small-M M=%d: %s" % (Ms, extra["small_m"]["M%d_K12288_N4096" % Ms]))
    cpu = None
    if not args.no_cpu_baseline:
        rows = args.cpu_rows or M
        log("bench: timing the CPU oracle on %d rows" % rows)
        cpu, sec, rows = cpu_baseline(spec, rows)
        if small:  # weight bytes streamed per full pass over the M tokens
            cpu["value"] = round(lin.weight_bytes() / (sec * M / rows) / 1e9, 4)
            cpu["unit"] = "GB/s"
        else:
            cpu["value"] = round(lin.ops() * rows / M / sec / 1e12, 6)
            cpu["unit"] = "TOPS"
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": {8: "int8", 4: "int4", 16: "bf16"}[bits],
        "data": "synthetic", "config": dict(cfg, parallelism="single-gpu"),
        "roofline": roof, "cpu_baseline": cpu, "detail": extra,
    }
    print(json.dumps(out), flush=True)


def time_layer(args, dev, spec):
    """Time one linear: per-launch durations of its kernels (HIP events around a graph of K
    back-to-back launches of each) and the wall time of K whole steps (one graph replay).
    Returns dict(lin, fused, t_rq, t_mm, wall, ncopy, kernel)."""
    import torch
    import int4_weight_quantized_block_amd as w4
    name, X, W, bias, g, bits, asym = spec[:7]
    gw = spec[7] if len(spec) > 7 else 0
    lin = Linear(X.to(dev), W.to(dev), bias.to(dev), g, bits, asym, gw=gw)
    # distinct copies of the inputs so the timed loop streams from HBM
    per_copy = lin.X.numel() * lin.X.element_size() + lin.packed.numel() + lin.s_w.numel() * lin.s_w.element_size()
    ncopy = max(1, min(64, math.ceil(2 * MALL_BYTES / per_copy)))
    Xs = [lin.X] + [lin.X.clone() for _ in range(ncopy - 1)]
    Ps = [(lin.packed, lin.s_w, lin.zp)] + [(lin.packed.clone(), lin.s_w.clone(),
                                            lin.zp.clone() if lin.zp is not None else None)
                                           for _ in range(ncopy - 1)]
    M, K, N = lin.M, lin.K, lin.N
    abits = 8 if bits == 16 else bits
    qbuf = torch.empty((M, K if abits == 8 else K // 2), dtype=torch.int8 if abits == 8 else torch.uint8, device=dev)
    sx = torch.empty((M,), dtype=torch.float32, device=dev)
    rs = torch.empty((M,), dtype=torch.int32, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L = w4.load_library()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    # argument tuples built once, so the timed loop costs little host time per launch and the
    # GPU never waits for the host
    xdt = w4.W4_BF16 if lin.X.dtype == torch.bfloat16 else w4.W4_F32
    bptr = lin.bias.data_ptr()
    if gw:
        wsg = torch.empty((max(256, w4.w4_linear_grouped_workspace_bytes(M, N, K, bits, gw)),), dtype=torch.uint8,
                          device=dev)
        wsc = torch.empty((max(256, w4.w4_grouped_workspace_bytes(M, N, K, bits, gw)),), dtype=torch.uint8,
                          device=dev)
        rq_args = [(x.data_ptr(), xdt, M, K, g, abits, qbuf.data_ptr(), sx.data_ptr(), rs.data_ptr(), sptr)
                   for x in Xs]
        if bits == 16:   # W4A16: the GEMM reads X itself
            mm_args = [(x.data_ptr(), xdt, M, K, 0, 16, p.data_ptr(), s.data_ptr(), gw, bptr, w4.W4_BF16, None, N,
                        Y.data_ptr(), w4.W4_OUT_BF16, wsg.data_ptr(), wsg.numel(), sptr) for x, (p, s, _) in zip(Xs, Ps)]
            f_mm = L.w4_linear_grouped
        else:
            mm_args = [(qbuf.data_ptr(), sx.data_ptr(), bits, p.data_ptr(), s.data_ptr(), gw, bptr, w4.W4_BF16, None,
                        M, N, K, Y.data_ptr(), w4.W4_OUT_BF16, wsc.data_ptr(), wsc.numel(), sptr) for p, s, _ in Ps]
            f_mm = L.w4_linear_cached_rot_grouped
        lin_args = [(x.data_ptr(), xdt, M, K, g, bits, p.data_ptr(), s.data_ptr(), gw, bptr, w4.W4_BF16, None, N,
                     Y.data_ptr(), w4.W4_OUT_BF16, wsg.data_ptr(), wsg.numel(), sptr) for x, (p, s, _) in zip(Xs, Ps)]
        f_lin = L.w4_linear_grouped
        fused = False
        kernel = "k_grp_stream" if M <= 16 and gw >= 64 and K % 1024 == 0 else "k_gemm_grp"
    else:
        lrp = None
        if getattr(args, "lowrank", 0):
            # the branch's t = x . L1 precomputed (untimed); the GEMM adds t . L2 in its epilogue
            gen = torch.Generator(device=dev).manual_seed(2011)
            R = args.lowrank
            t_lr = (torch.randn(M, R, generator=gen, device=dev) * 0.5).contiguous()
            l2_lr = (torch.randn(R, N, generator=gen, device=dev) * 0.01).to(torch.bfloat16).contiguous()
            lr_c = w4.LowRank(l2=l2_lr, t=t_lr).as_c()
            lr_keep = (t_lr, l2_lr, lr_c)
            lrp = ctypes.byref(lr_c)
        rq_args = [(x.data_ptr(), xdt, M, K, g, bits, qbuf.data_ptr(), sx.data_ptr(), rs.data_ptr(), sptr) for x in Xs]
        # the GEMM half with the workspace w4_linear gives it (K-split partials where planned),
        # so the per-launch time is that of the step's kernels
        wsm = torch.zeros((max(256, w4.w4_workspace_bytes(M, N, K, bits, 0)),), dtype=torch.uint8, device=dev)
        mm_args = [(qbuf.data_ptr(), sx.data_ptr(), rs.data_ptr(), bits, p.data_ptr(), s.data_ptr(),
                    z.data_ptr() if z is not None else None, bptr, w4.W4_BF16, lrp, M, N, K,
                    Y.data_ptr(), w4.W4_OUT_BF16, wsm.data_ptr(), wsm.numel(), sptr) for p, s, z in Ps]
        # the step: the whole layer through w4_linear (rotate + quantize into its workspace, then
        # the GEMM; one fused launch for a single token, see w4_linear_fused)
        wsl = torch.empty((max(256, w4.w4_linear_workspace_bytes(M, N, K, bits)),), dtype=torch.uint8, device=dev)
        lin_args = [(x.data_ptr(), xdt, M, K, g, bits, p.data_ptr(), s.data_ptr(),
                     z.data_ptr() if z is not None else None, bptr, w4.W4_BF16, lrp, N, Y.data_ptr(),
                     w4.W4_OUT_BF16, wsl.data_ptr(), wsl.numel(), sptr) for x, (p, s, z) in zip(Xs, Ps)]
        f_mm, f_lin = L.w4_linear_cached_rot, L.w4_linear
        fused = bool(L.w4_linear_fused(M, N, K, g, bits, xdt))
        kernel = "k_gemv_fused" if fused else ("k_gemv" if M <= 64 else "k_gemm")
    f_rq = L.w4_rotate_quant_act

    def step(i):
        rc = f_lin(*lin_args[i % ncopy])
        if rc:
            w4._check(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("bench: %s: %d copies of the inputs (%.0f MB), %d warmup steps done" % (
        name, ncopy, ncopy * per_copy / 1e6, args.warmup))

    # per-launch durations: each kernel launched K times back to back between two HIP events.
    # The K launches are captured once in a HIP graph and the replay is timed, so the events
    # see the kernels and the GPU's own launch gaps, not the host's per-call cost (a ctypes
    # call takes longer than a small-M kernel runs); --eager times plain launches instead.
    def per_launch(f, argl):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.eager:
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.steps):
                w4._check(f(*argl[i % ncopy]))
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps * 1e-3
        side = torch.cuda.Stream()
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk, stream=side):
            sk = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                w4._check(f(*(argl[i % ncopy][:-1] + (sk,))))
        gk.replay()
        torch.cuda.synchronize()
        # two replays back to back; the events bracket the second, which the host has
        # submitted while the first still runs, so they see K launches and not the graph's
        # submission latency
        gk.replay()
        e0.record(stream)
        gk.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e-3

    if fused:  # one kernel per step
        t_rq, t_mm = None, per_launch(f_lin, lin_args)
        log("bench: fused rotate+quant+GEMM %.2f us per launch" % (t_mm * 1e6))
    elif bits == 16:
        t_rq, t_mm = None, per_launch(f_mm, mm_args)
        log("bench: W4A16 GEMM %.2f us per launch" % (t_mm * 1e6))
    else:
        t_rq, t_mm = per_launch(f_rq, rq_args), per_launch(f_mm, mm_args)
        log("bench: rotate+quant %.2f us, GEMM %.2f us per launch" % (t_rq * 1e6, t_mm * 1e6))
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # the timed steps: one HIP graph holding the K steps' launches in order (step i on
        # input copy i % ncopy), captured once untimed and replayed once, so the GPU runs the
        # steps back to back without waiting for the host
        side = torch.cuda.Stream()
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph, stream=side):
            st2 = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                w4._check(f_lin(*(lin_args[i % ncopy][:-1] + (st2,))))
        gph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return {"lin": lin, "fused": fused, "t_rq": t_rq, "t_mm": t_mm, "wall": wall, "ncopy": ncopy, "kernel": kernel}


def summarize_trace(path, steps):
    """Per-kernel statistics of a rocprofv3 kernel trace (CSV), and for each kernel the mean
    duration over its longest run of back-to-back dispatches, last `steps` of them: the
    graph replay that bench.py times with HIP events for the roofline."""
    import csv
    if path.endswith(".db"):   # rocprofv3's default (rocpd SQLite) output
        import sqlite3
        q = sqlite3.connect(path).execute("select name, start, end from kernels")
        rows = [{"Kernel_Name": n, "Start_Timestamp": s, "End_Timestamp": e} for n, s, e in q]
    else:
        rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| kernel | calls | mean us | min us | max us |")
    print("|---|---|---|---|---|")
    for k, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print("| %s | %d | %.3f | %.3f | %.3f |" % (k[:90], len(d), sum(d) / len(d) / 1e3, min(d) / 1e3, max(d) / 1e3))
    # runs of consecutive dispatches of one kernel
    runs = []
    cur = None
    for r in rows:
        k = r["Kernel_Name"]
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if cur and cur[0] == k:
            cur[1].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        else:
            cur = [k, [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]))]]
            runs.append(cur)
        del dur
    print()
    print("| kernel | back-to-back launches (last of its longest run) | mean kernel us | mean start-to-start us |")
    print("|---|---|---|---|")
    best = {}
    for k, seq in runs:
        if len(seq) >= steps and len(seq) >= len(best.get(k, [])):
            best[k] = seq
    for k, seq in best.items():
        seq = seq[-steps:]
        mean = sum(e - s for s, e in seq) / len(seq) / 1e3
        span = (seq[-1][1] - seq[0][0]) / len(seq) / 1e3
        print("| %s | %d | %.3f | %.3f |" % (k[:90], len(seq), mean, span))


def measured_traffic(kernel, cfg):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    short = "k_gemv" if kernel.startswith("k_gemv") else kernel  # counters are kept per source file
    key = "%s:%s" % (short, traffic_workload(cfg["workload"], cfg.get("M"), cfg.get("K")))
    ent = data.get(key)
    if not ent:
        return None
    src = os.path.join(ROOT, "int4_weight_quantized_block_amd", "csrc", ent["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != ent["sha256"]:
        return None  # the kernel changed since the counters were taken
    return ent["bytes"]


def probe_library():
    """libw4probe.so: the measurement probes (include/w4_probe.h), built beside libw4.so."""
    path = os.path.join(ROOT, "int4_weight_quantized_block_amd", "libw4probe.so")
    if not os.path.exists(path):
        raise SystemExit("libw4probe.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    lib.w4_probe_mfma_rate.restype = ctypes.c_int
    lib.w4_probe_mfma_rate.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.w4_probe_read_rate.restype = ctypes.c_int
    lib.w4_probe_read_rate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p]
    return lib


def bench_hbm_peak(args, dev):
    """The HBM read rate a plain streaming kernel reaches on a buffer the size of one small-M
    linear's weights (K = 12288 -> N = 4096: 25.2 MB), cycling through copies larger than the
    256 MB Infinity Cache, for a few grid sizes: the practical ceiling the small-M kernels'
    HBM fractions should be read against.  Not a step of the layer."""
    import torch
    P = probe_library()
    nbytes = args.probe_mb * 1000 * 1000 // 16 * 16
    ncopy = max(2, math.ceil(2 * MALL_BYTES / nbytes))
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(ncopy)]
    st = torch.cuda.current_stream(dev)
    best = None
    rates = {}
    for blocks in (256, 512, 1024, 2048, 4096):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        for i in range(2):
            assert P.w4_probe_read_rate(bufs[i % ncopy].data_ptr(), nbytes, blocks, sink.data_ptr(), st.cuda_stream) == 0
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            s2 = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                assert P.w4_probe_read_rate(bufs[i % ncopy].data_ptr(), nbytes, blocks, sink.data_ptr(), s2) == 0
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / args.steps * 1e-3
        rates[blocks] = {"us": round(t * 1e6, 3), "gbs": round(nbytes / t / 1e9, 1)}
        log("bench: read %d MB with %d workgroups: %.2f us, %.0f GB/s" % (nbytes // 1000000, blocks, t * 1e6,
                                                                          nbytes / t / 1e9))
        if best is None or t < best[1]:
            best = (blocks, t)
    gbs = nbytes / best[1] / 1e9
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "kernel": "k_read_rate", "traffic": None, "launch_us": round(best[1] * 1e6, 3)}
    out = {
        "metric": "plain streaming read rate (probe)", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": 2, "ms_per_step": round(best[1] * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "hbm_peak", "bytes": nbytes, "copies": ncopy, "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": None, "detail": {"by_workgroups": rates, "best_workgroups": best[0]},
    }
    print(json.dumps(out), flush=True)


def bench_mfma_peak(args, dev):
    """The chip's sustained dense int8 MFMA rate: the library's probe (back-to-back
    v_mfma_i32_32x32x32_i8, eight waves per SIMD) with pseudo-random and with constant
    operands, K launches each between HIP events.  Not a step of the layer: it measures the
    ceiling the GEMM's roofline fraction should be read against."""
    import torch
    L = probe_library()
    blocks, iters = 256 * 8, 4000
    ops = blocks * 4.0 * iters * 4 * 2 * 32 ** 3
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)
    rate = {}
    for rnd in (0, 1):
        for _ in range(2):
            assert L.w4_probe_mfma_rate(blocks, iters, rnd, sink.data_ptr(), st.cuda_stream) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(args.steps):
            assert L.w4_probe_mfma_rate(blocks, iters, rnd, sink.data_ptr(), st.cuda_stream) == 0
        e1.record(st)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / args.steps * 1e-3
        rate[rnd] = ops / t / 1e12
        log("bench: probe %s operands: %.1f TOPS (%.3f ms per launch)" % ("random" if rnd else "constant", rate[rnd],
                                                                          t * 1e3))
    roof = {"bound": "mfma", "achieved": rate[1], "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
            "frac": rate[1] / PEAK_INT8_TOPS, "kernel": "k_mfma_rate", "traffic": None}
    out = {
        "metric": "sustained dense int8 MFMA rate (probe, random operands)", "value": round(rate[1], 1),
        "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": 2, "ms_per_step": round(ops / rate[1] / 1e9, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "mfma_peak", "blocks": blocks, "iters_per_wave": iters,
                   "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": None,
        "detail": {"constant_operands_tops": round(rate[0], 1), "random_operands_tops": round(rate[1], 1)},
    }
    print(json.dumps(out), flush=True)


def bench_double_block(args, dev):
    import torch
    import synth
    import int4_weight_quantized_block_amd as w4
    nb = synth.N_BLOCKS
    M = args.M or synth.DOUBLE_BLOCK_TOKENS
    blocks = []
    cpu_block = None  # block 0's inputs on the host, for the CPU oracle baseline
    for b in range(nb):
        blk = synth.double_block(b, dev, M=M)
        if b == 0 and not args.no_cpu_baseline:
            cpu_block = {"x": blk["x"].cpu(), "attn": blk["attn"].cpu()}
            for name, _, _ in synth.DOUBLE_BLOCK_LINEARS:
                cpu_block[name] = {key: blk[name][key].cpu() for key in ("W", "bias", "L1", "L2")}
        lins = {}
        for name, k, n in synth.DOUBLE_BLOCK_LINEARS:
            p = blk[name]
            packed, s_w, _ = w4.w4_pack_weights(p["W"], 256, False)
            lins[name] = (packed, s_w, p["bias"], p["L1"], p["L2"])
            del p["W"]
        # QKV and MLP-up read the block input: their L1 factors are stacked once (a load-time
        # step) so one pass gives both low-rank inputs along with the shared codes
        lins["x_l1"] = torch.cat([blk["qkv"]["L1"], blk["up"]["L1"]], dim=0).contiguous()
        blocks.append((blk["x"], blk["attn"], lins))
        log("bench: block %d packed" % b)
    torch.cuda.synchronize()
    K = synth.DIT_HIDDEN
    ops = sum(2.0 * M * k * n for _, k, n in synth.DOUBLE_BLOCK_LINEARS) * nb
    h = torch.empty((M, synth.DIT_MLP), dtype=torch.bfloat16, device=dev)
    outs = {name: torch.empty((M, n), dtype=torch.bfloat16, device=dev) for name, _, n in synth.DOUBLE_BLOCK_LINEARS}
    t_bufs = {name: torch.empty((M, synth.LOWRANK), dtype=torch.float32, device=dev)
              for name, _, _ in synth.DOUBLE_BLOCK_LINEARS}
    stream = torch.cuda.current_stream(dev)
    gemm_times = []

    r = synth.LOWRANK

    def timed(record, fn):
        e0 = torch.cuda.Event(enable_timing=True) if record else None
        if record:
            e0.record(stream)
        fn()
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            gemm_times.append((e0, e1))

    def lin_out(lins, name, t):
        packed, s_w, bias, L1, L2 = lins[name]
        return w4.LinearOut(packed=packed, row_scale=s_w, bias=bias, lowrank=w4.LowRank(l2=L2, t=t), out=outs[name])

    def step(record):
        for x, attn, lins in blocks:
            cache = w4.RotationCache()
            # QKV and MLP-up read the block input: one rotate-quant pass gives the codes and
            # x . L1 of both, and their GEMMs run as one launch
            q, sx, rs, tt = cache.get(x, 256, 8, l1=lins["x_l1"])
            pair = [lin_out(lins, "qkv", tt[:, :r]), lin_out(lins, "up", tt[:, r:2 * r])]
            timed(record, lambda: w4.w4_linear_cached_rot_multi(q, sx, rs, 8, pair))
            q, sx, rs, tt = cache.get(attn, 256, 8, l1=lins["out"][3])
            o = lin_out(lins, "out", tt)
            timed(record, lambda: w4.w4_linear_cached_rot(q, sx, rs, 8, o.packed, o.row_scale, bias=o.bias,
                                                          lowrank=o.lowrank, out=o.out))
            torch.nn.functional.gelu(outs["up"], out=h)  # host glue between the MLP linears
            packed, s_w, bias, L1, L2 = lins["down"]
            q, sx, rs, t = w4.w4_rotate_quant_act_lowrank(h, 256, 8, L1)
            w4.w4_linear_cached_rot(q, sx, rs, 8, packed, s_w, bias=bias, lowrank=w4.LowRank(l2=L2, t=t),
                                    out=outs["down"])
            cache.clear()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # GEMM launch durations: one eager pass with events around each GEMM launch
    step(True)
    torch.cuda.synchronize()
    if args.eager:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(False)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # the timed steps: one step (all launches of the 20 blocks, host GELU included)
        # captured as a HIP graph once, untimed, and replayed K times back to back
        side = torch.cuda.Stream()
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph, stream=side):
            step(False)
        gph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            gph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3
    value = ops / (wall / args.steps) / 1e12
    g_ops = 2.0 * M * K * (synth.DIT_QKV + synth.DIT_MLP + synth.DIT_HIDDEN)
    t_g = sum(a.elapsed_time(b) for a, b in gemm_times) * 1e-3 / nb
    roof = {"bound": "mfma", "achieved": g_ops / t_g / 1e12, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "k_gemm"
    roof["traffic"] = None  # four GEMM shapes per block: no single per-launch figure
    if args.copy_calibration:
        copy_calibration(dev)
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "double_block", "blocks": nb, "M": M, "g": 256, "act_bits": 8,
                   "lowrank": synth.LOWRANK, "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": None,
    }
    if cpu_block is not None:
        rows = args.cpu_rows or 3072
        log("bench: timing the CPU oracle on block 0, %d rows" % rows)
        out["cpu_baseline"] = cpu_baseline_block(cpu_block, rows, M, nb)
    print(json.dumps(out), flush=True)


def cpu_baseline_block(blk, rows, M, nb):
    """The oracle as it stands on this host's cores over the first ``rows`` token rows of
    block 0: the same step as the GPU's (rotation shared by QKV and MLP-up, low-rank branch
    on every linear, host GELU between the MLP linears); rows are independent, so the rate
    extrapolates to the whole workload.  Weight packing is done before timing."""
    import oracle
    import synth
    pw = {name: oracle.pack_weights(blk[name]["W"], 256, False) for name, _, _ in synth.DOUBLE_BLOCK_LINEARS}
    x, attn = blk["x"][:rows], blk["attn"][:rows]

    def lin(name, inp, qa):
        p = blk[name]
        lr = oracle.lowrank(inp, p["L1"].t(), p["L2"])  # L1 is held rank-major, [r, K]
        return oracle.linear_from_codes(qa["q"], qa["scale"], pw[name]["packed"], pw[name]["scale"], None, False,
                                        p["bias"], lr)

    t1 = time.perf_counter()
    qx = oracle.rotate_quant_act(x, 256, 8)  # shared by QKV and MLP-up
    lin("qkv", x, qx)
    up = lin("up", x, qx)
    lin("out", attn, oracle.rotate_quant_act(attn, 256, 8))
    h = oracle.gelu_bf16(up["y"])
    lin("down", h, oracle.rotate_quant_act(h, 256, 8))
    sec = time.perf_counter() - t1
    ops = sum(2.0 * rows * k * n for _, k, n in synth.DOUBLE_BLOCK_LINEARS)
    return {"cores": oracle.num_threads(), "kind": "oracle",
            "sample": "block 0 of %d: %d of %d token rows, all four linears with the rotation cache, low-rank "
                      "branches and GELU (rate extrapolates: rows and blocks are independent)" % (nb, rows, M),
            "seconds": round(sec, 3), "value": round(ops / sec / 1e12, 6), "unit": "TOPS"}


if __name__ == "__main__":
    main()
