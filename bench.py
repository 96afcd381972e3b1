#!/usr/bin/env python3
"""Benchmark of the quantized recurrent-state update on one MI355X.

Default workload (the headline): one decode token of a Mamba-2 370m-shaped
stack -- 48 layers x 32 heads x 64 x 128, batch 256, int4 asymmetric state
with a per-row fp32 scale and zero point, from a seeded random state
(N(0,1) rows, 5% of rows x20).  A "step" is one token through all 48
layers: 48 ssq_decode_step launches, captured once in a hipGraph and
replayed.  Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line: state-update throughput (GB/s of algorithmic bytes:
every state byte read and written once, plus x, y, dt, B, C), its fraction
of the 8 TB/s HBM peak, decode steps/s, the roofline of the dominant kernel
(per-launch duration from HIP events on the launch stream) and the CPU
oracle timed on a bounded sample on the host.

Other workloads (--workload) cover the remaining benchmark shapes; they
print the same schema.
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

METRIC = "state-update GB/s + % of HBM peak; decode steps/s at batch 256"
HBM_PEAK_GBPS = 8000.0
# wall time of the workload's kernel on a scratch state before the warm-up steps, to bring the
# device to steady clocks
DEVICE_WARMUP_MS = 150.0
# VALU roofline of the on-chip paths, in lane-operations/s: the fp32 vector peak (157.3 TFLOP/s,
# an fma counted as two flops) is 78.6 T fp32 operations per second (256 CUs x 4 SIMDs x 32
# lanes x 2.4 GHz).  The kernels are built without packed fp32: a wave64 fp32 add, multiply or
# fma issues in 2.5-2.7 cycles per SIMD (about 60 T lane-ops/s over the part), conversions,
# min3/max3, perm, DPP forms and fp64 in 4.3-4.8 (about 35 T/s), measured.
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
VALU_PEAK_TOPS = SIMDS * 32 * CLOCK_HZ / 1e12
# What holds each kernel, from the profiles: every step kernel but the int8 one takes the same
# time with its state cache-resident (--shared-state) and issues VALU instructions for most of
# its launch; the int8 decode runs at about 90% of the streaming copy; the scans and the
# prefill keep the state on-chip for all their tokens.
LIMITED_BY = {
    "valu_issue": "the launch takes the same time with the state cache-resident (--shared-state), and its "
                  "VALU instructions at their measured issue costs fill most of it (roofline.valu)",
    "hbm": "about 90% of the streaming copy's bandwidth in the same run (frac_of_copy)",
    "valu_issue_on_chip": "the state stays on-chip for all T tokens: VALU issue",
}

WORKLOADS = {
    # name: kind, layers, batch, heads, rows_per_head, format, init, tokens (scan), instances
    "m2_370m_int4": dict(kind="m2", layers=48, B=256, H=32, P=64, fmt="int4_asym", init="random",
                         desc="Mamba-2 370m-shaped decode step: 48 layers x 32 heads x 64 x 128, batch 256, "
                              "int4 asymmetric state (per-row fp32 scale + zero point), seeded random state "
                              "with 5% x20 outlier rows"),
    "m2_370m_int4_sr": dict(kind="m2", layers=48, B=256, H=32, P=64, fmt="int4_asym", init="random",
                            rounding="stochastic",
                            desc="as m2_370m_int4 with stochastic rounding of the codes (SplitMix64 "
                                 "uniforms per entry); each graph replay draws the next token"),
    "delta_int8": dict(kind="delta", layers=30, B=256, H=32, P=128, fmt="int8_asym", init="random",
                       desc="Delta-rule (GDN/KDA-style) decode step: 30 layers x 32 heads x 128 x 128, batch 256, "
                            "int8 asymmetric per-row state, seeded random state with 5% x20 outlier rows"),
    "damp_int8": dict(kind="delta", layers=30, B=256, H=32, P=128, fmt="damp", init="random",
                      desc="Two-tier delta-rule decode step: 30 layers x 32 heads x 128 x 128, batch 256, key "
                           "rows 0..15 in half precision and 16..127 as uint8 with scale and zero point, rows "
                           "rotated by a 128-point Hadamard transform; seeded random state with 5% x20 outlier rows"),
    "kda_int8": dict(kind="kda", layers=30, B=256, H=32, P=128, fmt="int8_asym", init="random",
                     desc="KDA-style decode step (a decay per key channel): 30 layers x 32 heads x 128 x 128, "
                          "batch 256, int8 asymmetric per-row state, seeded random state with 5% x20 outlier rows"),
    "m2_8b_int8sym": dict(kind="m2", layers=8, B=256, H=128, P=64, fmt="int8_sym", init="zero", rotate=True,
                          desc="Mamba-2 8B-shaped decode layer: 128 heads x 64 x 128, batch 256, int8 symmetric; "
                               "8 state instances in rotation so that the state is not cache resident"),
    "m2_8b_int4": dict(kind="m2", layers=8, B=256, H=128, P=64, fmt="int4_asym", init="zero", rotate=True,
                       desc="Mamba-2 8B-shaped decode layer: 128 heads x 64 x 128, batch 256, int4 asymmetric; "
                            "8 state instances in rotation so that the state is not cache resident"),
    "m2_130m_scan_int8asym": dict(kind="scan", layers=24, B=32, H=24, P=64, fmt="int8_asym", init="zero", T=2048,
                                  desc="Mamba-2 130m-shaped stack: 24 layers x 24 heads x 64 x 128, batch 32, "
                                       "2048-token scan per layer, int8 asymmetric state rounded every token"),
    "m2_130m_scan_int8sym": dict(kind="scan", layers=24, B=32, H=24, P=64, fmt="int8_sym", init="zero", T=2048,
                                 desc="as m2_130m_scan_int8asym with the int8 symmetric grid"),
    "m2_130m_scan_fp32": dict(kind="scan", layers=24, B=32, H=24, P=64, fmt="fp32", init="zero", T=2048,
                              desc="as m2_130m_scan_int8asym with the fp32 control state"),
    "m2_130m_prefill_int8asym": dict(kind="prefill", layers=24, B=32, H=24, P=64, fmt="int8_asym", init="zero",
                                     T=2048, chunk=64,
                                     desc="Mamba-2 130m-shaped stack: 24 layers x 24 heads x 64 x 128, batch 32, "
                                          "2048-token prompt per layer, fp32 recurrence inside chunks of 64 tokens, "
                                          "int8 asymmetric state written at each chunk end"),
    "m2_8b_scan_int8sym": dict(kind="scan", layers=1, B=8, H=128, P=64, fmt="int8_sym", init="zero", T=8192,
                               desc="Mamba-2 8B-shaped layer: batch 8, 8192-token scan, int8 symmetric, state "
                                    "rounded every token"),
    "m2_8b_scan_int4": dict(kind="scan", layers=1, B=8, H=128, P=64, fmt="int4_asym", init="zero", T=8192,
                            desc="Mamba-2 8B-shaped layer: batch 8, 8192-token scan, int4 asymmetric"),
}

# The pages' own figures for this path, with the hardware they were taken on (context; none of
# them is a state-update GB/s, steps/s or fraction of HBM for this workload)
PAGES_CONTEXT = [
    {"figure": "24.3% of decode latency spent on recurrent-state updates; about 15 GB of FP32 "
               "recurrent state at decode batch 256 (30 Gated DeltaNet layers)",
     "hardware": "not stated in the excerpt",
     "source": "Mamba state quantization for inference, Recurrent state is fixed per request, not free"},
    {"figure": "DAMP's fused mixed FP16/INT8 recurrent-update kernel 1.46-1.65x (GDN) and 1.81-2.01x "
               "(KDA) faster than FP32 from batch 32 to 256",
     "hardware": "not stated in the excerpt",
     "source": "Mamba state quantization for inference, Mixed precision spends bits on persistent channels"},
    {"figure": "sequential per-token scan with the state rounded every step (fp32 Mamba-2 130M/370M); "
               "no speed published",
     "hardware": "one RTX 3070 (8 GB)",
     "source": "ssm-state-quantization README, Setup"},
    {"figure": "Quamba2 whole-model time per output token 22.73 ms (FP16) to 12.61 ms (W8A8), "
               "Mamba2-8B at batch 1 (weight and activation quantization, not the state path)",
     "hardware": "A5000",
     "source": "Quamba2 summary"},
]

KERNEL_NAMES = {"m2": "k_m2_step", "delta": "k_delta_step", "kda": "k_delta_step", "scan": "k_m2_scan",
                "prefill": "k_m2_prefill"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default depends on the workload)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--device-warmup-ms", type=float, default=DEVICE_WARMUP_MS,
                    help="wall time of the workload's kernel on a scratch state before the warm-up steps")
    ap.add_argument("--workload", default="m2_370m_int4", choices=sorted(WORKLOADS))
    ap.add_argument("--eager", action="store_true", help="time back-to-back launches instead of graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--shared-state", action="store_true",
                    help="diagnostic: every launch updates one state instance, which then stays in the "
                         "last-level cache when it fits (separates the kernel's own time from HBM)")
    ap.add_argument("--layers", type=int, default=None,
                    help="fewer layers than the workload names (quick checks only; recorded in config)")
    ap.add_argument("--batch", type=int, default=None,
                    help="another batch size than the workload names (a sweep over batch; recorded in config)")
    return ap.parse_args()


KERNEL_SOURCES = {"m2": "ssq_mamba2.hip", "scan": "ssq_mamba2.hip", "prefill": "ssq_mamba2.hip",
                  "delta": "ssq_delta.hip", "kda": "ssq_delta.hip"}


def _code_only(text: str) -> str:
    """C++ source without its comments and whitespace: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def src_hash(kind: str) -> str:
    """Hash of the code a workload's kernel is built from, comments and whitespace left out
    (the committed traffic figures hold only while it is unchanged)."""
    h = hashlib.sha256()
    for name in ("ssq_device.h", "ssq_internal.h", KERNEL_SOURCES[kind]):
        h.update(_code_only(open(os.path.join(ROOT, "mamba_decode_amd", "csrc", name)).read()).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the state update needs no inter-GPU exchange and every "
              f"box here has one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mamba_decode_amd as ssq
    import synth

    wl = dict(WORKLOADS[args.workload])
    if args.layers is not None:
        if args.layers < 1:
            raise SystemExit("--layers must be positive")
        wl["layers"] = args.layers
    if args.batch is not None:
        if args.batch < 1:
            raise SystemExit("--batch must be positive")
        wl["B"] = args.batch
    kind = wl["kind"]
    seq = kind in ("scan", "prefill")  # T tokens per launch, the state on-chip
    steps = args.steps if args.steps is not None else (3 if seq else 100)
    warmup = args.warmup if args.warmup is not None else (1 if seq else 10)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    L, B, H, P, fmt = wl["layers"], wl["B"], wl["H"], wl["P"], wl["fmt"]
    N = 128
    T = wl.get("T", 1)
    rows = B * H * P
    fmt_id = ssq.FORMAT_NAMES[fmt]
    skind = ssq.SSQ_DELTA if kind in ("delta", "kda") else ssq.SSQ_MAMBA2
    desc = ssq.make_desc(skind, fmt, B, H, P, N)
    lay = ssq.ssq_state_layout(desc)
    meta = 0 if fmt == "fp32" else (8 if fmt.endswith("asym") else 4)
    state_bytes_layer = 2 * rows * (lay.row_bytes + meta)  # read once + written once
    if fmt == "damp":  # 112 uint8 rows (128 B + scale + zero) and 16 half rows (256 B) per matrix
        mats = rows // P
        state_bytes_layer = 2 * mats * ((P - ssq.SSQ_DAMP_NHI) * (128 + 8) + ssq.SSQ_DAMP_NHI * 256)
    log(f"[bench] workload {args.workload}: {L} layer(s), {rows} rows/layer, {fmt}, "
        f"{lay.total_bytes / 2**20:.1f} MiB state/layer")

    # ---------------- states (seeded random or zero), resident in HBM ----------------
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    states, storages = [], []
    for layer in range(1 if args.shared_state else L):
        storage = torch.empty(lay.total_bytes, dtype=torch.uint8, device=dev)
        if wl["init"] == "random":
            h = torch.randn(rows, N, generator=gen, device=dev)
            out = torch.rand(rows, 1, generator=gen, device=dev) < 0.05
            h = torch.where(out, h * 20.0, h).contiguous()
            st = ssq.ssq_alloc_state(desc, storage=storage, init=h)
            torch.cuda.synchronize()
            del h, out
        else:
            st = ssq.ssq_alloc_state(desc, storage=storage)
        if wl.get("rounding") == "stochastic":
            ssq.ssq_set_rounding(st, ssq.SSQ_ROUND_STOCHASTIC, args.seed * 1000 + layer, 0)
        states.append(st)
        storages.append(storage)
    if args.shared_state:
        states = states * L
    torch.cuda.synchronize()

    # ---------------- inputs (synth, seeded), resident in HBM ----------------
    import ctypes
    vp = ctypes.c_void_p
    ins, calls = [], []
    if kind == "m2":
        for layer in range(L):
            x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(args.seed, layer, B, H, 1, P, N)
            t = [torch.from_numpy(a).to(dev) for a in (x, dt, A, Bm, Cm, D)]
            y = torch.empty(rows, device=dev)
            ins.append((t, y))
        io_bytes = 4 * (rows * 2 + B * H + 2 * B * N + 2 * H)

        def launch(layer, stream, st=None):
            (x, dt, A, Bm, Cm, D), y = ins[layer]
            return ssq.lib.ssq_decode_step((st or states[layer]).handle, vp(x.data_ptr()), vp(dt.data_ptr()),
                                           vp(A.data_ptr()), vp(Bm.data_ptr()), vp(Cm.data_ptr()),
                                           vp(D.data_ptr()), vp(y.data_ptr()), 0, stream)
    elif kind in ("delta", "kda"):
        for layer in range(L):
            q, k, v, al, be = synth.delta_inputs(args.seed, layer, B, H, P, N)
            if kind == "kda":
                al = synth.kda_alpha(args.seed, layer, B, H, P)
            t = [torch.from_numpy(a).to(dev) for a in (q, k, v, al, be)]
            o = torch.empty(B * H * N, device=dev)
            ins.append((t, o))
        io_bytes = 4 * (B * H * (2 * P + 2 * N) + 2 * B * H) + (4 * B * H * (P - 1) if kind == "kda" else 0)
        step_fn = ssq.lib.ssq_kda_step if kind == "kda" else ssq.lib.ssq_delta_step

        def launch(layer, stream, st=None):
            (q, k, v, al, be), o = ins[layer]
            return step_fn((st or states[layer]).handle, vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
                           vp(al.data_ptr()), vp(be.data_ptr()), vp(o.data_ptr()), 0, stream)
    else:  # scan / prefill: one layer's inputs drawn on the device, shared by every layer
        g2 = torch.Generator(device=dev)
        g2.manual_seed(args.seed + 1)
        A_np, D_np, bias = synth.mamba2_head_params(args.seed, 0, H)
        x = torch.randn(B, T, H, P, generator=g2, device=dev)
        dtn = torch.randn(B, T, H, generator=g2, device=dev, dtype=torch.float64)
        dt = torch.nn.functional.softplus(dtn + torch.from_numpy(bias).to(dev)).float().contiguous()
        Bm = (torch.randn(B, T, 1, N, generator=g2, device=dev) / N ** 0.5).contiguous()
        Cm = (torch.randn(B, T, 1, N, generator=g2, device=dev) / N ** 0.5).contiguous()
        A = torch.from_numpy(A_np).to(dev)
        D = torch.from_numpy(D_np).to(dev)
        y = torch.empty_like(x)
        ins.append(((x, dt, A, Bm, Cm, D), y))
        io_bytes = 4 * (2 * rows * T + B * T * H + 2 * B * T * N + 2 * H)

        def launch(layer, stream, st=None):
            (x, dt, A, Bm, Cm, D), y = ins[0]
            ptrs = [vp(t.data_ptr()) for t in (x, dt, A, Bm, Cm, D, y)]
            if kind == "prefill":
                return ssq.lib.ssq_prefill((st or states[layer]).handle, T, wl["chunk"], *ptrs, 0, stream)
            return ssq.lib.ssq_scan((st or states[layer]).handle, T, *ptrs, 0, stream)
    torch.cuda.synchronize()
    bytes_per_launch = (state_bytes_layer if not seq else 0) + io_bytes

    def run_step():
        s = vp(torch.cuda.current_stream().cuda_stream)
        for layer in range(L):
            rc = launch(layer, s)
            if rc != 0:
                raise RuntimeError(f"launch failed: {ssq.ssq_last_error()}")

    # ---------------- graph capture of one step ----------------
    use_graph = not args.eager and not seq
    graph = None
    if use_graph:
        run_step()  # warm the launch path before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step()
        torch.cuda.synchronize()

    def do_step():
        if graph is not None:
            graph.replay()
        else:
            run_step()

    # ---------------- copy bandwidth in the same run (context) ----------------
    # the library's streaming copy over 2 GiB (4 GiB of traffic), and the runtime's copy
    nbytes = 1 << 31
    src = torch.empty(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    ssq.ssq_stream_copy(dst, src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        ssq.ssq_stream_copy(dst, src)
    c1.record()
    c1.synchronize()
    copy_gbps = 2 * nbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    n1 = (1 << 30) // 4  # the runtime's copy of 1 GiB (the traffic passes are calibrated on it)
    dst[:n1].copy_(src[:n1])
    torch.cuda.synchronize()
    c0.record()
    for _ in range(5):
        dst[:n1].copy_(src[:n1])
    c1.record()
    c1.synchronize()
    runtime_copy_gbps = 2 * (1 << 30) * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    # ---------------- device warm-up on a scratch state (not a step) ----------------
    # A few steps are too short for the part to reach its steady clocks (the first blocks of a
    # short run were 5-8% slower than the last), so the workload's own kernel first runs for
    # about DEVICE_WARMUP_MS on one extra state of the same shape with layer 0's inputs; the
    # states the steps update are untouched until the warm-up steps.
    warm_storage = torch.empty(lay.total_bytes, dtype=torch.uint8, device=dev)
    warm_state = ssq.ssq_alloc_state(desc, storage=warm_storage)
    if wl.get("rounding") == "stochastic":
        ssq.ssq_set_rounding(warm_state, ssq.SSQ_ROUND_STOCHASTIC, args.seed * 1000 + 999, 0)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    warm_launches = 0
    ws = vp(torch.cuda.current_stream().cuda_stream)
    while (time.perf_counter() - t_warm) * 1e3 < args.device_warmup_ms:
        for _ in range(8):
            if launch(0, ws, warm_state) != 0:
                raise RuntimeError(f"launch failed: {ssq.ssq_last_error()}")
        torch.cuda.synchronize()
        warm_launches += 8
    device_warmup_ms = (time.perf_counter() - t_warm) * 1e3
    warm_state.free()
    del warm_state, warm_storage

    log(f"[bench] warmup {warmup} step(s)")
    for _ in range(warmup):
        do_step()
    torch.cuda.synchronize()

    # ---------------- timed region: `steps` steps in 5 consecutive blocks ----------------
    # Events on the launch stream mark the blocks; the step time is the median over the
    # blocks of their mean step time (the mean over all steps is reported beside it).
    log(f"[bench] timing {steps} step(s)")
    nblk = min(5, steps)
    bounds = [round(i * steps / nblk) for i in range(nblk + 1)]
    evs_blk = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
    torch.cuda.synchronize()
    evs_blk[0].record()
    for b in range(nblk):
        for _ in range(bounds[b], bounds[b + 1]):
            do_step()
        evs_blk[b + 1].record()
    evs_blk[-1].synchronize()
    torch.cuda.synchronize()
    block_ms = [evs_blk[b].elapsed_time(evs_blk[b + 1]) / (bounds[b + 1] - bounds[b]) for b in range(nblk)]
    ms_per_step = float(np.median(block_ms))
    ms_per_step_mean = evs_blk[0].elapsed_time(evs_blk[-1]) / steps

    # ---------------- eager per-launch time (events around each launch, same stream): context ----------------
    kreps = max(1, min(steps, 20 if not seq else 2))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(kreps * L)]
    s = vp(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    i = 0
    for _ in range(kreps):
        for layer in range(L):
            evs[i][0].record()
            launch(layer, s)
            evs[i][1].record()
            i += 1
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in evs]
    eager_ms_median = float(np.median(kms))
    # every launch of a step runs the dominant kernel, so its average duration over the
    # timed region is the step time over the launches per step (gaps between launches
    # included, which makes the figure conservative)
    kernel_ms_mean = ms_per_step / L

    # ---------------- eager back-to-back steps (no events between launches): context ----------------
    if not seq:
        s = vp(torch.cuda.current_stream().cuda_stream)
        run_step()
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(kreps):
            run_step()
        b1.record()
        b1.synchronize()
        eager_ms_per_step = b0.elapsed_time(b1) / kreps
    else:
        eager_ms_per_step = None

    total_bytes_step = bytes_per_launch * L
    total_gbps = total_bytes_step / (ms_per_step * 1e-3) / 1e9
    state_gbps = state_bytes_layer * L / (ms_per_step * 1e-3) / 1e9 if not seq else None
    # the headline: state-update GB/s (the state read and written once per step); the scans keep
    # the state on-chip, so theirs is the GB/s of the per-token inputs and outputs
    value = state_gbps if not seq else total_gbps
    achieved = bytes_per_launch / (kernel_ms_mean * 1e-3) / 1e9

    # traffic and VALU instruction counts from the committed rocprofv3 counter runs, only while
    # the kernels are unchanged
    traffic = None
    valu = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        tr = json.load(open(tpath)).get(args.workload)
        if tr and tr.get("src_hash") == src_hash(kind) and args.batch is None and not args.shared_state:
            traffic = tr.get("hbm_bytes_per_launch")
            if tr.get("valu_insts_per_launch"):
                # wave64 VALU instructions issued per SIMD and cycle of this run's launch time: at
                # 2.1-4.5 cycles per instruction (by kind), 0.25 or more means the instruction
                # stream occupies most of the launch
                per_cycle = tr["valu_insts_per_launch"] / (SIMDS * kernel_ms_mean * 1e-3 * CLOCK_HZ)
                valu = {"insts_per_launch": tr["valu_insts_per_launch"],
                        "insts_per_wave": tr.get("valu_insts_per_wave"),
                        "insts_per_simd_cycle": round(per_cycle, 4),
                        "source": tr.get("summary")}

    limited = ("valu_issue_on_chip" if seq else ("hbm" if fmt.startswith("int8") and kind == "m2" else "valu_issue"))
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "timing": {"blocks": nblk, "block_ms_per_step": [round(b, 5) for b in block_ms],
                   "statistic": "median over the blocks of their mean step time",
                   "ms_per_step_mean_all_steps": round(ms_per_step_mean, 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl["desc"],
            "name": args.workload,
            "layers": L, "batch": B, "heads": H, "rows_per_head": P, "row_len": N, "format": fmt,
            "tokens": T if seq else 1,
            "launch": ("hipGraph replay of " if graph is not None else "back-to-back launches of ")
                      + f"{L} per-layer kernels per step",
            "parallelism": "single GPU",
            "state_instances": 1 if args.shared_state else L,
            **({"layers_reduced_from": WORKLOADS[args.workload]["layers"]} if args.layers is not None else {}),
            **({"batch_changed_from": WORKLOADS[args.workload]["B"]} if args.batch is not None else {}),
        },
        "value_kind": "state GB/s (state bytes read and written once per step)" if not seq
                      else "GB/s of the per-token inputs and outputs (the state stays on-chip)",
        "total_GBps": round(total_gbps, 2),
        "hbm_frac": round(total_gbps / HBM_PEAK_GBPS, 4),
        # a rotated workload times one layer on several state instances: each launch is one token
        "decode_steps_per_s": (round(1000.0 * (L if wl.get("rotate") else 1) / ms_per_step, 2)
                               if not seq else None),
        "tokens_per_s": round(B * T / (ms_per_step * 1e-3 / L), 1) if seq else None,
        "state_GBps": round(state_gbps, 2) if state_gbps else None,
        "decode_steps_per_s_eager": (round(1000.0 * (L if wl.get("rotate") else 1) / eager_ms_per_step, 2)
                                     if eager_ms_per_step else None),
        "copy_GBps": round(copy_gbps, 1),
        "copy_kind": "ssq_stream_copy, 2 GiB (4 GiB of traffic), same run",
        "device_warmup": {"kind": "the workload's kernel on a scratch state of the same shape, before the "
                                  "warm-up steps (not steps)",
                          "ms": round(device_warmup_ms, 1), "launches": warm_launches},
        "frac_of_copy": round(total_gbps / copy_gbps, 4),
        "runtime_copy_GBps": round(runtime_copy_gbps, 1),
        "roofline": {
            "bound": "hbm" if not seq else "alu",
            "kernel": KERNEL_NAMES[kind] + f"<{fmt}>",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": bytes_per_launch,
            "kernel_ms_mean": round(kernel_ms_mean, 5),
            "kernel_ms_source": "HIP events around the timed region, step time / launches per step",
            "eager_launch_ms_median": round(eager_ms_median, 5),
            "valu": valu,
            "limited_by": limited,
            "limited_by_evidence": LIMITED_BY[limited],
        },
        "device": torch.cuda.get_device_name(0),
        "pages_context": PAGES_CONTEXT,
    }
    if seq:
        # the state stays on-chip for all T tokens: the scan is bound by VALU issue.  Algorithmic
        # work per entry-step, in VALU lane-instructions, of the reconstruct-then-recur step: the
        # reconstruction s*(c - z) (the scan carries c - z from token to token), the write term
        # w*B and the fma of the update, the row's extremes (min3 and max3 each take two new
        # entries: one per entry; the symmetric grid's |.| max3: one half), the rounding fma,
        # and c' - z' plus one fma for the readout of the new codes; fp32: w*B, the fma and the
        # readout fma.  The prefill runs the fp32 step (3) and, once per chunk, the extremes,
        # the rounding and the reconstruction (c - z, times s): 4 more per chunk
        ops = 3 if fmt == "fp32" else (7 if fmt.endswith("asym") else 6.5)
        if kind == "prefill":
            ops = 3 + 4.0 / wl["chunk"]
        achieved_ops = rows * N * T * ops / (kernel_ms_mean * 1e-3) / 1e12
        rec["roofline"].update({
            "bound": "alu", "achieved": round(achieved_ops, 3), "peak": VALU_PEAK_TOPS,
            "unit": "T lane-ops/s", "frac": round(achieved_ops / VALU_PEAK_TOPS, 4),
            "ops_per_entry_step": ops, "io_GBps": round(achieved, 2),
        })

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args, wl, bytes_per_launch, rows)
    print(json.dumps(rec), flush=True)


def cpu_baseline(args, wl, bytes_per_launch, rows_per_layer):
    """The oracle as it stands on the host: K workers (the process's CPU affinity, at most 16),
    each single-threaded on a disjoint slice of sequences, over the workload's rows (bounded for
    the long scans); and one worker on a fixed slice for a bounded time."""
    import oracle

    k_leg = _cpu_kcore(args, wl, bytes_per_launch, rows_per_layer)
    single = _cpu_single(args, wl, bytes_per_launch, rows_per_layer)
    out = {"value": k_leg["GBps"], "unit": "GB/s", "cores": k_leg["cores"], "kind": "oracle",
           "sample": k_leg["sample"], "wall_s": k_leg["wall_s"], "cpu": _cpu_model(),
           "affinity_cpus": len(os.sched_getaffinity(0)), "workers_cap": 16}
    for key in ("decode_steps_per_s", "tokens_per_s"):
        if key in k_leg:
            out[key] = k_leg[key]
    out["single_core"] = single
    assert k_leg["cores"] == oracle.workers()
    return out


def _cpu_kcore(args, wl, bytes_per_launch, rows_per_layer):
    import numpy as np

    import oracle
    import synth

    K = oracle.workers()
    kind, fmt, B, H, P, N = wl["kind"], wl["fmt"], wl["B"], wl["H"], wl["P"], 128
    T = wl.get("T", 1)
    layers = 1 if wl.get("rotate") else wl["layers"]
    wall = 0.0

    def timed(fn, *a, **kw):
        nonlocal wall
        t0 = time.perf_counter()
        r = fn(*a, **kw)
        wall += time.perf_counter() - t0
        return r

    out = {"cores": K}
    if kind == "m2":
        # one step through every layer of the workload (each layer's own inputs), all rows; the
        # layers start from copies of one drawn state
        rows = B * H * P
        base = (oracle.make_state(fmt, rows, N, synth.init_state(args.seed, 0, rows, N, threads=K))
                if wl["init"] == "random" else oracle.make_state(fmt, rows, N))
        sr = wl.get("rounding") == "stochastic"
        for layer in range(layers):
            st = base.copy()
            x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(args.seed, layer, B, H, 1, P, N)
            timed(oracle.mamba2_step_par, st, x, dt, A, Bm, Cm, D, k=K,
                  sr=(args.seed * 1000 + layer, 0) if sr else None)
            del st
        done_bytes = bytes_per_launch * layers
        out["decode_steps_per_s"] = round(1.0 / wall, 5)
        out["sample"] = (f"one decode step of the whole workload: {layers} layer(s) x {rows} rows ({fmt}), "
                         f"each layer from a copy of one drawn state")
    elif kind in ("delta", "kda"):
        rows = B * H * P
        init = synth.init_state(args.seed, 0, rows, N, threads=K)
        if fmt == "damp":
            base = oracle.damp_from_fp32_par(init.reshape(B, H, P, N), B, H, k=K)
        else:
            base = oracle.make_state(fmt, rows, N, init)
        del init
        for layer in range(layers):
            st = base.copy()
            q, k, v, al, be = synth.delta_inputs(args.seed, layer, B, H, P, N)
            if kind == "kda":
                al = synth.kda_alpha(args.seed, layer, B, H, P)
                timed(oracle.kda_step_par, st, q, k, v, al, be, B, H, k=K)
            elif fmt == "damp":
                timed(oracle.damp_step_par, st, q, k, v, al, be, B, H, k=K)
            else:
                timed(oracle.delta_step_par, st, q, k, v, al, be, B, H, k=K)
            del st
        done_bytes = bytes_per_launch * layers
        out["decode_steps_per_s"] = round(1.0 / wall, 5)
        out["sample"] = (f"one step of the whole workload: {layers} layer(s) x {B * H} matrices ({fmt}), "
                         f"each layer from a copy of one drawn state")
    elif kind in ("scan", "prefill") and H * P * B * T <= (1 << 27):
        # one layer, the first min(B, K) sequences, every token
        nb = min(B, K)
        x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(args.seed, 0, nb, T, H, 1, P, N, threads=K)
        st = oracle.make_state(fmt, nb * H * P, N)
        if kind == "prefill":
            timed(oracle.mamba2_prefill_par, st, x, dt, A, Bm, Cm, D, chunk=wl["chunk"], k=K)
        else:
            timed(oracle.mamba2_scan_par, st, x, dt, A, Bm, Cm, D, k=K)
        done_bytes = bytes_per_launch * nb / B
        out["tokens_per_s"] = round(nb * T / wall, 1)
        out["sample"] = f"{nb} of {B} sequences of one layer ({nb * H * P} rows, {fmt}), all {T} tokens"
    else:
        # long scans: four rows of every (sequence, head), every token (rows are independent: the
        # oracle scans every sequence and head with those four rows' x)
        psel = np.linspace(0, P - 1, 4).astype(int)
        x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(args.seed, 0, B, T, H, 1, P, N, threads=K)
        xs = np.ascontiguousarray(x[:, :, :, psel])
        del x
        st = oracle.make_state(fmt, B * H * len(psel), N)
        timed(oracle.mamba2_scan_par, st, xs, dt, A, Bm, Cm, D, k=K)
        done_bytes = bytes_per_launch * len(psel) / P
        out["tokens_per_s"] = round(B * T / wall * len(psel) / P, 1)
        out["sample"] = (f"{B * H * len(psel)} rows of one layer (four in every (sequence, head), {fmt}), "
                         f"all {T} tokens")
    out["wall_s"] = round(wall, 3)
    out["GBps"] = round(done_bytes / wall / 1e9, 4)
    return out


def _cpu_single(args, wl, bytes_per_launch, rows_per_layer):
    """The oracle as it stands, single-threaded, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    import synth

    kind, fmt, B, H, P, N = wl["kind"], wl["fmt"], wl["B"], wl["H"], wl["P"], 128
    if kind in ("delta", "kda"):
        nmat = 64
        init = synth.init_state(args.seed, 0, nmat * P, N)
        q, k, v, al, be = synth.delta_inputs(args.seed, 0, 1, nmat, P, N)
        if fmt == "damp":
            st = oracle.damp_from_fp32(init.reshape(1, nmat, P, N), 1, nmat)
            step = oracle.damp_step
        else:
            st = oracle.make_state(fmt, nmat * P, N, init)
            step = oracle.delta_step
        if kind == "kda":
            al = synth.kda_alpha(args.seed, 0, 1, nmat, P)
            step = oracle.kda_step
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            step(st, q, k, v, al, be, 1, nmat)
            done += nmat * P
        sample = f"{nmat} matrices (128 x 128, {fmt}) of the delta layer, one step per call"
    elif kind == "prefill":
        Tc = 256
        x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(args.seed, 0, 1, Tc, H, 1, P, N)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            st = oracle.make_state(fmt, H * P, N)
            oracle.mamba2_prefill(st, x, dt, A, Bm, Cm, D, chunk=wl["chunk"])
            done += H * P * Tc
        sample = f"one sequence ({H * P} rows, {fmt}) over a {Tc}-token prompt in chunks of {wl['chunk']}"
    else:
        R = 32768
        srows = np.arange(R, dtype=np.int64)
        init = synth.init_state_rows(args.seed, 0, srows, N) if wl["init"] == "random" else None
        st = oracle.make_state(fmt, R, N, init)
        T = 1
        x, dt, Bm, Cm, A, D = synth.mamba2_rows_scan_inputs(args.seed, 0, B, T, H, 1, P, N, srows)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.mamba2_rows_scan(st, x, dt, A, Bm, Cm, D)
            done += R
        sample = f"{R} rows ({fmt}) of layer 0, one token per call"
    el = time.perf_counter() - t0
    rows_per_s = done / el  # row updates (one row, one token) per second
    gbps = rows_per_s * (bytes_per_launch / (rows_per_layer * wl.get("T", 1))) / 1e9
    out = {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": sample + f", repeated for {el:.1f} s", "rows_per_s": round(rows_per_s, 1)}
    if kind not in ("scan", "prefill"):
        layers = 1 if wl.get("rotate") else wl["layers"]
        out["decode_steps_per_s"] = round(rows_per_s / (rows_per_layer * layers), 5)
    return out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
