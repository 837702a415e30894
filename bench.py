#!/usr/bin/env python3
"""Benchmark of the MiX hot path on one MI355X.

One step = MiX-4.5b quantization of the activations X [4096 x 3584] (bf16; one kernel writes the
MiX codes and the GEMM's decoded A image) followed by the A-MiX x W-MXFP4 product with
W^T [18944 x 3584] (bf16 output) -- the Qwen2-VL-7B-shaped prefill linear layer. The weights are
MX-coded and imaged once before timing (offline in deployment); their quantizer is timed
separately and reported beside the step.

Prints ONE JSON line. ``value`` is the step's throughput in TFLOP/s (2 M N K per step over the
timed wall time, inputs resident in HBM). ``roofline`` reports the dominant kernel (the GEMM)
against the dense block-scaled FP8 MFMA peak; per-kernel times come from HIP events recorded on
the stream the kernels run on. ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same workload.

By default the same line also carries the other workloads as sections (``vision_linear``,
``attention_prefill``, ``decode``), each with its kernel time, algorithmic work, roofline fraction
and its own ``cpu_baseline``, and ``streaming_ceiling``: what this GPU reads and copies in practice,
measured in the same run. ``--workload`` prints one workload's line alone.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense, block-scaled FP8 (E4M3 A operand sets the rate)
TRAFFIC_SOURCE = ("stored figure: profiles/traffic.json, from rocprofv3 FETCH_SIZE and WRITE_SIZE runs scaled by a "
                  "plain copy's counts; null once the kernel's sources differ from those it was taken on")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the step untimed for this long before the warm-up steps (clock ramp of an idle GPU)")
    ap.add_argument("--workload", default="all",
                    choices=["all", "prefill_linear", "vision_linear", "attention_prefill", "decode"],
                    help="all (default): the prefill-linear line with the other workloads as sections")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time only hipBLASLt (torch._scaled_mm) on the prefill linear shape, as context")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class KernelTimer:
    """HIP events on the current stream around named launches; averages per name."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append(e)
        return e

    @staticmethod
    def ms(a, b):
        return a.elapsed_time(b)


def measured_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel, from the FETCH_SIZE / WRITE_SIZE counter runs
    recorded in profiles/traffic.json (scaled by a plain copy's counts); None if none was recorded or the
    kernel's sources changed since."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(root, "profiles", "traffic.json"))).get(workload)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["source_files"]:
        try:
            h.update(open(os.path.join(root, f), "rb").read())
        except OSError:
            return None
    return rec["traffic_bytes"] if h.hexdigest() == rec["source_sha256"] else None


# VALU issue peak: 256 CUs x 4 SIMDs, a wave64 instruction every 4 cycles per SIMD (16 lanes a
# cycle; the published 157.3 TFLOP/s fp32 vector figure counts packed two-element FMAs), 2.4 GHz
VALU_PEAK_GINSTS = 256 * 4 * 2.4e9 / 4 / 1e9


def measured_valu(workload):
    """VALU wave-instructions per call of the workload, from the SQ_INSTS_VALU counter run recorded in
    profiles/valu.json; None if none was recorded or the sources changed since."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(root, "profiles", "valu.json"))).get(workload)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["source_files"]:
        try:
            h.update(open(os.path.join(root, f), "rb").read())
        except OSError:
            return None
    return rec if h.hexdigest() == rec["source_sha256"] else None


def settle(torch, fn, ms):
    """Run fn(i) untimed for at least `ms` of wall time (synchronizing every few calls, so that the GPU
    is busy throughout). An idle MI355X needs tens of ms of sustained load to reach its steady clocks:
    the prefill GEMM measured 256-313 us per launch in its first ~10 ms and ~223 us from ~30 ms on,
    the quantizer ~13.5 us, then 12.3 us. Timing starts from that steady state."""
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        fn(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def rotating(n_bytes_each, min_total=320 << 20):
    """How many copies of a buffer are needed to exceed the 256 MB last-level cache."""
    return max(1, math.ceil(min_total / max(1, n_bytes_each)))


# ---------------------------------------------------------------- CPU baseline (oracle)

def cpu_baseline_linear(x_bits, w_t_bits, a_fmt, b_fmt, rows, cols, label):
    import oracle.gemm as og
    import oracle.mix as om
    import oracle.mx as ox
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    xs = x_bits[:rows]
    ws = w_t_bits[:cols]
    bc, bs = ox.mx_quantize(ws, b_fmt, "bf16")  # weights offline, as on the GPU
    t0 = time.perf_counter()
    ac, as_ = om.mix_quantize(xs, a_fmt, "bf16")
    c = og.gemm_ref(om.mix_dequantize(ac, as_, a_fmt), ox.mx_dequantize(bc, bs, b_fmt))
    dt = time.perf_counter() - t0
    K = xs.shape[1]
    flops = 2.0 * rows * cols * K
    assert np.isfinite(c).all()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{label}: rows 0..{rows - 1} of X x columns 0..{cols - 1} of W (MiX quantize, decode, fp64 "
                      f"product; the weights' MX codes made before timing), {dt:.1f} s"}


# ---------------------------------------------------------------- workloads

def bench_linear(torch, q, args, which):
    from quantized_gemm_algorithm_amd import synth
    if which == "prefill_linear":
        g = synth.prefill_linear()
        a_fmt, b_fmt, wl = "4.5b", "fp4", "qwen2vl7b_prefill_linear"
    else:
        g = synth.vision_linear()
        a_fmt, b_fmt, wl = "4.25b", "int4", "vision_encoder_linear"
    M, K = g["x"].shape
    N = g["w_t"].shape[0]
    dev = torch.device("cuda")

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    x0 = to_bf16(g["x"])
    w = to_bf16(g["w_t"])
    nrot = rotating(x0.numel() * 2)
    xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
    # weights: MX-coded and imaged once (offline in deployment; the quantizer is timed separately)
    bc, bs = q.mx_quantize(w, b_fmt)
    bimg = q.mx_gemm_b_image(bc, bs, b_fmt)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # per step: MiX codes + the GEMM's A image in one pass, then the GEMM from the images
    bufs = [q.mix_quantize_gemm(x, a_fmt) for x in xs[:2]]

    def step(i, marks=None):
        x = xs[i % nrot]
        ac, as_, aimg = bufs[i % 2]
        e0 = marks.mark() if marks else None
        q.mix_quantize_gemm(x, a_fmt, codes=ac, shared=as_, image=aimg)
        e1 = marks.mark() if marks else None
        q.mix_mx_gemm_images(aimg, bimg, out=out)
        e2 = marks.mark() if marks else None
        return e0, e1, e2

    settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # the timed steps: the two launches back to back, nothing recorded between them (an event marker
    # between launches costs about 3 us of the step each: 216.1 us with none, 225.3 us with three)
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    # the same steps again with events around each launch: the kernels' own durations
    timer = KernelTimer(torch)
    evs = []
    t_start.record()
    for i in range(args.steps):
        evs.append(step(i, timer))
    t_end.record()
    torch.cuda.synchronize()
    ms_step_marked = t_start.elapsed_time(t_end) / args.steps
    q_ms = np.mean([KernelTimer.ms(a, b) for a, b, _ in evs])
    g_ms = np.mean([KernelTimer.ms(b, c) for _, b, c in evs])

    # the quantizer's throughput: back-to-back launches on rotating inputs between two events (the
    # in-step events above also hold the dispatch gap around each event); the codes-only kernel (the
    # quantizer as the pages define it) and the step's variant that also writes the A image
    qrep = 20

    def q_stream(fn):
        for i in range(qrep):
            fn(i)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(qrep):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / qrep

    q_stream_ms = q_stream(lambda i: q.mix_quantize_gemm(xs[i % nrot], a_fmt, codes=bufs[i % 2][0],
                                                         shared=bufs[i % 2][1], image=bufs[i % 2][2]))
    q_codes_ms = q_stream(lambda i: q.mix_quantize(xs[i % nrot], a_fmt, codes=bufs[i % 2][0], shared=bufs[i % 2][1]))

    # weight quantizer, timed on its own (offline in deployment)
    wq_ms = []
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record(); q.mx_quantize(w, b_fmt); b.record()
        torch.cuda.synchronize()
        wq_ms.append(a.elapsed_time(b))
    wq_ms = float(np.median(wq_ms))

    # the Eq. (6) shift-and-add path on the vector ALUs (the comparison), same operands
    ac0, as0, _ = bufs[0]
    eq6_ms = []
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record(); q.mix_mx_gemm_eq6(ac0, as0, a_fmt, bc, bs, b_fmt, out=out); b.record()
        torch.cuda.synchronize()
        eq6_ms.append(a.elapsed_time(b))
    eq6_ms = float(np.median(eq6_ms))

    # the output quantized for a next layer (MiX-4.5b codes + its A image): in the GEMM epilogue
    # against the unfused chain (bf16 C, then the quantizer reading it back); N % 128 == 0
    fq = None
    if a_fmt == "4.5b" and N % 128 == 0:
        nq = q.mix_gemm_a_image_bytes(M, N)
        qc = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
        qs = torch.empty((M, N // 32), dtype=torch.int16, device=dev)
        qi = torch.empty((nq,), dtype=torch.uint8, device=dev)

        def chain(i, fused):
            x = xs[i % nrot]
            ac, as_, aimg = bufs[i % 2]
            q.mix_quantize_gemm(x, a_fmt, codes=ac, shared=as_, image=aimg)
            if fused:
                q.mix_mx_gemm_images_quantize(aimg, bimg, keep_c=False, codes=qc, shared=qs, q_image=qi)
            else:
                q.mix_mx_gemm_images(aimg, bimg, out=out)
                q.mix_quantize_gemm(out, "4.5b", codes=qc, shared=qs, image=qi)

        fq = {}
        for name, fused in (("unfused_ms", False), ("fused_ms", True)):
            for i in range(args.warmup):
                chain(i, fused)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(args.steps):
                chain(i, fused)
            b.record()
            torch.cuda.synchronize()
            fq[name] = a.elapsed_time(b) / args.steps
        fq["what"] = ("step that also codes the output as MiX-4.5b with its A image: quantize X, GEMM, then "
                      "quantize C (unfused, bf16 C through HBM) or the GEMM epilogue codes C (fused, no C)")
        fq["speedup"] = fq["unfused_ms"] / fq["fused_ms"]

    # MiX-INT4g16 (MiX-4.5b activations x MXINT4g16 weights, one exponent per 16 weight elements):
    # the same A image against the folded E4M3 B image of the g16 weights
    g16 = None
    if a_fmt == "4.5b":
        def evt_ms(fn, reps):
            ts = []
            for _ in range(reps):
                a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
                a.record(); fn(); b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return float(np.median(ts))
        gc, gs = q.mx_quantize(w, "int4g16")
        gwq_ms = evt_ms(lambda: q.mx_quantize(w, "int4g16"), 5)
        gimg = q.mx_gemm_b_image(gc, gs, "int4g16")
        gimg_ms = evt_ms(lambda: q.mx_gemm_b_image(gc, gs, "int4g16", out=gimg.buf), 5)
        aimg0 = bufs[0][2]
        settle(torch, lambda i, marks=None: q.mix_mx_gemm_images(aimg0, gimg, out=out), 100)
        gg_ms = evt_ms(lambda: q.mix_mx_gemm_images(aimg0, gimg, out=out), 10)
        g16 = {"pairing": "MiX-INT4g16 (MiX-4.5b x MXINT4g16)", "kernel": "k_gemm_f8 (E4M3 B image)",
               "gemm_ms": gg_ms, "TFLOP/s": 2.0 * M * N * K / (gg_ms * 1e-3) / 1e12,
               "frac_mfma": 2.0 * M * N * K / (gg_ms * 1e-3) / 1e12 / FP8_MFMA_PEAK_TFLOPS,
               "weight_quantizer_ms": gwq_ms, "image_build_ms": gimg_ms,
               "unfoldable_blocks": int(gimg.unfoldable.item())}
        del gc, gs, gimg  # free before the CPU baseline

    flops = 2.0 * M * N * K
    sh_bytes = 2 if a_fmt == "4.5b" else 1
    tiles_m, tiles_n = -(-M // 256), -(-N // 256)
    a_img_bytes = M * K + (K // 128) * tiles_m * 1024
    # quantizer: bf16 in; codes + shared fields out (the algorithmic bytes), + the A image (the step's variant)
    q_codes_bytes = M * K * 2 + M * K // 2 + M * (K // 32) * sh_bytes
    q_bytes = q_codes_bytes + a_img_bytes
    wq_bytes = N * K * 2 + N * K // 2 + N * (K // 32)
    b_bytes = (N * K // 2 if b_fmt == "fp4" else N * K) + (K // 128) * tiles_n * 1024
    gemm_bytes = a_img_bytes + b_bytes + M * N * 2  # each operand once + C
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    res = {
        "metric": "A-MiX4.5b x W-MXFP4 GEMM TFLOP/s + quantizer GB/s (% of MI355X peak)" if which == "prefill_linear"
        else "A-MiX4.25b x W-MXINT4 GEMM TFLOP/s + quantizer GB/s (% of MI355X peak)",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3xe2m1->f32" if b_fmt == "fp4" else "e4m3xe4m3->f32",
        "data": "synthetic",
        "config": {"workload": wl, "M": M, "K": K, "N": N, "a_format": "MiX-" + a_fmt,
                   "b_format": "MX" + b_fmt.upper(), "out": "bf16"},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": gemm_tflops / FP8_MFMA_PEAK_TFLOPS, "traffic": measured_traffic(which),
                     "traffic_source": TRAFFIC_SOURCE, "kernel": "k_gemm_f8",
                     "kernel_ms": g_ms, "algorithmic_flops": flops, "operand_bytes": gemm_bytes,
                     "timing": f"{args.steps} steps with HIP events around each launch, run right after the "
                               f"{args.steps} timed steps (which carry no events between launches; "
                               f"{ms_step_marked:.4f} ms per step with them)"},
        "quantizer": {"kernel": "k_mix_quantize (codes and shared fields)", "ms": q_codes_ms,
                      "GB/s": q_codes_bytes / (q_codes_ms * 1e-3) / 1e9,
                      "frac_hbm": q_codes_bytes / (q_codes_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "algorithmic_bytes": q_codes_bytes,
                      "timing": f"{qrep} back-to-back launches between two HIP events",
                      "traffic": measured_traffic(which + "_quantizer_codes"), "traffic_source": TRAFFIC_SOURCE,
                      "rotating_buffers": nrot,
                      "with_a_image": {"kernel": "k_mix_quantize (codes + the GEMM's A image, the step's variant)",
                                       "ms": q_stream_ms, "bytes": q_bytes,
                                       "GB/s": q_bytes / (q_stream_ms * 1e-3) / 1e9,
                                       "frac_hbm": q_bytes / (q_stream_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "frac_hbm_on_algorithmic_bytes":
                                           q_codes_bytes / (q_stream_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "traffic": measured_traffic(which + "_quantizer"),
                                       "in_step_ms": q_ms}},
        "weight_quantizer": {"kernel": "k_mx_quantize", "ms": wq_ms, "GB/s": wq_bytes / (wq_ms * 1e-3) / 1e9,
                             "frac_hbm": wq_bytes / (wq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": wq_bytes},
        "eq6_valu_gemm": {"kernel": "k_gemm_eq6", "ms": eq6_ms, "TFLOP/s": flops / (eq6_ms * 1e-3) / 1e12},
    }
    if fq is not None:
        res["fused_output_quantization"] = fq
    if g16 is not None:
        res["g16_weights"] = g16
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_linear(g["x"], g["w_t"], a_fmt, b_fmt, M, N, wl)
    return res


def bench_decode(torch, q, args):
    """Decode step (batch 16): x [16, 3584] -> MiX-4.5b -> product with the MXFP4 weights
    [18944, 3584] -> y bf16, and attention of q [16, 28, 128] over 8192 MX-coded cached tokens per
    row (the new token at position 8191 smoothed with the frozen prefill mean and appended), all in
    one mix_decode_step call (three launches)."""
    from quantized_gemm_algorithm_amd import synth
    g = synth.decode_step()
    B, L, Hkv, d = g["k_hist"].shape
    Hq = g["q"].shape[1]
    N, K = g["w_t"].shape
    dev = torch.device("cuda")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x = bf16(g["x"])
    qd = bf16(g["q"])
    w = bf16(g["w_t"])
    bc, bs = q.mx_quantize(w, "fp4")
    del w
    # one set = weights (image) and a KV cache; sets rotate to defeat the 256 MB MALL
    w_bytes = N * K // 2 + N * (K // 32)
    kv_bytes = 2 * B * Hkv * L * (d // 2 + d // 32)
    nset = rotating(w_bytes + kv_bytes, min_total=600 << 20)
    pos = torch.full((B,), L - 1, dtype=torch.int32, device=dev)
    k_new = bf16(g["k_hist"][:, L - 1])
    v_new = bf16(g["v_hist"][:, L - 1])
    sets = []
    mus = []
    for b in range(B):
        kd = bf16(g["k_hist"][b, :L - 1])
        mus.append(q.mix_kmean(kd.reshape(L - 1, Hkv * d)).reshape(Hkv, d))
    mu = torch.stack(mus)
    for si in range(nset):
        bci, bsi = (bc, bs) if si == 0 else (bc.clone(), bs.clone())
        cache = q.KVCache(B, L, Hkv, d)
        for b in range(B):
            q.mix_kv_cache_prefill(cache, b, bf16(g["k_hist"][b, :L - 1]), bf16(g["v_hist"][b, :L - 1]), mu[b])
        sets.append((q.mx_gemm_b_image(bci, bsi, "fp4"), cache))
    torch.cuda.synchronize()
    y = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((q._lib_().mix_decode_step_workspace_bytes(B, K, Hq, Hkv, d, L - 1),), dtype=torch.uint8,
                     device=dev)

    def step(i):
        bimg, cache = sets[i % nset]
        q.mix_decode_step(x, bimg, qd, k_new, v_new, cache, pos, L - 1, mu, y=y, o=o, workspace=ws)

    # the step captured once per weight/cache set as a HIP graph and replayed (outputs checked
    # against the eager step)
    step(0)
    torch.cuda.synchronize()
    y_ref, o_ref = y.clone(), o.clone()
    graphs = []
    for si in range(nset):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step(si)
        graphs.append(gr)
    settle(torch, lambda i: graphs[i % nset].replay(), args.settle_ms)
    for i in range(args.warmup):
        graphs[i % nset].replay()
    torch.cuda.synchronize()
    if not (torch.equal(y, y_ref) and torch.equal(o, o_ref)):
        raise RuntimeError("graph replay of the decode step differs from the eager step")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        graphs[i % nset].replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / args.steps
    # the timed steps: back-to-back calls on the stream (three launches each), as for the other
    # workloads; the graph replay above is reported beside them
    settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # the same step in one cooperative launch (grid-wide barriers where the launch boundaries stand),
    # checked against the eager step and timed the same way
    def step_single(i):
        bimg, cache = sets[i % nset]
        q.mix_decode_step(x, bimg, qd, k_new, v_new, cache, pos, L - 1, mu, y=y, o=o, workspace=ws, single=True)

    step_single(0)
    torch.cuda.synchronize()
    if not (torch.equal(y, y_ref) and torch.equal(o, o_ref)):
        raise RuntimeError("the single-launch decode step differs from the three-launch step")
    for i in range(args.warmup):
        step_single(i)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step_single(i)
    t1.record()
    torch.cuda.synchronize()
    ms_single = t0.elapsed_time(t1) / args.steps

    # the same work as separate calls (quantize x with its A image, the weight-stream product,
    # attention alone), each timed as back-to-back launches in one graph over the rotating sets
    ac, as_, aimg = q.mix_quantize_gemm(x, "4.5b")
    wsa = torch.empty((q._lib_().mix_attn_decode_workspace_bytes(B, Hq, Hkv, d, L - 1),), dtype=torch.uint8,
                      device=dev)
    gv_nset = max(nset, rotating(w_bytes, 320 << 20))
    gv_imgs = [sets[i % nset][0] if i < nset else None for i in range(gv_nset)]
    for i in range(nset, gv_nset):
        gv_imgs[i] = q.mx_gemm_b_image(bc.clone(), bs.clone(), "fp4")

    def graph_ms(fn, reps):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(reps):
                fn(i)
        gr.replay()
        torch.cuda.synchronize()
        t0.record()
        gr.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    parts_q = graph_ms(lambda i: q.mix_quantize_gemm(x, "4.5b", codes=ac, shared=as_, image=aimg), 16)
    parts_gv = graph_ms(lambda i: q.mix_mx_gemm_images(aimg, gv_imgs[i % gv_nset], out=y), 2 * gv_nset)
    parts_at = graph_ms(lambda i: q.mix_attn_decode(qd, k_new, v_new, sets[i % nset][1], pos, L - 1, mu,
                                                    workspace=wsa), 2 * nset)
    del gv_imgs

    a_img_bytes = B * K + (K // 128) * 1024
    gv_bytes = N * K // 2 + (K // 128) * (-(-N // 256)) * 1024 + a_img_bytes + B * N * 2
    # the step's algorithmic bytes: x in; the weights (codes + scales) and the cached K and V codes +
    # scales of 8192 tokens read once; q, the new token in and out, mu; y and o out
    step_bytes = (B * K * 2 + w_bytes + kv_bytes + B * Hq * d * 2 + 2 * B * Hkv * d * 2 + B * Hkv * d * 4
                  + B * N * 2 + B * Hq * d * 2)
    at_bytes = kv_bytes + B * Hq * d * 2 * 2 + 2 * B * Hkv * d * 2 + B * Hkv * d * 4
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "decode GB/s (% of MI355X HBM peak)",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3xe2m1->f32", "data": "synthetic",
        "config": {"workload": "decode_step_b16_l8192", "B": B, "K": K, "N": N, "L": L, "Hq": Hq, "Hkv": Hkv,
                   "d": d, "bytes_per_step": step_bytes, "rotating_sets": nset},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode"),
                     "traffic_source": TRAFFIC_SOURCE,
                     "kernel": "mix_decode_step (k_decode_scores + k_decode_pv + k_decode_combine)",
                     "kernel_ms": ms_step, "timing": f"{args.steps} back-to-back steps between two HIP events",
                     "algorithmic_bytes": step_bytes},
        "parts": {"graph_replay_ms_per_step": ms_graph,
                  "single_launch_ms_per_step": ms_single,
                  "separate_calls": {"what": "the same work as separate calls, each timed as back-to-back launches "
                                             "in one graph",
                                     "quantize_x_ms": parts_q, "gemv_ms": parts_gv,
                                     "gemv_GB/s": gv_bytes / (parts_gv * 1e-3) / 1e9,
                                     "attention_ms": parts_at,
                                     "attention_GB/s": at_bytes / (parts_at * 1e-3) / 1e9,
                                     "sum_ms": parts_q + parts_gv + parts_at}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(g, w_bytes, kv_bytes // B)
    return res


def cpu_baseline_decode(g, w_bytes, kv_bytes_row, rows=2):
    import oracle.attention as oa
    import oracle.gemm as og
    import oracle.mix as om
    import oracle.mx as ox
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    bc, bs = ox.mx_quantize(g["w_t"], "fp4", "bf16")  # weights offline, as on the GPU
    L = g["k_hist"].shape[1]
    mu = np.stack([oa.kmean_ref(g["k_hist"][b, :L - 1], "bf16") for b in range(rows)])  # prefill's, frozen
    t0 = time.perf_counter()
    ac, as_ = om.mix_quantize(g["x"], "4.5b", "bf16")
    og.gemm_ref(om.mix_dequantize(ac, as_, "4.5b"), ox.mx_dequantize(bc, bs, "fp4"))
    oa.attn_decode_ref(g["q"][:rows], g["k_hist"][:rows], g["v_hist"][:rows], mu, np.full(rows, L))
    dt = time.perf_counter() - t0
    byts = w_bytes + rows * kv_bytes_row
    return {"value": byts / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"decode step: the full x x W product (weights MX-coded before timing) and attention of batch "
                      f"rows 0..{rows - 1} over {L} tokens (the oracle codes their K/V history itself), {dt:.1f} s; "
                      f"credited bytes = weights + those rows' cached K/V"}


def bench_attention(torch, q, args):
    """Prefill attention: q [4096, 28, 128], k/v [4096, 4, 128] bf16, causal, K-smoothed."""
    from quantized_gemm_algorithm_amd import synth
    g = synth.attention_qkv()
    T, Hq, d = g["q"].shape
    Hkv = g["k"].shape[1]
    dev = torch.device("cuda")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    qd, kd, vd = bf16(g["q"]), bf16(g["k"]), bf16(g["v"])
    wsb = q._lib_().mix_attn_prefill_workspace_bytes(T, Hq, Hkv, d)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)

    def step():
        q.mix_attn_prefill(qd, kd, vd, causal=True, workspace=ws)

    settle(torch, lambda i: step(), args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # causal-exact work: row i attends to i + 1 keys; QK^T and PV each 2 d flops per (row, key)
    pairs = Hq * T * (T + 1) // 2
    flops = 2 * 2.0 * d * pairs
    tf = flops / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "prefill attention TFLOP/s (causal-exact flops)",
        "value": tf, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3xe2m1->f32", "data": "synthetic",
        "config": {"workload": "prefill_attention_t4096_h28_kv4_d128", "T": T, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "causal": True, "workspace_bytes": wsb},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / FP8_MFMA_PEAK_TFLOPS, "traffic": measured_traffic("attention_prefill"),
                     "traffic_source": TRAFFIC_SOURCE,
                     "kernel": "mix_attn_prefill (all kernels of the call)", "kernel_ms": ms_step},
    }
    vr = measured_valu("attention_prefill")
    if vr is not None:
        gis = vr["valu_insts_per_call"] / (ms_step * 1e-3) / 1e9
        res["roofline_valu"] = {
            "bound": "alu", "achieved": gis, "peak": VALU_PEAK_GINSTS, "unit": "G wave-instructions/s",
            "frac": gis / VALU_PEAK_GINSTS, "kernel": "mix_attn_prefill (all kernels of the call)",
            "valu_insts_per_call": vr["valu_insts_per_call"],
            "source": "stored figure: profiles/valu.json (rocprofv3 SQ_INSTS_VALU, device total per kernel); null "
                      "once the sources differ from those it was taken on",
            "dominant_kernel": {"kernel": "k_attn_pcode", "valu_insts": vr["valu_insts_per_kernel"]["k_attn_pcode<false>"],
                                "valu_time_floor_ms": vr["valu_insts_per_kernel"]["k_attn_pcode<false>"] /
                                                      (VALU_PEAK_GINSTS * 1e9) * 1e3}}
    res["underflow_map"] = underflow_section(torch, q, kd.view(T, Hkv * d))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_attention(g, d)
    return res


def cpu_baseline_attention(g, d, nrows=64):
    """The oracle's prefill (K-mean, coding, S, softmax, P coding, O) for every head over the last
    nrows query rows (which see the most keys); credited with their causal-exact flops."""
    import oracle.attention as oa
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    T, Hq, _ = g["q"].shape
    rows = np.arange(T - nrows, T)
    t0 = time.perf_counter()
    oa.attn_prefill_ref(g["q"], g["k"], g["v"], "bf16", causal=True, rows=rows)
    dt = time.perf_counter() - t0
    flops = 2 * 2.0 * d * Hq * float(np.sum(rows + 1))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"prefill attention: query rows {T - nrows}..{T - 1} of all {Hq} heads against all keys (the "
                      f"oracle codes the full K and V itself), {dt:.1f} s; credited with those rows' causal flops"}


def underflow_section(torch, q, k2d):
    """The underflow ("dead zone") map of the keys [T, Hkv d], blocks of 32 along the head dimension,
    raw and K-smoothed: per format the fraction of nonzero elements coded to zero, and the time of
    one mix_underflow_map call (three launches: clear, amax, map; the operand is read twice)."""
    mu = q.mix_kmean(k2d)
    out = {"what": "fraction of nonzero key elements each format codes to zero (32-element blocks)",
           "operand": list(k2d.shape)}
    for name, m in (("raw", None), ("smoothed", mu)):
        counts, _ = q.mix_underflow_map(k2d, mu=m)
        tot = counts.sum(dim=1).cpu().numpy()
        out[name] = {kind: float(tot[i]) / max(float(tot[-1]), 1.0) for i, kind in enumerate(q.UF_KINDS[:-1])}
    ws = torch.empty((q.mix_underflow_map_workspace_bytes(*k2d.shape),), dtype=torch.uint8, device=k2d.device)
    reps = 20
    for _ in range(3):
        q.mix_underflow_map(k2d, workspace=ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        q.mix_underflow_map(k2d, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 2 * k2d.numel() * k2d.element_size()
    out["call_ms"] = ms
    out["timing"] = f"{reps} back-to-back calls between two HIP events"
    out["read_GB/s"] = nbytes / (ms * 1e-3) / 1e9
    return out


def streaming_ceiling(torch):
    """What this GPU streams in practice, measured in the same run: a plain read (a sum over 1 GiB
    of int64) and a device-to-device copy (1 GiB each way), each the best of 5."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    s64 = src.view(torch.int64)
    torch.cuda.synchronize()

    def best(fn):
        ts = []
        for _ in range(6):
            a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
            a.record(); fn(); b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts[1:])

    read_ms = best(lambda: s64.sum())
    copy_ms = best(lambda: dst.copy_(src))
    out = {"read_GB/s": n / (read_ms * 1e-3) / 1e9, "copy_GB/s": 2 * n / (copy_ms * 1e-3) / 1e9,
           "what": "torch int64 sum over 1 GiB (read) and a 1 GiB device copy (read + write), best of 5"}
    out["read_frac_hbm"] = out["read_GB/s"] / HBM_PEAK_GBS
    out["copy_frac_hbm"] = out["copy_GB/s"] / HBM_PEAK_GBS
    del src, dst
    torch.cuda.empty_cache()
    return out


def same_size_stream(torch, nbytes, kind, reps=20):
    """A device copy (nbytes moved: nbytes / 2 read, nbytes / 2 written) or an int64 sum (nbytes
    read) of the size one call of a streaming kernel moves, timed like that kernel: `reps`
    back-to-back launches between two HIP events over buffers rotating through >= 320 MB, so each
    launch reads from HBM. This is the rate a launch of that size reaches, start-up included."""
    n = (nbytes // 2 if kind == "copy" else nbytes) // 256 * 256
    nrot = max(2, -(-320_000_000 // n))
    srcs = [torch.ones(n // 8, dtype=torch.int64, device="cuda") for _ in range(nrot)]
    dsts = [torch.empty_like(srcs[0]) for _ in range(2)]
    fn = (lambda i: dsts[i % 2].copy_(srcs[i % nrot])) if kind == "copy" else (lambda i: srcs[i % nrot].sum())
    for i in range(2 * nrot):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    moved = 2 * n if kind == "copy" else n
    del srcs, dsts
    torch.cuda.empty_cache()
    return {"bytes": moved, "ms": ms, "GB/s": moved / (ms * 1e-3) / 1e9,
            "what": f"torch {'device copy' if kind == 'copy' else 'int64 sum'} of the same bytes, "
                    f"{reps} back-to-back launches over rotating buffers"}


def section(res):
    """A workload's result as a section of the default line (the contract keys dropped)."""
    keep = {k: v for k, v in res.items() if k not in ("n_gpus", "steps", "warmup", "settle_ms", "higher_is_better",
                                                      "scaling", "vs_baseline", "data")}
    return keep


def calibrate_copy(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}))


def vendor_gemm(torch, args):
    """hipBLASLt through torch._scaled_mm on the prefill linear shape (M=4096, N=18944, K=3584, bf16
    out): tensorwise FP8, block-scaled MXFP8 (E8M0 per 32) and MXFP4 x MXFP4. Context for the
    block-scaled MFMA GEMM's roofline, not part of the step."""
    M, K, N = 4096, 3584, 18944
    dev = "cuda"
    flop = 2.0 * M * N * K
    gen = torch.Generator(device=dev).manual_seed(0)

    def timeit(fn):
        settle(torch, lambda i: fn(), args.settle_ms)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        return {"us": ms * 1e3, "TFLOP/s": flop / ms / 1e9}

    out = {"workload": "vendor_gemm_4096x18944x3584", "library": "hipBLASLt via torch._scaled_mm"}
    a = (torch.randn(M, K, device=dev, generator=gen) * 0.5).to(torch.float8_e4m3fn)
    b = (torch.randn(N, K, device=dev, generator=gen) * 0.5).to(torch.float8_e4m3fn)
    one = torch.tensor(1.0, device=dev)
    e8 = torch.float8_e8m0fnu
    sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev).view(e8)
    sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev).view(e8)
    cases = {
        "fp8_tensorwise": lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16),
        "mxfp8": lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16),
    }
    a4 = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=gen).view(torch.float4_e2m1fn_x2)
    b4 = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=gen).view(torch.float4_e2m1fn_x2)
    cases["mxfp4"] = lambda: torch._scaled_mm(a4, b4.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
    for name, fn in cases.items():
        try:
            out[name] = timeit(fn)
        except Exception as e:  # a format this torch/hipBLASLt build does not offer
            out[name] = {"error": repr(e)[:200]}
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is not sharded across GPUs. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.vendor_gemm:
        vendor_gemm(torch, args)
        return
    import quantized_gemm_algorithm_amd as q
    q._lib_()  # fail loudly if the HIP library is missing
    if args.workload in ("prefill_linear", "vision_linear"):
        res = bench_linear(torch, q, args, args.workload)
    elif args.workload == "decode":
        res = bench_decode(torch, q, args)
    elif args.workload == "attention_prefill":
        res = bench_attention(torch, q, args)
    else:
        # the headline workload's line, then the other workloads as sections of it, then what this GPU
        # streams in practice (the ceiling the HBM-bound kernels are compared with besides 8 TB/s)
        res = bench_linear(torch, q, args, "prefill_linear")
        log("prefill_linear done")
        torch.cuda.empty_cache()
        res["vision_linear"] = section(bench_linear(torch, q, args, "vision_linear"))
        log("vision_linear done")
        torch.cuda.empty_cache()
        res["attention_prefill"] = section(bench_attention(torch, q, args))
        log("attention_prefill done")
        torch.cuda.empty_cache()
        res["decode"] = section(bench_decode(torch, q, args))
        log("decode done")
        torch.cuda.empty_cache()
        ceil = streaming_ceiling(torch)
        qz = res["quantizer"]
        ceil["quantizer_frac_of_copy"] = qz["GB/s"] / ceil["copy_GB/s"]
        ceil["quantizer_with_image_frac_of_copy"] = qz["with_a_image"]["GB/s"] / ceil["copy_GB/s"]
        ceil["decode_frac_of_read"] = res["decode"]["value"] / ceil["read_GB/s"]
        # the same measurement at the size one call moves: a launch of 38 MB or 108 MB does not reach
        # the 1 GiB rate (start-up and drain are a larger share of it)
        cq = same_size_stream(torch, qz["algorithmic_bytes"], "copy")
        cq["quantizer_frac"] = qz["GB/s"] / cq["GB/s"]
        ceil["copy_quantizer_bytes"] = cq
        rd = same_size_stream(torch, res["decode"]["roofline"]["algorithmic_bytes"], "read")
        rd["decode_frac"] = res["decode"]["value"] / rd["GB/s"]
        ceil["read_decode_bytes"] = rd
        res["streaming_ceiling"] = ceil
    print(json.dumps(res))


if __name__ == "__main__":
    main()
