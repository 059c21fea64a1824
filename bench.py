#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: the W4A16 decode GEMV of an 8B-shaped MLP gate+up
projection, M in {1, 4, 16} tokens, K = 4096, N = 24576, group 128 (fp16
activations with 0.5% x20 outlier channels; uniform 4-bit weights and zero
points; fp16 scales in [0.005, 0.02]). One step = one GEMV at each of
M = 1, 4, 16, on weights in the decode layout (mq_w4a16_block_weights, run
once per weight set before anything is timed, as a serving engine converts
its checkpoint at load); the same steps on the AWQ [K, N/8] layout
(mq_w4a16_gemv) are reported as `gemv_awq_layout`. Every call reads a different one of `--sets` weight sets
(52 MB each, 520 MB in all), so a set is read again only after more than the
256 MB Infinity Cache and the 32 MB of L2 have been swept: the weight stream
comes from HBM. Inputs are resident in HBM before the timed region. The
steps are captured once in a HIP graph and replayed, so host launch overhead
is not timed.

value = algorithmic bytes of a step (x + qweight + scales + qzeros + y, for
the three calls) / wall time of a step, between device synchronizations.

Also reported (same line):
  roofline     one GEMV call, the unit that dominates the step: one launch of
               w4a16_gemv_blocked_kernel (K is not split at N = 24576, so no
               reduce kernel follows). achieved = algorithmic bytes per call /
               average call duration from HIP events recorded on that stream
               around the timed graph replay, against 8 TB/s; `traffic` =
               FETCH_SIZE + WRITE_SIZE per call from a committed
               rocprofv3 counter summary when it matches the current kernel
               source, else null.
  gemv_bf16    the headline steps with bf16 activations (decode layout).
  prefill      W8A8 prefill (per-token quant + scaled int8 GEMM, M=2048,
               K=N=4096; also with bf16 activations and output) and W4A16
               prefill GEMMs (M=4096, K=4096/12288, N=4096; K=4096 also with
               bf16 activations): kernel time and TOPS against the dense MFMA
               peaks.
  layers       the linear layers of an 8B-shaped decoder layer (qkv 4096->6144,
               o_proj 4096->4096, gate_up 4096->24576, down 12288->4096) at
               M = 1, 8, 64 and 2048 under W4A16 (decode-layout GEMV up to 64
               tokens, GEMM above) and W8A8_INT8 (mq_w8a8_linear: quantizer fused
               into the decode kernel for one token): microseconds per call with
               weights rotating over copies of >= 640 MB per layer; `set` = the
               four layers of a scheme in one graph, microseconds per layer set.
  groups       W4A16 with groups of 64 and 32 rows (LMDeploy quantizes the
               vision tower's attention with groups of 64): the gate+up GEMV
               (M = 1, 4, 16) in GB/s, a ViT-L fused qkv projection (K=1024,
               N=3072) at 1 and 16 tokens (GEMV) and 577 and 4096 tokens
               (GEMM), and the 4096^3 prefill GEMM, cold weights, graph replays.
  kv_quant     online KV-cache quantization (per head, per token, INT8 and
               INT4) of one layer's K: a 4096-token prefill (32 heads x 128,
               rotating copies >= 320 MB) and a 128-sequence decode append;
               microseconds and GB/s of x + codes + (scale, min).
  checkpoint   one-time checkpoint-layout conversions at the 8B gate_up size
               (field reorder, 4-bit transpose, scale transpose), warm.
  roofline_prefill  the prefill GEMMs against their MFMA peaks: the W8A8 GEMM
               at M=2048, K=N=4096 (int8, 5.0 POP/s) and the W4A16 GEMMs at
               M=4096, N=4096, K=4096/12288 (fp16, 2.5 PFLOP/s); achieved =
               2MNK / event-timed average launch; HBM traffic and MFMA-busy
               fraction from a committed rocprofv3 counter summary while it
               matches the kernel sources, else null.
  fp16_matmul_context  torch.matmul in fp16 at the decode and prefill shapes,
               context for the 4-bit vs fp16 ratio (not a target).
  cpu_baseline the CPU oracle on one step of the same workload (one weight
               set), on every core of this process's affinity set and again
               on one thread, about --cpu-seconds in all, in the same unit;
               with the host's CPU model.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0

METRIC = "W4A16 decode GEMV GB/s (% HBM peak); W8A8/W4A16 prefill TOPS (% MFMA peak)"
GEMV_K, GEMV_N, GROUP = 4096, 24576, 128
GEMV_MS = (1, 4, 16)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_c1_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_gemm_counters.json")
# Reading of "int8 weights from N(0, 0.02)": drawn in fp32, rounded to fp16 (the
# served dtype), then quantized per output channel by the per-token quantizer.
W8A8_WEIGHTS = "fp32 N(0, 0.02) rounded to fp16, then symmetric int8 per output channel (absmax/127)"
GEMV_SOURCES = ["w4a16_gemv_blocked.hip", "w4a16_gemv_blocked.h", "w4a16_split.h", "w4a16_common.h",
                "device_common.h"]


def w4a16_bytes(M, K, N, G=GROUP):
    rows = 1 if G == -1 else K // G  # group -1: one parameter row (per-channel)
    return M * K * 2 + K * N // 2 + rows * N * 2 + rows * (N // 8) * 4 + M * N * 2


def gemv_source_hash():
    """Hash of what the GEMV kernels are built from: their sources and flags."""
    from weight_activation_quantized_amd import _build
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, "weight_activation_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(repr((_build.FLAGS[:-2], _build.SOURCE_FLAGS.get("w4a16_gemv_blocked.hip", []))).encode())
    return h.hexdigest()[:16]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=10, help="rotating weight sets (52 MB each)")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-layers", action="store_true", help="skip the decoder-layer linear set")
    ap.add_argument("--no-groups", action="store_true", help="skip the group-64 / group-32 measurements")
    ap.add_argument("--no-kv", action="store_true", help="skip the KV-cache quantization measurements")
    ap.add_argument("--no-checkpoint", action="store_true", help="skip the checkpoint-layout conversions")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-context", action="store_true", help="skip the torch fp16 matmul context timings")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-kernel", action="store_true",
                    help="also run a plain 256 MB device copy (counter calibration under rocprofv3)")
    return ap.parse_args(argv)


def capture(torch, fn, n_calls_hint=""):
    """Capture fn() into a HIP graph (after one eager run) and return it."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_replay(torch, g):
    """Replay g once between synchronizations; return (wall s, event s)."""
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, ev0.elapsed_time(ev1) / 1e3


def bench_gemv(torch, mq, synth, args, log):
    """The headline steps on the decode weight layout (converted once per weight
    set before anything is timed, as at model load), then the same steps on the
    AWQ [K, N/8] layout for comparison."""
    dev = torch.device("cuda", 0)
    log(f"generating {args.sets} weight sets of K={GEMV_K} N={GEMV_N}")
    sets = []
    for s in range(args.sets):
        w = synth.w4a16_weights(GEMV_K, GEMV_N, GROUP, tag=1, seed=1000 + s)
        t = {k: torch.from_numpy(v).to(dev) for k, v in w.items()}
        t["qblocked"] = mq.w4a16_block_weights(t["qweight"])
        sets.append(t)
    xs, ys, wss = {}, {}, {}
    for M in GEMV_MS:
        x = synth.w4a16_inputs(M, GEMV_K, 8, GROUP, outlier_frac=0.005, tag=1, seed=M)["x"]
        xs[M] = torch.from_numpy(x).to(dev)
        ys[M] = torch.empty((M, GEMV_N), dtype=torch.float16, device=dev)
        nbytes = max(mq.w4a16_gemv_blocked_workspace_bytes(M, GEMV_N, GEMV_K, GROUP),
                     mq.w4a16_gemv_workspace_bytes(M, GEMV_N, GEMV_K, GROUP))
        wss[M] = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    counter = [0]

    def steps(n, blocked):
        def run():
            for _ in range(n):
                for M in GEMV_MS:
                    w = sets[counter[0] % len(sets)]
                    counter[0] += 1
                    if blocked:
                        mq.w4a16_gemv_blocked(xs[M], w["qblocked"], w["scales"], w["qzeros"], GROUP, out=ys[M],
                                              workspace=wss[M])
                    else:
                        mq.w4a16_gemv(xs[M], w["qweight"], w["scales"], w["qzeros"], GROUP, out=ys[M],
                                      workspace=wss[M])
        return run

    # the same steps with bf16 activations (bf16 copies of the same x)
    xs_bf = {M: xs[M].float().to(torch.bfloat16) for M in GEMV_MS}
    ys_bf = {M: torch.empty((M, GEMV_N), dtype=torch.bfloat16, device=dev) for M in GEMV_MS}

    def steps_bf16(n):
        def run():
            for _ in range(n):
                for M in GEMV_MS:
                    w = sets[counter[0] % len(sets)]
                    counter[0] += 1
                    mq.w4a16_gemv_blocked(xs_bf[M], w["qblocked"], w["scales"], w["qzeros"], GROUP, out=ys_bf[M],
                                          workspace=wss[M])
        return run

    res = {}
    log("bf16 decode layout: capturing and timing")
    g_warm = capture(torch, steps_bf16(max(args.warmup, 1)))
    g_timed = capture(torch, steps_bf16(args.steps))
    g_warm.replay()
    torch.cuda.synchronize()
    res["bf16"] = timed_replay(torch, g_timed)
    del g_warm, g_timed
    for blocked in (True, False):
        name = "blocked" if blocked else "awq"
        log(f"{name}: capturing warmup ({args.warmup}) and timed ({args.steps}) steps")
        g_warm = capture(torch, steps(max(args.warmup, 1), blocked))
        g_timed = capture(torch, steps(args.steps, blocked))
        g_warm.replay()
        torch.cuda.synchronize()
        log(f"{name}: timed region")
        res[name] = timed_replay(torch, g_timed)
        del g_warm, g_timed
    wall, ev = res["blocked"]
    step_bytes = sum(w4a16_bytes(M, GEMV_K, GEMV_N) for M in GEMV_MS)
    launches = args.steps * len(GEMV_MS)
    workspace_bytes = {M: mq.w4a16_gemv_blocked_workspace_bytes(M, GEMV_N, GEMV_K, GROUP) for M in GEMV_MS}
    awq_wall, awq_ev = res["awq"]
    bf_wall, bf_ev = res["bf16"]
    return {
        "wall_s": wall, "event_s": ev, "step_bytes": step_bytes, "launches": launches,
        "kernel_avg_us": ev / launches * 1e6, "workspace_bytes": workspace_bytes,
        "bytes_per_launch_avg": step_bytes / len(GEMV_MS),
        "awq_layout": {"GBps": round(step_bytes / (awq_wall / args.steps) / 1e9, 1),
                       "us_per_call": round(awq_ev / launches * 1e6, 3),
                       "kernel": "w4a16_gemv_lds_kernel + w4a16_gemv_reduce (K split 8 ways)"},
        "bf16": {"GBps": round(step_bytes / (bf_wall / args.steps) / 1e9, 1),
                 "us_per_call": round(bf_ev / launches * 1e6, 3),
                 "kernel": "w4a16_gemv_blocked_kernel, bf16 activations (same steps, decode layout)"},
    }, sets, xs


def bench_prefill(torch, mq, synth, oracle_free_quant, args, log):
    """W8A8 prefill (quant + GEMM) and W4A16 prefill GEMMs; kernel times from event-timed graph replays
    (the median of three)."""
    import numpy as np
    dev = torch.device("cuda", 0)
    out = {}
    R = args.prefill_reps

    def time_fn(fn):
        # median of three timed replays of R calls each (one warm replay first)
        g = capture(torch, lambda: [fn() for _ in range(R)])
        g.replay()
        evs = sorted(timed_replay(torch, g)[1] for _ in range(3))
        return evs[1] / R

    # W8A8: M=2048, K=N=4096; weights quantized per output channel on the GPU
    M, K, N = 2048, 4096, 4096
    d = synth.w8a8_inputs(M, K, N, outlier_frac=0.01, tag=2)
    x = torch.from_numpy(d["x"]).to(dev)
    wq, s_ch = oracle_free_quant(torch.from_numpy(d["wf"]).to(dev))
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    s_tok = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    log("prefill: w8a8 quant")
    t_q = time_fn(lambda: mq.quant_per_token_int8(x, out=xq, s_out=s_tok))
    log("prefill: w8a8 gemm")
    t_g = time_fn(lambda: mq.w8a8_scaled_mm(xq, s_tok, wq, s_ch, out=y))
    ops = 2.0 * M * N * K
    out["w8a8_c2"] = {
        "shape": [M, N, K], "quant_us": t_q * 1e6, "quant_GBps": (M * K * 3 + M * 4) / t_q / 1e9,
        "gemm_us": t_g * 1e6, "gemm_TOPS": ops / t_g / 1e12,
        "gemm_frac_int8_peak": ops / t_g / 1e12 / INT8_PEAK_TOPS,
        "layer_TOPS": ops / (t_q + t_g) / 1e12,
        "weights": W8A8_WEIGHTS,
    }
    # the same layer with bf16 activations and output (same draws rounded to bf16)
    db = synth.w8a8_inputs_bf16(M, K, N, outlier_frac=0.01, tag=2)
    xb = torch.from_numpy(db["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    log("prefill: w8a8 bf16 quant + gemm")
    t_qb = time_fn(lambda: mq.quant_per_token_int8(xb, out=xq, s_out=s_tok))
    t_gb = time_fn(lambda: mq.w8a8_scaled_mm(xq, s_tok, wq, s_ch, out=yb))
    out["w8a8_c2_bf16"] = {
        "shape": [M, N, K], "quant_us": t_qb * 1e6, "gemm_us": t_gb * 1e6, "gemm_TOPS": ops / t_gb / 1e12,
        "gemm_frac_int8_peak": ops / t_gb / 1e12 / INT8_PEAK_TOPS,
    }
    del x, wq, s_ch, xq, s_tok, y, xb, yb
    for name, K in (("w4a16_c3a", 4096), ("w4a16_c3b", 12288)):
        M, N = 4096, 4096
        dd = synth.w4a16_inputs(M, K, N, GROUP, tag=3 if K == 4096 else 4)
        t = {k: torch.from_numpy(v).to(dev) for k, v in dd.items()}
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        log(f"prefill: {name}")
        ws = torch.empty(max(mq.w4a16_gemm_workspace_bytes(M, N, K, GROUP), 16), dtype=torch.uint8, device=dev)
        tg = time_fn(lambda: mq.w4a16_gemm(t["x"], t["qweight"], t["scales"], t["qzeros"], GROUP, out=y,
                                           workspace=ws))
        ops = 2.0 * M * N * K
        out[name] = {"shape": [M, N, K], "gemm_us": tg * 1e6, "gemm_TFLOPS": ops / tg / 1e12,
                     "gemm_frac_fp16_peak": ops / tg / 1e12 / FP16_PEAK_TFLOPS}
        del t, y
    # bf16 activations: the o_proj-shaped prefill GEMM (bf16 MFMA, same peak as fp16)
    M, N, K = 4096, 4096, 4096
    db = synth.w4a16_inputs_bf16(M, K, N, GROUP, tag=3)
    xb = torch.from_numpy(db["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    t = {k: torch.from_numpy(db[k]).to(dev) for k in ("qweight", "scales", "qzeros")}
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    log("prefill: w4a16_c3a_bf16")
    tg = time_fn(lambda: mq.w4a16_gemm(xb, t["qweight"], t["scales"], t["qzeros"], GROUP, out=yb))
    ops = 2.0 * M * N * K
    out["w4a16_c3a_bf16"] = {"shape": [M, N, K], "gemm_us": tg * 1e6, "gemm_TFLOPS": ops / tg / 1e12,
                             "gemm_frac_bf16_peak": ops / tg / 1e12 / FP16_PEAK_TFLOPS}
    return out


def bench_layers(torch, mq, synth, args, log):
    """The linear layers of an 8B-shaped decoder layer at decode batches 1, 8, 64 and a
    2048-token prefill, under W4A16 (decode-layout GEMV for M <= 64, GEMM above) and
    W8A8_INT8 (mq_w8a8_linear: one fused kernel for M <= 16, quantize + scaled GEMM
    above). Weights rotate over copies totalling >= 640 MB per layer so every call
    reads them from HBM; times are per call from event-timed graph replays. `set` is
    the four layers of one scheme captured together in one graph (qkv, o_proj,
    gate_up, down in a row, as a decoder layer issues them)."""
    dev = torch.device("cuda", 0)
    R = 20
    out = {"w4a16": {}, "w8a8": {}, "set": {"w4a16": {}, "w8a8": {}}}

    def time_calls(fn):
        g = capture(torch, lambda: [fn(r) for r in range(R)])
        g.replay()
        best = min(timed_replay(torch, g)[1] for _ in range(3))
        return best / R

    def copies(tensors, nbytes):
        n = max(2, -(-640 * 2**20 // nbytes))
        return [tensors] + [{k: v.clone() for k, v in tensors.items()} for _ in range(n - 1)]

    fns = {"w4a16": {}, "w8a8": {}}  # scheme -> M -> [per-layer fn]
    keep = []
    for li, (name, shp) in enumerate(synth.LAYER_SET.items()):
        K, N = shp["K"], shp["N"]
        log(f"layers: {name} K={K} N={N}")
        w = synth.w4a16_weights(K, N, GROUP, tag=300 + li)
        w = {k: torch.from_numpy(v).to(dev) for k, v in w.items()}
        w["qblocked"] = mq.w4a16_block_weights(w["qweight"])
        wsets = copies(w, K * N // 2)
        keep.append(wsets)
        del w
        out["w4a16"][name] = {}
        for M in synth.LAYER_SET_MS:
            x = torch.from_numpy(synth.w4a16_inputs(M, K, 8, GROUP, outlier_frac=0.005, tag=310 + li,
                                                    seed=M)["x"]).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            if M <= mq.GEMV_MAX_M:
                ws = torch.zeros(max(mq.w4a16_gemv_blocked_workspace_bytes(M, N, K, GROUP), 16), dtype=torch.uint8,
                                 device=dev)

                def fn(r, x=x, y=y, ws=ws, wsets=wsets):
                    s = wsets[r % len(wsets)]
                    mq.w4a16_gemv_blocked(x, s["qblocked"], s["scales"], s["qzeros"], GROUP, out=y, workspace=ws)
            else:
                ws = torch.empty(max(mq.w4a16_gemm_workspace_bytes(M, N, K, GROUP), 16), dtype=torch.uint8,
                                 device=dev)

                def fn(r, x=x, y=y, wsets=wsets, ws=ws):
                    s = wsets[r % len(wsets)]
                    mq.w4a16_gemm(x, s["qweight"], s["scales"], s["qzeros"], GROUP, out=y, workspace=ws)
            fns["w4a16"].setdefault(M, []).append(fn)
            t = time_calls(fn)
            nbytes = w4a16_bytes(M, K, N)
            out["w4a16"][name][str(M)] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                                          "TFLOPS": round(2.0 * M * N * K / t / 1e12, 1)}

        d = synth.w8a8_inputs(8, K, N, outlier_frac=0.01, tag=320 + li)
        wq, s_ch = mq.quant_per_token_int8(torch.from_numpy(d["wf"]).to(dev))
        qsets = copies({"wq": wq, "s_ch": s_ch}, K * N)
        keep.append(qsets)
        del wq, s_ch
        out["w8a8"][name] = {}
        for M in synth.LAYER_SET_MS:
            x = torch.from_numpy(synth.w8a8_inputs(M, K, 8, outlier_frac=0.01, tag=330 + li, seed=M)["x"]).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = torch.empty(max(mq.w8a8_linear_workspace_bytes(M, K), 16), dtype=torch.uint8, device=dev)

            def fn(r, x=x, y=y, ws=ws, qsets=qsets):
                s = qsets[r % len(qsets)]
                mq.w8a8_linear(x, s["wq"], s["s_ch"], out=y, workspace=ws)
            fns["w8a8"].setdefault(M, []).append(fn)
            t = time_calls(fn)
            nbytes = M * K * 2 + K * N + N * 4 + M * N * 2
            out["w8a8"][name][str(M)] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                                         "TOPS": round(2.0 * M * N * K / t / 1e12, 1)}
    for scheme in ("w4a16", "w8a8"):
        for M in synth.LAYER_SET_MS:
            log(f"layers: {scheme} set M={M}")
            t = time_calls(lambda r, fl=fns[scheme][M]: [f(r) for f in fl])
            out["set"][scheme][str(M)] = round(t * 1e6, 2)
    del fns, keep
    torch.cuda.empty_cache()
    return out


def bench_groups(torch, mq, synth, log):
    """W4A16 with groups of 64 and 32 rows and with per-channel parameters
    (group -1, reported as "per_channel"): GEMV and GEMM shapes, cold weights
    (copies totalling >= 640 MB), microseconds per call from graph replays."""
    dev = torch.device("cuda", 0)
    R = 20

    def time_calls(fn):
        g = capture(torch, lambda: [fn(r) for r in range(R)])
        g.replay()
        best = min(timed_replay(torch, g)[1] for _ in range(3))
        return best / R

    out = {}
    shapes = [("gate_up", 4096, 24576, (1, 4, 16)), ("vit_qkv", 1024, 3072, (1, 16, 577, 4096)),
              ("o_proj_prefill", 4096, 4096, (4096,))]
    for G in (64, 32, -1):
        key = "per_channel" if G == -1 else f"g{G}"
        out[key] = {}
        for name, K, N, Ms in shapes:
            log(f"groups: G={G} {name} K={K} N={N}")
            w = {k: torch.from_numpy(v).to(dev) for k, v in synth.w4a16_weights(K, N, G, tag=400 + abs(G)).items()}
            w["qblocked"] = mq.w4a16_block_weights(w["qweight"])
            wbytes = K * N // 2
            n = max(2, -(-640 * 2**20 // wbytes))
            wsets = [w] + [{k: v.clone() for k, v in w.items()} for _ in range(n - 1)]
            del w
            res = {}
            for M in Ms:
                x = torch.from_numpy(synth.w4a16_inputs(M, K, 8, G, outlier_frac=0.005 if M <= 64 else 0.0,
                                                        tag=410 + abs(G), seed=M)["x"]).to(dev)
                y = torch.empty((M, N), dtype=torch.float16, device=dev)
                if M <= mq.GEMV_MAX_M:
                    ws = torch.zeros(max(mq.w4a16_gemv_blocked_workspace_bytes(M, N, K, G), 16), dtype=torch.uint8,
                                     device=dev)

                    def fn(r, x=x, y=y, ws=ws):
                        s = wsets[r % len(wsets)]
                        mq.w4a16_gemv_blocked(x, s["qblocked"], s["scales"], s["qzeros"], G, out=y, workspace=ws)
                else:
                    ws = torch.empty(max(mq.w4a16_gemm_workspace_bytes(M, N, K, G), 16), dtype=torch.uint8,
                                     device=dev)

                    def fn(r, x=x, y=y, ws=ws):
                        s = wsets[r % len(wsets)]
                        mq.w4a16_gemm(x, s["qweight"], s["scales"], s["qzeros"], G, out=y, workspace=ws)
                t = time_calls(fn)
                nbytes = w4a16_bytes(M, K, N, G)
                flops = 2.0 * M * N * K
                res[str(M)] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                               "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4),
                               "TFLOPS": round(flops / t / 1e12, 1),
                               "fp16_frac": round(flops / t / 1e12 / FP16_PEAK_TFLOPS, 4)}
            out[key][name] = res
            del wsets
            torch.cuda.empty_cache()
    return out


def bench_kv_quant(torch, mq, log):
    """Online KV-cache quantization of one layer's K (or V): a 4096-token prefill
    and a 128-sequence decode append, 32 heads x 128, INT8 and INT4. The prefill
    rotates over copies totalling >= 320 MB, so x comes from HBM."""
    import numpy as np
    dev = torch.device("cuda", 0)
    R = 20
    out = {}

    def time_calls(fn):
        g = capture(torch, lambda: [fn(r) for r in range(R)])
        g.replay()
        best = min(timed_replay(torch, g)[1] for _ in range(3))
        return best / R

    rng = np.random.default_rng(77)
    for name, T in (("prefill_4096", 4096), ("decode_128seq", 128)):
        shape = (T, 32, 128)
        x0 = torch.from_numpy(rng.standard_normal(shape).astype(np.float16)).to(dev)
        nbytes_x = x0.numel() * 2
        n = max(2, -(-320 * 2**20 // nbytes_x)) if T > 1024 else 2
        xs = [x0] + [x0.clone() for _ in range(n - 1)]
        rows = T * 32
        for bits in (8, 4):
            codes = torch.empty((T, 32, 128 if bits == 8 else 64), dtype=torch.uint8, device=dev)
            params = torch.empty((T, 32, 2), dtype=torch.float32, device=dev)
            log(f"kv_quant: {name} bits={bits}")
            t = time_calls(lambda r, codes=codes, params=params: mq.kv_quant(xs[r % n], bits, codes=codes,
                                                                             params=params))
            nbytes = rows * 128 * 2 + rows * 128 * bits // 8 + rows * 8
            out[f"{name}_int{bits}"] = {"rows": rows, "head_dim": 128, "us": round(t * 1e6, 2),
                                        "GBps": round(nbytes / t / 1e9, 1),
                                        "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4)}
        del xs
        torch.cuda.empty_cache()
    return out


def bench_checkpoint(torch, mq, log):
    """One-time checkpoint-layout conversions at the 8B gate_up size: an
    AWQ-order qweight [4096, 3072] words reordered, a K-packed [24576, 512]
    transposed to [4096, 3072], and scales [24576, 32] transposed. Each is
    run 20 times in a graph (the same buffers: warm), microseconds per call
    and GB/s of read + write."""
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    w_kn = torch.randint(-2 ** 31, 2 ** 31 - 1, (4096, 3072), dtype=torch.int32, device=dev, generator=g)
    w_nk = torch.randint(-2 ** 31, 2 ** 31 - 1, (24576, 512), dtype=torch.int32, device=dev, generator=g)
    s_nk = torch.rand((24576, 32), device=dev, generator=g).half()
    o1, o2 = torch.empty_like(w_kn), torch.empty((4096, 3072), dtype=torch.int32, device=dev)
    o3 = torch.empty((32, 24576), dtype=torch.float16, device=dev)
    R = 20
    out = {}
    for name, fn, nbytes in (
            ("int4_reorder_4096x3072", lambda: mq.int4_reorder(w_kn, mq.AWQ_FIELD_ORDER, out=o1), 2 * w_kn.numel() * 4),
            ("int4_transpose_24576x4096", lambda: mq.int4_transpose(w_nk, mq.AWQ_FIELD_ORDER, out=o2),
             2 * w_nk.numel() * 4),
            ("u16_transpose_24576x32", lambda: mq.u16_transpose(s_nk, out=o3), 2 * s_nk.numel() * 2)):
        log(f"checkpoint: {name}")
        gr = capture(torch, lambda fn=fn: [fn() for _ in range(R)])
        gr.replay()
        t = min(timed_replay(torch, gr)[1] for _ in range(3)) / R
        out[name] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1)}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, log):
    """The oracle on one step of the headline workload (one weight set), on the
    host cores this process may run on: BLAS threads = len(sched_getaffinity),
    then again with one thread. Each leg repeats the step for about
    --cpu-seconds / 2 (at least once)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import synth
    affinity = len(os.sched_getaffinity(0))
    w = synth.w4a16_weights(GEMV_K, GEMV_N, GROUP, tag=1, seed=1000)
    xs = {M: synth.w4a16_inputs(M, GEMV_K, 8, GROUP, outlier_frac=0.005, tag=1, seed=M)["x"] for M in GEMV_MS}
    step_bytes = sum(w4a16_bytes(M, GEMV_K, GEMV_N) for M in GEMV_MS)

    def leg(threads):
        with threadpool_limits(limits=threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            reps, t_total = 0, 0.0
            while True:
                t0 = time.perf_counter()
                for M in GEMV_MS:
                    y = oracle.w4a16_ref(xs[M], w["qweight"], w["scales"], w["qzeros"], GROUP)
                    assert np.all(np.isfinite(y))
                t_total += time.perf_counter() - t0
                reps += 1
                if t_total >= args.cpu_seconds / 2 or reps >= 20:
                    break
        log(f"cpu baseline: {reps} steps in {t_total:.1f} s with {used} BLAS thread(s)")
        return step_bytes * reps / t_total / 1e9, used, reps, t_total

    v_all, used_all, reps_all, t_all = leg(affinity)
    v_one, _, reps_one, t_one = leg(1)
    return {"value": round(v_all, 4), "unit": "GB/s", "cores": used_all, "kind": "oracle",
            "sample": f"{reps_all} step(s) of the headline workload (M=1,4,16 against one 52 MB weight set) in "
                      f"{t_all:.1f} s; NumPy unpack/dequant single-threaded, float64 BLAS matmul on "
                      f"{used_all} thread(s)",
            "cpu_model": cpu_model(), "affinity_cores": affinity,
            "single_thread": {"value": round(v_one, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{reps_one} step(s) in {t_one:.1f} s"}}


def bench_fp16_context(torch, synth, log):
    """Context only: torch.matmul in fp16 (hipBLASLt) at the headline decode
    shapes (weights [K, N] fp16, two rotating 201 MB copies so each call reads
    HBM) and at the two W4A16 prefill shapes, microseconds per call from graph
    replays; for the 4-bit vs fp16 ratio the pages quote for whole models."""
    dev = torch.device("cuda", 0)
    R = 20
    out = {}

    def time_calls(fn):
        g = capture(torch, lambda: [fn(r) for r in range(R)])
        g.replay()
        return min(timed_replay(torch, g)[1] for _ in range(3)) / R

    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    ws = [(torch.randn((GEMV_K, GEMV_N), device=dev, generator=gen) * 0.02).half() for _ in range(2)]
    for M in GEMV_MS:
        x = torch.from_numpy(synth.w4a16_inputs(M, GEMV_K, 8, GROUP, outlier_frac=0.005, tag=1, seed=M)["x"]).to(dev)
        y = torch.empty((M, GEMV_N), dtype=torch.float16, device=dev)
        log(f"fp16 context: matmul M={M} K={GEMV_K} N={GEMV_N}")
        t = time_calls(lambda r, x=x, y=y: torch.matmul(x, ws[r % 2], out=y))
        nbytes = M * GEMV_K * 2 + GEMV_K * GEMV_N * 2 + M * GEMV_N * 2
        out[f"decode_M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1)}
    del ws
    for name, K in (("prefill_c3a", 4096), ("prefill_c3b", 12288)):
        M, N = 4096, 4096
        x = (torch.randn((M, K), device=dev, generator=gen)).half()
        w = (torch.randn((K, N), device=dev, generator=gen) * 0.02).half()
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        log(f"fp16 context: matmul {name}")
        t = time_calls(lambda r, x=x, w=w, y=y: torch.matmul(x, w, out=y))
        out[name] = {"us": round(t * 1e6, 2), "TFLOPS": round(2.0 * M * N * K / t / 1e12, 1)}
        del x, w, y
    torch.cuda.empty_cache()
    return out


def load_traffic(launch_bytes):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("source_hash") != gemv_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


PREFILL_SOURCES = {"w8a8_c2": ["w8a8_gemm.hip", "device_common.h", "launch.h"],
                   "w4a16_c3a": ["w4a16_gemm.hip", "w4a16_common.h", "device_common.h", "launch.h"],
                   "w4a16_c3b": ["w4a16_gemm.hip", "w4a16_common.h", "device_common.h", "launch.h"]}


def source_hash(files):
    from weight_activation_quantized_amd import _build
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "weight_activation_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(repr(_build.FLAGS[:-2]).encode())
    return h.hexdigest()[:16]


def prefill_roofline(prefill):
    """Roofline objects for the prefill GEMMs: achieved = 2MNK per launch /
    event-timed average launch duration, against the dense MFMA peak of the
    kernel's operand type; `traffic` and MFMA-busy from the committed counter
    summary while it matches the kernel's sources, else null."""
    counters = {}
    if os.path.exists(PREFILL_TRAFFIC_FILE):
        with open(PREFILL_TRAFFIC_FILE) as f:
            counters = json.load(f).get("kernels", {})
    out = {}
    for key, kernel, peak, unit in (("w8a8_c2", "w8a8_gemm_kernel<true, false>", INT8_PEAK_TOPS, "TOP/s"),
                                    ("w4a16_c3a", "w4a16_gemm_kernel<4, false>", FP16_PEAK_TFLOPS, "TFLOP/s"),
                                    ("w4a16_c3b", "w4a16_gemm_kernel<4, false>", FP16_PEAK_TFLOPS, "TFLOP/s")):
        p = prefill.get(key)
        if not p:
            continue
        M, N, K = p["shape"]
        ach = p.get("gemm_TOPS", p.get("gemm_TFLOPS"))
        c = counters.get(key, {})
        fresh = c.get("source_hash") == source_hash(PREFILL_SOURCES[key])
        out[key] = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": unit,
                    "frac": round(ach / peak, 4),
                    "traffic": c.get("hbm_bytes_per_launch") if fresh else None,
                    "mfma_busy": c.get("mfma_busy") if fresh else None,
                    "kernel": kernel, "avg_launch_us": round(p["gemm_us"], 3),
                    "algorithmic_ops_per_launch": 2 * M * N * K}
    return out


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on one GPU only; "
                                   "the layer's shards are the single-GPU kernels at smaller N or K"}))
        return 2
    rank = int(os.environ.get("RANK", "0"))

    def log(msg):
        sys.stderr.write(f"[bench] {msg}\n")
        sys.stderr.flush()

    import torch

    import synth
    import weight_activation_quantized_amd as mq

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    mq.library()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)

    res, sets, xs = bench_gemv(torch, mq, synth, args, log)
    if args.copy_kernel:
        a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    del sets
    torch.cuda.empty_cache()

    ms_per_step = res["wall_s"] / args.steps * 1e3
    value = res["step_bytes"] / (res["wall_s"] / args.steps) / 1e9
    achieved = res["bytes_per_launch_avg"] / (res["kernel_avg_us"] * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "W4A16 decode GEMV (8B MLP gate+up): M in {1,4,16}, K=4096, N=24576, group 128; "
                        f"{args.sets} rotating weight sets (cold HBM); one step = one GEMV per M; weights in the "
                        "decode layout (converted once before timing)",
            "M": list(GEMV_MS), "K": GEMV_K, "N": GEMV_N, "group": GROUP, "weight_sets": args.sets,
            "gemv_workspace_bytes": res["workspace_bytes"], "parallelism": "single GPU",
            "w8a8_weights": W8A8_WEIGHTS,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(res["bytes_per_launch_avg"]),
            "kernel": "w4a16_gemv_blocked_kernel (one launch per call; K is not split at N=24576)",
            "avg_launch_us": round(res["kernel_avg_us"], 3),
            "algorithmic_bytes_per_launch": res["bytes_per_launch_avg"],
        },
        "gemv_awq_layout": res["awq_layout"],
        "gemv_bf16": res["bf16"],
    }
    if not args.no_prefill:
        line["prefill"] = bench_prefill(torch, mq, synth, mq.quant_per_token_int8, args, log)
        line["roofline_prefill"] = prefill_roofline(line["prefill"])
    if not args.no_fp16_context:
        line["fp16_matmul_context"] = bench_fp16_context(torch, synth, log)
    if not args.no_layers:
        line["layers"] = bench_layers(torch, mq, synth, args, log)
    if not args.no_groups:
        line["groups"] = bench_groups(torch, mq, synth, log)
    if not args.no_kv:
        line["kv_quant"] = bench_kv_quant(torch, mq, log)
    if not args.no_checkpoint:
        line["checkpoint"] = bench_checkpoint(torch, mq, log)
    if not args.no_cpu_baseline and rank == 0:
        line["cpu_baseline"] = cpu_baseline(args, log)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
