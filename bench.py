#!/usr/bin/env python3
"""Throughput of the fused dequant-matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

One step = the Whisper large-v3-turbo decoder GEMV set at M=1 in NF4 with
double-quant: the fused Q/K/V projection (one wq_matmul_qkv, 3840x1280), the
out-projection (1280x1280), fc1 (5120x1280) and fc2 (1280x5120).  Steps cycle
through a pool of weight copies of >= 1 GiB so every step streams its weights
from HBM (the 256 MB Infinity Cache cannot hold them); the launches of all pool
slots are captured once in a HIP graph and replayed.  `value` is weight bytes
(codes + scales) per second over exactly K timed steps.

Also reported (same JSON line): the encoder GEMM at M=1500 in NVFP4 (fc1 + fc2,
TFLOP/s), the same GEMMs as NVFP4 W4A4 (runtime-quantized activations), one
encoder layer at batch 4 (M=6000) in q8_0 and q4_0, the decode
set at M=4 and M=16, a 433 MB streaming GEMV (NF4+DQ, M=1), the dominant
kernels' roofline fractions, an unfused ablation (dequantize, cast, library
GEMM) and a dense bf16 GEMM at the encoder and decode shapes, and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA
DECODER = [("qkv", 3840, 1280), ("out", 1280, 1280), ("fc1", 5120, 1280), ("fc2", 1280, 5120)]
ENC_D, ENC_FFN, ENC_M = 1280, 5120, 1500


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=416)
    ap.add_argument("--warmup", type=int, default=104)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="only the decode set (for profiling)")
    ap.add_argument("--encoder-only", action="store_true",
                    help="only the encoder GEMMs (NVFP4, M=1500), for MFMA counter runs")
    ap.add_argument("--stream-only", action="store_true",
                    help="only the 433 MB streaming GEMV (for profiling)")
    ap.add_argument("--w4a4-only", action="store_true",
                    help="only the NVFP4 W4A4 encoder GEMMs (M=1500), for profiling")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_bit_amd import wq
    from block_quantized_bit_amd.inputs import linear_case

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()          # default priority

    def quantize_dev(fmt, w_dev, dq):
        n, k = w_dev.shape
        d = wq.desc(fmt, n, k, dq)
        cb, sb = wq.wq_packed_size(d)
        codes = torch.empty(cb, dtype=torch.uint8, device=dev)
        scales = torch.empty(sb, dtype=torch.uint8, device=dev)
        wq.wq_quantize(d, w_dev, codes, scales)
        return d, codes, scales

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    # plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
    cal = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()

    # a device copy of 512 MiB each way (1 GiB of traffic) evicts the 256 MB Infinity Cache
    flush_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    timing_info = {}

    def capture(enqueue, n_slots, count, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            enqueue(start % n_slots, stream)            # untimed eager pass before capture
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for s in range(count):
                    enqueue((start + s) % n_slots, stream)
        return g

    def run_graph_steps(enqueue, n_slots, steps, warmup, per_graph=None):
        """Time `steps` steps replayed from captured HIP graphs; step s of the run uses slot
        s % n_slots of a weight pool.  Warmup runs steps 0 .. warmup-1, the timed steps are
        warmup .. warmup+steps-1 (graphs of one full cycle of the pool, or of `per_graph`
        steps, then the remainder).  Every timed graph is replayed once before the warmup (its
        first launch uploads it), and for a pool of several slots a 1 GiB device copy runs
        between the warmup and the timed steps, so the timed steps start with none of their
        weights in the Infinity Cache whatever `steps` and `warmup` are; within the timed steps
        a slot is read again only after the whole pool.  After the copy one step runs on the slot
        before the first timed one, so that only the timed weights are cold.  Returns seconds for
        the timed steps."""
        per = per_graph or n_slots
        start = warmup % n_slots
        full, rest = divmod(steps, per)
        timed = []
        if full:
            timed.append((capture(enqueue, n_slots, per, start), full))
        if rest:
            timed.append((capture(enqueue, n_slots, rest, start + full * per), 1))
        for g, _ in timed:
            g.replay()
        if warmup:
            wg = capture(enqueue, n_slots, min(warmup, per), 0)
            for _ in range(-(-warmup // per)):
                wg.replay()
        torch.cuda.synchronize()
        cold = n_slots > 1
        if cold:
            flush_dst.copy_(flush_src)
            # one step on the slot just before the first timed one: what every step shares (X, Y,
            # workspaces, the kernels' code, page-table entries) is warm again, as in a running
            # decoder, while the timed slots' weights stay cold (for steps < n_slots that slot is
            # not timed; otherwise it is read again only after the whole pool)
            with torch.cuda.stream(stream):
                enqueue((start - 1) % n_slots, stream)
            torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            # A device-side spin ahead of the start event keeps the GPU busy while the host
            # submits the start event and the graphs, so the timed region holds device work
            # only (a serving loop submits the next step while the current one runs).
            spin = hasattr(torch.cuda, "_sleep")
            if spin:
                torch.cuda._sleep(2_000_000)
            ev0.record(stream)
            for g, reps in timed:
                for _ in range(reps):
                    g.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        timing_info.clear()
        timing_info.update({"slots": n_slots, "timed_first_slot": start,
                            "cold": ("1 GiB device copy between warmup and the timed steps; a slot is re-read only "
                                     "after the whole pool; the shared buffers warmed by one step on the slot "
                                     "before the first timed one") if cold else "one weight set, reused (not cold)",
                            "host_submission": ("outside the timed region: the graphs are queued behind a device-side "
                                                "spin before the start event") if spin else "inside the timed region"})
        return ev0.elapsed_time(ev1) / 1e3

    def sclk_mhz():
        """Current shader clock from the driver's table (the entry marked '*'), or None."""
        import glob
        for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
            try:
                for line in open(f):
                    if line.strip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
            except (OSError, ValueError, IndexError):
                continue
        return None

    def enc_step(s_, st, layers, m):
        for e in layers:
            wq.wq_matmul(e["d"], m, e["x"], e["k"], e["c"], e["s"], e["b"], e["y"], wq.WQ_BF16, e["n"],
                         e["ws"] if e["nb"] else None, e["nb"], stream=st)

    def encoder_part():
        # ---- encoder GEMM, NVFP4, M = 1500: fc1 + fc2 ----
        enc = []
        enc_cases = []
        for i, (n, k) in enumerate([(ENC_FFN, ENC_D), (ENC_D, ENC_FFN)]):
            w, b, x = linear_case(3000 + i, n, k, ENC_M, row_lognormal_sigma=0.3)
            enc_cases.append((w, b, x))
            d, c, s = quantize_dev(wq.WQ_NVFP4, torch.from_numpy(w).to(dev), False)
            nb = wq.wq_workspace_size(d, ENC_M)
            enc.append(dict(d=d, c=c, s=s, b=bf16_dev(b), x=bf16_dev(x), n=n, k=k,
                            y=torch.empty((ENC_M, n), dtype=torch.int16, device=dev),
                            ws=torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev), nb=nb))

        reps = 50
        # ten steps per captured graph, so that graph launches do not count against the kernels
        te = run_graph_steps(lambda s_, st: enc_step(s_, st, enc, ENC_M), 1, reps, 10, per_graph=10)
        mhz = sclk_mhz()
        flops = sum(2.0 * ENC_M * e["n"] * e["k"] for e in enc)
        tflops = flops * reps / te / 1e12
        encoder = {
            "metric": "encoder TFLOP/s (M=1500)",
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "config": {"workload": "encoder fc1 1280->5120 and fc2 5120->1280, NVFP4 W4A16, X[1500,1280] bf16"},
            "us_per_step": round(te * 1e6 / reps, 2),
            "roofline": {"kernel": "k_gemm<NVFP4>", "bound": "mfma", "achieved": round(tflops, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("encoder_nvfp4_m1500", "traffic_bytes_per_step"),
                         "traffic_per": "step (fc1 + fc2 + K-split reduce)",
                         "algorithmic_bytes_per_step": sum(e["c"].numel() + e["s"].numel() + 2 * ENC_M * (e["k"] + e["n"])
                                                           + 2 * e["n"] for e in enc),
                         # the same against the dense peak at the shader clock the driver reported right
                         # after the timed steps (256 CUs x 4096 bf16 flop per clock); null if unreadable
                         "sclk_mhz": mhz,
                         "peak_at_sclk": round(256 * 4096 * mhz * 1e6 / 1e12, 1) if mhz else None,
                         "frac_at_sclk": round(tflops / (256 * 4096 * mhz * 1e6 / 1e12), 4) if mhz else None},
        }
        if not args.no_cpu:
            encoder["cpu_baseline"] = cpu_baseline_encoder(enc_cases)
        log(f"[bench] encoder NVFP4 M=1500: {encoder['us_per_step']} us, {tflops:.1f} TFLOP/s")
        encoder_part.layers = enc
        return encoder

    def w4a4_part(w4a16_us=None):
        """NVFP4 W4A4 at the encoder shape: fc1 (1280 -> 5120) and fc2 (5120 -> 1280) on
        X[1500, *] with activations quantized at run time.  Timed twice: the two
        wq_matmul_w4a4 calls on activations already packed (their producer quantizes them),
        and the whole W4A4 step with wq_quantize_act of each input in front."""
        lay = []
        for i, (n, k) in enumerate([(ENC_FFN, ENC_D), (ENC_D, ENC_FFN)]):
            w, b, x = linear_case(3000 + i, n, k, ENC_M, row_lognormal_sigma=0.3)
            d, c, s = quantize_dev(wq.WQ_NVFP4, torch.from_numpy(w).to(dev), False)
            cb, sb = wq.wq_act_packed_size(ENC_M, k)
            nb = wq.wq_w4a4_workspace_size(d, ENC_M)
            e = dict(d=d, c=c, s=s, b=bf16_dev(b), x=bf16_dev(x), n=n, k=k,
                     xc=torch.empty(cb, dtype=torch.uint8, device=dev), xs=torch.empty(sb, dtype=torch.uint8, device=dev),
                     y=torch.empty((ENC_M, n), dtype=torch.int16, device=dev),
                     ws=torch.zeros(nb, dtype=torch.uint8, device=dev), nb=nb)
            wq.wq_quantize_act(ENC_M, k, e["x"], k, e["xc"], e["xs"])
            lay.append(e)
        torch.cuda.synchronize()

        def mm_step(s_, st):
            for e in lay:
                wq.wq_matmul_w4a4(e["d"], ENC_M, e["xc"], e["xs"], e["c"], e["s"], e["b"], e["y"], wq.WQ_BF16, e["n"],
                                  e["ws"], e["nb"], stream=st)

        def full_step(s_, st):
            for e in lay:
                wq.wq_quantize_act(ENC_M, e["k"], e["x"], e["k"], e["xc"], e["xs"], stream=st)
                wq.wq_matmul_w4a4(e["d"], ENC_M, e["xc"], e["xs"], e["c"], e["s"], e["b"], e["y"], wq.WQ_BF16, e["n"],
                                  e["ws"], e["nb"], stream=st)

        def act_step(s_, st):
            for e in lay:
                wq.wq_quantize_act(ENC_M, e["k"], e["x"], e["k"], e["xc"], e["xs"], stream=st)

        reps = 50
        flops = sum(2.0 * ENC_M * e["n"] * e["k"] for e in lay)
        tm = run_graph_steps(mm_step, 1, reps, 10, per_graph=10)
        tf = run_graph_steps(full_step, 1, reps, 10, per_graph=10)
        ta = run_graph_steps(act_step, 1, reps, 10, per_graph=10)
        tfl_m = flops * reps / tm / 1e12
        out = {
            "config": {"workload": "encoder fc1 1280->5120 and fc2 5120->1280, NVFP4 W4A4, X[1500,*] quantized "
                                   "per 16 values at run time"},
            "matmul_us_per_step": round(tm * 1e6 / reps, 2),
            "TFLOPs": round(tfl_m, 2),
            "frac_bf16_peak": round(tfl_m / BF16_PEAK_TFLOPS, 4),
            "frac_fp4_peak": round(tfl_m / FP4_PEAK_TFLOPS, 4),
            "contraction_unit": "bf16 MFMA on exact e2m1*E4M3 expansions (E4M3 per 16 has no exact form on the "
                                "E8M0-per-32 fp4 MFMA)",
            "with_act_quant_us_per_step": round(tf * 1e6 / reps, 2),
            "TFLOPs_with_act_quant": round(flops * reps / tf / 1e12, 2),
            "act_quant_us_per_step": round(ta * 1e6 / reps, 2),
        }
        if w4a16_us:
            out["over_w4a16"] = round(tm * 1e6 / reps / w4a16_us, 3)
        log(f"[bench] w4a4: {out}")
        return out

    def streaming_part(by_format=False):
        """One launch streams 433 MB: the fc1 geometry (K = 1280) widened to N = 655360 rows,
        NF4 + double-quant, M = 1; 20 timed launches on one weight set (larger than the
        Infinity Cache, read in order, so every launch reads it from HBM).  by_format: the
        same matrix in every format as well (by_format key of the result)."""
        gen = torch.Generator(device=dev).manual_seed(7)
        ns, ks = 655360, 1280
        wbig = torch.randn((ns, ks), device=dev, generator=gen, dtype=torch.float32) * 0.02
        xs = bf16_dev(linear_case(9, 16, ks, 1)[2])
        ys = torch.empty((1, ns), dtype=torch.int16, device=dev)

        def one(fmt, dq):
            d_s, c_s, s_s = quantize_dev(fmt, wbig, dq)
            torch.cuda.synchronize()
            nbs = wq.wq_workspace_size(d_s, 1)
            wss_ = torch.zeros(max(nbs, 16), dtype=torch.uint8, device=dev)
            sbytes = c_s.numel() + s_s.numel()
            reps = 20
            ts = run_graph_steps(lambda s, st: wq.wq_matmul(d_s, 1, xs, ks, c_s, s_s, None, ys, wq.WQ_BF16, ns,
                                                            wss_ if nbs else None, nbs, stream=st), 1, reps, 5, per_graph=5)
            del c_s, s_s
            return {"bytes": sbytes, "us": round(ts * 1e6 / reps, 2), "GBps": round(sbytes * reps / ts / 1e9, 1),
                    "frac_hbm": round(sbytes * reps / ts / 1e9 / HBM_PEAK_GBS, 4)}

        out = {"shape": f"M=1 N={ns} K={ks} NF4+DQ", **one(wq.WQ_NF4, True)}
        log(f"[bench] streaming: {out}")
        if by_format:
            out["by_format"] = {}
            for name, fmt in (("nf4", wq.WQ_NF4), ("nvfp4", wq.WQ_NVFP4), ("q4_0", wq.WQ_Q4_0), ("q4_1", wq.WQ_Q4_1),
                              ("q5_0", wq.WQ_Q5_0), ("q4_k", wq.WQ_Q4_K), ("q6_k", wq.WQ_Q6_K), ("q8_0", wq.WQ_Q8_0)):
                out["by_format"][name] = one(fmt, False)
                torch.cuda.empty_cache()
            log(f"[bench] streaming by format: {out['by_format']}")
        del wbig
        torch.cuda.empty_cache()
        return out

    if args.encoder_only:
        print(json.dumps({"encoder": encoder_part()}), flush=True)
        return
    if args.w4a4_only:
        print(json.dumps({"w4a4": w4a4_part()}), flush=True)
        return
    if args.stream_only:
        print(json.dumps({"streaming_gemv": streaming_part()}), flush=True)
        return

    # ---------------- decode set: NF4 + double-quant, pool of weight copies ----------------
    t0 = time.time()
    base = []
    for i, (name, n, k) in enumerate(DECODER):
        w, b, x16 = linear_case(2000 + i, n, k, 16, outlier_frac=0.001)
        if name == "qkv":
            b = b.copy()
            b[1280:2560] = 0                      # key projection has no bias
        d, codes, scales = quantize_dev(wq.WQ_NF4, torch.from_numpy(w).to(dev), True)
        base.append(dict(name=name, n=n, k=k, d=d, codes=codes, scales=scales, bias=bf16_dev(b),
                         x16=bf16_dev(x16), w=w, b=b, xbits=x16))
    set_bytes = sum(e["codes"].numel() + e["scales"].numel() for e in base)
    pool_n = max(1, -(-(1 << 30) // set_bytes))               # >= 1 GiB of weights
    pool = [[(e["codes"].clone(), e["scales"].clone()) for e in base] for _ in range(pool_n)]
    torch.cuda.synchronize()
    log(f"[bench] decode set {set_bytes / 1e6:.3f} MB of packed weights, pool of {pool_n} copies "
        f"({pool_n * set_bytes / 2**30:.2f} GiB), built in {time.time() - t0:.1f}s")

    def decode_buffers(m):
        outs, wss = [], []
        for e in base:
            outs.append(torch.empty((m, e["n"]), dtype=torch.int16, device=dev))
            nb = wq.wq_workspace_size(e["d"], m)
            wss.append((torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev), nb))
        return outs, wss

    def enqueue_decode_step(m, slot, outs, wss, st):
        for j, e in enumerate(base):
            codes, scales = pool[slot][j]
            y = outs[j]
            ws, nb = wss[j]
            if e["name"] == "qkv":
                ys = [y.data_ptr(), y.data_ptr() + 2 * 1280, y.data_ptr() + 2 * 2560]
                wq.wq_matmul_qkv(e["d"], m, e["x16"], e["k"], codes, scales, e["bias"], [1280, 1280, 1280],
                                 ys, [e["n"]] * 3, wq.WQ_BF16, ws if nb else None, nb, stream=st)
            else:
                wq.wq_matmul(e["d"], m, e["x16"], e["k"], codes, scales, e["bias"], y, wq.WQ_BF16, e["n"],
                             ws if nb else None, nb, stream=st)

    def decode_bytes(m):
        """algorithmic bytes of one step: packed weights + X + Y (bf16) + bias"""
        return sum(e["codes"].numel() + e["scales"].numel() + 2 * m * e["k"] + 2 * m * e["n"] + 2 * e["n"]
                   for e in base)

    def ablation_part(enc, fused_enc_us, fused_dec_us):
        """The same Linears without fusion, for comparison (bench only, not part of the library):
        unfused = wq_dequantize to fp32, cast to bf16, then torch's GEMM (hipBLASLt);
        dense = torch's GEMM on the unquantized weights cast to bf16."""
        import torch.nn.functional as F
        out = {"how": "unfused: wq_dequantize -> fp32, cast to bf16, F.linear (hipBLASLt); "
                      "dense: F.linear on bf16 weights (no quantization); HIP graph replay"}
        # encoder, NVFP4, M = 1500
        for e in enc:
            e["w32"] = torch.empty((e["n"], e["k"]), dtype=torch.float32, device=dev)
            e["wq"] = torch.empty((e["n"], e["k"]), dtype=torch.bfloat16, device=dev)
            w, _, _ = linear_case(3000 + enc.index(e), e["n"], e["k"], ENC_M, row_lognormal_sigma=0.3)
            e["wd"] = torch.from_numpy(w).to(dev).to(torch.bfloat16)

        def enc_unfused(s_, st):
            for e in enc:
                wq.wq_dequantize(e["d"], e["c"], e["s"], e["w32"], stream=st)
                e["wq"].copy_(e["w32"])
                F.linear(e["x"].view(torch.bfloat16), e["wq"], e["b"].view(torch.bfloat16))

        def enc_dense(s_, st):
            for e in enc:
                F.linear(e["x"].view(torch.bfloat16), e["wd"], e["b"].view(torch.bfloat16))

        reps = 50
        tu = run_graph_steps(enc_unfused, 1, reps, 10, per_graph=10) * 1e6 / reps
        td = run_graph_steps(enc_dense, 1, reps, 10, per_graph=10) * 1e6 / reps
        out["encoder_nvfp4_m1500_fc1_fc2"] = {"fused_us": fused_enc_us, "unfused_us": round(tu, 2),
                                              "dense_bf16_us": round(td, 2),
                                              "unfused_over_fused": round(tu / fused_enc_us, 3),
                                              "fused_over_dense": round(fused_enc_us / td, 3)}
        for e in enc:
            del e["w32"], e["wq"], e["wd"]
        # decode set, NF4 + double-quant, M = 1: packed weights cycled over the >= 1 GiB pool as in the
        # fused step; the dense bf16 weights cycled over their own >= 1 GiB pool
        w32 = [torch.empty((e["n"], e["k"]), dtype=torch.float32, device=dev) for e in base]
        wqb = [torch.empty((e["n"], e["k"]), dtype=torch.bfloat16, device=dev) for e in base]
        x1 = [e["x16"][:1].view(torch.bfloat16) for e in base]
        bb = [e["bias"].view(torch.bfloat16) for e in base]

        def dec_unfused(slot, st):
            for j, e in enumerate(base):
                codes, scales = pool[slot][j]
                wq.wq_dequantize(e["d"], codes, scales, w32[j], stream=st)
                wqb[j].copy_(w32[j])
                F.linear(x1[j], wqb[j], bb[j])

        dense_bytes = sum(2 * e["n"] * e["k"] for e in base)
        dpool_n = max(1, -(-(1 << 30) // dense_bytes))
        dpool = [[torch.from_numpy(e["w"]).to(dev).to(torch.bfloat16) for e in base] for _ in range(dpool_n)]

        def dec_dense(slot, st):
            for j, e in enumerate(base):
                F.linear(x1[j], dpool[slot][j], bb[j])

        tu = run_graph_steps(dec_unfused, pool_n, pool_n * 2, pool_n) * 1e6 / (pool_n * 2)
        td = run_graph_steps(dec_dense, dpool_n, dpool_n * 4, dpool_n) * 1e6 / (dpool_n * 4)
        out["decode_nf4dq_m1_step"] = {"fused_us": round(fused_dec_us, 3), "unfused_us": round(tu, 2),
                                       "dense_bf16_us": round(td, 2),
                                       "unfused_over_fused": round(tu / fused_dec_us, 3),
                                       "fused_over_dense": round(fused_dec_us / td, 3)}
        del w32, wqb, dpool
        torch.cuda.empty_cache()
        log(f"[bench] unfused ablation: {out}")
        return out

    def decode_by_format():
        """The decode set (QKV as one wq_matmul_qkv, out, fc1, fc2; M = 1) quantized from the
        same fp32 weights in each format, each cycled over its own >= 1 GiB pool."""
        out = {}
        x1 = [e["x16"] for e in base]
        ys = [torch.empty((1, e["n"]), dtype=torch.int16, device=dev) for e in base]
        for name, fmt, dq in (("nf4", wq.WQ_NF4, False), ("nvfp4", wq.WQ_NVFP4, False),
                              ("q4_0", wq.WQ_Q4_0, False), ("q4_1", wq.WQ_Q4_1, False), ("q5_0", wq.WQ_Q5_0, False),
                              ("q4_k", wq.WQ_Q4_K, False), ("q6_k", wq.WQ_Q6_K, False), ("q8_0", wq.WQ_Q8_0, False)):
            mats = [quantize_dev(fmt, torch.from_numpy(e["w"]).to(dev), dq) for e in base]
            nbytes = sum(c.numel() + s_.numel() for _, c, s_ in mats)
            pn = max(1, -(-(1 << 30) // nbytes))
            fpool = [[(c.clone(), s_.clone()) for _, c, s_ in mats] for _ in range(pn)]

            def step(slot, st, mats=mats, fpool=fpool):
                for j, e in enumerate(base):
                    d = mats[j][0]
                    c, s_ = fpool[slot][j]
                    if e["name"] == "qkv":
                        p0 = ys[j].data_ptr()
                        wq.wq_matmul_qkv(d, 1, x1[j], e["k"], c, s_, e["bias"], [1280, 1280, 1280],
                                         [p0, p0 + 2 * 1280, p0 + 2 * 2560], [e["n"]] * 3, wq.WQ_BF16, stream=st)
                    else:
                        wq.wq_matmul(d, 1, x1[j], e["k"], c, s_, e["bias"], ys[j], wq.WQ_BF16, e["n"], stream=st)

            t = run_graph_steps(step, pn, pn * 2, pn) / (pn * 2)
            out[name] = {"us_per_step": round(t * 1e6, 2), "weight_bytes": nbytes,
                         "weight_GBps": round(nbytes / t / 1e9, 1)}
            del fpool, mats
            torch.cuda.empty_cache()
        log(f"[bench] decode M=1 by format: {out}")
        return out

    def quality_part():
        """Per format, on the same fp32 weights: the relative L2 error of one Linear's output
        against the unquantized fp32 product (a diagnostic of the format, not a gate), and
        the time of wq_quantize.  Matrices: decoder fc1 (5120 x 1280, 0.1 % outliers x 8) at
        M = 16 and encoder fc1 (5120 x 1280, per-row std from LogNormal(0, 0.3)) at M = 1500.
        The fp32 and bf16-weight references are torch matmuls in fp32 (TF32 off)."""
        torch.backends.cuda.matmul.allow_tf32 = False
        fmts = (("nf4", wq.WQ_NF4, False), ("nf4dq", wq.WQ_NF4, True), ("nvfp4", wq.WQ_NVFP4, False),
                ("q4_0", wq.WQ_Q4_0, False), ("q4_1", wq.WQ_Q4_1, False), ("q5_0", wq.WQ_Q5_0, False),
                ("q4_k", wq.WQ_Q4_K, False), ("q6_k", wq.WQ_Q6_K, False), ("q8_0", wq.WQ_Q8_0, False))
        cases = (("decoder_fc1_m16", linear_case(2002, ENC_FFN, ENC_D, 16, outlier_frac=0.001), 16),
                 ("encoder_fc1_m1500", linear_case(3000, ENC_FFN, ENC_D, ENC_M, row_lognormal_sigma=0.3), ENC_M))
        out = {"how": "rel_l2 = ||Y - Y_fp32|| / ||Y_fp32||, Y_fp32 = X W^T + b in fp32; "
                      "bf16_weights = the same with W rounded to bf16; quantize_us = one wq_quantize "
                      "(fp32 W in HBM), mean of 10 after a warm-up call"}
        for cname, (w, b, x), m in cases:
            n, k = w.shape
            W = torch.from_numpy(w).to(dev)
            X = bf16_dev(x)
            Xf = X.view(torch.bfloat16).float()
            Bf = bf16_dev(b).view(torch.bfloat16).float()
            ref = Xf @ W.t() + Bf
            nref = torch.linalg.vector_norm(ref).item()
            row = {"bf16_weights": round(torch.linalg.vector_norm(
                Xf @ W.to(torch.bfloat16).float().t() + Bf - ref).item() / nref, 6)}
            for name, fmt, dq in fmts:
                d, c, s_ = quantize_dev(fmt, W, dq)
                Y = torch.empty((m, n), dtype=torch.float32, device=dev)
                nb = wq.wq_workspace_size(d, m)
                ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
                wq.wq_matmul(d, m, X, k, c, s_, bf16_dev(b), Y, wq.WQ_F32, n, ws if nb else None, nb)
                rel = torch.linalg.vector_norm(Y - ref).item() / nref
                ent = {"rel_l2": round(rel, 6)}
                if cname == "decoder_fc1_m16":
                    with torch.cuda.stream(stream):
                        wq.wq_quantize(d, W, c, s_, stream=stream)
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for _ in range(10):
                            wq.wq_quantize(d, W, c, s_, stream=stream)
                        e1.record(stream)
                    torch.cuda.synchronize()
                    tq = e0.elapsed_time(e1) * 1e3 / 10
                    ent["quantize_us"] = round(tq, 1)
                    ent["quantize_GBps_fp32_in"] = round(n * k * 4 / tq / 1e3, 1)
                row[name] = ent
                del c, s_
            out[cname] = row
            del W
            torch.cuda.empty_cache()
        log(f"[bench] quality and quantize time: {out}")
        return out

    def sweep_part():
        """large-v3-turbo's 232 Linears as the export policy assigns them and its call plan
        groups them (block_quantized_bit_amd.policy, "nf4dq" requested: encoder q8_0, decoder
        NF4 + double-quant).  Per decoded token: 24 decoder calls (self-attention Q/K/V as one
        wq_matmul_qkv, self O, cross Q, cross O, fc1, fc2 per layer) at M = 1 and 16, cycled over a
        >= 1 GiB pool.  Once per utterance: the 4 cross-attention K/V calls (wq_matmul_qkv,
        2 splits, 2560 x 1280) at M = 1500 encoder frames, and the same 8 Linears as the plan's
        cross-layer merge (one wq_matmul, 10240 x 1280).  Encoder: 32 x {Q/K/V as one
        wq_matmul_qkv (3840 x 1280), O, fc1, fc2} = 128 calls at M = 1500 (668 MB of q8_0 weights,
        read from HBM on every pass).  Weights are drawn on the device from a seeded generator
        (only their shapes matter for timing); key projections have no bias."""
        from block_quantized_bit_amd import policy as P
        out = {}
        gen = torch.Generator(device=dev).manual_seed(5000)
        calls = P.plan(P.make_policy("nf4dq"))

        def make(c):
            w = torch.randn((c.n, c.k), device=dev, generator=gen, dtype=torch.float32) * 0.02
            d = P.fmt_desc(c.fmt, c.n, c.k)
            cb, sb = wq.wq_packed_size(d)
            cc = torch.empty(cb, dtype=torch.uint8, device=dev)
            ss = torch.empty(sb, dtype=torch.uint8, device=dev)
            wq.wq_quantize(d, w, cc, ss)
            bias = (torch.randn(c.n, device=dev, generator=gen) * 0.01).to(torch.bfloat16)
            col = 0
            for name, width in zip(c.names, c.split_n):
                if name.endswith(".k"):
                    bias[col:col + width] = 0
                col += width
            return dict(call=c, d=d, c=cc, s=ss, bias=bias)

        def enqueue(e, m, x, y, c_, s_, ws, nb, st):
            c = e["call"]
            if c.fused:
                p0 = y.data_ptr()
                offs = np.cumsum((0,) + c.split_n[:-1])
                wq.wq_matmul_qkv(e["d"], m, x, c.k, c_, s_, e["bias"], list(c.split_n),
                                 [p0 + 2 * int(o) for o in offs], [c.n] * len(c.split_n), wq.WQ_BF16,
                                 ws if nb else None, nb, stream=st)
            else:
                wq.wq_matmul(e["d"], m, x, c.k, c_, s_, e["bias"], y, wq.WQ_BF16, c.n, ws if nb else None, nb,
                             stream=st)

        # ---- per-token decoder calls, pooled ----
        dec = [make(c) for c in calls if c.rows == "tokens"]
        step_bytes = sum(e["c"].numel() + e["s"].numel() for e in dec)
        spool_n = max(1, -(-(1 << 30) // step_bytes))
        spool = [[(e["c"].clone(), e["s"].clone()) for e in dec] for _ in range(spool_n)]
        xk = {k: torch.randn((16, k), device=dev, generator=gen).to(torch.bfloat16) for k in (1280, 5120)}
        torch.cuda.synchronize()
        for m in (1, 16):
            ys = {n: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for n in (1280, 3840, 5120)}

            def dec_step(slot, st, m=m, ys=ys):
                for j, e in enumerate(dec):
                    c_, s_ = spool[slot][j]
                    enqueue(e, m, xk[e["call"].k], ys[e["call"].n], c_, s_, None, 0, st)

            t = run_graph_steps(dec_step, spool_n, spool_n * 2, spool_n) / (spool_n * 2)
            alg = step_bytes + sum(2 * m * (e["call"].k + e["call"].n) + 2 * e["call"].n for e in dec)
            out[f"decoder_step_m{m}"] = {"launches": len(dec), "linears": sum(len(e["call"].names) for e in dec),
                                         "us_per_step": round(t * 1e6, 2), "weight_bytes": step_bytes,
                                         "weight_GBps": round(step_bytes / t / 1e9, 1),
                                         "algorithmic_GBps": round(alg / t / 1e9, 1),
                                         "us_per_launch": round(t * 1e6 / len(dec), 3), "timing": dict(timing_info)}
            log(f"[bench] decoder step M={m}: {out[f'decoder_step_m{m}']}")
        del spool, dec
        torch.cuda.empty_cache()
        # the launch floor in the same setting: 24 one-element kernels per graph replay
        tiny = torch.zeros(1, device=dev)
        te_ = run_graph_steps(lambda s_, st: [tiny.add_(1.0) for _ in range(24)], 1, 20, 5, per_graph=5) / 20
        out["empty_launch_floor"] = {"launches": 24, "us_per_launch": round(te_ * 1e6 / 24, 3),
                                     "how": "24 one-element torch kernels per HIP graph step"}

        # ---- encoder-frame calls: cross-attention K/V (once per utterance) and the encoder ----
        xs = {k: torch.randn((ENC_M, k), device=dev, generator=gen).to(torch.bfloat16) for k in (1280, 5120)}
        ys = {n: torch.empty((ENC_M, n), dtype=torch.bfloat16, device=dev) for n in (1280, 2560, 3840, 5120, 10240)}
        merged = P.plan(P.make_policy("nf4dq"), merge_cross_kv=True)
        for key, plan_, sel, reps in (
                ("cross_kv_nf4dq_m1500", calls, lambda c: c.rows == "frames_once", 20),
                ("cross_kv_merged_nf4dq_m1500", merged, lambda c: c.rows == "frames_once", 20),
                ("encoder_sweep_q8_0_m1500", calls, lambda c: c.names[0].startswith("encoder"), 3)):
            lin = [make(c) for c in plan_ if sel(c)]
            for e in lin:
                e["nb"] = wq.wq_workspace_size(e["d"], ENC_M)
            wsz = max(e["nb"] for e in lin)
            wsb = torch.zeros(max(wsz, 16), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()

            def run_all(s_, st, lin=lin, wsb=wsb):
                for e in lin:
                    enqueue(e, ENC_M, xs[e["call"].k], ys[e["call"].n], e["c"], e["s"], wsb, e["nb"], st)

            t = run_graph_steps(run_all, 1, reps, 1, per_graph=1) / reps
            fl = sum(2.0 * ENC_M * e["call"].n * e["call"].k for e in lin)
            out[key] = {"launches": len(lin), "linears": sum(len(e["call"].names) for e in lin),
                        "us": round(t * 1e6, 1), "weight_bytes": sum(e["c"].numel() + e["s"].numel() for e in lin),
                        "TFLOPs": round(fl / t / 1e12, 2), "frac_mfma": round(fl / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
            log(f"[bench] {key}: {out[key]}")
            del lin
            torch.cuda.empty_cache()
        out["linears_232"] = {
            "what": "every Linear once: the encoder's 128 calls and the 4 cross-attention K/V calls at 1500 "
                    "frames, plus one decoded step of the 24 per-token calls at M = 16",
            "launches": out["encoder_sweep_q8_0_m1500"]["launches"] + out["cross_kv_nf4dq_m1500"]["launches"]
                        + out["decoder_step_m16"]["launches"],
            "linears": out["encoder_sweep_q8_0_m1500"]["linears"] + out["cross_kv_nf4dq_m1500"]["linears"]
                       + out["decoder_step_m16"]["linears"],
            "us": round(out["encoder_sweep_q8_0_m1500"]["us"] + out["cross_kv_nf4dq_m1500"]["us"]
                        + out["decoder_step_m16"]["us_per_step"], 1),
            "us_cross_kv_merged": round(out["encoder_sweep_q8_0_m1500"]["us"]
                                        + out["cross_kv_merged_nf4dq_m1500"]["us"]
                                        + out["decoder_step_m16"]["us_per_step"], 1)}
        return out

    outs1, wss1 = decode_buffers(1)
    t = run_graph_steps(lambda s, st: enqueue_decode_step(1, s, outs1, wss1, st), pool_n, args.steps, args.warmup)
    main_timing = dict(timing_info)
    ms_per_step = t * 1e3 / args.steps
    value = set_bytes * args.steps / t / 1e9
    per_launch_bytes = decode_bytes(1) / len(base)
    per_launch_s = t / (args.steps * len(base))
    achieved = per_launch_bytes / per_launch_s / 1e9
    log(f"[bench] decode M=1: {ms_per_step * 1e3:.2f} us/step, {value:.1f} GB/s weights, "
        f"{per_launch_s * 1e6:.2f} us/launch")

    result = {
        "metric": "decode GEMV weight GB/s (M=1) + encoder TFLOP/s (M=1500), % roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "whisper-large-v3-turbo decoder GEMV set, NF4 + double-quant (64-blocks, int8 absmax "
                        "in 256-block groups), M=1: fused QKV 1280->3840 (wq_matmul_qkv), out 1280->1280, "
                        "fc1 1280->5120, fc2 5120->1280; bf16 activations and outputs",
            "weights": f"{set_bytes} B per step, cycled over {pool_n} copies ({pool_n * set_bytes / 2**30:.2f} GiB)",
            "cold": main_timing["cold"],
            "timed_slots": f"{main_timing['timed_first_slot']} .. {(main_timing['timed_first_slot'] + args.steps - 1) % pool_n}"
                           f" (mod {pool_n})",
            "bytes_read_timed": set_bytes * args.steps,
            "launches_per_step": len(base),
            "timing": "HIP graph replay, HIP events on the launch stream; host submission "
                      + main_timing["host_submission"].split(":")[0],
        },
        "roofline": {
            "kernel": "k_gemv<NF4,dq,1>",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_gemv_nf4dq_m1"),
            "bytes_per_launch": int(per_launch_bytes),
            "us_per_launch": round(per_launch_s * 1e6, 3),
        },
    }

    if not args.no_extras:
        extras = {}
        # ---- decode set at M = 4 and 16 (16 concurrent requests) ----
        for m in (4, 16):
            o, w_ = decode_buffers(m)
            tm = run_graph_steps(lambda s, st: enqueue_decode_step(m, s, o, w_, st), pool_n, pool_n * 2, pool_n)
            extras[f"decode_m{m}"] = {"us_per_step": round(tm * 1e6 / (pool_n * 2), 3),
                                      "weight_GBps": round(set_bytes * pool_n * 2 / tm / 1e9, 2),
                                      "algorithmic_GBps": round(decode_bytes(m) * pool_n * 2 / tm / 1e9, 2)}
            log(f"[bench] decode M={m}: {extras[f'decode_m{m}']}")

        extras["streaming_gemv"] = streaming_part(by_format=True)

        encoder = encoder_part()
        extras["unfused_ablation"] = ablation_part(encoder_part.layers, encoder["us_per_step"], ms_per_step * 1e3)
        encoder_part.layers = None
        extras["encoder_w4a4_nvfp4"] = w4a4_part(encoder["us_per_step"])

        # ---- the decode set (M = 1) in every format, same weights ----
        extras["decode_m1_by_format"] = decode_by_format()

        # ---- output error of each format against fp32 weights, and wq_quantize time ----
        extras["quality_and_quantize_time"] = quality_part()

        # ---- large-v3-turbo sweep: the whole per-token decoder step and the q8_0 encoder ----
        extras.update(sweep_part())

        # ---- one encoder layer at batch 4 (M = 6000), q8_0 and q4_0 on identical weights: Q/K/V as
        # one wq_matmul_qkv over the concatenated weights (3840 x 1280), then O, fc1, fc2 ----
        mb4 = 4 * ENC_M
        for fmt_name, fmt in (("q8_0", wq.WQ_Q8_0), ("q4_0", wq.WQ_Q4_0), ("q4_1", wq.WQ_Q4_1), ("q5_0", wq.WQ_Q5_0),
                              ("q4_k", wq.WQ_Q4_K), ("q6_k", wq.WQ_Q6_K)):
            parts = [linear_case(4000 + i, ENC_D, ENC_D, mb4) for i in range(4)] + \
                    [linear_case(4004, ENC_FFN, ENC_D, mb4), linear_case(4005, ENC_D, ENC_FFN, mb4)]
            spec = [(np.concatenate([p[0] for p in parts[:3]]), np.concatenate([parts[0][1], np.zeros_like(parts[1][1]),
                                                                               parts[2][1]]), parts[0][2], 3)]
            spec += [(p[0], p[1], p[2], 1) for p in parts[3:]]
            lay = []
            for w, b, x, nsplit in spec:
                n, k = w.shape
                d, c, s = quantize_dev(fmt, torch.from_numpy(w).to(dev), False)
                nb = wq.wq_workspace_size(d, mb4)
                lay.append(dict(d=d, c=c, s=s, b=bf16_dev(b), x=bf16_dev(x), n=n, k=k, nsplit=nsplit,
                                y=torch.empty((mb4, n), dtype=torch.int16, device=dev),
                                ws=torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev), nb=nb))

            def layer_step(s_, st, lay=lay):
                for e in lay:
                    if e["nsplit"] == 3:
                        p0 = e["y"].data_ptr()
                        wq.wq_matmul_qkv(e["d"], mb4, e["x"], e["k"], e["c"], e["s"], e["b"], [ENC_D] * 3,
                                         [p0, p0 + 2 * ENC_D, p0 + 4 * ENC_D], [e["n"]] * 3, wq.WQ_BF16,
                                         e["ws"] if e["nb"] else None, e["nb"], stream=st)
                    else:
                        wq.wq_matmul(e["d"], mb4, e["x"], e["k"], e["c"], e["s"], e["b"], e["y"], wq.WQ_BF16, e["n"],
                                     e["ws"] if e["nb"] else None, e["nb"], stream=st)

            reps = 10
            tl = run_graph_steps(layer_step, 1, reps, 5, per_graph=5)
            fl = sum(2.0 * mb4 * e["n"] * e["k"] for e in lay)
            extras[f"encoder_layer_b4_{fmt_name}"] = {"launches": len(lay), "us_per_layer": round(tl * 1e6 / reps, 1),
                                                      "TFLOPs": round(fl * reps / tl / 1e12, 2),
                                                      "frac_mfma": round(fl * reps / tl / 1e12 / BF16_PEAK_TFLOPS, 4)}
            log(f"[bench] layer b4 {fmt_name}: {extras[f'encoder_layer_b4_{fmt_name}']}")
            del lay
        result["encoder"] = encoder
        result["extras"] = extras

    # ---------------- CPU oracle baseline (bounded sample) ----------------
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(base, set_bytes)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")

    print(json.dumps(result), flush=True)


def source_digest(paths):
    """sha256 over the named kernel sources (relative to the repository root), in order."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def measured_traffic(key, field="traffic_bytes_per_launch"):
    """HBM bytes (per launch, or per step for the encoder) from the committed rocprofv3
    counter runs, or None when the kernel sources changed since those counters were taken
    (each record names its sources and their sha256)."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[key]
        digest = source_digest(rec["sources"])
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if digest != rec.get("sources_sha256"):
        return None
    return rec[field]


def cpu_baseline(base, set_bytes):
    """The plain C oracle, as it stands, doing the same step on the host: decode
    every packed weight of the set (double-quant absmax, NF4 levels) and run the
    fp32 matmul for one token.  Runs whole steps until 10 s have passed."""
    cores = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(cores)
    from oracle import oracle as O
    prepared = []
    for e in base:
        q = O.nf4_quantize(e["w"])
        codes, a = q
        qq, d, mu = O.nf4_double_quant(a)
        prepared.append((codes, qq, d, mu, e["xbits"][:1], e["b"]))
    steps = 0
    t0 = time.perf_counter()
    while True:
        for codes, qq, d, mu, x, b in prepared:
            ahat = O.nf4_dq_absmax(qq, d, mu)
            w_hat = O.nf4_dequantize(codes, ahat)
            O.matmul(x, w_hat, b)
        steps += 1
        el = time.perf_counter() - t0
        if el > 10.0:
            break
    return {"value": round(set_bytes * steps / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} whole decode steps (4 matrices, M=1: dequantize to fp32 + fp32 matmul) "
                      f"in {el:.1f} s; dequantize single-threaded, matmul OpenMP over rows"}


def cpu_baseline_encoder(cases):
    """The plain C oracle, as it stands, on the encoder step (NVFP4 fc1 + fc2, M = 1500): each
    matrix is quantized and dequantized to fp32 once (not timed), then the fp32 matmul runs over
    row blocks of X (OpenMP over rows) until 10 s have passed; TFLOP/s counts the rows done."""
    cores = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(cores)
    from oracle import oracle as O
    prepared = []
    for w, b, x in cases:
        q = O.quantize(2, w, False)        # NVFP4
        prepared.append((x, q["w_hat"], b, w.shape[0], w.shape[1]))
    rows = np.arange(64)
    flop = 0.0
    t0 = time.perf_counter()
    blocks = 0
    while True:
        for x, w_hat, b, n, k in prepared:
            r = (rows + 64 * blocks) % x.shape[0]
            O.matmul(x, w_hat, b, rows=r)
            flop += 2.0 * len(r) * n * k
        blocks += 1
        el = time.perf_counter() - t0
        if el > 10.0:
            break
    return {"value": round(flop / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{blocks} blocks of 64 rows of X through fc1 and fc2 (fp32 matmul on the oracle's "
                      f"dequantized NVFP4 weights) in {el:.1f} s; quantize/dequantize not timed"}


if __name__ == "__main__":
    main()
