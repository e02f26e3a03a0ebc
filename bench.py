"""Benchmark of the W4A8 linear layer on one MI355X.

Workload: the 7B MLP projection K=4096 -> N=11008, swept over token counts
M in {1, 8, 32, 256, 4096} (one decode token up to a 4096-token prefill).  One
step = for every M, the per-token activation quantization followed by the W4A8
GEMM, exactly what a serving engine runs per linear layer (the weights were
quantized offline, once).  Inputs are seeded synthetic tensors resident in HBM
before timing starts; every GEMM call reads a different copy of the packed
weights, rotating through enough copies to exceed the 256 MB Infinity Cache,
so weight bytes really come from HBM.

Prints one JSON line: whole-step throughput (TOPS), the roofline of the
dominant kernel (the M=4096 GEMM), per-M kernel figures, every shape of the
five workload configurations ("configs": µs, GB/s, TOPS, fractions of the HBM
and INT8 peaks and of the measured streaming-read ceiling), and the CPU oracle
timed on a bounded sample of the same workload.  Two separate objects, not
part of the step or of `value`, measure the other entry points on the same
tensors against the HBM roofline, each with its oracle beside it:
"norm_quant" (the fused LayerNorm + INT8 producer, norm_quantize_act_i8) and
"w4a16" (the W4A16 GEMM on the same packed weights, gemm_w4a16, at the
decode token counts, next to the W4A8 GEMM's times) and "kv4_attention"
(decode attention over the 4-bit KV cache, attention_kv4_decode, on the
reference 7B at a 4,096-token context, multi-head and with 8 kv heads).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8 GEMM TOPS + achieved HBM GB/s (% roofline), K=4096 N=11008 M=1..4096"
K_DIM, N_DIM = 4096, 11008
MS = (1, 8, 32, 256, 4096)
FAMILY = 3          # weight / activation value distributions of the prefill family
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=50, help="calls per per-M kernel timing loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="token rows per M in the oracle sample (default: every row, one whole step)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration block")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the path runs on a single MI355X); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from w4a8_quantized_linear_amd import _lib, accounting as A, workloads
    from w4a8_quantized_linear_amd.tuning import graph_time
    from w4a8_quantized_linear_amd import (gemm_w4a8, gemm_w4a16, norm_quantize_act_i8,
                                           quantize_act_per_token_i8, quantize_weights_w4g128)
    from w4a8_quantized_linear_amd._lib import w4a8_hbm_read
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs (host-generated, seeded), resident in HBM before timing ----
    w_np = workloads.weights(FAMILY, K_DIM, N_DIM)
    wq = quantize_weights_w4g128(torch.from_numpy(w_np).to(dev), canonical=False)
    wbytes = wq["wpacked"].numel()
    nrot = max(2, math.ceil(ROTATE_BYTES / wbytes))
    wcopies = [wq["wpacked"]] + [wq["wpacked"].clone() for _ in range(nrot - 1)]
    s0 = wq["s0"]
    xs, qxs, sas, ys = {}, {}, {}, {}
    for M in MS:
        xs[M] = torch.from_numpy(workloads.activations(FAMILY, M, K_DIM, N_DIM)).to(dev)
        qxs[M] = torch.empty((M, K_DIM), dtype=torch.int8, device=dev)
        sas[M] = torch.empty((M,), dtype=torch.float32, device=dev)
        ys[M] = torch.empty((M, N_DIM), dtype=torch.float16, device=dev)
    ws = _lib.workspace(dev, max(_lib.gemm_w4a8_workspace_bytes(M, N_DIM, K_DIM) for M in MS))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    counter = [0]
    dom_M = MS[-1]
    ev_pairs = []

    def step(record, st=None):
        st = st or stream
        for M in MS:
            quantize_act_per_token_i8(xs[M], qx=qxs[M], s_a=sas[M], stream=st)
            wp = wcopies[counter[0] % nrot]
            counter[0] += 1
            if record and M == dom_M:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                gemm_w4a8(qxs[M], sas[M], wp, s0, N_DIM, y=ys[M], ws=ws, stream=st)
                e1.record(st)
                ev_pairs.append((e0, e1))
            else:
                gemm_w4a8(qxs[M], sas[M], wp, s0, N_DIM, y=ys[M], ws=ws, stream=st)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # ---- the steps launched one call at a time from the host (eager): the
    # calls' own events give eager_step_avg_us; this figure includes the
    # host's launch rate and is kept as eager_ms_per_step --------------------
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step(True)
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = t_start.elapsed_time(t_end) / args.steps
    dom_us = 1e3 * sum(a.elapsed_time(b) for a, b in ev_pairs) / len(ev_pairs)

    # ---- timed region: exactly `steps` steps, captured once in a HIP graph
    # (the weight copies keep rotating from step to step inside it) and
    # replayed: every kernel of every step runs, without the host's per-call
    # launch cost.  One untimed replay first. --------------------------------
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(args.steps):
                step(False, side)
    stream.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    graph.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    ops_step = sum(A.gemm_ops(M, N_DIM, K_DIM) for M in MS)
    value = ops_step / (ms_per_step * 1e-3) / 1e12

    # ---- per-M kernel figures: `reps` calls captured in one HIP graph and
    # replayed under events, so that small-M figures are the kernels' own time
    # and not the host's launch rate ----------------------------------------
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    ceil_us = graph_time(lambda r: w4a8_hbm_read(wcopies[r % nrot], sink), args.reps)
    per_m = []
    for M in MS:
        rec = {"M": M}
        for kind in ("act_quant", "gemm"):
            if kind == "act_quant":
                us = graph_time(lambda r: quantize_act_per_token_i8(xs[M], qx=qxs[M], s_a=sas[M]), args.reps)
                nbytes = A.act_quant_bytes(M, K_DIM)
                rec["act_quant_us"] = round(us, 3)
                rec["act_quant_GBps"] = round(nbytes / us * 1e-3, 1)
            else:
                us = graph_time(lambda r: gemm_w4a8(qxs[M], sas[M], wcopies[r % nrot], s0, N_DIM, y=ys[M],
                                                    ws=ws), args.reps)
                nbytes = A.gemm_bytes(M, N_DIM, K_DIM)
                ops = A.gemm_ops(M, N_DIM, K_DIM)
                rec["gemm_us"] = round(us, 3)
                rec["gemm_GBps"] = round(nbytes / us * 1e-3, 1)
                rec["gemm_TOPS"] = round(ops / us * 1e-6, 2)
                rec["hbm_frac"] = round(nbytes / us * 1e-3 / (A.MI355X_HBM_BYTES_PER_S / 1e9), 4)
                rec["mfma_frac"] = round(ops / us * 1e-6 / (A.MI355X_INT8_OPS_PER_S / 1e12), 4)
                rec["ceiling_frac"] = round(ceil_us / us, 4)
        per_m.append(rec)

    # ---- roofline of the dominant kernel (M=4096 GEMM, MFMA-bound) ---------
    # Its duration is the graph-timed per-M figure (HIP events around replays of
    # `reps` back-to-back launches on the launch stream): the kernel's own time,
    # which a rocprofv3 kernel trace of this command reproduces.  The events
    # bracketing it inside the eager step also cover the markers' cache flush
    # and dispatch; that figure is kept as eager_step_avg_us.
    dom_ops = A.gemm_ops(dom_M, N_DIM, K_DIM)
    dom_graph_us = next(r for r in per_m if r["M"] == dom_M)["gemm_us"]
    achieved = dom_ops / (dom_graph_us * 1e-6) / 1e12
    peak = A.MI355X_INT8_OPS_PER_S / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(),
                "kernel": "gemm_w4a8 M=%d N=%d K=%d" % (dom_M, N_DIM, K_DIM),
                "avg_us": round(dom_graph_us, 3), "eager_step_avg_us": round(dom_us, 3),
                "ops_per_launch": dom_ops}

    # ---- fused normalization + quantizer (not part of the step) -----------
    gam = torch.from_numpy(workloads.norm_affine(K_DIM)[0]).to(dev)
    bet = torch.from_numpy(workloads.norm_affine(K_DIM)[1]).to(dev)
    nq = []
    for M in MS:
        us = graph_time(lambda r: norm_quantize_act_i8(xs[M], gam, bet, eps=1e-5, qx=qxs[M], s_a=sas[M]),
                        args.reps)
        nbytes = A.norm_quant_bytes(M, K_DIM)
        nq.append({"M": M, "us": round(us, 3), "GBps": round(nbytes / us * 1e-3, 1),
                   "hbm_frac": round(nbytes / us * 1e-3 / (A.MI355X_HBM_BYTES_PER_S / 1e9), 4)})
    big = nq[-1]
    norm_quant = {
        "kernel": "norm_quantize_act_i8 (LayerNorm, gamma + beta) K=%d" % K_DIM,
        "per_m": nq,
        "roofline": {"bound": "hbm", "achieved": big["GBps"], "peak": A.MI355X_HBM_BYTES_PER_S / 1e9,
                     "unit": "GB/s", "frac": big["hbm_frac"], "traffic": None,
                     "bytes_per_launch": A.norm_quant_bytes(MS[-1], K_DIM), "M": MS[-1]},
        "unfused_bytes_per_launch": A.unfused_norm_quant_bytes(MS[-1], K_DIM),
    }

    # ---- W4A16 on the same weights at the decode token counts (not part of the step)
    w16 = []
    for M in [m for m in MS if m <= 32]:
        us = graph_time(lambda r: gemm_w4a16(xs[M], wcopies[r % nrot], s0, N_DIM, y=ys[M]), args.reps)
        nbytes = A.w4a16_bytes(M, N_DIM, K_DIM)
        w8 = next(r for r in per_m if r["M"] == M)
        w16.append({"M": M, "us": round(us, 3), "GBps": round(nbytes / us * 1e-3, 1),
                    "hbm_frac": round(nbytes / us * 1e-3 / (A.MI355X_HBM_BYTES_PER_S / 1e9), 4),
                    "w4a8_act_quant_plus_gemm_us": round(w8["act_quant_us"] + w8["gemm_us"], 3)})
    w4a16 = {"kernel": "gemm_w4a16 K=%d N=%d" % (K_DIM, N_DIM), "per_m": w16,
             "roofline": {"bound": "hbm", "achieved": w16[0]["GBps"], "peak": A.MI355X_HBM_BYTES_PER_S / 1e9,
                          "unit": "GB/s", "frac": w16[0]["hbm_frac"], "traffic": None, "M": w16[0]["M"],
                          "bytes_per_launch": A.w4a16_bytes(w16[0]["M"], N_DIM, K_DIM)}}

    kv4 = bench_kv4(args, stream)
    configs = None if args.no_configs else bench_configs(args)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "W4A8 linear K=4096 N=11008 (7B MLP projection), one step = "
                               "act-quant + GEMM at each M in [1, 8, 32, 256, 4096]",
                   "K": K_DIM, "N": N_DIM, "M": list(MS), "group": 128,
                   "weight_copies": nrot, "wall_s": round(wall, 4)},
        "roofline": roofline,
        "hbm_read_ceiling": {"bytes": wbytes, "us": round(ceil_us, 3),
                             "GBps": round(wbytes / ceil_us * 1e-3, 1),
                             "kernel": "w4a8_hbm_read (the weight stream read once, nothing computed)"},
        "per_m": per_m,
        "targets": targets(per_m, configs),
        "configs": configs,
        "norm_quant": norm_quant,
        "w4a16": w4a16,
        "kv4_attention": kv4,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w_np, args.cpu_rows)
        norm_quant["cpu_baseline"] = cpu_baseline_norm_quant()
        w4a16["cpu_baseline"] = cpu_baseline_w4a16(w_np)
        kv4["cpu_baseline"] = cpu_baseline_kv4()

    print(json.dumps(out), flush=True)


DECODE_HBM_TARGET = 0.70     # fraction of 8 TB/s for the decode GEMM at M <= 32
PREFILL_MFMA_TARGET = 0.50   # fraction of 5.0 POPS for the prefill GEMM at M = 4096


def targets(per_m, configs):
    """The two performance bars of the path, and the measured rows that fall short
    of them, stated in the output next to the figures (met: every row reaches it)."""
    rows = configs if configs else [dict(r, K=K_DIM, N=N_DIM) for r in per_m]
    dec = [r for r in rows if r["M"] <= 32]
    pre = [r for r in rows if r["M"] == 4096]
    dec_below = [{"M": r["M"], "K": r["K"], "N": r["N"], "hbm_frac": r["hbm_frac"],
                  "ceiling_frac": r.get("ceiling_frac")} for r in dec if r["hbm_frac"] < DECODE_HBM_TARGET]
    pre_below = [{"M": r["M"], "K": r["K"], "N": r["N"], "mfma_frac": r["mfma_frac"],
                  "with_act_quant": r.get("total_mfma_frac")}
                 for r in pre if min(r["mfma_frac"], r.get("total_mfma_frac", 1.0)) < PREFILL_MFMA_TARGET]
    return {"decode_hbm_frac": DECODE_HBM_TARGET, "decode_met": not dec_below,
            "decode_rows": len(dec), "decode_rows_below": dec_below,
            "prefill_mfma_frac": PREFILL_MFMA_TARGET, "prefill_met": not pre_below,
            "prefill_rows": len(pre), "prefill_rows_below": pre_below}


def bench_configs(args):
    """Every shape of the five workload configurations: the GEMM (and for the
    prefill configuration the activation quantizer before it) timed as HIP-graph
    replays, weights rotated through 1 GiB of copies so that their bytes come
    from HBM, beside the streaming-read ceiling of the same weight bytes.
    Inputs follow each configuration's recipe, drawn on the GPU from a seeded
    generator (the full-size host draws of the parity tests take far longer):
    weights N(0, 0.02) -- Student-t(4) scaled to the same spread for the
    heavy-tailed configuration -- quantized by quantize_weights_w4g128;
    activations N(0, 1) with the configuration's outlier channels scaled up,
    quantized per token."""
    import torch

    from w4a8_quantized_linear_amd import (_lib, accounting as A, gemm_w4a8, quantize_act_per_token_i8,
                                           quantize_weights_w4g128, workloads as W)
    from w4a8_quantized_linear_amd._lib import w4a8_hbm_read
    from w4a8_quantized_linear_amd.tuning import graph_time
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    reps = max(10, args.reps // 2)
    hbm, ops_peak = A.MI355X_HBM_BYTES_PER_S, A.MI355X_INT8_OPS_PER_S
    ridge = ops_peak / hbm
    out = []
    for fam in W.FAMILIES:
        for (K, N) in fam.kns:
            gen.manual_seed(0x57A8 * 1000 + fam.index * 100 + K % 97 + N % 89)
            w = torch.randn((N, K), device=dev, generator=gen)
            if fam.w_dist == "student_t4":     # z / sqrt(chi2_4 / 4), then the population std sqrt(2) out
                chi2 = sum(torch.randn((N, K), device=dev, generator=gen) ** 2 for _ in range(4))
                w = w / torch.sqrt(chi2 / 4) / math.sqrt(2.0)
            wq = quantize_weights_w4g128((w * 0.02).float().contiguous(), canonical=False)
            del w
            wb = wq["wpacked"].numel()
            views = [wq["wpacked"]] + [wq["wpacked"].clone() for _ in range(max(2, math.ceil(ROTATE_BYTES / wb)) - 1)]
            s0 = wq["s0"]
            cus = graph_time(lambda r: w4a8_hbm_read(views[r % len(views)], sink), reps)
            n_out = int(round(0.01 * K)) if fam.n_outlier < 0 else fam.n_outlier
            outl = torch.randperm(K, device=dev, generator=gen)[:n_out]
            for M in fam.ms:
                x = torch.randn((M, K), device=dev, generator=gen)
                x[:, outl] *= fam.outlier_scale
                x = x.half()
                qx, sa = quantize_act_per_token_i8(x)
                y = torch.empty((M, N), dtype=torch.float16, device=dev)
                ws = _lib.workspace(dev, _lib.gemm_w4a8_workspace_bytes(M, N, K))
                us = graph_time(lambda r: gemm_w4a8(qx, sa, views[r % len(views)], s0, N, y=y, ws=ws), reps)
                nbytes, ops = A.gemm_bytes(M, N, K), A.gemm_ops(M, N, K)
                rec = {"config": fam.index, "M": M, "K": K, "N": N,
                       "bound": "hbm" if ops / nbytes < ridge else "mfma",
                       "gemm_us": round(us, 3), "GBps": round(nbytes / us * 1e-3, 1),
                       "TOPS": round(ops / us * 1e-6, 2), "hbm_frac": round(nbytes / us * 1e-3 / (hbm / 1e9), 4),
                       "mfma_frac": round(ops / us * 1e-6 / (ops_peak / 1e12), 4),
                       "ceiling_us": round(cus, 3), "ceiling_frac": round(cus / us, 4)}
                if fam.index == 3:
                    # prefill: the activation quantizer is part of the timed work
                    aus = graph_time(lambda r: quantize_act_per_token_i8(x, qx=qx, s_a=sa), reps)
                    tot = aus + us
                    rec.update({"act_quant_us": round(aus, 3), "total_us": round(tot, 3),
                                "total_TOPS": round(ops / tot * 1e-6, 2),
                                "total_mfma_frac": round(ops / tot * 1e-6 / (ops_peak / 1e12), 4)})
                out.append(rec)
                del x, qx, sa, y
            del views, wq
            torch.cuda.empty_cache()
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_w4a8_m4096_k4096_n11008.txt")
TRAFFIC_SOURCES = ("w4a8_quantized_linear_amd/csrc/gemm_prefill.hip",
                   "w4a8_quantized_linear_amd/csrc/kernel_common.h",
                   "w4a8_quantized_linear_amd/csrc/dispatch.hip")


def source_digest():
    """sha256 over the sources that decide the dominant kernel's memory traffic."""
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when the kernel sources changed
    since those counters were taken."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_sha256") != source_digest():
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w_np, rows):
    """The oracle, as it stands, on a bounded sample: every M of the sweep with at most `rows` token rows."""
    import numpy as np

    import oracle as orc
    from w4a8_quantized_linear_amd import accounting as A, workloads
    wq = orc.quantize_weights(w_np)
    total_ops, total_s, threads, sample = 0, 0.0, 1, []
    for M in MS:
        m = min(M, rows)
        x = workloads.activations(FAMILY, M, K_DIM, N_DIM)[:m]
        bufs = orc.linear_timed_buffers(m, N_DIM, K_DIM)
        t0 = time.perf_counter()
        threads = orc.linear_into(x, wq, bufs)
        total_s += time.perf_counter() - t0
        total_ops += A.gemm_ops(m, N_DIM, K_DIM)
        sample.append(m)
    return {"value": round(total_ops / total_s / 1e12, 6), "unit": "TOPS", "cores": threads,
            "kind": "oracle", "seconds": round(total_s, 3),
            "sample": "oracle act-quant + dequant + int64 GEMM + epilogue, K=4096 N=11008, token rows %s "
                      "(first rows of each M of the sweep)" % sample}


def cpu_baseline_norm_quant(rows: int = 4096):
    """The fused producer's oracle on a bounded sample: the first `rows` tokens of the M=4096 activations.
    The oracle is one serial C call per block of tokens; the blocks run on host threads (the C call
    releases the interpreter lock), as many as the oracle's GEMM uses, so the baselines are comparable."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle as orc
    from w4a8_quantized_linear_amd import accounting as A, workloads
    x = workloads.activations(FAMILY, MS[-1], K_DIM, N_DIM)[:rows]
    g, b = workloads.norm_affine(K_DIM)
    threads = max(1, min(orc.num_threads(), rows))
    blocks = [x[i * rows // threads:(i + 1) * rows // threads] for i in range(threads)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda blk: orc.norm_quantize_act(blk, g, b, eps=1e-5), blocks))
    s = time.perf_counter() - t0
    return {"value": round(A.norm_quant_bytes(rows, K_DIM) / s / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(s, 3),
            "sample": "oracle LayerNorm + per-token INT8, K=%d, the first %d tokens of M=%d, in %d blocks on "
                      "%d host threads" % (K_DIM, rows, MS[-1], threads, threads)}


def bench_kv4(args, stream):
    """Decode attention over the 4-bit KV cache on each configuration (every sequence
    at the full context), and the one-token append that precedes it in a decode step."""
    import torch

    from w4a8_quantized_linear_amd import (accounting as A, attention_kv4_decode, kv4_attention_workspace_bytes,
                                           kv4_cache_alloc, quantize_kv4, workloads as W)
    from w4a8_quantized_linear_amd.tuning import graph_time
    dev = torch.device("cuda:0")
    res = {}
    for name, cfg in sorted(W.KV_CONFIGS.items()):
        B, Hq, Hkv, S = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"]
        kc, vc = kv4_cache_alloc(B, Hkv, S, device=dev)
        for part in range(S // 256):
            k, v = W.kv_rows_torch(41, B, 256, Hkv, part, dev)
            quantize_kv4(k, v, torch.full((B,), part * 256, dtype=torch.int32, device=dev), kc, vc, S, stream=stream)
        del k, v
        q = torch.from_numpy(W.kv_query(41, B, Hq)).to(dev)
        lens = torch.full((B,), S, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        ws = torch.empty(max(1, kv4_attention_workspace_bytes(B, Hq, S)), dtype=torch.uint8, device=dev)
        sm = 1.0 / math.sqrt(128)
        attention_kv4_decode(q, kc, vc, S, Hkv, lens, sm, out=out, ws=ws, stream=stream)
        torch.cuda.synchronize()
        reps = max(10, args.reps // 2)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            attention_kv4_decode(q, kc, vc, S, Hkv, lens, sm, out=out, ws=ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        nbytes = A.kv4_attention_bytes([S] * B, Hq, Hkv)
        # the decode step's append: one new token per sequence, written at position S - 1
        k1, v1 = W.kv_rows_torch(42, B, 1, Hkv, 0, dev)
        pos = torch.full((B,), S - 1, dtype=torch.int32, device=dev)
        # (a few-microsecond kernel: timed as HIP-graph replays, not at the host's launch rate)
        qus = graph_time(lambda r: quantize_kv4(k1, v1, pos, kc, vc, S), reps)
        res[name] = {"B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "head_dim": 128, "attention_us": round(us, 3),
                     "bytes_per_launch": nbytes, "GBps": round(nbytes / us * 1e-3, 1),
                     "hbm_frac": round(nbytes / us * 1e-3 / (A.MI355X_HBM_BYTES_PER_S / 1e9), 4),
                     "tokens_per_s": round(B / us * 1e6, 1), "append_one_token_us": round(qus, 3)}
        del kc, vc, ws
        torch.cuda.empty_cache()
    first = res[sorted(res)[0]]
    return {"kernel": "attention_kv4_decode (kv4_attn_kernel + kv4_combine_kernel), every sequence at S",
            "configs": res,
            "roofline": {"bound": "hbm", "achieved": first["GBps"], "peak": A.MI355X_HBM_BYTES_PER_S / 1e9,
                         "unit": "GB/s", "frac": first["hbm_frac"], "traffic": None, "config": sorted(res)[0],
                         "bytes_per_launch": first["bytes_per_launch"]}}


def cpu_baseline_kv4(seqs: int = 2):
    """The oracle's KV4 attention (double) on a bounded sample: `seqs` sequences of the
    multi-head configuration at the full context, all 32 heads."""
    import numpy as np

    import oracle as orc
    from w4a8_quantized_linear_amd import accounting as A, workloads as W
    cfg = W.KV_CONFIGS["7b_mha"]
    Hq, Hkv, S = cfg["Hq"], cfg["Hkv"], cfg["S"]
    k, v = W.kv_rows(43, seqs, S, Hkv)
    kq = orc.quantize_kv4(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    vq = orc.quantize_kv4(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    q = W.kv_query(43, seqs, Hq)
    lens = np.full(seqs, S, np.int32)
    calls, t0 = 0, time.perf_counter()
    while calls == 0 or time.perf_counter() - t0 < 2.0:
        orc.kv4_attention(q, kq, vq, lens, 1.0 / math.sqrt(128))
        calls += 1
    s = (time.perf_counter() - t0) / calls
    return {"value": round(A.kv4_attention_bytes([S] * seqs, Hq, Hkv) / s / 1e9, 3), "unit": "GB/s",
            "cores": orc.num_threads(), "kind": "oracle", "seconds": round(s * calls, 3),
            "sample": "oracle KV4 decode attention (double), 7b_mha: %d sequences x %d tokens x %d heads, "
                      "%d calls" % (seqs, S, Hq, calls)}


def cpu_baseline_w4a16(w_np, rows: int = 8):
    """The W4A16 oracle (double products and sums) on a bounded sample: the M = 8 activations."""
    import oracle as orc
    from w4a8_quantized_linear_amd import accounting as A, workloads
    wq = orc.quantize_weights(w_np)
    r, _ = orc.dequant_i8(wq["q4"], wq["s1"], wq["z"])
    x = workloads.activations(FAMILY, rows, K_DIM, N_DIM)
    t0 = time.perf_counter()
    orc.gemm_w4a16(x, r, wq["s0"])
    s = time.perf_counter() - t0
    return {"value": round(A.w4a16_bytes(rows, N_DIM, K_DIM) / s / 1e9, 3), "unit": "GB/s",
            "cores": orc.num_threads(), "kind": "oracle", "seconds": round(s, 3),
            "sample": "oracle W4A16 (double), K=%d N=%d, M=%d" % (K_DIM, N_DIM, rows)}


if __name__ == "__main__":
    main()
