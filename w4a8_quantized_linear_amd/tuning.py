"""Offline profiling of the decode GEMM plans, the training data of the learned
plan selector (QFactory reading notes, 6.2: the kernel-efficiency model is
trained on measured runs of randomly drawn configurations).

For each shape (M <= 64 tokens, K, N) every plan that can run
(gemm_w4a8_decode_candidates) is timed, its weight bytes coming from HBM (the
calls rotate over copies in a 1 GiB buffer), and the achieved fraction of the
8 TB/s HBM peak is recorded.  The calls are captured in a HIP graph and the
graph is replayed under HIP events, so small kernels are timed without the
host's per-call launch cost:

    python -m w4a8_quantized_linear_amd.tuning OUT.csv [--shapes 120] [--seed 0] [--eval]

--eval measures the 7B / 70B decode shapes instead of random ones (the
held-out set).  --compare re-times, on those shapes and the 7B MLP shape
(K = 4096, N = 11008), the rule table's plan against the selector's
(W4A8_SELECTOR=0 versus the compiled-in model), interleaved, 50 calls per
graph, three rounds, medians.  Needs a GPU; the weights are random bytes (every byte is a
valid code pair and group parameter), timing does not depend on the values.

--launch M1,M2,..  --n N --k K [--calls C] makes C eager calls per token count with the
plan gemm_w4a8 picks (rotating weight copies, as above) and prints the plans: the
program that profiler runs (rocprofv3 --pmc ...) trace for the decode counters.

--route OUT.csv times, at 72..256 tokens on the 7B / 70B layers and on narrow layers,
the best decode plan (every candidate) against the many-token kernel at each TM and
K split, and the plan gemm_w4a8 picks: the evidence behind sending 65..128 tokens to
the decode kernels when the many-token tiles are few, and 129..1024 tokens when the
layer has at most 2^20 outputs.

--splits OUT.csv times the many-token kernel at 96..768 tokens on long-K layers for TM 4
and 8 with every tile split into s = 1, 2, 3, 4, 6, 8 equal K ranges (W4A8_PREFILL_P =
tiles x s) and TM 16 whole, next to the plan gemm_w4a8 picks.

--wide OUT.csv [--shapes 150 --seed 5] times, on random shapes with 129..256 tokens and
at most 2^20 outputs, every decode plan, the many-token kernel at TM 4 / 8 with 1..4
K ranges per tile, and the plan gemm_w4a8 picks (--wide-m and --outputs move the token
and M x N ranges); --wide-layers does the same on 15 7B / 70B layers at 136..512 tokens.  The data behind the 129..256-token route and
its decode plan tree.  --mid does the same on random shapes with 65..128 tokens
that the dispatcher sends to the decode kernels, --mid-layers on the 7B / 70B and
narrow layers above at 72..128 tokens.

--w16 OUT.csv times gemm_w4a16 at 17, 32, 48 and 64 tokens on the 7B layers for
every (tiles per workgroup, token tiles per workgroup) and the launcher's own
choice, and checks that two token tiles give the bits of one.
"""
from __future__ import annotations

import argparse
import csv
import math
import os
import sys

import numpy as np

FIELDS = ("set", "M", "N", "K", "mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n", "rules", "us", "util")
EVAL_SHAPES = [(M, N, K) for M in (1, 8, 16, 32, 64)
               for (K, N) in ((4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096),
                              (8192, 10240), (8192, 57344), (28672, 8192))]


def random_shapes(n, seed, m_lo=1, m_hi=64):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(round(2 ** rng.uniform(math.log2(m_lo), math.log2(m_hi))))
        K = 128 * int(round(2 ** rng.uniform(2, math.log2(224))))
        N = 16 * int(round(2 ** rng.uniform(5, math.log2(3584))))
        if N * K // 2 <= 512 << 20:
            out.append((M, N, K))
    return out


def graph_time(call, reps, replays=3):
    """Microseconds per call: `reps` calls (call(r)) captured once in a HIP graph,
    replayed `replays` times under events after one warm replay."""
    import torch
    call(0)                                   # eager: plan, workspace, kernel attributes
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for r in range(reps):
                call(r + 1)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * reps)


def measure(shapes, tag, writer, reps=10, wave_n=None):
    import torch

    from w4a8_quantized_linear_amd import (accounting as A, gemm_w4a8, gemm_w4a8_decode_candidates,
                                           gemm_w4a8_plan, w4a8_packed_weight_bytes)
    dev = torch.device("cuda:0")
    pool = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev)
    for (M, N, K) in shapes:
        wb = w4a8_packed_weight_bytes(N, K)
        stride = (wb + 4095) // 4096 * 4096
        copies = max(1, (1 << 30) // stride)
        views = [pool[i * stride:i * stride + wb] for i in range(min(copies, 64))]
        qx = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        sa = torch.rand(M, device=dev) * 0.01
        s0 = (torch.rand(N, device=dev) * 1e-3).half()
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        os.environ["W4A8_SELECTOR"] = "0"
        rules = gemm_w4a8_plan(M, N, K)
        rules_t = tuple(rules[f] for f in ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n"))
        nbytes = A.gemm_bytes(M, N, K)
        for c in gemm_w4a8_decode_candidates(M, N, K):
            if wave_n is not None and c[6] != wave_n:
                continue
            os.environ["W4A8_DECODE_PLAN"] = ",".join(str(v) for v in c)
            got = gemm_w4a8_plan(M, N, K)
            if tuple(got[f] for f in ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")) != c:
                continue
            us = graph_time(lambda r: gemm_w4a8(qx, sa, views[r % len(views)], s0, N, y=y), reps)
            writer.writerow([tag, M, N, K, *c, int(c == rules_t), round(us, 3),
                             round(nbytes / us * 1e-6 / 8.0, 5)])
        del os.environ["W4A8_DECODE_PLAN"]
        print("measured %s M=%d N=%d K=%d" % (tag, M, N, K), flush=True)
    os.environ.pop("W4A8_SELECTOR", None)


COMPARE_FIELDS = ("M", "N", "K", "rules_plan", "selector_plan", "rules_us", "selector_us", "ratio")
ROUTE_FIELDS = ("M", "N", "K", "decode_best_us", "decode_best_plan", "prefill_best_us", "prefill_best_cfg",
                "picked_plan", "picked_us")
W16_FIELDS = ("M", "N", "K", "nt", "mt", "us", "default_us")
SPLIT_FIELDS = ("M", "N", "K", "tm", "splits", "ranges", "us", "picked_plan", "picked_us")
SPLIT_LAYERS = ((8192, 10240), (11008, 4096), (28672, 8192), (8192, 8192), (14336, 4096), (4096, 11008),
                (4096, 4096), (8192, 28672))
ROUTE_LAYERS = ((4096, 11008), (11008, 4096), (8192, 10240), (4096, 22016), (4096, 12288), (28672, 8192))
# narrow layers (N <= 6144) outside the set the 129..256-token plan rule was fitted on
ROUTE_NARROW_LAYERS = ((3072, 3072), (6144, 2048), (18432, 4096), (7168, 4096), (12288, 1536), (5120, 5120),
                       (8192, 3072))
W16_LAYERS = ((4096, 11008), (4096, 4096), (4096, 22016), (11008, 4096), (4096, 12288))


def _weight_views(pool, N, K):
    from w4a8_quantized_linear_amd import w4a8_packed_weight_bytes
    wb = w4a8_packed_weight_bytes(N, K)
    stride = (wb + 4095) // 4096 * 4096
    return [pool[i * stride:i * stride + wb] for i in range(min(max(1, (1 << 30) // stride), 64))]


def route(writer, ms=(72, 96, 112, 128, 136, 160, 192, 256), reps=10):
    """Best decode plan against the many-token kernel's best TM and K split per shape."""
    import torch

    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, gemm_w4a8_decode_candidates, gemm_w4a8_plan
    dev = torch.device("cuda:0")
    pool = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev)
    keys = ("W4A8_DECODE_PLAN", "W4A8_PREFILL_TM", "W4A8_PREFILL_P")
    fields = ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")
    ws = _lib.workspace(dev, 1 << 30)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for (K, N) in ROUTE_LAYERS + ROUTE_NARROW_LAYERS:
        views = _weight_views(pool, N, K)
        nblk = -(-N // 256)
        for M in ms:
            if M > 128 and (K, N) in ROUTE_LAYERS and M not in (160, 256):
                continue
            qx = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
            sa = torch.rand(M, device=dev) * 0.01
            s0 = (torch.rand(N, device=dev) * 1e-3).half()
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            call = lambda r: gemm_w4a8(qx, sa, views[r % len(views)], s0, N, y=y, ws=ws)
            best_d, plan_d = float("inf"), ""
            for c in gemm_w4a8_decode_candidates(M, N, K):
                os.environ["W4A8_DECODE_PLAN"] = ",".join(str(v) for v in c)
                if tuple(gemm_w4a8_plan(M, N, K)[f] for f in fields) != c:
                    continue
                us = graph_time(call, reps)
                if us < best_d:
                    best_d, plan_d = us, ",".join(str(v) for v in c)
            os.environ.pop("W4A8_DECODE_PLAN", None)
            best_p, cfg_p = float("inf"), ""
            for tm in (4, 8, 16):
                tiles = -(-M // (16 * tm)) * nblk
                for s in ((1, 2, 3, 4) if tm < 16 else (1,)):
                    if s > 1 and (tiles * s > cus or (K // 128) // s < 16):
                        continue
                    os.environ["W4A8_PREFILL_TM"] = str(tm)
                    os.environ["W4A8_PREFILL_P"] = str(tiles * s if s > 1 else 0)
                    us = graph_time(call, reps)
                    if us < best_p:
                        best_p, cfg_p = us, "tm%d s%d" % (tm, s)
            for k in keys:
                os.environ.pop(k, None)
            p = gemm_w4a8_plan(M, N, K)
            picked = ("%d:" % p["kind"]) + ",".join(str(p[f]) for f in fields)
            us = graph_time(call, reps)
            writer.writerow([M, N, K, round(best_d, 3), plan_d, round(best_p, 3), cfg_p, picked, round(us, 3)])
            print("route M=%d N=%d K=%d decode %.2f us prefill %.2f us picked %s %.2f us"
                  % (M, N, K, best_d, best_p, picked, us), flush=True)


WIDE_FIELDS = ("M", "N", "K", "kind", "plan", "us")
# 15 layers of the 7B / 70B family and their tensor-parallel shards (K, N)
WIDE_LAYERS = ((11008, 4096), (14336, 4096), (28672, 4096), (8192, 4096), (5120, 4096), (4096, 4096),
               (11008, 2048), (8192, 2048), (4096, 2048), (28672, 2048), (13824, 5120), (8192, 6144),
               (4096, 6144), (8192, 1024), (2048, 4096))


def wide_shapes(n, seed, outputs=(0, 1 << 20), tokens=(129, 256)):
    """Random (M, N, K) with M in `tokens` (default 129..256) and M x N in
    the `outputs` range (default: at most 2^20): M uniform, K log-uniform in
    2048..28672, N log-uniform in max(512, lo / M)..hi / M (multiples of
    128)."""
    rng = np.random.default_rng(seed)
    lo, hi = outputs
    out = []
    while len(out) < n:
        M = int(rng.integers(tokens[0], tokens[1] + 1))
        K = 128 * int(round(2 ** rng.uniform(math.log2(16), math.log2(224))))
        N = 128 * int(round(2 ** rng.uniform(math.log2(max(512, lo // M) / 128), math.log2((hi // M) / 128))))
        if N >= 512 and lo < M * N <= hi:
            out.append((M, N, K))
    return out


def mid_shapes(n, seed):
    """Random (M, N, K) with 65..128 tokens on which gemm_w4a8 takes the decode
    kernels (the 64 x 256 many-token tiles fill under half of 256 CUs): M
    uniform, K log-uniform in 2048..28672, N log-uniform in 512..16384
    (multiples of 128)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(65, 129))
        K = 128 * int(round(2 ** rng.uniform(math.log2(16), math.log2(224))))
        N = 128 * int(round(2 ** rng.uniform(math.log2(4), math.log2(128))))
        if -(-M // 64) * -(-N // 256) * 2 < 256:
            out.append((M, N, K))
    return out


def wide(writer, shapes, reps=10):
    """129..1024 tokens: every decode candidate, the many-token kernel at TM 4 / 8
    with every tile split into s = 1..4 K ranges, and the plan gemm_w4a8 picks."""
    import torch

    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, gemm_w4a8_decode_candidates, gemm_w4a8_plan
    dev = torch.device("cuda:0")
    pool = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev)
    ws = _lib.workspace(dev, 1 << 30)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    fields = ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")
    keys = ("W4A8_DECODE_PLAN", "W4A8_PREFILL_TM", "W4A8_PREFILL_P")
    ratios, route = [], []
    for (M, N, K) in shapes:
        views = _weight_views(pool, N, K)
        qx = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        sa = torch.rand(M, device=dev) * 0.01
        s0 = (torch.rand(N, device=dev) * 1e-3).half()
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        call = lambda r: gemm_w4a8(qx, sa, views[r % len(views)], s0, N, y=y, ws=ws)
        dec, pre = {}, {}
        for c in gemm_w4a8_decode_candidates(M, N, K):
            os.environ["W4A8_DECODE_PLAN"] = ",".join(str(v) for v in c)
            if tuple(gemm_w4a8_plan(M, N, K)[f] for f in fields) == c:
                dec[os.environ["W4A8_DECODE_PLAN"]] = graph_time(call, reps)
        os.environ.pop("W4A8_DECODE_PLAN", None)
        nblk = -(-N // 256)
        for tm in (4, 8):
            tiles = -(-M // (16 * tm)) * nblk
            for sp in (1, 2, 3, 4):
                if sp > 1 and (tiles * sp > cus or (K // 128) // sp < 16):
                    continue
                os.environ["W4A8_PREFILL_TM"] = str(tm)
                os.environ["W4A8_PREFILL_P"] = str(tiles * sp if sp > 1 else 0)
                pre["tm%d s%d" % (tm, sp)] = graph_time(call, reps)
        for k in keys:
            os.environ.pop(k, None)
        p = gemm_w4a8_plan(M, N, K)
        picked = ("%d:" % p["kind"]) + ",".join(str(p[f]) for f in fields)
        us = graph_time(call, reps)
        for kind, d in (("decode", dec), ("prefill", pre)):
            for plan, t in d.items():
                writer.writerow([M, N, K, kind, plan, round(t, 3)])
        writer.writerow([M, N, K, "picked", picked, round(us, 3)])
        bd, bp = min(dec.values()), min(pre.values())
        if p["kind"] == 0:
            ratios.append(us / bd)
        route.append((p["kind"], bp / us if p["kind"] == 0 else bd / us))
        print("wide M=%d N=%d K=%d best decode %.2f us best prefill %.2f us picked %s %.2f us"
              % (M, N, K, bd, bp, picked, us), flush=True)
    if ratios:
        geo = math.exp(sum(math.log(r) for r in ratios) / len(ratios))
        print("picked decode plan / best decode plan: geomean %.3f, max %.3f over %d shapes"
              % (geo, max(ratios), len(ratios)))
    for kind in (0, 1):
        r = [v for k, v in route if k == kind]
        if r:
            print("picked %s: the other kernel's best at %.2f-%.2fx the picked time (%d shapes)"
                  % ("decode" if kind == 0 else "many-token", min(r), max(r), len(r)), flush=True)


def splits(writer, ms=(96, 160, 256, 384, 512, 768), reps=10):
    """Many-token kernel: TM 4 / 8 with each tile split into s equal K ranges, TM 16 whole."""
    import torch

    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, gemm_w4a8_plan
    dev = torch.device("cuda:0")
    pool = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev)
    ws = _lib.workspace(dev, 1 << 30)
    keys = ("W4A8_PREFILL_TM", "W4A8_PREFILL_P")
    for (K, N) in SPLIT_LAYERS:
        views = _weight_views(pool, N, K)
        s0 = (torch.rand(N, device=dev) * 1e-3).half()
        nblk = -(-N // 256)
        for M in ms:
            qx = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
            sa = torch.rand(M, device=dev) * 0.01
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            call = lambda r: gemm_w4a8(qx, sa, views[r % len(views)], s0, N, y=y, ws=ws)
            for k in keys:
                os.environ.pop(k, None)
            p = gemm_w4a8_plan(M, N, K)
            picked = "%d:%d:%d" % (p["kind"], p["mt"], p["splitk"])
            picked_us = graph_time(call, reps)
            runs = [(tm, s) for tm in (4, 8) for s in (1, 2, 3, 4, 6, 8)] + [(16, 1)]
            for tm, s in runs:
                tiles = -(-M // (16 * tm)) * nblk
                P = tiles * s if s > 1 else 0
                if P > 512 or (s > 1 and (K // 128) // s < 4):
                    continue
                os.environ["W4A8_PREFILL_TM"], os.environ["W4A8_PREFILL_P"] = str(tm), str(P)
                writer.writerow([M, N, K, tm, s, P, round(graph_time(call, reps), 3), picked, round(picked_us, 3)])
            for k in keys:
                os.environ.pop(k, None)
            print("splits M=%d N=%d K=%d picked %s %.2f us" % (M, N, K, picked, picked_us), flush=True)


def w16(writer, ms=(17, 32, 48, 64), reps=20):
    """gemm_w4a16 over (NT, MT); MT = 2 must give the bits of MT = 1."""
    import torch

    from w4a8_quantized_linear_amd import gemm_w4a16
    dev = torch.device("cuda:0")
    pool = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev)
    keys = ("W4A8_W16_NT", "W4A8_W16_MT")
    for (K, N) in W16_LAYERS:
        views = _weight_views(pool, N, K)
        s0 = (torch.rand(N, device=dev) * 1e-3).half()
        for M in ms:
            x = (torch.randn((M, K), device=dev) * 0.5).half()
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            call = lambda r: gemm_w4a16(x, views[r % len(views)], s0, N, y=y)
            for k in keys:
                os.environ.pop(k, None)
            default = graph_time(call, reps)
            for nt in (1, 2, 4):
                ref = None
                for mt in (1, 2):
                    os.environ["W4A8_W16_NT"], os.environ["W4A8_W16_MT"] = str(nt), str(mt)
                    out = gemm_w4a16(x, views[0], s0, N)
                    if ref is None:
                        ref = out
                    elif not torch.equal(out, ref):
                        raise SystemExit("two token tiles differ from one: M=%d N=%d K=%d NT=%d" % (M, N, K, nt))
                    writer.writerow([M, N, K, nt, mt, round(graph_time(call, reps), 3), round(default, 3)])
            for k in keys:
                os.environ.pop(k, None)
            print("w16 M=%d N=%d K=%d default %.2f us" % (M, N, K, default), flush=True)


def compare(shapes, writer, reps=50, rounds=3):
    import torch

    from w4a8_quantized_linear_amd import gemm_w4a8, gemm_w4a8_plan, w4a8_packed_weight_bytes
    dev = torch.device("cuda:0")
    pool = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev)
    fields = ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")
    for (M, N, K) in shapes:
        wb = w4a8_packed_weight_bytes(N, K)
        stride = (wb + 4095) // 4096 * 4096
        views = [pool[i * stride:i * stride + wb] for i in range(min(max(1, (1 << 30) // stride), 64))]
        qx = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        sa = torch.rand(M, device=dev) * 0.01
        s0 = (torch.rand(N, device=dev) * 1e-3).half()
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        plans, times = {}, {"0": [], "1": []}
        for _ in range(rounds):
            for sel in ("0", "1"):
                os.environ["W4A8_SELECTOR"] = sel
                plans[sel] = gemm_w4a8_plan(M, N, K)
                times[sel].append(graph_time(lambda r: gemm_w4a8(qx, sa, views[r % len(views)], s0, N, y=y), reps))
        os.environ.pop("W4A8_SELECTOR", None)
        desc = lambda p: "%d:%s" % (p["kind"], ",".join(str(p[f]) for f in fields))
        tr, ts = float(np.median(times["0"])), float(np.median(times["1"]))
        writer.writerow([M, N, K, desc(plans["0"]), desc(plans["1"]), round(tr, 3), round(ts, 3), round(ts / tr, 4)])
        print("compared M=%d N=%d K=%d rules %.2f us selector %.2f us" % (M, N, K, tr, ts), flush=True)


def launch(ms, N, K, calls):
    """`calls` eager gemm_w4a8 calls per token count, weights rotated past the caches."""
    import torch
    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, w4a8_packed_weight_bytes
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    nbytes = w4a8_packed_weight_bytes(N, K)
    nrot = max(2, math.ceil((1 << 30) / nbytes))
    wbuf = torch.randint(0, 256, (nrot, nbytes), dtype=torch.uint8, device=dev, generator=g)
    s0 = torch.full((N,), 0.01, dtype=torch.float16, device=dev)
    ws = _lib.workspace(dev, max(_lib.gemm_w4a8_workspace_bytes(M, N, K) for M in ms))
    for M in ms:
        qx = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        sa = torch.full((M,), 0.01, dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        print("M=%d N=%d K=%d plan %s" % (M, N, K, _lib.gemm_w4a8_plan_detail(M, N, K)), flush=True)
        for c in range(calls):
            gemm_w4a8(qx, sa, wbuf[c % nrot], s0, N, y=y, ws=ws)
        torch.cuda.synchronize()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("out", nargs="?")
    ap.add_argument("--launch", default=None, help="M1,M2,..: eager calls of the chosen plan (profiler runs)")
    ap.add_argument("--n", type=int, default=11008)
    ap.add_argument("--k", type=int, default=4096)
    ap.add_argument("--calls", type=int, default=30)
    ap.add_argument("--shapes", type=int, default=120)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--eval", action="store_true")
    ap.add_argument("--compare", action="store_true")
    ap.add_argument("--route", action="store_true", help="decode against many-token kernel at 72..256 tokens")
    ap.add_argument("--w16", action="store_true", help="gemm_w4a16 tiles-per-workgroup sweep at 17..64 tokens")
    ap.add_argument("--splits", action="store_true", help="many-token kernel: splits per tile at 96..768 tokens")
    ap.add_argument("--wide", action="store_true",
                    help="129..256 tokens: every decode plan and many-token split, random shapes (--shapes, --seed)")
    ap.add_argument("--wide-layers", action="store_true", help="as --wide, on 15 7B / 70B layers at 136..512 tokens")
    ap.add_argument("--mid", action="store_true", help="as --wide, on random shapes with 65..128 tokens")
    ap.add_argument("--outputs", default="0,1048576", help="lo,hi: the M x N range of --wide's random shapes")
    ap.add_argument("--wide-m", default="129,256", help="lo,hi: the token counts of --wide's random shapes")
    ap.add_argument("--mid-layers", action="store_true", help="as --wide, on 7B / 70B and narrow layers at 72..128 tokens")
    ap.add_argument("--wave-n", type=int, default=None,
                    help="time only the candidates of this decode kernel family (0, 1, 2)")
    ap.add_argument("--shapes-from", default=None,
                    help="time the (M, N, K) shapes of an earlier sweep's CSV (M <= --max-m)")
    ap.add_argument("--max-m", type=int, default=64)
    ap.add_argument("--m-range", default="1,64", help="lo,hi: token counts of the random shapes (log-uniform)")
    ap.add_argument("--part", default="0/1", help="i/n: time every n-th shape from the i-th (to split a sweep)")
    args = ap.parse_args(argv)
    if args.launch:
        launch([int(v) for v in args.launch.split(",")], args.n, args.k, args.calls)
        return 0
    if args.out is None:
        ap.error("the output CSV is required")
    if args.wide or args.wide_layers or args.mid or args.mid_layers:
        if args.mid:
            shapes = mid_shapes(args.shapes, args.seed)
        elif args.mid_layers:
            layers = sorted(set(ROUTE_LAYERS + ROUTE_NARROW_LAYERS + WIDE_LAYERS))
            shapes = [(M, N, K) for (K, N) in layers for M in (72, 96, 112, 128)
                      if -(-M // 64) * -(-N // 256) * 2 < 256]
        elif args.wide:
            shapes = wide_shapes(args.shapes, args.seed, tuple(int(v) for v in args.outputs.split(",")),
                                 tuple(int(v) for v in args.wide_m.split(",")))
        else:
            shapes = [(M, N, K) for (K, N) in WIDE_LAYERS for M in (136, 160, 192, 224, 256, 320, 384, 448, 512)
                      if M * N <= (1 << 20)]
        with open(args.out, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(WIDE_FIELDS)
            wide(w, shapes)
        return 0
    if args.route or args.w16 or args.splits:
        fields, fn = {"route": (ROUTE_FIELDS, route), "w16": (W16_FIELDS, w16),
                      "splits": (SPLIT_FIELDS, splits)}[next(k for k in ("route", "w16", "splits") if getattr(args, k))]
        with open(args.out, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(fields)
            fn(w)
        return 0
    if args.compare:
        shapes = EVAL_SHAPES + [(M, 11008, 4096) for M in (1, 8, 16, 32, 64)]
        with open(args.out, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(COMPARE_FIELDS)
            compare(shapes, w)
        return 0
    m_lo, m_hi = (int(v) for v in args.m_range.split(","))
    shapes = EVAL_SHAPES if args.eval else random_shapes(args.shapes, args.seed, m_lo, m_hi)
    if args.shapes_from:
        import gzip
        with (gzip.open(args.shapes_from, "rt") if args.shapes_from.endswith(".gz") else open(args.shapes_from)) as f:
            shapes = sorted({(int(r["M"]), int(r["N"]), int(r["K"])) for r in csv.DictReader(f)})
    shapes = [s for s in shapes if s[0] <= args.max_m]
    part, nparts = (int(v) for v in args.part.split("/"))
    shapes = shapes[part::nparts]
    with open(args.out, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(FIELDS)
        measure(shapes, "eval" if args.eval else "train", w, wave_n=args.wave_n)
    return 0


if __name__ == "__main__":
    sys.exit(main())
