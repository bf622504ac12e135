"""Benchmark: one head-wise sparse global-attention layer at S = 100 frames.

A step is one pass of the whole hot path on one synthetic sequence: the
correspondence index build (DINO cosine top-K over other frames), the
vertical heads' mean-query probe + top-K, and the 16-head sparse attention
(shared-key heads on the matrix cores, per-query correspondence sets on the
gather path).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  Besides the contract fields it carries:
  breakdown    per launch group, ms per step (HIP events on the stream)
  attn_only_ms the layer with the index cached (what every later layer costs)
  dense_ms     the in-house dense flash attention at the same shape
  roofline     the dominant kernel against the MI355X peak, with counter figures;
               roofline_other.*.alone: the gather and the shared-key kernels each
               timed on their own heads
  sequence_lengths  the step, the cached-index layer and the dense kernel at
               S = 32 and S = 500 (latency against sequence length)
  cpu_baseline the CPU oracle, timed on a bounded row sample, extrapolated
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms per 16-head sparse global-attn layer at S=100 frames; HBM GB/s & MFMA % of peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

# Counter readings of the step's kernel groups on the S = 100 workload
# (rocprofv3 --pmc, one pass per group of counters; per step: the index
# build's cosine GEMM is 1 seed-bound + 1 symmetric launch, the fused
# per-frame build's GEMM 1 sampled + 1 filtered symmetric launch, the
# shared-key attention its launch(es) of one layer, the others one;
# shared_attention_alone: the 13 shared-key heads on their own, no gather
# beside them, full occupancy).  executed_tflop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
# FLOP; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x
# 1024 SIMDs), the share of SIMD cycles the matrix cores were busy while the
# kernel ran; fetch/write = FETCH_SIZE / WRITE_SIZE in KiB, scaled by what
# the counters read for a plain device copy in the same run (WRITE_SIZE reads
# the copied KiB exactly, FETCH_SIZE half of them).  A group's figures hold
# for the kernel source with the recorded digest only; after any change they
# are reported as null until the counters are taken again.
COUNTERS = {
    "config": 3,
    "fetch_scale": 1.99993,
    "write_scale": 1.0,
    "groups": {
        "cosine_gemm": {"source": ["head_wise_dynamic_amd/csrc/corr_cos.hip", "head_wise_dynamic_amd/csrc/corr_index.hip"],
            "sha256": "bddb6f37cfe3da0e81df60bc8b8afe971104fa7b5dd0fcbca6c6f787b96d5421",
            "executed_tflop": 20.034, "mfma_busy": 0.4367,
            "fetch_kib": 38557448.1, "write_kib": 2028201.8},
        "per_frame_gemm": {"source": ["head_wise_dynamic_amd/csrc/corr_cos.hip", "head_wise_dynamic_amd/csrc/corr_index.hip"],
            "sha256": "bddb6f37cfe3da0e81df60bc8b8afe971104fa7b5dd0fcbca6c6f787b96d5421",
            "executed_tflop": 22.8345, "mfma_busy": 0.3475,
            "fetch_kib": 40189044.6, "write_kib": 6029793.2},
        "shared_attention": {"source": ["head_wise_dynamic_amd/csrc/attn_mfma.hip", "head_wise_dynamic_amd/csrc/api.cpp"],
            "sha256": "ac511e4027adae7c4bc1b54987e0e2f7fde363fc5c4989dd9c5c43f9c5330ce3",
            "executed_tflop": 2.7005, "mfma_busy": 0.3127,
            "fetch_kib": 454424.6, "write_kib": 229973.2},
        "shared_attention_alone": {"source": ["head_wise_dynamic_amd/csrc/attn_mfma.hip", "head_wise_dynamic_amd/csrc/api.cpp"],
            "sha256": "ac511e4027adae7c4bc1b54987e0e2f7fde363fc5c4989dd9c5c43f9c5330ce3",
            "executed_tflop": 2.6465, "mfma_busy": 0.447,
            "fetch_kib": 347761.8, "write_kib": 223275.0},
        "dense": {"source": ["head_wise_dynamic_amd/csrc/attn_mfma.hip", "head_wise_dynamic_amd/csrc/api.cpp"],
            "sha256": "ac511e4027adae7c4bc1b54987e0e2f7fde363fc5c4989dd9c5c43f9c5330ce3",
            "executed_tflop": 77.3724, "mfma_busy": 0.4934,
            "fetch_kib": 6825756.2, "write_kib": 274800.4},
        "gather_attention": {"source": ["head_wise_dynamic_amd/csrc/attn_valu.hip", "head_wise_dynamic_amd/csrc/api.cpp"],
            "sha256": "b3ebddeb6183537036f1220e4c0328f5c48983fa7b5e18cb434fe94dfc1add00",
            "executed_tflop": 0.0, "mfma_busy": None,
            "fetch_kib": 12567492.6, "write_kib": 51337.5},
    },
}


def counters_for(group, config):
    """The recorded counter figures of a kernel group, with its HBM traffic in
    GB, or None for another workload or when the sources no longer match the
    ones they were taken on (the kernel's file, or a list of files: the
    kernel and the code that schedules its launches; the digest is over
    their bytes in order)."""
    import hashlib
    rec = COUNTERS["groups"].get(group)
    if rec is None or config != COUNTERS["config"]:
        return None
    srcs = rec["source"] if isinstance(rec["source"], list) else [rec["source"]]
    h = hashlib.sha256()
    try:
        for src in srcs:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    if h.hexdigest() != rec["sha256"]:
        return None
    out = dict(rec)
    out["traffic_gb"] = (rec["fetch_kib"] * COUNTERS["fetch_scale"] + rec["write_kib"] * COUNTERS["write_scale"]) \
        * 1024 / 1e9
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload id (3 = S=100 VGGT-scale layer)")
    ap.add_argument("--reps", type=int, default=10, help="reps of each breakdown measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--block", type=int, default=37,
                    help="also time the block-wise index with blocks of this many patches (0: skip)")
    ap.add_argument("--block-k", type=int, default=7, help="blocks kept per query block for --block")
    ap.add_argument("--corr-stride", type=int, default=64,
                    help="also time the layer with its correspondence heads united with this stride (0: skip)")
    ap.add_argument("--broadcast-radius", type=int, default=1,
                    help="also time the layer with its position heads as broadcast heads of this window "
                         "radius on the patch grid (-1: skip)")
    ap.add_argument("--no-qk-index", action="store_true",
                    help="skip timing the index built from the first correspondence head's logits")
    ap.add_argument("--no-seq-lengths", action="store_true",
                    help="skip the S = 32 and S = 500 steps (latency against sequence length)")
    ap.add_argument("--no-alone", action="store_true",
                    help="skip timing the gather and the shared-key kernels each on their own heads")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip timing the 24-layer stack (index built once, the stack's per-layer plans)")
    ap.add_argument("--stack-inputs", type=int, default=3,
                    help="distinct per-layer Q/K/V sets the 24-layer stack rotates through")
    ap.add_argument("--no-profile", action="store_true",
                    help="skip timing one offline-profiling pass (Sec. 4.2) over this sequence")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device to device twice (a known-size kernel for HBM counters)")
    ap.add_argument("--per-frame-k", type=int, default=4,
                    help="also time the per-frame index build with this K per frame (0: skip)")
    ap.add_argument("--cpu-row-stride", type=int, default=5,
                    help="CPU baseline: attention on every n-th query row of every head")
    ap.add_argument("--cpu-corr-rows", type=int, default=512,
                    help="CPU baseline: correspondence index rows timed")
    return ap.parse_args()


def key_counts(w):
    """Per head: number of (query, key) pairs the head's key sets hold."""
    g = w.geom
    S, ns, P, N, T = g.S, g.ns, g.P, g.N, g.T
    out = []
    for role, budget, anchor, _ in w.plan:
        if role == 0:       # position
            per_frame = [ns * S + P + (P if f != anchor else 0) for f in range(S)]
            out.append(("shared", T * sum(per_frame)))
        elif role == 1:     # vertical
            out.append(("shared", N * min(budget, N)))
        elif role == 3:     # scanning
            on = -(-N // budget)
            sp_on = sum(1 for f in range(S) for t in range(ns) if (f * T + t) % budget == 0)
            out.append(("shared", N * (on + ns * S - sp_on)))
        elif role == 4:
            out.append(("shared", N * N))
        else:               # correspondence: special rows dense, patch rows gathered
            out.append(("shared", ns * S * N))
            out.append(("gather", g.Np * min(w.corr_K, (S - 1) * P)))
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    import head_wise_dynamic_amd as saf
    from workload import make_inputs

    t_gen = time.time()
    w = make_inputs(args.config)
    g = w.geom
    print(f"[bench] generated {w.name} N={g.N} in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v, dino = dev(w.q), dev(w.k), dev(w.v), dev(w.dino)
    o = torch.empty_like(q)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        ctx.build_corr_index(dino, w.corr_K)
        ctx.sparse_attention(w.plan, q, k, v, o=o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # ---- breakdown: per launch group, events recorded by the library
    ctx.set_kernel_timing(True)
    ctx.read_kernel_timing()
    groups = {}
    for _ in range(args.reps):
        step()
        torch.cuda.synchronize()
        per = {}
        for name, ms in ctx.read_kernel_timing():
            per[name] = per.get(name, 0.0) + ms
            per["launches:" + name] = per.get("launches:" + name, 0) + 1
        for name, ms in per.items():
            groups.setdefault(name, []).append(ms)
    launches = {}   # per layer: summed time of each launch group
    for _ in range(args.reps):
        ctx.sparse_attention(w.plan, q, k, v, o=o)
        torch.cuda.synchronize()
        per = {}
        for name, ms in ctx.read_kernel_timing():
            per[name] = per.get(name, 0.0) + ms
        for name, ms in per.items():
            launches.setdefault(name, []).append(ms)
    ctx.set_kernel_timing(False)
    launch_counts = {n.split(":", 1)[1]: int(v[0]) for n, v in groups.items() if n.startswith("launches:")}
    breakdown = {n: round(statistics.median(v), 4) for n, v in groups.items() if not n.startswith("launches:")}

    # layer with the index cached (every layer after the first of a sequence)
    attn = []
    for _ in range(args.reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ctx.sparse_attention(w.plan, q, k, v, o=o)
        e1.record(stream)
        torch.cuda.synchronize()
        attn.append(e0.elapsed_time(e1))
    attn_ms = statistics.median(attn)

    # each kernel group on its own heads (contexts of their own, the same
    # per-head data): the gathered heads alone, and the other heads alone, so
    # the in-layer rates (the two kernels share the chip) can be read against
    # the rates each reaches by itself
    alone = None
    if not args.no_alone:
        corr_h = [h for h, r in enumerate(w.plan) if r[0] == 2]
        other_h = [h for h, r in enumerate(w.plan) if r[0] != 2]

        def group_alone(heads, name):
            sub = saf.Context(g.S, g.ns, g.P, len(heads), g.d, torch.bfloat16)
            qs, ks, vs = (t[heads].contiguous() for t in (q, k, v))
            os_ = torch.empty_like(qs)
            plan = [w.plan[h] for h in heads]
            if any(r[0] == 2 for r in plan):
                sub.set_corr_index(ctx.get_corr_index())
            sub.sparse_attention(plan, qs, ks, vs, o=os_)
            torch.cuda.synchronize()
            sub.set_kernel_timing(True)
            sub.read_kernel_timing()
            ts = []
            for _ in range(args.reps):
                sub.sparse_attention(plan, qs, ks, vs, o=os_)
                torch.cuda.synchronize()
                ts.append(sum(ms for n, ms in sub.read_kernel_timing() if n == name))
            sub.set_kernel_timing(False)
            sub.close()
            del qs, ks, vs, os_
            return statistics.median(ts)

        alone = {"gather_attention_ms": round(group_alone(corr_h, "gather_attention"), 4),
                 "shared_attention_ms": round(group_alone(other_h, "shared_attention"), 4),
                 "heads": {"gather": corr_h, "shared": other_h}}

    # cold caches: 1 GiB scrub before each rep
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold = []
    for _ in range(max(3, args.reps // 2)):
        scrub.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del scrub

    # per-step spread: every step timed on its own (warm caches)
    single = []
    for _ in range(max(10, args.reps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        single.append(e0.elapsed_time(e1))
    single.sort()
    pct = lambda p: single[min(len(single) - 1, int(round(p * (len(single) - 1))))]
    step_spread = {"p10": round(pct(0.1), 3), "p50": round(pct(0.5), 3), "p90": round(pct(0.9), 3),
                   "n": len(single)}

    # the 24-layer stack of the same geometry: the index built once, then the
    # stack's 24 per-layer plans (roles permuted per layer; layers 10-16 with
    # six correspondence heads).  Every layer reads Q/K/V buffers other than
    # its predecessor's: --stack-inputs distinct layers' inputs (the stack
    # workload's own seeds for layers 0, 1, ...) are generated and layer l
    # uses set l mod that count, so no layer finds the previous layer's K/V
    # in the caches (each set is 845 MB, the last-level cache 256 MB).
    stack = None
    if not args.no_stack and args.config == 3 and args.stack_inputs > 0:
        from workload import layer_roles, make_inputs as make_layer_inputs
        t_gen = time.time()
        sets = []
        for l in range(args.stack_inputs):
            wl = make_layer_inputs(4, layer=l, dino=False)
            sets.append(tuple(dev(a) for a in (wl.q, wl.k, wl.v)))
            del wl
            if args.stack_inputs > 3:
                print(f"[bench] stack input set {l + 1}/{args.stack_inputs}", file=sys.stderr, flush=True)
        print(f"[bench] generated {len(sets)} stack input sets in {time.time() - t_gen:.1f}s", file=sys.stderr,
              flush=True)
        plans = []
        for l in range(24):
            roles, budgets = layer_roles(4, l)
            plans.append([(r, b, 0, 0) for r, b in zip(roles, budgets)])

        def run_stack():
            for l, pl in enumerate(plans):
                ql, kl, vl = sets[l % len(sets)]
                ctx.sparse_attention(pl, ql, kl, vl, o=o)

        ctx.build_corr_index(dino, w.corr_K)
        run_stack()
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        ctx.build_corr_index(dino, w.corr_K)
        e1.record(stream)
        run_stack()
        e2.record(stream)
        torch.cuda.synchronize()
        stack = {"layers": 24, "distinct_qkv_sets": len(sets), "index_ms": round(e0.elapsed_time(e1), 3),
                 "layers_ms": round(e1.elapsed_time(e2), 3), "total_ms": round(e0.elapsed_time(e2), 3)}
        del sets

    dense_ms = None
    if not args.no_dense:
        od = torch.empty_like(q)
        ctx.dense_attention(q, k, v, o=od)
        torch.cuda.synchronize()
        dn = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ctx.dense_attention(q, k, v, o=od)
            e1.record(stream)
            torch.cuda.synchronize()
            dn.append(e0.elapsed_time(e1))
        dense_ms = statistics.median(dn)
        del od

    # per-frame index (K best of every other frame), built in a context of its
    # own so the step's cached index is untouched; not part of the step
    per_frame = None
    if args.per_frame_k > 0:
        pctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)

        def build_ms(mode):
            pctx.build_corr_index(dino, args.per_frame_k, mode=mode)
            torch.cuda.synchronize()
            pf = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                pctx.build_corr_index(dino, args.per_frame_k, mode=mode)
                e1.record(stream)
                torch.cuda.synchronize()
                pf.append(e0.elapsed_time(e1))
            return statistics.median(pf)

        stored_ms = build_ms(saf.SAF_CORR_PER_FRAME_STORED)
        pf_ms = build_ms(saf.SAF_CORR_PER_FRAME)
        per_frame = {"K_per_frame": args.per_frame_k, "row_length": pctx.corr_k(), "build_ms": round(pf_ms, 3),
                     "recomputed_rows": len(pctx.recomputed_rows()),
                     "tflops": round(2.0 * g.Np * g.Np * w.Df / (pf_ms * 1e-3) / 1e12, 2),
                     "stored_cosines_build_ms": round(stored_ms, 3)}
        pctx.close()

    # the index taken from the first correspondence head's logits (K as the
    # DINO index), in a context of its own; not part of the step
    qk = None
    if not args.no_qk_index:
        h0 = [h for h, p in enumerate(w.plan) if p[0] == 2][0]
        qctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
        qctx.build_corr_index_qk(q, k, h0, w.corr_K)
        torch.cuda.synchronize()
        qt = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            qctx.build_corr_index_qk(q, k, h0, w.corr_K)
            e1.record(stream)
            torch.cuda.synchronize()
            qt.append(e0.elapsed_time(e1))
        qk = {"head": h0, "K": w.corr_K, "build_ms": round(statistics.median(qt), 3),
              "tflops": round(2.0 * g.Np * g.Np * g.d / (statistics.median(qt) * 1e-3) / 1e12, 2)}
        qctx.close()

    # the layer with its correspondence heads as correspondence top-K united
    # with a stride (cached total index); not part of the step
    corr_stride = None
    if args.corr_stride > 0:
        csplan = [(5, args.corr_stride, a, f) if r == 2 else (r, b, a, f) for (r, b, a, f) in w.plan]
        ctx.sparse_attention(csplan, q, k, v, o=o)
        torch.cuda.synchronize()
        ct = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ctx.sparse_attention(csplan, q, k, v, o=o)
            e1.record(stream)
            torch.cuda.synchronize()
            ct.append(e0.elapsed_time(e1))
        corr_stride = {"stride": args.corr_stride, "attn_only_ms": round(statistics.median(ct), 4)}

    # the layer with its position heads as broadcast heads (the local window
    # of every frame around the query's grid position); not part of the step
    broadcast = None
    if args.broadcast_radius >= 0:
        gw = math.isqrt(g.P) if math.isqrt(g.P) ** 2 == g.P else 0
        bplan = [(6, args.broadcast_radius, gw, f) if r == 0 else (r, b, a, f) for (r, b, a, f) in w.plan]
        ctx.sparse_attention(bplan, q, k, v, o=o)
        torch.cuda.synchronize()
        bt = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ctx.sparse_attention(bplan, q, k, v, o=o)
            e1.record(stream)
            torch.cuda.synchronize()
            bt.append(e0.elapsed_time(e1))
        side = 2 * args.broadcast_radius + 1
        broadcast = {"radius": args.broadcast_radius, "grid_width": gw,
                     "heads": sum(1 for p in w.plan if p[0] == 0),
                     "keys_per_interior_patch_query": g.ns * g.S + g.S * (side * side if gw else side),
                     "attn_only_ms": round(statistics.median(bt), 4)}

    # block-wise index (blocks of --block patches, --block-k blocks per query
    # block) and the layer on it, in a context of its own; not part of the step
    block = None
    if args.block > 0 and g.P % args.block == 0:
        bctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
        bplan = [(r, 0 if r == 2 else b, a, f) for (r, b, a, f) in w.plan]
        bctx.build_corr_index_blocks(dino, args.block, args.block_k)
        bctx.sparse_attention(bplan, q, k, v, o=o)
        torch.cuda.synchronize()
        bt, ba = [], []
        for _ in range(3):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
            bctx.build_corr_index_blocks(dino, args.block, args.block_k)
            e1.record(stream)
            bctx.sparse_attention(bplan, q, k, v, o=o)
            e2.record(stream)
            torch.cuda.synchronize()
            bt.append(e0.elapsed_time(e1))
            ba.append(e1.elapsed_time(e2))
        block = {"block": args.block, "K_blocks": args.block_k, "row_length": bctx.corr_k(),
                 "build_ms": round(statistics.median(bt), 3), "attn_only_ms": round(statistics.median(ba), 4),
                 "step_ms": round(statistics.median(bt) + statistics.median(ba), 3)}
        bctx.close()

    # one offline-profiling pass (Sec. 4.2) with this sequence as the single
    # calibration sample: dense reference, baseline at sigma = 0.85 and eight
    # candidates (the broadcast one on the patch grid), per-head errors and the
    # selection; not part of the step
    prof = None
    if not args.no_profile:
        from head_wise_dynamic_amd import profiling
        pctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
        grid_w = math.isqrt(g.P) if math.isqrt(g.P) ** 2 == g.P else 0
        cands = [(1, 1024, 0), (1, 2048, 0), (1, 4096, 0), (2, 128, 0), (2, 256, 0), (0, 0, 0), (3, 16, 0),
                 (6, 1, grid_w)]
        smp = dict(q=q, k=k, v=v, dino=dino)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = profiling.profile_heads(pctx, [smp], cands, sigma=0.85)
        torch.cuda.synchronize()
        t_prof = time.perf_counter() - t0
        full = pctx.dense_attention(q, k, v)
        sums = pctx.head_nmse(full, o)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pctx.head_nmse(full, o, out=sums)
        e1.record(stream)
        torch.cuda.synchronize()
        nmse_ms = e0.elapsed_time(e1)
        names = {0: "position", 1: "vertical", 2: "correspondence", 3: "scanning", 4: "dense", 6: "broadcast"}
        prof = {"sigma": 0.85, "configs": [f"{names[r]}:{b}" for r, b, _ in res["configs"]],
                "choice_per_head": [int(c) for c in res["choice"]], "wall_ms": round(t_prof * 1e3, 1),
                "error_kernel_ms": round(nmse_ms, 4),
                "error_kernel_gbs": round(2 * g.H * g.N * g.d * 2 / (nmse_ms * 1e-3) / 1e9, 1)}
        del full
        pctx.close()

    # latency against sequence length (SAF3R Sec. 5.2, Fig. 6): the same step
    # (index build + layer) on the S = 32 and S = 500 workloads, the layer
    # with the index cached, and the dense kernel once; S = 100 is this line.
    # Each workload is generated, run in a context of its own and released;
    # not part of the step.
    seq = None
    if not args.no_seq_lengths and args.config == 3:
        seq = {f"S={g.S}": {"N": g.N, "step_ms": round(ms_per_step, 3), "attn_only_ms": round(attn_ms, 3),
                            "dense_ms": round(dense_ms, 3) if dense_ms else None}}
        for cid in (2, 5):
            t_gen = time.time()
            wl = make_inputs(cid)
            gl = wl.geom
            ql, kl, vl, dl = dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.dino)
            print(f"[bench] generated {wl.name} N={gl.N} in {time.time() - t_gen:.1f}s", file=sys.stderr,
                  flush=True)
            ol = torch.empty_like(ql)
            cl = saf.Context(gl.S, gl.ns, gl.P, gl.H, gl.d, torch.bfloat16)

            def timed_l(fn, reps):
                fn()
                torch.cuda.synchronize()
                ts = []
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1))
                return statistics.median(ts)

            def step_l():
                cl.build_corr_index(dl, wl.corr_K)
                cl.sparse_attention(wl.plan, ql, kl, vl, o=ol)

            st_ms = timed_l(step_l, 3)
            ix_ms = timed_l(lambda: cl.build_corr_index(dl, wl.corr_K), 3)
            at_ms = timed_l(lambda: cl.sparse_attention(wl.plan, ql, kl, vl, o=ol), 3)
            dn_ms = None
            if not args.no_dense:
                dn_ms = timed_l(lambda: cl.dense_attention(ql, kl, vl, o=ol), 1)
            seq[f"S={gl.S}"] = {"N": gl.N, "step_ms": round(st_ms, 3), "index_ms": round(ix_ms, 3),
                                "attn_only_ms": round(at_ms, 3), "dense_ms": round(dn_ms, 3) if dn_ms else None,
                                "speedup_attn_vs_dense": round(dn_ms / at_ms, 2) if dn_ms else None}
            print(f"[bench] {wl.name}: step {st_ms:.2f} ms, layer {at_ms:.2f} ms", file=sys.stderr, flush=True)
            cl.close()
            del wl, ql, kl, vl, dl, ol
            torch.cuda.empty_cache()

    # ---- roofline of the dominant kernel (largest single-kernel share)
    pairs = key_counts(w)
    shared_pairs = sum(p for kind, p in pairs if kind == "shared")
    gather_pairs = sum(p for kind, p in pairs if kind == "gather")
    n_corr = sum(1 for r in w.plan if r[0] == 2)
    d = g.d
    shared_flops = 4.0 * d * shared_pairs
    gather_bytes = gather_pairs * (2 * d * 2) + g.Np * w.corr_K * 4 + n_corr * g.Np * (2 * d * 2)
    cand = {}
    if "shared_attention" in launches:
        t = statistics.median(launches["shared_attention"])
        cand["shared_attention"] = dict(bound="mfma", achieved=shared_flops / (t * 1e-3) / 1e12,
                                        peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", ms=t)
    if "gather_attention" in launches:
        t = statistics.median(launches["gather_attention"])
        cand["gather_attention"] = dict(bound="hbm", achieved=gather_bytes / (t * 1e-3) / 1e9,
                                        peak=PEAK_HBM_GBS, unit="GB/s", ms=t)
    if "cosine_gemm" in groups:
        # the index build's GEMM phases: algorithmic work 2 (S P)^2 Df per
        # step (every pair counted once per direction); the kernel computes the
        # square part of the pair space once per unordered pair
        t = statistics.median(groups["cosine_gemm"])
        cand["cosine_gemm"] = dict(bound="mfma", achieved=2.0 * g.Np * g.Np * w.Df / (t * 1e-3) / 1e12,
                                   peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", ms=t,
                                   launches=launch_counts.get("cosine_gemm", 0))
    dom = max(cand, key=lambda n: cand[n]["ms"])

    def counter_view(name, ms):
        """Counter-based figures of a kernel group at the live time ms: FLOP
        the matrix cores executed (and that rate against the peak), their
        busy share, and the calibrated HBM bytes (and that rate)."""
        c = counters_for(name, args.config)
        if c is None:
            return None
        v = {"mfma_busy": c["mfma_busy"], "traffic_gb": round(c["traffic_gb"], 3),
             "traffic_gbs": round(c["traffic_gb"] / (ms * 1e-3), 1),
             "traffic_frac": round(c["traffic_gb"] / (ms * 1e-3) / PEAK_HBM_GBS, 4)}
        if c["executed_tflop"]:
            v["executed_tflop"] = c["executed_tflop"]
            v["executed_tflops"] = round(c["executed_tflop"] / (ms * 1e-3), 2)
            v["executed_frac"] = round(c["executed_tflop"] / (ms * 1e-3) / PEAK_BF16_TFLOPS, 4)
        return v

    r = cand[dom]
    cv = counter_view(dom, r["ms"])
    roofline = {"kernel": dom, "bound": r["bound"], "achieved": round(r["achieved"], 2), "peak": r["peak"],
                "unit": r["unit"], "frac": round(r["achieved"] / r["peak"], 4),
                "achieved_is": "algorithmic work (every pair of the cosine matrix once per direction) / live time",
                "traffic": cv["traffic_gb"] if cv else None,
                "traffic_unit": "GB of HBM traffic per step (all launches of the kernel), from counters",
                "counters": cv,
                "kernel_ms_per_step": round(r["ms"], 4), "launches_per_step": r.get("launches", 1)}
    others = {n: {"achieved": round(c["achieved"], 2), "unit": c["unit"], "peak": c["peak"],
                  "frac": round(c["achieved"] / c["peak"], 4), "kernel_ms": round(c["ms"], 4),
                  "counters": counter_view(n, c["ms"])}
              for n, c in cand.items() if n != dom}
    if alone:
        # the same algorithmic work per kernel, at its time on its own heads
        alone["gather_attention_gbs"] = round(gather_bytes / (alone["gather_attention_ms"] * 1e-3) / 1e9, 1)
        alone["gather_attention_frac"] = round(alone["gather_attention_gbs"] / PEAK_HBM_GBS, 4)
        # without the correspondence heads, whose dense special rows also run
        # on the matrix cores in the layer
        other_flops = 4.0 * d * (shared_pairs - n_corr * g.ns * g.S * g.N)
        alone["shared_attention_tflops"] = round(other_flops / (alone["shared_attention_ms"] * 1e-3) / 1e12, 2)
        alone["shared_attention_frac"] = round(alone["shared_attention_tflops"] / PEAK_BF16_TFLOPS, 4)
        for n in ("gather_attention", "shared_attention"):
            if n in others:
                others[n]["alone"] = {k: v for k, v in alone.items() if k.startswith(n)}
        if "shared_attention" in others:
            # full occupancy, no gather beside it
            others["shared_attention"]["alone"]["counters"] = counter_view("shared_attention_alone",
                                                                            alone["shared_attention_ms"])
    if dense_ms:
        others["dense"] = {"achieved": round(4.0 * d * g.H * g.N * g.N / (dense_ms * 1e-3) / 1e12, 2),
                           "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
                           "frac": round(4.0 * d * g.H * g.N * g.N / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "kernel_ms": round(dense_ms, 4), "counters": counter_view("dense", dense_ms)}
    corr_flops = 2.0 * g.Np * g.Np * w.Df
    corr_ms = breakdown.get("corr_index")

    def per_frame_counters(pf):
        """The fused per-frame build's two GEMM launches (sampled bounds,
        filtered square): executed FLOP against the whole build's time."""
        c = counters_for("per_frame_gemm", args.config) if pf["K_per_frame"] == 4 else None
        if c is None:
            return None
        return {"gemm_executed_tflop": c["executed_tflop"], "gemm_mfma_busy": c["mfma_busy"],
                "gemm_traffic_gb": round(c["traffic_gb"], 3),
                "executed_frac_of_build": round(c["executed_tflop"] / (pf["build_ms"] * 1e-3) / PEAK_BF16_TFLOPS, 4)}

    # ---- CPU oracle on a bounded sample, extrapolated to the full step
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_row_stride, args.cpu_corr_rows)

    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator standing in for 7Scenes/ScanNet-shaped sequences)",
        "config": {"workload": f"{w.name}: one global-attention layer, S={g.S} frames x (5 special + "
                               f"{g.P} patch) tokens, N={g.N}, H=16, d=64, heads 4 position / 3 vertical "
                               f"(top-{w.plan[4][1]}) / 3 correspondence (top-{w.corr_K}, Df={w.Df}) / "
                               f"6 scanning (stride {w.plan[-1][1]}); step = corr index build + layer",
                   "S": g.S, "N": g.N, "H": g.H, "d": g.d},
        "wall_s_timed_region": round(wall, 3),
        "attn_only_ms": round(attn_ms, 4),
        "cold_step_ms_median": round(statistics.median(cold), 4),
        "step_ms_spread": step_spread,
        "stack_24_layers": stack,
        "breakdown_ms": breakdown,
        "corr_index_tflops": round(corr_flops / (corr_ms * 1e-3) / 1e12, 2) if corr_ms else None,
        "dense_ms": round(dense_ms, 3) if dense_ms else None,
        "dense_tflops": round(4.0 * d * g.H * g.N * g.N / (dense_ms * 1e-3) / 1e12, 2) if dense_ms else None,
        "speedup_attn_vs_dense": round(dense_ms / attn_ms, 2) if dense_ms else None,
        "speedup_step_vs_dense": round(dense_ms / ms_per_step, 2) if dense_ms else None,
        "per_frame_index": dict(per_frame, counters=per_frame_counters(per_frame)) if per_frame else None,
        "sequence_lengths": seq,
        "block_index": block,
        "corr_stride_layer": corr_stride,
        "broadcast_layer": broadcast,
        "qk_index": qk,
        "offline_profiling": prof,
        "sparsity": round(1.0 - (shared_pairs + gather_pairs) / (g.H * g.N * g.N), 4),
        "roofline": roofline,
        "roofline_other": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()


def cpu_baseline(w, row_stride: int, corr_rows: int):
    """Oracle time per step, from every row_stride-th query row and corr_rows
    index rows, scaled up by the pair / row counts."""
    import numpy as np

    import oracle

    g = w.geom
    rows = np.arange(0, g.N, row_stride, dtype=np.int64)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    vert_sets = {}
    for h in w.heads(1):
        ids, _, _, _ = oracle.vertical_index(w.q[h], w.k[h], w.plan[h][1])
        vert_sets[h] = ids
    t_vert = time.perf_counter() - t0
    t0 = time.perf_counter()
    u = np.random.default_rng(0).choice(g.Np, corr_rows, replace=False)
    idx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, w.corr_K, u)
    t_corr = (time.perf_counter() - t0) * g.Np / corr_rows
    # attention on the sampled rows; correspondence rows of sampled patches
    # reuse the sampled index rows (cycled) so the pair count is exact
    t = rows % g.T
    pr = (rows // g.T) * g.P + t - g.ns
    corr = {int(p): idx[i % corr_rows] for i, p in enumerate(pr[t >= g.ns])}
    sets, _, _ = oracle.layer_sets(g, w.plan, w.q, w.k, w.v, w.dino, w.corr_K, rows=rows, corr_rows=corr)
    sample_pairs = 0
    t0 = time.perf_counter()
    for h in range(g.H):
        row_set, s = sets[h]
        oracle.attention_sets(w.q[h], w.k[h], w.v[h], rows, row_set, s)
        lens = np.array([len(x) for x in s])
        sample_pairs += int(lens[row_set].sum())
    t_attn = time.perf_counter() - t0
    full_pairs = sum(p for _, p in key_counts(w))
    t_attn_full = t_attn * full_pairs / sample_pairs
    total_s = t_vert + t_corr + t_attn_full
    return {"value": round(total_s * 1e3, 1), "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": (f"attention on every {row_stride}th query row of all 16 heads ({rows.size} rows, "
                       f"{sample_pairs} pairs, {t_attn:.1f}s) scaled by pair count; correspondence index on "
                       f"{corr_rows} random rows scaled by row count; vertical probe + top-K in full "
                       f"({t_vert:.1f}s); extrapolated"),
            "attn_ms_extrapolated": round(t_attn_full * 1e3, 1),
            "corr_index_ms_extrapolated": round(t_corr * 1e3, 1)}


if __name__ == "__main__":
    main()
