#!/usr/bin/env python3
"""Benchmark of one routed MoE FFN layer with MXFP4 experts on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

Default workload: one-token decode (T=1, d=7168, E=896 experts, top-16,
f=1536) over 1000 distinct seeded tokens; one step = one moe_layer_forward
call on one batch (router, top-k, grouping, gate/up + SwiGLU, down,
combine), cycling through the batches so that no token is timed twice in a
row.  Inputs are synthetic and resident in HBM before timing starts.  The
other workloads (batched-decode T=64, zipf-prefill T=4096, long-prefill
T=32768) time the same call on their own shapes.  ``--tail`` times the
pre-norm block instead (moe_block_forward: RMSNorm before the router, a bf16
shared expert and the residual add around the same routed layer).

Prints one JSON line: throughput (tokens/s), the roofline of the dominant
kernel (HIP events on the library's own stream inside the timed region):
the gate/up GEMV against HBM bandwidth for decode-sized T, the scaled-MFMA
gate/up GEMM against the MXFP4 matrix peak for prefill-sized T; and the
CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
WORKLOADS = {"tiny": 0, "decode": 1, "batched-decode": 2, "zipf-prefill": 3, "long-prefill": 4,
             "mimo-decode": 5, "mimo-prefill": 6, "fp8-decode": 7, "fp8-prefill": 8}
DEFAULT_STEPS = {"tiny": 1000, "decode": 1000, "batched-decode": 200, "zipf-prefill": 20,
                 "long-prefill": 5, "mimo-decode": 1000, "mimo-prefill": 20, "fp8-decode": 1000,
                 "fp8-prefill": 3}
KERNELS = ("router_logits", "topk_softmax", "router_norms", "router_filter_gemm",
           "router_select", "router_refine", "permute", "topk_permute", "gemv_gate_up",
           "down_combine", "gemv_down", "mx_split_x", "gate_up_mfma", "down_mfma",
           "combine", "fp8_plan", "fp8_gate_up", "fp8_down")
# the pre-norm block's own kernels (--tail)
TAIL_KERNELS = ("rmsnorm", "shared_gate_up", "shared_down_add", "shared_gemm_gate_up",
                "shared_gemm_down")
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense MXFP4 / MXFP6, published
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16, published
MFMA_MIN_T = 128                # the library's scaled-MFMA path starts here (no per-expert choice)
FUSE_MAX_T = 4                  # up to here the library keeps the fused GEMV token path


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: decode 1000, batched-decode 200, "
                         "zipf-prefill 20, long-prefill 5, tiny 1000, mimo-decode 1000, "
                         "mimo-prefill 20)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 20 decode-sized, 2 prefill)")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode")
    ap.add_argument("--act", choices=("bf16", "mx"), default="bf16",
                    help="expert activations: bf16 (the W4A16 result; default) or mx (the "
                         "activation-MX mode: x and h rounded to one MX E2M3 term per 32)")
    ap.add_argument("--tail", action="store_true",
                    help="time the pre-norm MoE block (moe_block_forward: RMSNorm, the routed "
                         "layer, a bf16 shared expert of width f, the residual add) instead of "
                         "the routed layer alone")
    ap.add_argument("--packed", action="store_true",
                    help="prefill workloads: the experts re-laid once (before timing) in the "
                         "scaled-MFMA GEMM's operand order (moe_prepack_experts), timed through "
                         "moe_layer_forward_packed; the same bytes and the same results")
    ap.add_argument("--cpu-sample", type=int, default=24,
                    help="tokens of the workload the CPU oracle runs on the host's threads "
                         "(0: skip the CPU baseline)")
    ap.add_argument("--cpu-one-core-sample", type=int, default=2,
                    help="tokens of the workload the CPU oracle runs on one thread, the "
                         "per-core reference (0: skip)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel timing passes after the timed region")
    ap.add_argument("--gemv-max-rows", type=int, default=None, metavar="N",
                    help="diagnostic: override the per-expert crossover (experts with at most "
                         "N rows take the GEMVs in a scaled-MFMA call; 0..16)")
    ap.add_argument("--crossover", action="store_true",
                    help="only measure the per-expert crossover of the expert paths: "
                         "moe_expert_ffn at the K3 shape with every expert given n rows, all "
                         "experts on the grouped GEMVs against all on scaled-MFMA tiles, for "
                         "n = 1..16; prints one JSON line and exits")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure this GPU's ceilings: one-launch streaming reads of "
                         "several sizes and the matrix instructions' issue rate per operand "
                         "format; prints one JSON line and exits")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 device copy (torch.neg) of MIB MiB five "
                         "times, the reference for scaling HBM traffic counters, and exit")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    """Reads and writes exactly mib MiB per launch: what a traffic counter
    reads for it gives the counter's scale."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                      "launches": 5}))


def stream_read_gbps(nbytes: int, reps: int = 5, _buf={}):
    """The best bandwidth (GB/s) of one launch reading nbytes (rounded down to
    16 B) with the library's plain streaming-read kernel, over reps launches
    at each of a few grid sizes: what a kernel reading the same bytes in one
    launch can reach here, ramp-up and tail included."""
    import torch
    from routed_expert_mxfp4_amd import moe
    nbytes -= nbytes % 16
    if _buf.get("n", 0) < nbytes:
        _buf.clear()
        torch.cuda.synchronize()
        _buf["t"] = torch.randint(-2 ** 31, 2 ** 31 - 1, ((nbytes + 3) // 4,), dtype=torch.int32,
                                  device="cuda:0")
        _buf["out"] = torch.empty(1 << 16, dtype=torch.int32, device="cuda:0")
        _buf["n"] = nbytes
    buf, out = _buf["t"], _buf["out"]
    best = (float("inf"), 0)
    for blocks in (1024, 2048, 4096, 8192):
        moe.diag_stream_read(buf, nbytes, out, blocks)          # warm
        moe.diag_time_kernel("stream_read", capacity=reps)
        for i in range(reps):
            moe.diag_stream_read(buf, nbytes, out, blocks)
        torch.cuda.synchronize()
        best = min([best] + [(ms * 1e-3, blocks) for ms in moe.diag_kernel_times(reps)])
    moe.diag_time_kernel(None, 0)
    return nbytes / best[0] / 1e9, best[1]


def mfma_rate_tflops(kind: str, reps: int = 3):
    """The best rate (TFLOP/s) of the matrix instruction of this kind issued
    from registers by two, four and eight waves per SIMD."""
    import torch
    from routed_expert_mxfp4_amd import moe
    out = torch.empty(4 * 2048, dtype=torch.float32, device="cuda:0")
    best = 0.0
    for blocks, iters in ((512, 2048), (1024, 1024), (2048, 512)):
        flops = moe.diag_mfma_rate(kind, blocks, iters, out)   # warm
        moe.diag_time_kernel("mfma_rate", capacity=reps)
        for i in range(reps):
            moe.diag_mfma_rate(kind, blocks, iters, out)
        torch.cuda.synchronize()
        best = max([best] + [flops / (ms * 1e-3) / 1e12 for ms in moe.diag_kernel_times(reps)])
    moe.diag_time_kernel(None, 0)
    return best


def peaks() -> None:
    """Measured ceilings next to the published ones."""
    from routed_expert_mxfp4_amd import synth
    cfg = synth.CONFIGS[1]
    gu, dn = cfg.k * cfg.gate_up_bytes, cfg.k * (cfg.expert_bytes - cfg.gate_up_bytes)
    reads = []
    for label, n in (("16 MiB", 16 << 20), ("decode down, 16 experts", dn),
                     ("decode gate/up, 16 experts", gu), ("decode layer, 16 experts", gu + dn),
                     ("1 GiB", 1 << 30), ("4 GiB", 4 << 30)):
        gbps, blocks = stream_read_gbps(n)
        reads.append({"what": label, "bytes": n - n % 16, "GBps": gbps, "blocks": blocks,
                      "frac_of_published": gbps / HBM_PEAK_GBPS})
    rates = {}
    for kind, pub in (("fp6xfp4", MXFP4_PEAK_TFLOPS), ("fp4xfp4", MXFP4_PEAK_TFLOPS),
                      ("fp6xfp4_32x32x64", MXFP4_PEAK_TFLOPS),
                      ("fp4xfp4_32x32x64", MXFP4_PEAK_TFLOPS),
                      ("fp8xfp4", None), ("fp8xfp8", FP8_PEAK_TFLOPS), ("bf16", BF16_PEAK_TFLOPS)):
        r = mfma_rate_tflops(kind)
        rates[kind] = {"TFLOPs": r, "published_TFLOPs": pub,
                       "frac_of_published": None if pub is None else r / pub}
    print(json.dumps({"stream_read": reads, "mfma_rate": rates,
                      "published": {"hbm_GBps": HBM_PEAK_GBPS, "mxfp4_TFLOPs": MXFP4_PEAK_TFLOPS,
                                    "fp8_TFLOPs": FP8_PEAK_TFLOPS,
                                    "bf16_TFLOPs": BF16_PEAK_TFLOPS}}))


def crossover(reps: int = 10) -> None:
    """Time moe_expert_ffn on the K3 shape (d=7168, E=896, top-16, f=1536)
    with exactly n rows per expert (T = n*E/k tokens, token t's slot j on
    expert (t*k + j) mod E), once with every expert on the grouped GEMVs
    (crossover override 16) and once with every expert on 128-row
    scaled-MFMA tiles (override 0).  The crossover is the largest n up to
    which the GEMVs are faster at every n."""
    import torch
    from routed_expert_mxfp4_amd import moe, synth
    cfg = synth.CONFIGS[4]
    dev = torch.device("cuda:0")
    E, k, d, f = cfg.E, cfg.k, cfg.d, cfg.f
    experts = synth.gen_experts(cfg, device=dev)
    ns = (1, 2, 3, 4, 5, 6, 8, 10, 12, 16)
    xs = synth.gen_x(cfg, tokens=range(max(ns) * E // k)).to(dev)
    table = []
    for n in ns:
        T = n * E // k
        t = torch.arange(T, dtype=torch.int64)[:, None] * k + torch.arange(k)[None, :]
        ids = (t % E).to(torch.int32).to(dev)
        _, offsets, sr, _ = moe.moe_permute(ids, E)
        x = xs[:T].contiguous()
        row = {"rows_per_expert": n, "tokens": T}
        for path, R in (("gemv", 16), ("mfma", 0)):
            moe.diag_set_gemv_max_rows(R)
            ws = moe.workspace(moe.dims_of(T, d, E, k, f), moe.ENTRY_EXPERT_FFN, dev)
            for _ in range(3):
                moe.moe_expert_ffn(x, experts, offsets, sr, k, ws=ws)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
            for i in range(reps):
                ev[2 * i].record()
                moe.moe_expert_ffn(x, experts, offsets, sr, k, ws=ws)
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            ms = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps))
            row[path + "_ms"] = ms[reps // 2]
            row[path + "_us_per_expert"] = 1e3 * ms[reps // 2] / E
        moe.diag_set_gemv_max_rows(None)
        table.append(row)
        print("rows/expert %2d: gemv %.3f ms, mfma %.3f ms" % (n, row["gemv_ms"], row["mfma_ms"]),
              file=sys.stderr, flush=True)
    cross = 0
    for row in table:
        if row["gemv_ms"] < row["mfma_ms"]:
            cross = row["rows_per_expert"]
        else:
            break
    print(json.dumps({"crossover_rows": cross, "built_in": moe.diag_gemv_max_rows(),
                      "shape": {"d": d, "E": E, "k": k, "f": f}, "median_of": reps,
                      "table": table}))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def usable_cores():
    """Threads the CPU baseline runs: the cores this process may use, at most
    16 (the host share of one GPU)."""
    return max(1, min(affinity_cores(), 16))


def affinity_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def traffic_from_profiles(kernel: str, workload: str, src_sha: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the kernel source as it is now; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != src_sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, n_tokens, n_one_core):
    """The oracle, as it stands, on the first tokens of the workload: router +
    top-k over all experts, the k expert rows, combine.  n_tokens tokens run
    with the k rows of a token in parallel threads (the C code releases the
    GIL), then n_one_core further tokens on a single thread, the per-core
    reference.  Weight generation is excluded from the timing."""
    import numpy as np
    import oracle
    from routed_expert_mxfp4_amd import synth
    wr16 = synth.as_u16(synth.gen_router_w(cfg))
    bias = synth.gen_bias(cfg)
    bias_np = None if bias is None else bias.numpy()
    threads = usable_cores()
    fp8 = cfg.wfmt == "fp8"
    gen = synth.gen_experts_fp8 if fp8 else synth.gen_experts
    erow = oracle.expert_row_fp8 if fp8 else oracle.expert_row

    def token(n, pool):
        batch, t = (n, 0) if cfg.T == 1 else (0, n)
        x16 = synth.as_u16(synth.gen_x(cfg, batch, tokens=[t]))
        t0 = time.perf_counter()
        lg = oracle.router_logits(x16, wr16, bias_np)
        ids, w = oracle.topk_softmax(lg, cfg.k)
        spent = time.perf_counter() - t0
        W = {k: v.numpy() for k, v in gen(cfg, experts=[int(e) for e in ids[0]]).items()}

        def row(j):
            return erow(x16[0], W["gu_codes"][j], W["gu_scales"][j],
                        W["dn_codes"][j], W["dn_scales"][j], cfg.d, cfg.f)[1]
        t0 = time.perf_counter()
        rows = pool.map(row, range(cfg.k)) if pool is not None else map(row, range(cfg.k))
        oracle.combine_token(w[0], np.stack(list(rows)))
        return spent + time.perf_counter() - t0

    spent = 0.0
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for n in range(n_tokens):
            spent += token(n, pool)
    one = None
    if n_one_core > 0:
        s1 = sum(token(n_tokens + n, None) for n in range(n_one_core))
        one = {"value": n_one_core / s1, "unit": "tokens/s", "cores": 1, "seconds": s1,
               "sample": "%d further token(s), every step on one thread" % n_one_core}
    return {"value": n_tokens / spent, "unit": "tokens/s", "cores": min(threads, cfg.k),
            "kind": "oracle",
            "sample": "%d token(s) of the %s workload, all %d expert rows each (one thread "
                      "per row, up to %d at once), oracle (plain C, fp64) on %s"
                      % (n_tokens, cfg.name, cfg.k, threads, cpu_model()),
            "seconds": spent, "nproc": os.cpu_count(), "affinity_cores": affinity_cores(),
            "one_core": one}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py runs on one GPU only: the multi-GPU (expert-parallel) path is "
                  "not built; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from routed_expert_mxfp4_amd import moe, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy)
        return
    if args.crossover:
        crossover()
        return
    if args.peaks:
        peaks()
        return
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[WORKLOADS[args.workload]]
    if args.steps is None:
        args.steps = DEFAULT_STEPS[args.workload]
    if args.warmup is None:
        args.warmup = 2 if cfg.T >= MFMA_MIN_T else 20
    # the kernel that dominates the step: the expert-weight stream of the
    # gate/up GEMV (HBM-bound) for decode-sized T, the scaled-MFMA gate/up
    # GEMM (matrix-core-bound) for prefill-sized T
    fp8 = cfg.wfmt == "fp8"
    if fp8 and (args.tail or args.act != "bf16"):
        print("the FP8 expert variant runs the routed layer in bf16 activations only",
              file=sys.stderr)
        sys.exit(2)
    # the expert path the library takes (moe_abi.cpp's choice, mirrored): the
    # scaled-MFMA GEMMs once some expert can hold more than the crossover's
    # rows (bf16, canonical store), from MFMA_MIN_T tokens on otherwise; in
    # such a call experts with at most gemv_max rows stay on the GEMVs
    shape_ok = cfg.d % 512 == 0 and cfg.f % 256 == 0
    per_expert = (args.act == "bf16" and not args.packed and cfg.f % 32 == 0 and cfg.d <= 8192
                  and cfg.f <= 4096)
    if args.gemv_max_rows is not None:
        moe.diag_set_gemv_max_rows(args.gemv_max_rows)
    gemv_max = moe.diag_gemv_max_rows() if per_expert else 0
    mfma = (not fp8) and shape_ok and cfg.T > FUSE_MAX_T and (
        cfg.T > gemv_max if per_expert else cfg.T >= MFMA_MIN_T)
    if args.packed and not (mfma and cfg.f % 512 == 0 and not args.tail):
        print("--packed needs a prefill workload on the scaled-MFMA path (d, f % 512 == 0), "
              "without --tail", file=sys.stderr)
        sys.exit(2)
    dominant = "fp8_gate_up" if fp8 else ("gate_up_mfma" if mfma else "gemv_gate_up")
    # the counter summary that belongs to this exact run variant
    traffic_key = (args.workload + ("-packed" if args.packed else "") +
                   ("-mx" if args.act == "mx" else "") + ("-block" if args.tail else ""))
    L = moe.lib()

    # ---- inputs, resident in HBM before timing --------------------------------
    experts = synth.gen_experts_fp8(cfg, device=dev) if fp8 else synth.gen_experts(cfg, device=dev)
    wr = synth.gen_router_w(cfg).to(dev)
    bias = synth.gen_bias(cfg)
    bias = None if bias is None else bias.to(dev)
    n_batches = min(cfg.batches, max(1, args.steps + args.warmup))
    xs = [synth.gen_x(cfg, b).to(dev) for b in range(n_batches)]
    act = moe.ACT_MX_E2M3 if args.act == "mx" else moe.ACT_BF16
    if args.packed:
        experts = moe.moe_prepack_experts(experts, cfg.d, cfg.f)   # outside the timed region
        torch.cuda.synchronize()
        layer = moe.PackedLayer(experts, wr, cfg.k, bias, T=cfg.T, act=act)
    elif fp8:
        layer = moe.Fp8Layer(experts, wr, cfg.k, bias, T=cfg.T)
    elif args.tail:
        tail = {n: (v.to(dev) if hasattr(v, "to") else v)
                for n, v in synth.gen_tail(cfg).items()}
        layer = moe.Block(experts, wr, cfg.k, tail, bias, T=cfg.T, act=act)
    else:
        layer = moe.Layer(experts, wr, cfg.k, bias, T=cfg.T, act=act)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    dims = moe.dims_of(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, act)
    ex = moe.fp8_experts_of(experts) if fp8 else moe.experts_of(experts)
    ws = layer._ws
    bptr = None if bias is None else ctypes.c_void_p(bias.data_ptr())
    if args.tail:
        argsets = [(ctypes.byref(dims), ctypes.c_void_p(x.data_ptr()), ctypes.byref(layer._tw),
                    ctypes.c_void_p(wr.data_ptr()), bptr, ctypes.byref(ex),
                    ctypes.c_void_p(y.data_ptr()), None, None, ctypes.c_void_p(ws.data_ptr()),
                    ws.numel(), sptr) for x in xs]
        fwd, fname = L.moe_block_forward, "moe_block_forward"
    elif fp8:
        argsets = [(ctypes.byref(dims), ctypes.c_void_p(x.data_ptr()),
                    ctypes.c_void_p(wr.data_ptr()), bptr, ctypes.byref(ex),
                    ctypes.c_void_p(y.data_ptr()), None, None, ctypes.c_void_p(ws.data_ptr()),
                    ws.numel(), sptr) for x in xs]
        fwd, fname = L.moe_layer_forward_fp8, "moe_layer_forward_fp8"
    elif args.packed:
        argsets = [(ctypes.byref(dims), ctypes.c_void_p(x.data_ptr()),
                    ctypes.c_void_p(wr.data_ptr()), bptr, ctypes.byref(ex),
                    ctypes.c_void_p(y.data_ptr()), None, None, ctypes.c_void_p(ws.data_ptr()),
                    ws.numel(), sptr) for x in xs]
        fwd, fname = L.moe_layer_forward_packed, "moe_layer_forward_packed"
    else:
        argsets = [(ctypes.byref(dims), ctypes.c_void_p(x.data_ptr()),
                    ctypes.c_void_p(wr.data_ptr()), bptr, ctypes.byref(ex),
                    ctypes.c_void_p(y.data_ptr()), None, None, ctypes.c_void_p(ws.data_ptr()),
                    ws.numel(), sptr) for x in xs]
        fwd, fname = L.moe_layer_forward, "moe_layer_forward"

    def run(n0, count):
        for i in range(count):
            st = fwd(*argsets[(n0 + i) % n_batches])
            if st != 0:
                raise moe.MoeError(st, fname)

    run(0, args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: K steps, dominant kernel timed with HIP events ------------
    # one launch in `every` carries the events (a 1000-step decode run: 125
    # timed launches), so the events' own cost is not in most steps
    every = 8 if args.steps >= 200 else 1
    moe.diag_time_kernel(dominant, capacity=max(1, args.steps), every=every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_launch = moe.diag_kernel_times(max(1, args.steps))
    dom_ms, dom_n = sum(per_launch), len(per_launch)
    moe.diag_time_kernel(None, 0)
    elapsed = t1 - t0


    # ---- per-kernel breakdown (separate passes, outside the timed region) -------
    breakdown = {}
    if not args.no_breakdown:
        for kname in KERNELS + (TAIL_KERNELS if args.tail else ()):
            moe.diag_time_kernel(kname, capacity=max(1, args.steps))
            run(args.warmup, args.steps)
            torch.cuda.synchronize()
            ms, n = moe.diag_kernel_time()
            if n:
                breakdown[kname] = {"avg_us": 1e3 * ms / n, "launches": n}
        moe.diag_time_kernel(None, 0)
        t2 = time.perf_counter()
        run(args.warmup, args.steps)
        torch.cuda.synchronize()
        breakdown["steps_without_events_ms_per_step"] = 1e3 * (time.perf_counter() - t2) / args.steps

    # ---- algorithmic work ------------------------------------------------------------
    ids_probe = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    per_expert_gu = cfg.gate_up_bytes
    touched, on_mfma, rows_mfma = [], [], []
    for b in range(min(n_batches, 64)):
        if args.tail:
            layer.forward(xs[b], out=y, topk_ids=ids_probe)
        else:
            layer.forward(xs[b], y=y, topk_ids=ids_probe)
        counts = torch.bincount(ids_probe.flatten().long(), minlength=cfg.E)
        touched.append(int((counts > 0).sum()))
        big = counts > gemv_max
        on_mfma.append(int(big.sum()))
        rows_mfma.append(int(counts[big].sum()))
    torch.cuda.synchronize()
    mean_touched = sum(touched) / len(touched)
    # the dominant GEMM's own share: the experts on the MFMA tiles and their rows
    mean_on_mfma = sum(on_mfma) / len(on_mfma)
    mean_rows_mfma = sum(rows_mfma) / len(rows_mfma)
    avg_launch_s = (dom_ms / dom_n) * 1e-3 if dom_n else float("nan")
    pl = sorted(per_launch)

    def pct(q):
        return 1e3 * pl[min(len(pl) - 1, int(q * (len(pl) - 1) + 0.5))] if pl else None
    launch_pct = {"p10_us": pct(0.10), "p50_us": pct(0.50), "p90_us": pct(0.90)}
    tokens = args.steps * cfg.T
    value = tokens / elapsed
    layer_bytes = mean_touched * cfg.expert_bytes
    layer_flops = 2.0 * cfg.T * cfg.k * 3 * cfg.d * cfg.f
    if fp8 and cfg.T >= MFMA_MIN_T:
        # FP8 experts on the bf16 matrix cores (codes converted exactly to
        # bf16): the gate/up GEMM against the bf16 matrix peak past the bf16
        # ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B), else against HBM
        flops_per_launch = 2.0 * cfg.T * cfg.k * 2 * cfg.f * cfg.d
        bytes_per_launch = mean_touched * per_expert_gu
        tflops = flops_per_launch / avg_launch_s / 1e12
        src = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc", "ffn_fp8_mfma.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        common = {"kernel": dominant, "traffic": traffic_from_profiles(dominant, traffic_key, sha),
                  "algorithmic_flops_per_launch": flops_per_launch,
                  "algorithmic_bytes_per_launch": bytes_per_launch,
                  "layer_flop_per_byte": layer_flops / layer_bytes,
                  "bf16_tflops": tflops, "bf16_frac": tflops / BF16_PEAK_TFLOPS,
                  "avg_launch_us": avg_launch_s * 1e6, "launches_timed": dom_n}
        if layer_flops / layer_bytes >= BF16_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3:
            roofline = dict(common, bound="mfma", achieved=tflops, peak=BF16_PEAK_TFLOPS,
                            unit="TFLOP/s", frac=tflops / BF16_PEAK_TFLOPS)
        else:
            achieved = bytes_per_launch / avg_launch_s / 1e9
            roofline = dict(common, bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS,
                            unit="GB/s", frac=achieved / HBM_PEAK_GBPS)
    elif mfma and layer_flops / layer_bytes >= MXFP4_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3:
        # past the ridge (10.1 PFLOP/s / 8 TB/s = 1262 flop/B): the matrix
        # cores bound the gate/up GEMM (its rows times [2f x d])
        flops_per_launch = 2.0 * mean_rows_mfma * 2 * cfg.f * cfg.d
        achieved = flops_per_launch / avg_launch_s / 1e12
        src = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc", "ffn_mfma.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": achieved,
                    "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / MXFP4_PEAK_TFLOPS,
                    "traffic": traffic_from_profiles(dominant, traffic_key, sha),
                    "algorithmic_flops_per_launch": flops_per_launch,
                    "mfma_passes_per_product": 1 if act else 2,
                    "avg_launch_us": avg_launch_s * 1e6, "launches_timed": dom_n}
    elif mfma:
        # below the ridge: HBM bounds the layer (every touched expert's
        # weights read once); the gate/up GEMM's bytes are its experts'
        # gate/up matrices, its flops are reported beside them
        bytes_per_launch = mean_on_mfma * per_expert_gu
        flops_per_launch = 2.0 * mean_rows_mfma * 2 * cfg.f * cfg.d
        achieved = bytes_per_launch / avg_launch_s / 1e9
        src = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc", "ffn_mfma.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": traffic_from_profiles(dominant, traffic_key, sha),
                    "algorithmic_bytes_per_launch": bytes_per_launch,
                    "experts_on_mfma_per_launch": mean_on_mfma,
                    "experts_on_gemv_per_launch": mean_touched - mean_on_mfma,
                    "layer_flop_per_byte": layer_flops / layer_bytes,
                    "mxfp4_tflops": flops_per_launch / avg_launch_s / 1e12,
                    "mxfp4_frac": flops_per_launch / avg_launch_s / 1e12 / MXFP4_PEAK_TFLOPS,
                    "mfma_passes_per_product": 1 if act else 2,
                    "avg_launch_us": avg_launch_s * 1e6, "launches_timed": dom_n}
    else:
        bytes_per_launch = mean_touched * per_expert_gu
        achieved = bytes_per_launch / avg_launch_s / 1e9
        src = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc",
                           "ffn_fp8.hip" if fp8 else "ffn_gemv.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": traffic_from_profiles(dominant, traffic_key, sha),
                    "algorithmic_bytes_per_launch": bytes_per_launch,
                    "avg_launch_us": avg_launch_s * 1e6, "launches_timed": dom_n}

    roofline["launch_us_percentiles"] = launch_pct
    roofline["timed_every"] = every
    # the same launch against what this GPU measurably sustains for its bound
    if roofline["bound"] == "hbm" and roofline["algorithmic_bytes_per_launch"] >= 16:
        # (a crossover override can leave the scaled-MFMA call no expert)
        mp, blocks = stream_read_gbps(int(roofline["algorithmic_bytes_per_launch"]))
        roofline["measured_peak"] = {
            "value": mp, "unit": "GB/s", "frac": roofline["achieved"] / mp,
            "what": "one launch of a plain streaming read of the same bytes (%d blocks; "
                    "bench.py --peaks)" % blocks}
    elif roofline["bound"] == "mfma":
        kind = "bf16" if fp8 else "fp6xfp4"
        mp = mfma_rate_tflops(kind)
        roofline["measured_peak"] = {
            "value": mp, "unit": "TFLOP/s", "frac": roofline["achieved"] / mp,
            "what": "%s scaled 16x16x128 matrix instructions issued from registers "
                    "(bench.py --peaks)" % kind}
    out = {
        "metric": "MoE-layer tokens/s + expert-weight GB/s (decode) / MXFP4 TFLOP/s (prefill), 1 GPU",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6xfp4" if act and mfma else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "f": cfg.f, "distinct_batches": n_batches,
                   "weights": ("FP8 (E4M3FN codes + fp32 scale per 128x128 block), resident in HBM"
                               if fp8 else
                               "MXFP4 (E2M1 codes + E8M0 scale per 32), resident in HBM" +
                               (", in the GEMM's operand order (re-laid once before timing; "
                                "same bytes)" if args.packed else "")),
                   "activations": ("MX E2M3, one term per 32 (activation-MX mode)" if act
                                   else "bf16"), "accumulate": "fp32",
                   "expert_path": (("FP8 codes -> bf16 matrix-core GEMMs" if cfg.T >= MFMA_MIN_T
                                    else "FP8 dequant-GEMV") if fp8 else
                                   "scaled MFMA" if mfma else "GEMV")},
        "block": (None if not args.tail else {
            "entry": "moe_block_forward",
            "steps": "RMSNorm (canonical fp64) -> routed layer on xn -> bf16 SwiGLU shared "
                     "expert of width f -> residual add",
            "shared_expert_bytes": 3 * cfg.d * cfg.f * 2,
            "norm_bytes_per_token": 2 * 2 * cfg.d}),
        "expert_weight_GBps": layer_bytes * args.steps / elapsed / 1e9,
        "expert_weight_hbm_frac": layer_bytes * args.steps / elapsed / 1e9 / HBM_PEAK_GBPS,
        "tflops": layer_flops * args.steps / elapsed / 1e12,
        "mxfp4_frac": layer_flops * args.steps / elapsed / 1e12 / MXFP4_PEAK_TFLOPS,
        "roofline": roofline,
        "cpu_baseline": None,
        "breakdown": breakdown,
    }
    if args.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample, args.cpu_one_core_sample)
        if args.tail:
            out["cpu_baseline"]["note"] = "the routed layer's oracle (the block's dominant work)"
    print(json.dumps(out))


if __name__ == "__main__":
    main()
