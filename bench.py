#!/usr/bin/env python3
"""Benchmark of the W4A4 hot path on one MI355X.

Workload: the LLaMA-2-7B q_proj linear layer, X 2048x4096 fp16 (8 fixed
outlier channels x30), W 4096x4096 fp16 ~N(0, 0.02), 128-wide Hadamard
blocks (--had full: one 4096-point Hadamard), symmetric INT4 per token and
per output channel.  Synthetic, seeded inputs from `workloads`.

One step = one pass of the whole path over one batch, on one HIP stream:
    quant_weight_offline(W) -> rotate_quant_act(X) -> w4a4_gemm
Inputs sit in HBM before the timed region; 8 copies of the inputs and
outputs are cycled so that a step never finds its operands in the 256 MiB
last-level cache.  The GEMM launch of every timed step carries a pair of
HIP events armed through w4a4_time_next_launch: the runtime stamps the
kernel's own start and end into them, so its average is the device
duration taken live over the timed steps, with no marker packets between
kernels.  The two rotate+quantize kernels are timed the same way in a second
pass after the timed region (arming every launch makes the step host-bound).
(Running the weight and activation steps on two streams, eagerly or as a
captured HIP graph, measured slower here: the cross-stream waits and graph
launches cost more host time than the overlap saves.)

Prints one JSON line; value = 2*M*N*K / step time (TOPS of the whole step).
`--suite` instead prints one line per kernel and configuration (cold and
warm timings of every entry point, with rooflines).
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
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS
FP4_PEAK_TOPS = 10100.0        # MI355X dense fp4 MFMA (MXFP4 products), TFLOP/s
NSETS = 8


def src_hash(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "rotation_w4a4_quantization_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_traffic(kernel_key: str, src: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_hash(?:\s*\([^)]*\))?:\s*(\w+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != src:
        return None
    return float(m_b.group(1))


def cpu_baseline(min_seconds: float = 10.0, min_reps: int = 3) -> dict:
    """The CPU oracle on the same q_proj step, timed on this host's cores:
    whole steps repeated until about `min_seconds` of work (at least
    `min_reps` steps)."""
    import oracle as O
    import workloads as WL
    from threadpoolctl import threadpool_info

    d = WL.qproj()
    times = []
    while len(times) < min_reps or sum(times) < min_seconds:
        t0 = time.perf_counter()
        wq = O.quant_weight_offline(d["W"], 128)
        a = O.rotate_quant_act(d["X"], 128, "sym")
        acc = O.int_gemm(a["codes"], wq["codes"])
        O.epilogue_sym_f32(acc, a["scale"], wq["scale"])
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    M, N, K = 2048, 4096, 4096
    return {"value": round(2 * M * N * K / dt / 1e12, 5), "unit": "TOPS", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(times)} full q_proj steps (weight rotate+quant, activation rotate+quant, exact "
                      f"integer GEMM, fp32 epilogue) at M=2048 N=K=4096, {dt:.3f} s per step, "
                      f"{sum(times):.1f} s in all; numpy float64 + BLAS"}


def _time_kernel(torch, fn, flush, n=30, warm_n=50):
    """Device duration of the kernel one call of `fn` launches: median / p10 /
    p90 after flushing the caches (cold), and the mean over back-to-back
    launches (warm).  Each launch carries its own events through
    w4a4_time_next_launch, so the figures are kernel durations only."""
    from rotation_w4a4_quantization_amd.timing import HipEvents
    hev = HipEvents()
    for _ in range(3):
        fn()
    cold = []
    ev = [hev.pair() for _ in range(max(n, warm_n))]
    for i in range(n):
        flush()
        hev.arm(*ev[i])
        fn()
        cold.append(hev.elapsed(*ev[i]))
    cold.sort()
    torch.cuda.synchronize()
    for i in range(warm_n):
        hev.arm(*ev[i])
        fn()
    warm = sum(hev.elapsed(*e) for e in ev[:warm_n]) / warm_n
    hev.close()
    return dict(cold_ms_median=cold[len(cold) // 2], cold_ms_p10=cold[len(cold) // 10],
                cold_ms_p90=cold[(9 * len(cold)) // 10], warm_ms=warm)


def run_suite(torch, R, WL):
    """One JSON line per (entry point, configuration): cold (caches flushed by
    reading 512 MiB, which leaves no dirty lines to write back during the
    timed launch) and warm timings, with the roofline each kernel answers to."""
    dev = torch.device("cuda:0")
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def flush():
        scratch.amax()

    def emit(kernel, config, t, nbytes=None, ops=None, peak=("int8", INT8_PEAK_TOPS)):
        rec = dict(kernel=kernel, config=config, **{k: round(v, 5) for k, v in t.items()})
        if nbytes is not None:
            gbs = nbytes / (t["cold_ms_median"] * 1e-3) / 1e9
            rec.update(bytes=nbytes, bound="hbm", cold_GBps=round(gbs, 1),
                       cold_frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
                       warm_GBps=round(nbytes / (t["warm_ms"] * 1e-3) / 1e9, 1))
        if ops is not None:
            tops = ops / (t["cold_ms_median"] * 1e-3) / 1e12
            rec.update(ops=ops, bound="mfma", cold_TOPS=round(tops, 1),
                       **{f"cold_frac_{peak[0]}": round(tops / peak[1], 4)},
                       warm_TOPS=round(ops / (t["warm_ms"] * 1e-3) / 1e12, 1))
        print(json.dumps(rec), flush=True)

    def T(a):
        return torch.from_numpy(a).to(dev)

    def act_bytes(M, K, asym=False):
        return 2 * M * K + M * K // 2 + (5 * M * (K // 128) if asym else 4 * M)

    def mx_bytes(M, K):
        return 2 * M * K + M * K // 2 + M * K // 32

    FP4 = ("fp4", FP4_PEAK_TOPS)

    # q_proj family M x 4096 x 4096 (both Hadamard widths), decode rows, down_proj, gate/up
    wq = T(WL.qproj_weight())
    for block in (128, "full"):
        tag = "128" if block == 128 else "full"
        wc, ws, wg = R.quant_weight_offline(wq, block)
        emit("quant_weight_offline", f"qproj W 4096x4096 had{tag}",
             _time_kernel(torch, lambda: R.quant_weight_offline(wq, block), flush),
             nbytes=2 * 4096 * 4096 + 4096 * 2048 + 4 * 4096 + 4 * 4096 * 32)
        for M in (1, 4, 16, 256, 2048, 8192, 32768):
            x = T(WL.qproj(M=min(M, 2048), with_w=False)["X"])
            if M > 2048:
                x = x.repeat(M // 2048, 1)
            xc, xs, _ = R.rotate_quant_act(x, block)
            emit("rotate_quant_act", f"qproj X {M}x4096 had{tag}",
                 _time_kernel(torch, lambda: R.rotate_quant_act(x, block), flush), nbytes=act_bytes(M, 4096))
            y = torch.empty((M, 4096), dtype=torch.float32, device=dev)
            emit("w4a4_gemm", f"{M}x4096x4096 had{tag}",
                 _time_kernel(torch, lambda: R.w4a4_gemm(xc, xs, None, wc, ws, out=y), flush),
                 nbytes=(M * 2048 + 4 * M + 4096 * 2048 + 4 * 4096 + 4 * M * 4096) if M <= 16 else None,
                 ops=2 * M * 4096 * 4096)
    # decode linear in one launch (activation rotate+quant fused into the decode GEMM);
    # compare with the rotate_quant_act + w4a4_gemm lines above
    wc, ws, _ = R.quant_weight_offline(wq, 128)
    for M in (1, 4, 16):
        x = T(WL.decode(M, with_w=False)["X"])
        y = torch.empty((M, 4096), dtype=torch.float32, device=dev)
        emit("w4a4_decode_fused", f"{M}x4096x4096 had128",
             _time_kernel(torch, lambda: R.w4a4_decode_fused(x, wc, ws, out=y), flush),
             nbytes=2 * M * 4096 + 4096 * 2048 + 4 * 4096 + 4 * M * 4096, ops=2 * M * 4096 * 4096)
    # MXFP4 on the same shapes (128-wide blocks)
    wmc, wme = R.rotate_quant_mxfp4(wq, 128)
    emit("rotate_quant_mxfp4", "qproj W 4096x4096 had128",
         _time_kernel(torch, lambda: R.rotate_quant_mxfp4(wq, 128), flush), nbytes=mx_bytes(4096, 4096))
    for M in (1, 16, 256, 2048, 8192):
        x = T(WL.qproj(M=min(M, 2048), with_w=False)["X"])
        if M > 2048:
            x = x.repeat(M // 2048, 1)
        xmc, xme = R.rotate_quant_mxfp4(x, 128)
        emit("rotate_quant_mxfp4", f"qproj X {M}x4096 had128",
             _time_kernel(torch, lambda: R.rotate_quant_mxfp4(x, 128), flush), nbytes=mx_bytes(M, 4096))
        y = torch.empty((M, 4096), dtype=torch.float32, device=dev)
        emit("mxfp4_gemm", f"{M}x4096x4096 had128",
             _time_kernel(torch, lambda: R.mxfp4_gemm(xmc, xme, wmc, wme, out=y), flush),
             nbytes=(M * 2048 + M * 128 + 4096 * 2048 + 4096 * 128 + 4 * M * 4096) if M <= 16 else None,
             ops=2 * M * 4096 * 4096, peak=FP4)
    del wq, wmc
    d = WL.downproj()
    x, w = T(d["X"]), T(d["W"])
    del d
    xc, xs, _ = R.rotate_quant_act(x, 128)
    wc, ws, _ = R.quant_weight_offline(w, 128)
    emit("rotate_quant_act", "downproj X 4096x14336 had128",
         _time_kernel(torch, lambda: R.rotate_quant_act(x, 128), flush), nbytes=act_bytes(4096, 14336))
    emit("quant_weight_offline", "downproj W 4096x14336 had128",
         _time_kernel(torch, lambda: R.quant_weight_offline(w, 128), flush),
         nbytes=2 * 4096 * 14336 + 4096 * 7168 + 4 * 4096 + 4 * 4096 * 112)
    y = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
    emit("w4a4_gemm", "downproj 4096x4096x14336",
         _time_kernel(torch, lambda: R.w4a4_gemm(xc, xs, None, wc, ws, out=y), flush),
         ops=2 * 4096 * 4096 * 14336)
    xmc, xme = R.rotate_quant_mxfp4(x, 128)
    wmc, wme = R.rotate_quant_mxfp4(w, 128)
    emit("rotate_quant_mxfp4", "downproj X 4096x14336 had128",
         _time_kernel(torch, lambda: R.rotate_quant_mxfp4(x, 128), flush), nbytes=mx_bytes(4096, 14336))
    emit("mxfp4_gemm", "downproj 4096x4096x14336",
         _time_kernel(torch, lambda: R.mxfp4_gemm(xmc, xme, wmc, wme, out=y), flush),
         ops=2 * 4096 * 4096 * 14336, peak=FP4)
    del x, w, xc, wc, y, xmc, wmc
    d = WL.gateup()
    x, w = T(d["X"]), T(d["W"])
    del d
    xc, xs, xz = R.rotate_quant_act(x, 128, "asym")
    wc, ws, _ = R.quant_weight_offline(w, 128)
    emit("rotate_quant_act", "gateup X 8192x8192 asym g128",
         _time_kernel(torch, lambda: R.rotate_quant_act(x, 128, "asym"), flush),
         nbytes=act_bytes(8192, 8192, asym=True))
    emit("quant_weight_offline", "gateup W 28672x8192 had128",
         _time_kernel(torch, lambda: R.quant_weight_offline(w, 128), flush, n=10),
         nbytes=2 * 28672 * 8192 + 28672 * 4096 + 4 * 28672 + 4 * 28672 * 64)
    y = torch.empty((8192, 28672), dtype=torch.float32, device=dev)
    emit("w4a4_gemm", "gateup asym 8192x28672x8192",
         _time_kernel(torch, lambda: R.w4a4_gemm(xc, xs, xz, wc, ws, act_mode="asym", out=y), flush, n=10,
                      warm_n=10),
         ops=2 * 8192 * 28672 * 8192)
    del xc, wc
    xmc, xme = R.rotate_quant_mxfp4(x, 128)
    wmc, wme = R.rotate_quant_mxfp4(w, 128)
    emit("mxfp4_gemm", "gateup 8192x28672x8192",
         _time_kernel(torch, lambda: R.mxfp4_gemm(xmc, xme, wmc, wme, out=y), flush, n=10, warm_n=10),
         ops=2 * 8192 * 28672 * 8192, peak=FP4)
    del x, w, y, xmc, wmc
    kv = T(WL.kv()["KV"])
    emit("kv_rotate_quant4", "kv 8x32x4096x128",
         _time_kernel(torch, lambda: R.kv_rotate_quant4(kv), flush),
         nbytes=2 * kv.numel() + kv.numel() // 2 + 5 * (kv.numel() // 128))
    # decode attention over the INT4 cache (K = the KV workload, V = its heads reversed)
    kc, ks, kz = R.kv_rotate_quant4(kv)
    vc, vs, vz = R.kv_rotate_quant4(kv.flip(1).contiguous())
    q = T(WL.small_random(123, 8 * 32, 128).reshape(8, 32, 128))
    o = torch.empty((8, 32, 128), dtype=torch.float32, device=dev)
    emit("kv4_attention_decode", "q 8x32 over kv 8x32x4096x128 int4",
         _time_kernel(torch, lambda: R.kv4_attention_decode(q, kc, ks, kz, vc, vs, vz, out=o), flush),
         nbytes=attn_bytes(8, 32, 4096))
    del kc, vc
    # few heads, long caches: the single pass against tokens split over
    # workgroups (the split line times both of its kernels)
    for B, H, S in ((1, 32, 4096), (1, 8, 32768)):
        src = kv.reshape(-1)[:B * H * S * 128].reshape(B, H, S, 128)
        kc, ks, kz = R.kv_rotate_quant4(src)
        vc, vs, vz = R.kv_rotate_quant4(src.flip(1).contiguous())
        q = T(WL.small_random(124, B * H, 128).reshape(B, H, 128))
        o = torch.empty((B, H, 128), dtype=torch.float32, device=dev)
        ws = torch.empty((max(R.kv4_attention_workspace_bytes(B, H, S), 16),), dtype=torch.uint8, device=dev)
        cfg = f"q {B}x{H} over kv {B}x{H}x{S}x128 int4"
        emit("kv4_attention_decode", cfg,
             _time_kernel(torch, lambda: R.kv4_attention_decode(q, kc, ks, kz, vc, vs, vz, out=o), flush),
             nbytes=attn_bytes(B, H, S))
        emit("kv4_attention_decode_ws", cfg,
             _time_kernel(torch, lambda: R.kv4_attention_decode_split(q, kc, ks, kz, vc, vs, vz, out=o,
                                                                      workspace=ws), flush),
             nbytes=attn_bytes(B, H, S))
        del kc, vc, src


def attn_bytes(B: int, H: int, S: int) -> int:
    """Algorithmic bytes of one decode-attention launch: the K and V codes,
    scales and zero-points of every cached token, the query and the output."""
    return B * H * (S * (64 + 64 + 4 + 4 + 1 + 1) + 128 * 2 + 128 * 4)


def run_only(torch, R, WL, which, steps, had):
    """Launch one entry point `steps` times on its workload (q_proj unless named)."""
    dev = torch.device("cuda:0")
    block = 128 if had == "128" else "full"

    def T(a):
        return torch.from_numpy(a).to(dev)

    if which == "copy":
        # plain device copy of 256 MiB: the reference kernel for the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)                                           # noqa: E731
    elif which in ("gemm", "act", "weight", "decode"):
        d = WL.qproj() if which != "decode" else WL.decode(16)
        x, w = T(d["X"]), T(d["W"])
        wc, ws, _ = R.quant_weight_offline(w, block)
        xc, xs, _ = R.rotate_quant_act(x, block)
        y = torch.empty((x.shape[0], w.shape[0]), dtype=torch.float32, device=dev)
        fn = {"gemm": lambda: R.w4a4_gemm(xc, xs, None, wc, ws, out=y),
              "decode": lambda: R.w4a4_gemm(xc, xs, None, wc, ws, out=y),
              "act": lambda: R.rotate_quant_act(x, block),
              "weight": lambda: R.quant_weight_offline(w, block)}[which]
    elif which == "fused":
        d = WL.decode(16)
        x, w = T(d["X"]), T(d["W"])
        wc, ws, _ = R.quant_weight_offline(w, 128)
        y = torch.empty((16, w.shape[0]), dtype=torch.float32, device=dev)
        fn = lambda: R.w4a4_decode_fused(x, wc, ws, out=y)                    # noqa: E731
    elif which in ("mx", "mxact", "mxdecode"):
        d = WL.qproj() if which != "mxdecode" else WL.decode(16)
        x, w = T(d["X"]), T(d["W"])
        wc, we = R.rotate_quant_mxfp4(w, 128)
        xc, xe = R.rotate_quant_mxfp4(x, 128)
        y = torch.empty((x.shape[0], w.shape[0]), dtype=torch.float32, device=dev)
        fn = {"mx": lambda: R.mxfp4_gemm(xc, xe, wc, we, out=y),
              "mxdecode": lambda: R.mxfp4_gemm(xc, xe, wc, we, out=y),
              "mxact": lambda: R.rotate_quant_mxfp4(x, 128)}[which]
    elif which == "downproj":
        d = WL.downproj()
        x, w = T(d["X"]), T(d["W"])
        wc, ws, _ = R.quant_weight_offline(w, 128)
        xc, xs, _ = R.rotate_quant_act(x, 128)
        y = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        fn = lambda: R.w4a4_gemm(xc, xs, None, wc, ws, out=y)                  # noqa: E731
    elif which == "gateup":
        d = WL.gateup()
        x, w = T(d["X"]), T(d["W"])
        wc, ws, _ = R.quant_weight_offline(w, 128)
        xc, xs, xz = R.rotate_quant_act(x, 128, "asym")
        y = torch.empty((8192, 28672), dtype=torch.float32, device=dev)
        fn = lambda: R.w4a4_gemm(xc, xs, xz, wc, ws, act_mode="asym", out=y)   # noqa: E731
    elif which in ("downact", "gateact"):
        x = T((WL.downproj(with_w=False) if which == "downact" else WL.gateup(with_w=False))["X"])
        mode = "sym" if which == "downact" else "asym"
        fn = lambda: R.rotate_quant_act(x, 128, mode)                         # noqa: E731
    elif which == "attn":
        kv = T(WL.kv()["KV"])
        kc, ks, kz = R.kv_rotate_quant4(kv)
        vc, vs, vz = R.kv_rotate_quant4(kv.flip(1).contiguous())
        del kv
        q = T(WL.small_random(123, 8 * 32, 128).reshape(8, 32, 128))
        o = torch.empty((8, 32, 128), dtype=torch.float32, device=dev)
        fn = lambda: R.kv4_attention_decode(q, kc, ks, kz, vc, vs, vz, out=o)  # noqa: E731
    elif which == "attnsplit":
        # 1 x 8 heads x 32768 tokens: tokens split over workgroups
        kv = T(WL.kv()["KV"]).reshape(-1)[:8 * 32768 * 128].reshape(1, 8, 32768, 128)
        kc, ks, kz = R.kv_rotate_quant4(kv)
        vc, vs, vz = R.kv_rotate_quant4(kv.flip(1).contiguous())
        del kv
        q = T(WL.small_random(124, 8, 128).reshape(1, 8, 128))
        o = torch.empty((1, 8, 128), dtype=torch.float32, device=dev)
        ws = torch.empty((R.kv4_attention_workspace_bytes(1, 8, 32768),), dtype=torch.uint8, device=dev)
        fn = lambda: R.kv4_attention_decode_split(q, kc, ks, kz, vc, vs, vz, out=o, workspace=ws)  # noqa: E731
    else:
        kv = T(WL.kv()["KV"])
        fn = lambda: R.kv_rotate_quant4(kv)                                    # noqa: E731
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    print(f"ran {which} x{steps}", flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first; a few hundred let the clocks settle")
    ap.add_argument("--min-warmup-s", type=float, default=1.0,
                    help="keep running untimed steps until this much wall time has passed, "
                         "whatever --warmup says, so that short runs still time settled clocks")
    ap.add_argument("--had", choices=["128", "full"], default="128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true", help="per-kernel lines for every configuration")
    ap.add_argument("--only", choices=["gemm", "act", "weight", "kv", "attn", "attnsplit", "decode", "gateup", "downproj", "copy",
                                       "mx", "mxact", "mxdecode", "fused", "downact", "gateact"],
                    help="launch one kernel --steps times back to back (for rocprofv3 runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "this path has no multi-GPU mode; rows shard with no communication.", file=sys.stderr)
        return 2

    import torch

    import rotation_w4a4_quantization_amd as R
    from rotation_w4a4_quantization_amd import _lib
    import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.suite:
        run_suite(torch, R, WL)
        return 0
    if args.only:
        run_only(torch, R, WL, args.only, args.steps, args.had)
        return 0

    dev = torch.device("cuda:0")
    M, N, K = 2048, 4096, 4096
    block = 128 if args.had == "128" else K
    hb = _lib.W4A4_HAD_128 if block == 128 else _lib.W4A4_HAD_FULL
    d = WL.qproj(M=M)
    X = torch.from_numpy(d["X"]).to(dev)
    W = torch.from_numpy(d["W"]).to(dev)
    sets = []
    for _ in range(NSETS):
        sets.append(dict(
            x=X.clone(), w=W.clone(),
            xc=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
            xs=torch.empty((M,), dtype=torch.float32, device=dev),
            wc=torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
            ws=torch.empty((N,), dtype=torch.float32, device=dev),
            wg=torch.empty((N, K // 128), dtype=torch.int32, device=dev),
            y=torch.empty((M, N), dtype=torch.float32, device=dev)))
    del X, W
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    lib = _lib.load()
    from rotation_w4a4_quantization_amd.timing import HipEvents
    hev = HipEvents()
    ptrs = [{k: v.data_ptr() for k, v in s.items()} for s in sets]

    def weight(s):
        return lib.quant_weight_offline(s["w"], N, K, K, hb, None, s["wc"], s["ws"], s["wg"], sp)

    def act(s):
        return lib.rotate_quant_act(s["x"], M, K, K, hb, None, _lib.W4A4_ACT_SYM_TOKEN, s["xc"], s["xs"], None,
                                    sp)

    def gemm(s):
        return lib.w4a4_gemm(s["xc"], s["xs"], None, _lib.W4A4_ACT_SYM_TOKEN, s["wc"], s["ws"], None,
                             M, N, K, s["y"], N, sp)

    def check(st):
        if st:
            raise RuntimeError(f"W4A4 call failed: {_lib.last_error()}")

    # untimed warm-up: --warmup steps, extended to --min-warmup-s seconds of
    # device work (the GPU clocks take a few hundred steps to settle)
    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        s = ptrs[i % NSETS]
        check(weight(s) | act(s) | gemm(s))
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_done = i

    # The GEMM launch of every timed step carries its own pair of events: the
    # runtime stamps the kernel's start and end into them (no marker packets
    # between kernels).  Arming every launch costs enough host time to make
    # the step launch-bound, so the two rotate+quantize kernels are timed the
    # same way in a second pass right after the timed region.
    arm = lib.w4a4_time_next_launch
    ev = [hev.pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = ptrs[i % NSETS]
        st = weight(s) | act(s)
        arm(*ev[i])
        st |= gemm(s)
        check(st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kt = {"w4a4_gemm": sum(hev.elapsed(*e) for e in ev) / args.steps}

    ev2 = [hev.pair() for _ in range(args.steps)]
    for i in range(args.steps):
        s = ptrs[i % NSETS]
        arm(*ev[i])
        st = weight(s)
        arm(*ev2[i])
        st |= act(s)
        st |= gemm(s)
        check(st)
    torch.cuda.synchronize()
    kt["quant_weight_offline"] = sum(hev.elapsed(*e) for e in ev) / args.steps
    kt["rotate_quant_act"] = sum(hev.elapsed(*e) for e in ev2) / args.steps
    hev.close()

    ops = 2.0 * M * N * K
    gemm_tops = ops / (kt["w4a4_gemm"] * 1e-3) / 1e12
    act_bytes = 2 * M * K + M * K // 2 + 4 * M
    w_bytes = 2 * N * K + N * K // 2 + 4 * N + 4 * N * (K // 128)
    act_gbs = act_bytes / (kt["rotate_quant_act"] * 1e-3) / 1e9
    w_gbs = w_bytes / (kt["quant_weight_offline"] * 1e-3) / 1e9

    traffic = profile_traffic(f"w4a4_gemm_qproj_had{args.had}", src_hash("gemm.hip", "common.h", "tile.h"))
    out = {
        "metric": "W4A4 GEMM TOPS (frac INT8 MFMA peak) + rotate+quant GB/s, M×4096×4096",
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_done,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes (int8 MFMA, int32 acc), fp32 transform/scales",
        "data": "synthetic (seeded N(0,1) activations with 8 outlier channels x30, N(0,0.02) weights)",
        "config": {"workload": f"LLaMA-2-7B q_proj W4A4 linear: M=2048, N=4096, K=4096, "
                               f"Hadamard block {block}, symmetric INT4 per token / per channel",
                   "M": M, "N": N, "K": K, "had_block": block},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": INT8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic, "kernel": "w4a4_gemm (gemm_adirect_kernel<8, 2, 4>, 256x128 tiles)",
                     "per_launch_ops": ops, "avg_launch_ms": round(kt["w4a4_gemm"], 5)},
        "kernels": {
            "w4a4_gemm": {"avg_ms": round(kt["w4a4_gemm"], 5), "TOPS": round(gemm_tops, 1),
                          "frac_int8_peak": round(gemm_tops / INT8_PEAK_TOPS, 4)},
            "rotate_quant_act": {"avg_ms": round(kt["rotate_quant_act"], 5), "GB/s": round(act_gbs, 1),
                                 "frac_hbm_peak": round(act_gbs / HBM_PEAK_GBS, 4),
                                 "bytes": act_bytes},
            "quant_weight_offline": {"avg_ms": round(kt["quant_weight_offline"], 5),
                                     "GB/s": round(w_gbs, 1),
                                     "frac_hbm_peak": round(w_gbs / HBM_PEAK_GBS, 4), "bytes": w_bytes},
        },
        # the online part of the layer alone (activation rotate+quant, then the
        # GEMM; the weights quantized once, offline): 2MNK over the sum of the
        # two kernels' device durations, without the gaps between launches
        "online_layer": {"ms": round(kt["rotate_quant_act"] + kt["w4a4_gemm"], 5),
                         "TOPS": round(ops / ((kt["rotate_quant_act"] + kt["w4a4_gemm"]) * 1e-3) / 1e12, 1)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
