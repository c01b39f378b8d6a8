#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer on one MI355X.

A step is one deepseek_moe_forward over one batch (router, routing, counting
sort, grouped SwiGLU experts + shared expert, combine) plus the bias update,
with the inputs resident in HBM. The default workload is the DeepSeek-V3-shaped
prefill layer in bf16 (T=8192, d=7168, 256 routed experts, top-8 in 8 groups of
32 with 4 groups per token, shared expert, intermediate 2048).

Prints ONE JSON line on stdout (progress goes to stderr). Besides the contract
fields it carries:
  roofline      the dominant kernel (gate/up grouped GEMM): algorithmic bytes
                and flops per launch over its mean duration, timed live with
                HIP events recorded by the library on its own stream;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload;
  extra         per-step median / p10 / p90, decode-sized batches
                (T = 16/64/256: per-call median with L2 and the Infinity Cache
                flushed by a 512 MB write before every call, HBM GB/s, and the
                warm back-to-back time beside it), the fp8 layer, its 100-step
                load-balancing loop beside the oracle's own loop, the small
                bf16 and tiny fp32 layers, the training step, the oracle's
                throughput per workload and the stage breakdown.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12}
STAGES = ["gate", "permute", "gemm_gate_up", "gemm_down", "combine"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def wsize(wl) -> float:
    return {"f32": 4.0, "bf16": 2.0, "fp8": 1.0}[wl.w]


def algorithmic(wl, T: int, n_touched: int) -> dict:
    """Algorithmic work per call: top-K sparse flops; every touched expert's
    weights, the router weights, x in and y out once (no intermediates)."""
    sw, sa = wsize(wl), (4.0 if wl.act == "f32" else 2.0)
    TK = T * wl.K
    w_routed = n_touched * 3.0 * wl.d * wl.I * sw
    w_shared = 3.0 * wl.d * wl.Is * sw
    layer_bytes = w_routed + w_shared + wl.E * wl.d * 4.0 + 2.0 * T * wl.d * sa
    layer_flops = T * wl.flops_per_token
    # gate/up grouped GEMM: its weights, x rows once, H written once
    g1_flops = 4.0 * wl.d * (TK * wl.I + T * wl.Is)
    g1_bytes = (n_touched * 2.0 * wl.I * wl.d + 2.0 * wl.Is * wl.d) * sw + T * wl.d * sa + \
        (TK + T) * wl.I * (1.0 if wl.w == "fp8" else sa)
    return {"layer_bytes": layer_bytes, "layer_flops": layer_flops,
            "g1_bytes": g1_bytes, "g1_flops": g1_flops}


def time_layer(layer, x, steps: int, warmup: int, bias_update: bool = True, stages: bool = True):
    import torch
    import sparse_mixture_experts_gate_amd as M
    T = x.shape[0]
    out = layer.alloc_outputs(T)
    layer.workspace(T)
    for _ in range(warmup):
        layer.forward(x, out, with_logits=False)
        if bias_update:
            layer.bias_update(out["counts"], T)
    torch.cuda.synchronize()
    evs = []
    if stages:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        for row in evs:
            for e in row:
                e.record()  # materialize the underlying hipEvent
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        if stages:
            M.moe_profile_events(evs[i])
        layer.forward(x, out, with_logits=False)
        if bias_update:
            layer.bias_update(out["counts"], T)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if stages:
        M.moe_profile_events(None)
    res = {"wall_ms_per_step": wall * 1e3 / steps,
           "gpu_ms_per_step": start.elapsed_time(end) / steps, "out": out}
    if stages:
        st = [[row[j].elapsed_time(row[j + 1]) for j in range(5)] for row in evs]
        res["stage_ms"] = {name: sum(s[j] for s in st) / steps for j, name in enumerate(STAGES)}
        res["step_ms_pctl"] = percentiles([row[0].elapsed_time(row[5]) for row in evs])
    return res


def percentiles(v) -> dict:
    """Median and p10/p90 of per-call times (ms)."""
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def time_cold(layer, x, calls: int, warmup: int) -> dict:
    """Per-call GPU time of the forward with L2 and the Infinity Cache flushed
    before every call: a 512 MB scratch buffer is written first (outside the
    timed events), so the weights come from HBM as in a real decode step."""
    import torch
    T = x.shape[0]
    out = layer.alloc_outputs(T)
    layer.workspace(T)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=x.device)
    for _ in range(warmup):
        layer.forward(x, out, with_logits=False)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for i, (a, b) in enumerate(evs):
        scratch.fill_(i & 0xFF)
        a.record()
        layer.forward(x, out, with_logits=False)
        b.record()
    torch.cuda.synchronize()
    del scratch
    return {"pctl": percentiles([a.elapsed_time(b) for a, b in evs]), "out": out}


def decode_record(wl, T: int, nt: int, warm: dict, cold: dict) -> dict:
    """A decode line: the cold per-call median is the measurement; the warm
    back-to-back wall time is kept beside it."""
    a = algorithmic(wl, T, nt)
    dms = cold["pctl"]["median"]
    return {"ms": dms, "ms_pctl": cold["pctl"], "tokens_per_s": T / (dms / 1e3),
            "hbm_GBps": a["layer_bytes"] / (dms / 1e3) / 1e9,
            "hbm_frac": a["layer_bytes"] / (dms / 1e3) / HBM_PEAK,
            "ms_warm_back_to_back": warm["wall_ms_per_step"], "n_touched": nt,
            "stage_ms_warm": warm["stage_ms"]}


def traffic_record(kernel: str, workload: str):
    """HBM traffic measured by rocprofv3 counters for `kernel`, valid only while
    the kernel's sources (every file its code comes from) are unchanged since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    # one digest over every source file of the kernel (comma-separated names)
    h = hashlib.sha256()
    for name in rec["source"].split(","):
        h.update(open(os.path.join(ROOT, "sparse_mixture_experts_gate_amd", "csrc", name),
                      "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["bytes_per_launch"]


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return int(max(blas) if blas else 1)


def cpu_baseline(wl, P, n_tokens: int, x=None) -> dict:
    """The CPU oracle, unchanged, on the first n_tokens tokens of the batch
    (of ``x`` when given): router product, routing and the fp64 experts.
    Weights of the experts those tokens use are copied to the host before the
    clock starts."""
    import numpy as np
    import oracle as O
    x = (P["x"] if x is None else x)[:n_tokens].float().cpu().numpy()
    wr = P["w_router"].cpu().numpy()
    b = P["bias"].cpu().numpy()
    u = O.router_logits(x, wr)
    rr = O.route(u, b, wl.K, wl.G, wl.M, wl.topn)
    need = np.unique(rr.idx)
    w13 = {int(e): P["w13"][int(e)].float().cpu().numpy() for e in need}
    w2 = {int(e): P["w2"][int(e)].float().cpu().numpy() for e in need}
    ws13 = P["ws13"].float().cpu().numpy() if wl.Is else None
    ws2 = P["ws2"].float().cpu().numpy() if wl.Is else None
    t0 = time.perf_counter()
    O.forward(x, wr, b, w13, w2, ws13, ws2, wl.K, wl.G, wl.M, wl.topn)
    secs = time.perf_counter() - t0
    return {"value": n_tokens / secs, "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{n_tokens} tokens of {wl.name} (T={wl.T}), full oracle forward "
                      f"(fp64 router product, routing, fp64 SwiGLU experts over the "
                      f"{len(need)} experts they use + shared), {secs:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


# Known-byte reads for counter calibration (bench.py --calibrate-loads), one
# per load path of the library's kernels: buffer loads straight into LDS with
# the default and the non-temporal policy (dsmoe_mb_hbm_dma[_default], 1280
# workgroups x 4 waves x 1 KB pieces, a whole number of 8-piece rounds per
# wave, so every byte is read exactly once), and 16-byte register loads with
# both policies (dsmoe_mb_hbm_read[_default], grid-stride, every byte once).
# Kernel-name substring -> bytes read per launch.
DMA_BLOCKS = 1280
DMA_BYTES = ((2 ** 31 - 1) // (8 * DMA_BLOCKS * 4 * 1024)) * 8 * DMA_BLOCKS * 4 * 1024
READ_BYTES = 1 << 30
LOAD_CALIBRATION = {"hbm_dma_kernel<false>": DMA_BYTES, "hbm_dma_kernel<true>": DMA_BYTES,
                    "hbm_read_kernel<false>": READ_BYTES, "hbm_read_kernel<true>": READ_BYTES}


def calibrate_loads() -> None:
    """Three launches of each calibration read (LOAD_CALIBRATION), for the
    counters of a profiled run; nothing is timed."""
    import ctypes
    import torch
    mb = ctypes.CDLL(os.path.join(ROOT, "sparse_mixture_experts_gate_amd",
                                  "libdsmoe_microbench.so"))
    for f in (mb.dsmoe_mb_hbm_dma, mb.dsmoe_mb_hbm_dma_default):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    for f in (mb.dsmoe_mb_hbm_read, mb.dsmoe_mb_hbm_read_default):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                      ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.ones(max(DMA_BYTES, READ_BYTES), dtype=torch.uint8, device="cuda")
    blocks = 8192
    sink = torch.empty(blocks * 256 * 4, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        for f in (mb.dsmoe_mb_hbm_dma_default, mb.dsmoe_mb_hbm_dma):
            if f(buf.data_ptr(), DMA_BYTES, DMA_BLOCKS, stream) != 0:
                raise RuntimeError("calibration launch failed")
        for f in (mb.dsmoe_mb_hbm_read_default, mb.dsmoe_mb_hbm_read):
            if f(buf.data_ptr(), READ_BYTES, blocks, sink.data_ptr(), stream) != 0:
                raise RuntimeError("calibration launch failed")
    torch.cuda.synchronize()
    del buf, sink


def achievable_peaks() -> dict:
    """Microbenchmarked peaks of this GPU (libdsmoe_microbench.so, hand-written
    HIP kernels): streaming reads far beyond the 256 MB Infinity Cache, once
    into registers (4 GiB) and once over the layer's own LDS-DMA load path
    (2 GiB), streaming writes of 4 GiB (4- and 16-byte stores, default and
    non-temporal), and back-to-back independent MFMAs with operands in registers,
    bf16 32x32x16 and FP8 32x32x64. Each is the best of 3 timed launches
    after a warm-up launch."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "sparse_mixture_experts_gate_amd", "libdsmoe_microbench.so")
    mb = ctypes.CDLL(path)
    mb.dsmoe_mb_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    mb.dsmoe_mb_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    mb.dsmoe_mb_hbm_dma.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 4 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    blocks = cus * 32
    sink = torch.empty(blocks * 256 * 4, dtype=torch.uint8, device="cuda")

    def best(launch, reps=3):
        launch()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = launch()
            b.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"microbenchmark launch failed: {rc}")
            times.append(a.elapsed_time(b) / 1e3)
        return min(times)

    t_read = best(lambda: mb.dsmoe_mb_hbm_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                               stream))
    dma_bytes = (2 << 30) - 1024
    t_dma = best(lambda: mb.dsmoe_mb_hbm_dma(buf.data_ptr(), dma_bytes, cus * 5, stream))
    res = {"hbm_read_GBps": nbytes / t_read / 1e9, "hbm_dma_GBps": dma_bytes / t_dma / 1e9}
    # writes: 4-byte and 16-byte stores, default and non-temporal policy
    mb.dsmoe_mb_hbm_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    for mode, key in ((0, "hbm_write_b32_GBps"), (1, "hbm_write_b32_nt_GBps"),
                      (2, "hbm_write_b128_GBps"), (3, "hbm_write_b128_nt_GBps")):
        t = best(lambda: mb.dsmoe_mb_hbm_write(buf.data_ptr(), nbytes, blocks, mode, stream))
        res[key] = nbytes / t / 1e9
    del buf
    for name, fp8, iters, flops in (("mfma_bf16_TFLOPs", 0, 20000, 32768.0),
                                    ("mfma_fp8_TFLOPs", 1, 10000, 131072.0)):
        t = best(lambda: mb.dsmoe_mb_mfma(fp8, iters, blocks, sink.data_ptr(), stream))
        res[name] = blocks * 4 * iters * 8 * flops / t / 1e12
    return res


def cpu_baseline_fp8(wl, layer_bf16_P, x, n_tokens: int, workers: int) -> dict:
    """The oracle's FP8 forward on n_tokens tokens: routing from its own fp64
    logits, x quantized in 1x128 tiles, the E4M3 experts (the oracle's own
    128x128 block quantization of the bf16 weights, done before the clock,
    like the library's once-per-weight-set preparation) with fp32 H
    re-quantized. The experts run on ``workers`` threads."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    P = layer_bf16_P
    xh = x[:n_tokens].float().cpu().numpy()
    u = O.router_logits(xh, P["w_router"].cpu().numpy())
    rr = O.route(u, P["bias"].cpu().numpy(), wl.K, wl.G, wl.M, wl.topn)
    need = [int(e) for e in np.unique(rr.idx)]

    def quant(e):
        return e, O.quantize_blocks_128(P["w13"][e].float().cpu().numpy()), \
            O.quantize_blocks_128(P["w2"][e].float().cpu().numpy())

    with ThreadPoolExecutor(workers) as ex:
        qs = {e: (a, b) for e, a, b in ex.map(quant, need)}
    sh13 = O.quantize_blocks_128(P["ws13"].float().cpu().numpy())
    sh2 = O.quantize_blocks_128(P["ws2"].float().cpu().numpy())

    class _Pick:
        def __init__(self, which, part):
            self.which, self.part = which, part

        def __getitem__(self, e):
            return qs[int(e)][self.which][self.part]

    t0 = time.perf_counter()
    u = O.router_logits(xh, P["w_router"].cpu().numpy())
    rr = O.route(u, P["bias"].cpu().numpy(), wl.K, wl.G, wl.M, wl.topn)
    O.layer_output_fp8(xh, rr.idx, rr.gate, _Pick(0, 0), _Pick(0, 1), _Pick(1, 0), _Pick(1, 1),
                       sh13[0], sh13[1], sh2[0], sh2[1], workers=workers)
    secs = time.perf_counter() - t0
    return {"value": n_tokens / secs, "unit": "tokens/s", "cores": max(workers, blas_threads()),
            "kind": "oracle",
            "sample": f"{n_tokens} tokens of {wl.name}: fp64 router product, routing, FP8 "
                      f"experts ({len(need)} routed + shared, E4M3 weights prepared before the "
                      f"clock) on {workers} threads, {secs:.1f} s"}


def small_record(dev, cpu: bool) -> dict:
    """The small bf16 layer (T = 4096, d = 2048, 64 experts of 1408, top-6,
    shared expert of 2816, clustered tokens): tokens/s, the layer's and the
    gate/up GEMM's fraction of the bf16 MFMA peak, and the oracle on all its
    tokens."""
    import sparse_mixture_experts_gate_amd as M
    from sparse_mixture_experts_gate_amd.workloads import CONFIGS, make_inputs
    wl = CONFIGS["small_bf16"]
    P = make_inputs(wl, dev)
    layer = M.MoELayer(wl, P)
    r = time_layer(layer, P["x"], 50, 5)
    nt = int((r["out"]["counts"] > 0).sum())
    a = algorithmic(wl, wl.T, nt)
    ms = r["wall_ms_per_step"]
    g1 = r["stage_ms"]["gemm_gate_up"]
    rec = {"T": wl.T, "ms": ms, "ms_pctl": r["step_ms_pctl"], "tokens_per_s": wl.T / (ms / 1e3),
           "layer_mfma_frac": a["layer_flops"] / (ms / 1e3) / MFMA_PEAK["bf16"],
           "layer_hbm_frac": a["layer_bytes"] / (ms / 1e3) / HBM_PEAK,
           "gemm_gate_up_ms": g1,
           "gemm_gate_up_mfma_frac": a["g1_flops"] / (g1 / 1e3) / MFMA_PEAK["bf16"],
           "stage_ms": r["stage_ms"], "n_touched": nt}
    if cpu:
        rec["cpu_oracle"] = cpu_baseline(wl, P, wl.T)
    return rec


def fp8_loop_record(layer8, wl8, P, dev, steps: int = 100) -> dict:
    """The FP8 layer's load-balancing loop: `steps` forwards + bias updates
    (gamma = 0.001) on fresh Zipf-skewed batches (seed 1000 + s), from the
    layer's initial bias. Beside it the oracle runs the same loop on its own:
    its own fp64 router logits, routing, counts and bias update on every
    token of every batch (routing only, timed on the host cores). Reports
    the max/mean expert load of both per step and their difference."""
    import numpy as np
    import torch
    import oracle as O
    from sparse_mixture_experts_gate_amd.workloads import make_tokens
    T, E, K = wl8.T, wl8.E, wl8.K
    mean = T * K / E
    layer8.bias.copy_(P["bias"])
    out = layer8.alloc_outputs(T)
    layer8.workspace(T)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    gpu = []
    for s in range(steps):
        x = make_tokens(wl8, T, 1000 + s, dev)
        ev[s][0].record()
        layer8.forward(x, out, with_logits=False)
        layer8.bias_update(out["counts"], T)
        ev[s][1].record()
        gpu.append(float(out["counts"].max().item()) / mean)
    torch.cuda.synchronize()
    step_ms = percentiles([a.elapsed_time(b) for a, b in ev])
    wr = P["w_router"].cpu().numpy()
    b = P["bias"].cpu().numpy()
    ora, secs = [], 0.0
    for s in range(steps):
        xh = make_tokens(wl8, T, 1000 + s, dev).float().cpu().numpy()
        t0 = time.perf_counter()
        rr = O.route(O.router_logits(xh, wr), b, K, wl8.G, wl8.M, wl8.topn)
        counts = np.bincount(rr.idx.ravel(), minlength=E)
        b = O.bias_update(b, counts, wl8.gamma, T, K)
        secs += time.perf_counter() - t0
        ora.append(float(counts.max()) / mean)
    diff = np.abs(np.asarray(gpu) - np.asarray(ora))
    return {"steps": steps, "gamma": wl8.gamma, "T": T,
            "gpu_step_ms": step_ms,
            "max_over_mean_gpu": [round(v, 4) for v in gpu],
            "max_over_mean_oracle": [round(v, 4) for v in ora],
            "abs_diff_max": float(diff.max()), "abs_diff_mean": float(diff.mean()),
            "first": {"gpu": gpu[0], "oracle": ora[0]},
            "final": {"gpu": gpu[-1], "oracle": ora[-1]},
            "mean_last10": {"gpu": float(np.mean(gpu[-10:])), "oracle": float(np.mean(ora[-10:]))},
            "oracle_loop": {"value": steps * T / secs, "unit": "tokens/s", "seconds": secs,
                            "cores": blas_threads(), "kind": "oracle",
                            "sample": f"{steps} steps x {T} tokens, routing only (fp64 router "
                                      f"product, routing, counts, bias update)"}}


# sequences of the balance loss: the pages fix no length; 4096 tokens, two
# sequences per 8192-token batch
BALANCE_SEQ_LEN = 4096
BALANCE_ALPHA = 1e-4


def time_train(layer, x, steps: int, warmup: int) -> dict:
    """One training step of the layer per iteration: the training forward
    (moe_forward_train), the sequence-level balance loss with its gradients
    (moe_seq_balance_loss) and the backward (moe_backward), each bracketed by
    HIP events on the current stream. dy is a seeded bf16 N(0, 1) tensor."""
    import torch
    T, d = x.shape
    L = BALANCE_SEQ_LEN if T % BALANCE_SEQ_LEN == 0 else T
    g = torch.Generator(device=x.device)
    g.manual_seed(99)
    dy = torch.randn(T, d, generator=g, device=x.device).to(torch.bfloat16)
    sv = layer.alloc_saved(T)
    grads = layer.alloc_grads()
    for _ in range(warmup):
        layer.forward_train(x, sv)
        layer.seq_balance_loss(x, sv, L, BALANCE_ALPHA)
        layer.backward(x, dy, sv, grads)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        layer.forward_train(x, sv)
        ev[i][1].record()
        layer.seq_balance_loss(x, sv, L, BALANCE_ALPHA)
        ev[i][2].record()
        layer.backward(x, dy, sv, grads)
        ev[i][3].record()
    torch.cuda.synchronize()
    fwd = [e[0].elapsed_time(e[1]) for e in ev]
    bal = [e[1].elapsed_time(e[2]) for e in ev]
    bwd = [e[2].elapsed_time(e[3]) for e in ev]
    return {"fwd_train_ms": percentiles(fwd)["median"], "bwd_ms": percentiles(bwd)["median"],
            "bwd_ms_pctl": percentiles(bwd), "balance_ms": percentiles(bal)["median"],
            "balance_ms_pctl": percentiles(bal), "balance_seq_len": L}


def train_record(wl, T: int, r: dict) -> dict:
    # expert GEMM flops of the forward (gate, up, down per routed pair and
    # shared row); the backward's input- and weight-gradient GEMMs are twice that
    fwd_fl = (6.0 * wl.d * wl.I * wl.K + 6.0 * wl.d * wl.Is) * T
    bwd_fl = 2.0 * fwd_fl
    tf = bwd_fl / (r["bwd_ms"] / 1e3)
    # balance loss: reads the logits, the selection, x and W_r once and writes
    # dx and dW_r (fp32); its two products take 2 T E d flops each
    bal_bytes = (T * wl.E * 4 + T * wl.K * 4 + T * wl.d * 2 + wl.E * wl.d * 4 + T * wl.d * 4
                 + wl.E * wl.d * 4)
    bal_s = r["balance_ms"] / 1e3
    return {"T": T, "fwd_train_ms": r["fwd_train_ms"], "bwd_ms": r["bwd_ms"],
            "bwd_ms_pctl": r["bwd_ms_pctl"],
            "bwd_gemm_tflop": bwd_fl / 1e12, "bwd_tflops": tf / 1e12,
            "bwd_mfma_frac": tf / MFMA_PEAK["bf16"],
            "balance_loss": {"ms": r["balance_ms"], "ms_pctl": r["balance_ms_pctl"],
                             "seq_len": r["balance_seq_len"], "alpha": BALANCE_ALPHA,
                             "alg_bytes": bal_bytes, "hbm_GBps": bal_bytes / bal_s / 1e9,
                             "hbm_frac": bal_bytes / bal_s / HBM_PEAK,
                             "gflop": 4.0 * T * wl.E * wl.d / 1e9},
            "train_step_tokens_per_s":
                T / ((r["fwd_train_ms"] + r["balance_ms"] + r["bwd_ms"]) / 1e3)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy three times, so that HBM byte "
                         "counters can be scaled against a kernel of known traffic")
    ap.add_argument("--calibrate-loads", action="store_true",
                    help="also read known byte counts through each load path of the kernels "
                         "(LDS-DMA and register loads, default and non-temporal policy)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-loop", action="store_true",
                    help="skip the FP8 layer's 100-step load-balancing loop and its oracle loop")
    ap.add_argument("--train-only", action="store_true",
                    help="only time the training step (forward, balance loss, backward) of the "
                         "workload and print that record (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer and runs on one GPU only; "
              "--gpus must be 1.", file=sys.stderr)
        return 2

    import torch
    import sparse_mixture_experts_gate_amd as M
    from sparse_mixture_experts_gate_amd.workloads import CONFIGS, make_inputs, make_tokens

    wl = CONFIGS[args.workload]
    dev = "cuda"
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.calibrate_loads:
        calibrate_loads()
    log(f"generating {wl.name} inputs")
    P = make_inputs(wl, dev)
    layer = M.MoELayer(wl, P)
    if args.train_only:
        log(f"timing the training step of {wl.name}: warmup {args.warmup}, steps {args.steps}")
        rec = train_record(wl, wl.T, time_train(layer, P["x"], args.steps, args.warmup))
        log(f"train: forward {rec['fwd_train_ms']:.3f} ms, balance loss "
            f"{rec['balance_loss']['ms']:.3f} ms, backward {rec['bwd_ms']:.3f} ms "
            f"({rec['bwd_tflops']:.0f} TFLOP/s)")
        if wl.w == "fp8":
            rec["bwd_mfma_frac_fp8"] = rec["bwd_tflops"] * 1e12 / MFMA_PEAK["fp8"]
        key = "train_fp8" if wl.w == "fp8" else "train_bf16"
        print(json.dumps({key: rec, "workload": wl.name}), flush=True)
        return 0
    log(f"timing {wl.name}: warmup {args.warmup}, steps {args.steps}")
    r = time_layer(layer, P["x"], args.steps, args.warmup)
    counts = r["out"]["counts"].cpu()
    n_touched = int((counts > 0).sum())
    near = int(r["out"]["near_tie"].item())
    ms = r["wall_ms_per_step"]
    tok_s = wl.T / (ms / 1e3)
    alg = algorithmic(wl, wl.T, n_touched)
    g1_ms = r["stage_ms"]["gemm_gate_up"]
    g1_bw = alg["g1_bytes"] / (g1_ms / 1e3)
    g1_fl = alg["g1_flops"] / (g1_ms / 1e3)
    bound = "hbm" if alg["g1_bytes"] / HBM_PEAK >= alg["g1_flops"] / MFMA_PEAK[wl.w] else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": g1_bw / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": g1_bw / HBM_PEAK}
    else:
        roof = {"bound": "mfma", "achieved": g1_fl / 1e12, "peak": MFMA_PEAK[wl.w] / 1e12,
                "unit": "TFLOP/s", "frac": g1_fl / MFMA_PEAK[wl.w]}
    roof.update({"kernel": "ffn1_bf16_kernel (grouped gate/up GEMM + SwiGLU)",
                 "traffic": traffic_record("ffn1_bf16", wl.name),
                 "ms_per_launch": g1_ms, "alg_bytes_per_launch": alg["g1_bytes"],
                 "alg_flops_per_launch": alg["g1_flops"],
                 "mfma_frac": g1_fl / MFMA_PEAK[wl.w], "hbm_frac": g1_bw / HBM_PEAK})
    if not args.no_extra:
        ach = achievable_peaks()
        log("achievable: " + json.dumps({k: round(v, 1) for k, v in ach.items()}))
        if bound == "hbm":
            hbm_ach = max(ach["hbm_read_GBps"], ach["hbm_dma_GBps"])
            roof.update({"achievable_peak": hbm_ach, "frac_of_achievable": g1_bw / 1e9 / hbm_ach})
        else:
            key = "mfma_fp8_TFLOPs" if wl.w == "fp8" else "mfma_bf16_TFLOPs"
            roof.update({"achievable_peak": ach[key], "frac_of_achievable": g1_fl / 1e12 / ach[key]})
    layer_mfma = alg["layer_flops"] / (ms / 1e3) / MFMA_PEAK[wl.w]
    layer_hbm = alg["layer_bytes"] / (ms / 1e3) / HBM_PEAK
    log(f"{wl.name}: {ms:.3f} ms/step, {tok_s/1e6:.3f} M tok/s, layer MFMA {layer_mfma:.1%}, "
        f"HBM {layer_hbm:.1%}; stages {json.dumps({k: round(v, 3) for k, v in r['stage_ms'].items()})}")

    extra = {"stage_ms": r["stage_ms"], "gpu_ms_per_step": r["gpu_ms_per_step"],
             "step_ms_pctl": r["step_ms_pctl"],
             "layer_mfma_frac": layer_mfma, "layer_hbm_frac": layer_hbm,
             "n_touched_experts": n_touched, "near_tie_tokens": near,
             "near_tie_frac": near / wl.T, "max_over_mean_load": float(counts.max()) / (wl.T * wl.K / wl.E)}
    if not args.no_extra:
        extra["achievable_peaks"] = ach
    if not args.no_extra and wl.name == "v3_prefill_bf16":
        dec = {}
        for T in (16, 64, 256):
            x = make_tokens(CONFIGS["v3_decode_bf16"], T, 3, dev)
            rd = time_layer(layer, x, 20, 3, bias_update=False)
            rc = time_cold(layer, x, 20, 3)
            nt = int((rd["out"]["counts"] > 0).sum())
            dec[str(T)] = decode_record(wl, T, nt, rd, rc)
            log(f"decode T={T}: {dec[str(T)]['ms']:.3f} ms (cold, median), "
                f"{dec[str(T)]['hbm_GBps']:.0f} GB/s, {nt} experts; warm back-to-back "
                f"{rd['wall_ms_per_step']:.3f} ms")
        extra["decode_bf16"] = dec
        tr = train_record(wl, wl.T, time_train(layer, P["x"], 5, 2))
        extra["train_bf16"] = tr
        log(f"train: forward {tr['fwd_train_ms']:.3f} ms, balance loss "
            f"{tr['balance_loss']['ms']:.3f} ms, backward {tr['bwd_ms']:.3f} ms "
            f"({tr['bwd_tflops']:.0f} TFLOP/s)")
        layer._bws = None
        layer._sws = None
        torch.cuda.empty_cache()
        try:
            wl8 = CONFIGS["v3_fp8"]
            layer8 = M.MoELayer(wl8, P)
            r8 = time_layer(layer8, P["x"], 10, 3)
            ms8 = r8["wall_ms_per_step"]
            a8 = algorithmic(wl8, wl8.T, int((r8["out"]["counts"] > 0).sum()))
            extra["fp8"] = {"ms": ms8, "tokens_per_s": wl8.T / (ms8 / 1e3),
                            "mfma_frac_fp8": a8["layer_flops"] / (ms8 / 1e3) / MFMA_PEAK["fp8"],
                            "hbm_frac": a8["layer_bytes"] / (ms8 / 1e3) / HBM_PEAK,
                            "stage_ms": r8["stage_ms"]}
            log(f"fp8: {ms8:.3f} ms, {wl8.T / ms8 * 1e3 / 1e6:.3f} M tok/s")
            dec8 = {}
            for T in (16, 64, 256):
                x = make_tokens(CONFIGS["v3_decode_bf16"], T, 3, dev)
                rd = time_layer(layer8, x, 20, 3, bias_update=False)
                rc = time_cold(layer8, x, 20, 3)
                nt = int((rd["out"]["counts"] > 0).sum())
                dec8[str(T)] = decode_record(wl8, T, nt, rd, rc)
                log(f"fp8 decode T={T}: {dec8[str(T)]['ms']:.3f} ms (cold, median), "
                    f"{dec8[str(T)]['hbm_GBps']:.0f} GB/s, {nt} experts; warm back-to-back "
                    f"{rd['wall_ms_per_step']:.3f} ms")
            extra["decode_fp8"] = dec8
            tr8 = train_record(wl8, wl8.T, time_train(layer8, P["x"], 5, 2))
            tr8["bwd_mfma_frac_fp8"] = tr8["bwd_tflops"] * 1e12 / MFMA_PEAK["fp8"]
            extra["train_fp8"] = tr8
            log(f"train fp8: forward {tr8['fwd_train_ms']:.3f} ms, balance loss "
                f"{tr8['balance_loss']['ms']:.3f} ms, backward {tr8['bwd_ms']:.3f} ms "
                f"({tr8['bwd_tflops']:.0f} TFLOP/s)")
            layer8._bws = None
            layer8._sws = None
            layer8._wt = layer8._wt_tensors = None
            torch.cuda.empty_cache()
            if not args.no_loop:
                log("fp8 load-balancing loop: 100 steps, then the oracle's own loop")
                lp = fp8_loop_record(layer8, wl8, P, dev)
                extra["fp8_bias_loop"] = lp
                log(f"fp8 loop: max/mean load gpu {lp['first']['gpu']:.3f} -> "
                    f"{lp['final']['gpu']:.3f}, oracle {lp['first']['oracle']:.3f} -> "
                    f"{lp['final']['oracle']:.3f}, max |diff| {lp['abs_diff_max']:.3f}; oracle "
                    f"loop {lp['oracle_loop']['value']:.0f} tokens/s")
            del layer8
        except M.MoeError as e:
            extra["fp8"] = {"error": str(e)}
            log(f"fp8: {e}")
        log("small bf16 layer")
        sm = small_record(dev, not args.no_cpu_baseline)
        extra["small_bf16"] = sm
        log(f"small_bf16: {sm['ms']:.3f} ms, {sm['tokens_per_s'] / 1e6:.2f} M tok/s, layer MFMA "
            f"{sm['layer_mfma_frac']:.1%}, gate/up GEMM MFMA {sm['gemm_gate_up_mfma_frac']:.1%}")
        tw = CONFIGS["tiny_f32"]
        Pt = make_inputs(tw, dev)
        rt = time_layer(M.MoELayer(tw, Pt), Pt["x"], 50, 5)
        extra["tiny_f32"] = {"T": tw.T, "ms": rt["wall_ms_per_step"],
                             "tokens_per_s": tw.T / (rt["wall_ms_per_step"] / 1e3)}
        if not args.no_cpu_baseline:
            cpus = {"tiny_f32": cpu_baseline(tw, Pt, tw.T)}
            xd = make_tokens(CONFIGS["v3_decode_bf16"], 64, 3, dev)
            cpus["v3_decode_bf16_T64"] = cpu_baseline(wl, P, 64, x=xd)
            workers = max(1, min(16, len(os.sched_getaffinity(0))))
            cpus["v3_fp8"] = cpu_baseline_fp8(CONFIGS["v3_fp8"], P, P["x"], 8, workers)
            extra["cpu_oracle_per_config"] = cpus
            log("cpu oracle per config: " + json.dumps(
                {k: round(v["value"], 1) for k, v in cpus.items()}))

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu oracle baseline on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(wl, P, args.cpu_tokens)
        log(f"cpu oracle: {cpu['value']:.2f} tokens/s on {cpu['cores']} BLAS threads")

    line = {"metric": "MoE-layer tokens/s at V3 shape (bf16, fp8) + % of MFMA/HBM roofline",
            "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": wl.w, "data": "synthetic",
            "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "n_experts": wl.E,
                       "top_k": wl.K, "groups": wl.G, "topk_groups": wl.M, "inter": wl.I,
                       "shared_inter": wl.Is, "parallelism": "single GPU"},
            "roofline": roof, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
