"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

One step = one W4A4 linear of the QKV projection of a 5B video DiT block:
activation amax + NVFP4 quantization of X bf16 [2640, 3072] + NVFP4 GEMM
against the pre-quantized weight W [9216, 3072] (16x16 tiles, four-over-six)
with fp32 accumulation and bf16 output -- one call of nvfp4_linear.
`value` is its throughput in TFLOP/s (2*M*N*K per step), inputs resident in
device memory, three rotating input/weight sets.

The same JSON line also carries
  step_ms_events  p10 / median / p90 of the per-step GPU times (events
                recorded between the timed steps);
  gpu_state     clock levels and board power (sysfs) read while the step
                runs (untimed), the device name and a SHA-256 stamp of the
                library sources;
  roofline      the GEMM kernel alone, timed with HIP events on its stream,
                against the fp16 MFMA peak (its operands are exact fp16);
  kv            NVFP4 KV-cache quantize and dequantize of K and V bf16
                [24, 18480, 128] in GB/s of algorithmic bytes, and against HBM;
  extra         the FFN pair, the QKV projection with a rank-128 LoRA
                branch, the long-sequence training shapes (forward, weight
                gradient with and without the Hadamard transform, data
                gradient), and for context the vendor library's dense
                fp16/bf16 GEMM on the QKV shape;
  cpu_baseline  the CPU oracle (fp32 quantizer, fp64 GEMM) on the full QKV
                step on the host cores;
  parity        the oracle's results of that leg against the library's on
                the same seeded inputs (the first timed input set): codes,
                scales and alpha bit-exact, fp32 output within relative
                Frobenius 1e-5, bf16 output = RNE of the fp32 one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--parts qkv,kv,extra,cpu]
       python bench.py --copy-calibration   (a plain 256 MiB device copy, for
                                             scaling rocprofv3 byte counters)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 W4A4 GEMM TFLOPS incl. act-quantize at DiT shapes; KV-quantize GB/s"
HBM_PEAK_GBPS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0       # dense fp16/bf16 MFMA, MI355X
FP4_MFMA_PEAK_TFLOPS = 10100.0       # context only
PEAK_SCLK_MHZ = 2400.0               # the shader clock the published peaks assume


# HBM bytes per launch of the QKV-shaped GEMM kernel, from rocprofv3 byte
# counters: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, the factors being what the two
# counters read for a plain 256 MiB device copy.  They hold for the GEMM
# sources they were taken with only (gemm.hip and the device.h it includes):
# null once either has changed.
GEMM_TRAFFIC = {"gemm_src_sha256": "f1c497d5a1005289773b45335bf58a0da255df806e3dcd28e5cddff1a83ceaff",
                "bytes_per_launch": 107723821}


def gemm_src_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in ("gemm.hip", "device.h"):
        with open(os.path.join(ROOT, "nvfp4_w4a4_quantized_04_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def gemm_traffic():
    return GEMM_TRAFFIC["bytes_per_launch"] if gemm_src_sha256() == GEMM_TRAFFIC["gemm_src_sha256"] else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def time_events(fn, iters: int, warmup: int = 3) -> float:
    """Average milliseconds per call of fn() measured with events on the
    current stream (where the library enqueues), after >= 0.5 s of warm-up."""
    import torch
    t_end = time.perf_counter() + 0.5
    i = 0
    while time.perf_counter() < t_end or i < warmup:
        fn(i)
        i += 1
        if i % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def linear_sets(nv, workloads, m, k, n, nsets, seed0):
    """Rotating (x, packed W, y, workspace) sets for one linear shape."""
    import torch
    sets = []
    for i in range(nsets):
        c = workloads.config2(seed=seed0 + 100 * i, m=m, k=k, n=n)
        x = dev_bf16(c["x"])
        w = nv.quantize(dev_bf16(c["w"]), "tile16", "4over6")
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = nv.linear_workspace(m, k)
        sets.append((x, w, y, ws))
    torch.cuda.synchronize()
    return sets


def bench_linear(nv, sets, steps, warmup):
    import torch

    def step(i):
        x, w, y, ws = sets[i % len(sets)]
        nv.linear(x, w, torch.bfloat16, out=y, workspace=ws)

    # clocks ramp up over the first few hundred milliseconds of sustained work
    t_end = time.perf_counter() + 1.0
    i = 0
    while time.perf_counter() < t_end or i < warmup:
        step(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # one event after each step (a marker on the stream, no sync): the gaps
    # between consecutive events are the per-step GPU times
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    q = lambda f: per[min(steps - 1, int(f * steps))]
    return ms, {"p10": round(q(0.1), 5), "median": round(q(0.5), 5), "p90": round(q(0.9), 5)}


def read_gpu_clocks():
    """Current shader/memory clock levels and board power from sysfs (the
    level marked '*' in pp_dpm_sclk / pp_dpm_mclk, hwmon power in W).  Plain
    file reads: no tool is started."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        info = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
                info[name] = cur[0] if cur else None
            except OSError:
                pass
        for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
            for pname in ("power1_average", "power1_input"):
                try:
                    with open(os.path.join(hw, pname)) as f:
                        info[pname + "_W"] = int(f.read().strip()) / 1e6
                except (OSError, ValueError):
                    pass
        if info:
            out[os.path.basename(os.path.dirname(dev))] = info
    return out or None


def sclk_mhz(state):
    """The shader clock in MHz from gpu_state's sysfs reading ("1: 2023Mhz *"),
    or None."""
    try:
        for card in (state or {}).get("clocks", {}).values():
            v = card.get("pp_dpm_sclk")
            if v:
                return float(v.split(":")[1].strip().lower().split("mhz")[0])
    except (AttributeError, IndexError, ValueError):
        return None
    return None


def gpu_state_under_load(step, seconds=2.0):
    """Clock levels and power read from sysfs halfway through `seconds` of the
    step running back to back (untimed), plus a stamp of the library
    sources."""
    import glob
    import hashlib
    import threading
    import torch
    out = {}

    def sample():
        time.sleep(seconds / 2)
        out["clocks"] = read_gpu_clocks()

    th = threading.Thread(target=sample)
    t_end = time.perf_counter() + seconds
    i = 0
    th.start()
    while time.perf_counter() < t_end or th.is_alive():
        step(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
        if time.perf_counter() > t_end + 5:
            break
    torch.cuda.synchronize()
    th.join(timeout=1)
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "nvfp4_w4a4_quantized_04_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    out["device"] = torch.cuda.get_device_name(0)
    out["csrc_sha256"] = h.hexdigest()
    return out


def bench_gemm_kernel(nv, sets, iters):
    """The GEMM kernel alone on pre-quantized activations (events)."""
    import torch
    packed = []
    for x, w, y, ws in sets:
        packed.append((nv.quantize(x, "row16", "4over6"), w, y))
    torch.cuda.synchronize()

    def call(i):
        a, w, y = packed[i % len(packed)]
        nv.gemm(a, w, torch.bfloat16, out=y)

    return time_events(call, iters)


def bench_kv(nv, workloads, iters):
    """KV-cache quantize (K and V bf16 [24, 18480, 128]) and dequantize.

    Two modes of nvfp4_kv_quantize: the amax computed inside the call (two
    passes over the tensor), and the amax handed in by the GEMM that produced
    K or V (its epilogue writes max |C|; one pass)."""
    import torch
    c = workloads.config4()
    heads, tokens, d = c["k"].shape
    n = heads * tokens * d
    wsz = nv.lib.nvfp4_quantize_workspace_size(heads * tokens, d)

    def entry(t):
        return (t, nv.empty_packed(heads * tokens, d, nv.ROW16),
                torch.empty((heads * tokens, d), dtype=torch.bfloat16, device="cuda"),
                torch.empty(wsz, dtype=torch.uint8, device="cuda"),
                t.float().abs().max().reshape(1).contiguous())

    sets = [entry(dev_bf16(c["k"])), entry(dev_bf16(c["v"]))]
    # a third tensor so consecutive calls never find their input in the
    # 256 MB last-level cache
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    sets.append(entry(torch.randn((heads, tokens, d), generator=g, device="cuda").to(torch.bfloat16)))
    torch.cuda.synchronize()

    def q2(i):
        kv, p, y, ws, am = sets[i % len(sets)]
        nv.kv_quantize(kv, "4over6", out=p, workspace=ws)

    def q1(i):
        kv, p, y, ws, am = sets[i % len(sets)]
        nv.kv_quantize(kv, "4over6", out=p, workspace=ws, amax=am)

    def dq(i):
        kv, p, y, ws, am = sets[i % len(sets)]
        nv.dequantize(p, torch.bfloat16, out=y)

    def copy(i):
        # context: a plain device copy of one 113.5 MB tensor (torch), the
        # rate a read-and-write stream reaches on this machine
        sets[i % len(sets)][2].view(heads, tokens, d).copy_(sets[(i + 1) % len(sets)][0])

    # the pages' granularity: one global scale per 8-frame chunk (7040 tokens:
    # chunks of 8, 8 and 5 frames) of K and of V, both tensors and all their
    # chunks in one call; two such [2, heads, tokens, d] pairs alternate
    tpc = 8 * 880
    pairs = [torch.stack((sets[0][0], sets[1][0])), torch.stack((sets[2][0], sets[0][0].neg()))]
    cpk = [nv.kv_quantize_chunked(p, tpc) for p in pairs]
    cy = [torch.empty_like(p) for p in pairs]
    cws = torch.empty(nv.lib.nvfp4_kv_chunked_workspace_size(2, heads, tokens, d, tpc), dtype=torch.uint8,
                      device="cuda")
    torch.cuda.synchronize()

    # the chunks' maxima as the pages' streaming inference has them: each
    # chunk's K and V come out of that chunk's projection, whose epilogue
    # reports max |C| (one read per call)
    nch = (tokens + tpc - 1) // tpc
    cam = [torch.stack([p[u, :, c * tpc:(c + 1) * tpc].float().abs().amax() for u in range(2) for c in range(nch)])
           .contiguous() for p in pairs]
    torch.cuda.synchronize()

    def qc(i):
        nv.kv_quantize_chunked(pairs[i % 2], tpc, out=cpk[i % 2], workspace=cws)

    def qc1(i):
        nv.kv_quantize_chunked(pairs[i % 2], tpc, out=cpk[i % 2], chunk_amax=cam[i % 2])

    def dqc(i):
        nv.kv_dequantize_chunked(cpk[i % 2], torch.bfloat16, out=cy[i % 2])

    t2 = time_events(q2, iters)
    t1 = time_events(q1, iters)
    tdq = time_events(dq, iters)
    tcp = time_events(copy, iters)
    tqc = time_events(qc, iters) / 2                  # per tensor: each call quantizes K and V
    tqc1 = time_events(qc1, iters) / 2
    tdqc = time_events(dqc, iters) / 2
    bytes_q = n * 2 + n * 9 / 16 + 4          # read bf16, write codes + scales + alpha
    bytes_dq = n * 9 / 16 + 4 + n * 2

    def rate(b, ms):
        gbps = b / (ms * 1e-3) / 1e9
        return round(gbps, 1), round(gbps / HBM_PEAK_GBPS, 4)

    r2, r1, rd = rate(bytes_q, t2), rate(bytes_q, t1), rate(bytes_dq, tdq)
    rc, rdc = rate(bytes_q + 4 * (nch - 1), tqc), rate(bytes_dq + 4 * (nch - 1), tdqc)
    rc1 = rate(bytes_q + 4 * (nch - 1), tqc1)
    del sets, pairs, cpk, cy, cam
    torch.cuda.empty_cache()
    win = bench_kv_window(nv, iters)
    return {
        "workload": f"K/V bf16 [{heads},{tokens},{d}], 16-blocks along head_dim, four-over-six",
        "quantize_ms_per_tensor": round(t2, 5), "quantize_GBps": r2[0], "quantize_frac_hbm": r2[1],
        "quantize_1pass_ms_per_tensor": round(t1, 5), "quantize_1pass_GBps": r1[0],
        "quantize_1pass_frac_hbm": r1[1],
        "dequantize_ms_per_tensor": round(tdq, 5), "dequantize_GBps": rd[0], "dequantize_frac_hbm": rd[1],
        "per_chunk_alpha": {
            "tokens_per_chunk": tpc, "chunks": nch,
            "quantize_ms_per_tensor": round(tqc, 5), "quantize_GBps": rc[0], "quantize_frac_hbm": rc[1],
            "quantize_1pass_ms_per_tensor": round(tqc1, 5), "quantize_1pass_GBps": rc1[0],
            "quantize_1pass_frac_hbm": rc1[1],
            "dequantize_ms_per_tensor": round(tdqc, 5), "dequantize_GBps": rdc[0], "dequantize_frac_hbm": rdc[1],
            "note": "one global scale per 8-frame chunk of the 21-frame tensor, K and V and all their chunks "
                    "in one call (amax partials per tensor and chunk, then the quantizer; quantize_1pass: the "
                    "chunks' maxima handed in, as each chunk's projection reports them); time per tensor is "
                    "half the call"},
        "context_device_copy": {"ms": round(tcp, 5), "GBps": round(2 * n * 2 / (tcp * 1e-3) / 1e9, 1),
                                "frac_hbm": round(2 * n * 2 / (tcp * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                "note": "torch copy of one bf16 tensor of the same size (read + write): the "
                                        "rate a plain read-and-write stream reaches here, context only"},
        "algorithmic_bytes_per_tensor": {"quantize": bytes_q, "dequantize": bytes_dq},
        "note": "GB/s = algorithmic bytes / event time per call, three rotating 113.5 MB tensors; quantize = amax "
                "pass inside the call (two reads of the tensor), quantize_1pass = amax supplied by the producing "
                "GEMM's epilogue (one read)",
        "window": win,
    }


def bench_kv_window(nv, iters):
    """Consumer side at the pages' inference configuration: 8-frame chunks of
    880 tokens x 24 heads x 128, keys smoothed and quantized per chunk; the
    attention window of the chunk at frame 64 (global sink frames 0-7, shot
    sink frames 16-23, the 32 frames before) rebuilt in one launch each for K
    and V."""
    import torch
    chunk_frames, frame_rows, d = 8, 880 * 24, 128
    rows = chunk_frames * frame_rows
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    kc, vc = [], []
    wsz = nv.lib.nvfp4_kv_smooth_workspace_size(rows, d)
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    kraw = []
    for c in range(8):
        k = (torch.randn((rows, d), generator=g, device="cuda") + 2.0).to(torch.bfloat16)
        v = torch.randn((rows, d), generator=g, device="cuda").to(torch.bfloat16)
        kc.append(nv.kv_quantize_smoothed(k, workspace=ws))
        vc.append(nv.kv_quantize(v, "4over6"))
        kraw.append(k)
    torch.cuda.synchronize()

    # the eight raw key chunks in turn (346 MB: no call finds its chunk in the
    # 256 MB last-level cache)
    def smooth(i):
        c = i % 8
        nv.kv_quantize_smoothed(kraw[c], out=kc[c][0], means=kc[c][1], workspace=ws)

    t_smooth = time_events(smooth, iters)
    runs = nv.kv_window_plan(64, chunk_frames, 32, 8, 16, 8)
    kparts = [(kc[c][0], kc[c][1], f0 * frame_rows, n * frame_rows) for c, f0, n in runs]
    vparts = [(vc[c], None, f0 * frame_rows, n * frame_rows) for c, f0, n in runs]
    del kraw
    wrows = sum(p[3] for p in kparts)
    kout = torch.empty((wrows, d), dtype=torch.bfloat16, device="cuda")
    vout = torch.empty((wrows, d), dtype=torch.bfloat16, device="cuda")

    def window(i):
        nv.kv_dequantize_window(kparts, out=kout)
        nv.kv_dequantize_window(vparts, out=vout)

    t_win = time_events(window, iters)
    n = wrows * d
    bytes_win = 2 * (n * 9 / 16 + n * 2) + wrows * 4          # K and V: packed in, bf16 out; K means
    bytes_smooth = rows * d * (2 + 9 / 16) + rows * 4          # keys read once, packed out, means
    gbps = bytes_win / (t_win * 1e-3) / 1e9
    gbs = bytes_smooth / (t_smooth * 1e-3) / 1e9
    return {"workload": f"window of the chunk at frame 64: {len(runs)} chunks x {rows} rows x {d}, K and V",
            "frames": wrows // frame_rows, "window_ms_k_and_v": round(t_win, 5), "window_GBps": round(gbps, 1),
            "window_frac_hbm": round(gbps / HBM_PEAK_GBPS, 4), "smoothed_k_quantize_ms_per_chunk": round(t_smooth, 5),
            "smoothed_k_quantize_GBps": round(gbs, 1),
            "note": "window GB/s = (packed K and V + K means read, bf16 K and V written) / time of the two launches "
                    "(518 MB of bf16 output per call between reuses of the packed chunks); smoothed quantize: "
                    "algorithmic bytes (keys read once, packed keys and means written), eight rotating chunks; the "
                    "call reads the keys twice (means and amax, then quantize)"}


def bench_extra(nv, workloads, iters):
    """FFN pair and long-sequence training shapes (fused act-quantize + GEMM)."""
    import torch
    out = {}
    for name, (m, k, n) in {"ffn_up_m2640_k3072_n14336": (2640, 3072, 14336),
                            "ffn_down_m2640_k14336_n3072": (2640, 14336, 3072),
                            "train_fwd_m32768_k3072_n3072": (32768, 3072, 3072)}.items():
        sets = linear_sets(nv, workloads, m, k, n, 2, 30)
        ms, _ = bench_linear(nv, sets, iters, 3)
        gms = bench_gemm_kernel(nv, sets, iters)
        tf, gtf = 2 * m * n * k / (ms * 1e-3) / 1e12, 2 * m * n * k / (gms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1), "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
                     "gemm_kernel_ms": round(gms, 4), "gemm_kernel_TFLOPs": round(gtf, 1),
                     "gemm_kernel_frac": round(gtf / FP16_MFMA_PEAK_TFLOPS, 4)}
        del sets
        torch.cuda.empty_cache()
    # the QKV projection with the rank-128 BF16 LoRA branch (alpha 128)
    m, k, n, r = 2640, 3072, 9216, 128
    sets = linear_sets(nv, workloads, m, k, n, 2, 40)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    la = (torch.randn((r, k), generator=g, device="cuda") / k ** 0.5).to(torch.bfloat16)
    lb = (torch.randn((n, r), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    u = torch.empty((m, r), dtype=torch.bfloat16, device="cuda")
    lws = torch.empty(nv.lib.nvfp4_linear_lora_workspace_size(m, k, r), dtype=torch.uint8, device="cuda")

    def lora_step(i):
        x_, w_, y_, ws_ = sets[i % len(sets)]
        nv.linear_lora(x_, w_, la, lb, 1.0, torch.bfloat16, out=y_, workspace=lws, u=u)

    ms = time_events(lora_step, iters)
    tf = 2 * m * (n * k + k * r + n * r) / (ms * 1e-3) / 1e12
    out["qkv_lora_r128_m2640_k3072_n9216"] = {
        "ms": round(ms, 4), "TFLOPs": round(tf, 1), "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
        "note": "flops of the NVFP4 product plus both LoRA products"}
    del sets
    torch.cuda.empty_cache()
    # weight gradient dW = dY^T X over 32768 tokens
    t, n, k = 32768, 3072, 3072
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = torch.randn((t, k), generator=g, device="cuda").to(torch.bfloat16)
    dy = (torch.randn((t, n), generator=g, device="cuda") * 1e-3).to(torch.bfloat16)
    dw = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    ws = nv.wgrad_workspace(t, n, k)

    def wg(i):
        nv.wgrad(dy, x, torch.bfloat16, out=dw, workspace=ws)

    def entry(ms, note=None):
        tf = 2 * t * n * k / (ms * 1e-3) / 1e12
        e = {"ms": round(ms, 4), "TFLOPs": round(tf, 1), "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}
        if note:
            e["note"] = note
        return e

    ms = time_events(wg, iters)
    out["train_wgrad_t32768_n3072_k3072"] = entry(ms, "amax of dY and X computed inside the call")
    # the forward already has max |X| (and the producing GEMM of dY its max):
    # handed in, the two amax passes drop out
    x_am = x.float().abs().max().reshape(1)
    dy_am = dy.float().abs().max().reshape(1)

    def wga(i):
        nv.wgrad(dy, x, torch.bfloat16, out=dw, workspace=ws, dy_amax=dy_am, x_amax=x_am)

    ms = time_events(wga, iters)
    out["train_wgrad_amax_in_t32768_n3072_k3072"] = entry(
        ms, "amax of dY and X handed in (the forward's / the producing GEMM's epilogue max), no amax pass")
    # the GEMM alone on the two COL16-packed operands
    pa = nv.quantize(dy, "col16", "4over6")
    pb = nv.quantize(x, "col16", "4over6")

    def wgk(i):
        nv.gemm(pa, pb, torch.bfloat16, out=dw)

    ms = time_events(wgk, iters)
    out["train_wgrad_gemm_kernel"] = entry(ms, "the dW GEMM alone on pre-packed operands")
    del pa, pb
    # the same with the random Hadamard transform on both operands
    def wgr(i):
        nv.wgrad(dy, x, torch.bfloat16, out=dw, workspace=ws, rht_signs=0xC39A)

    ms = time_events(wgr, iters)
    out["train_wgrad_rht_t32768_n3072_k3072"] = entry(ms)
    # data gradient dX = dY W: dY quantized along the 3072 output features, the
    # forward's TILE16 weight transposed once in packed form (not timed)
    w = nv.quantize((torch.randn((n, k), generator=g, device="cuda") * 0.02).to(torch.bfloat16), "tile16", "4over6")
    wt = nv.transpose_tile16(w)
    dx = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
    lws = nv.linear_workspace(t, n)

    def dg(i):
        nv.dgrad(dy, wt, torch.bfloat16, out=dx, workspace=lws)

    ms = time_events(dg, iters)
    out["train_dgrad_t32768_n3072_k3072"] = entry(ms)
    del x, dy, dw, ws, w, wt, dx, lws
    torch.cuda.empty_cache()
    # context: the vendor library's dense fp16 / bf16 GEMM (torch.matmul,
    # hipBLASLt) on the QKV shape, with 16-bit operands and no quantization
    m, k, n = 2640, 3072, 9216
    for dt, tag in ((torch.float16, "fp16"), (torch.bfloat16, "bf16")):
        pairs = [(torch.randn((m, k), generator=g, device="cuda").to(dt),
                  torch.randn((n, k), generator=g, device="cuda").to(dt)) for _ in range(3)]
        c = torch.empty((m, n), dtype=dt, device="cuda")

        def mm(i):
            a_, b_ = pairs[i % 3]
            torch.matmul(a_, b_.t(), out=c)

        ms = time_events(mm, iters)
        out[f"context_vendor_{tag}_gemm_m2640_k3072_n9216"] = {
            "ms": round(ms, 4), "TFLOPs": round(2 * m * n * k / (ms * 1e-3) / 1e12, 1),
            "note": "torch.matmul (hipBLASLt), dense 16-bit operands: context, not this library"}
        del pairs, c
    return out


def gpu_outputs_for_parity(nv, workloads):
    """The library's results on the first timed QKV input set (seed 2, full
    size), copied to the host: the quantized activation and weight, and the
    fused linear's fp32 and bf16 outputs."""
    import numpy as np
    import torch
    c = workloads.config2()
    x = dev_bf16(c["x"])
    w = nv.quantize(dev_bf16(c["w"]), "tile16", "4over6")
    a = nv.quantize(x, "row16", "4over6")
    y32 = nv.linear(x, w, torch.float32)
    y16 = nv.linear(x, w, torch.bfloat16)
    torch.cuda.synchronize()

    def packed(t):
        return (t.codes.cpu().numpy(), t.scales.cpu().numpy(), np.float32(t.alpha.cpu().numpy()[0]))

    out = {"a": packed(a), "w": packed(w), "y32": y32.cpu().numpy(),
           "y16": y16.cpu().view(torch.int16).numpy().view(np.uint16)}
    del x, w, a, y32, y16
    torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(workloads, m, k, n, gpu=None):
    """The oracle (fp32 quantizer, fp64 GEMM, OpenMP) on the full QKV step,
    repeated until about 10 s of host time have passed (at most 8 steps).
    With `gpu` (gpu_outputs_for_parity on the same seeded inputs) the oracle's
    results also check the library's at full size: codes, scale bytes and
    alpha bit for bit, the fp32 output within relative Frobenius 1e-5, and the
    bf16 output equal to the round-to-nearest-even of the fp32 one."""
    import numpy as np
    import oracle
    c = workloads.config2()
    W = oracle.quantize(c["w"], oracle.TILE16, oracle.FOUR_OVER_SIX)     # offline, untimed
    steps = 0
    t0 = time.perf_counter()
    while steps < 8 and (steps == 0 or time.perf_counter() - t0 < 10.0):
        A = oracle.quantize(c["x"], oracle.ROW16, oracle.FOUR_OVER_SIX)
        C = oracle.gemm_f64(A, W)
        steps += 1
    dt = (time.perf_counter() - t0) / steps
    out = {"value": round(2 * m * n * k / dt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle", "seconds_per_step": round(dt, 3), "steps": steps, "cpu_model": cpu_model(),
           "sample": f"{steps} full QKV steps: amax + four-over-six quantize of X [2640,3072] (fp32 steps) and "
                     "the fp64 GEMM against W [9216,3072] (W quantized once, untimed)"}
    # the KV round trip on a bounded sample of the KV workload: K of the first
    # 6 of 24 heads, [6 * 18480, 128], quantized (amax inside) and dequantized
    kv = workloads.config4()["k"][:6].reshape(-1, 128)
    t0 = time.perf_counter()
    R = oracle.quantize(kv, oracle.ROW16, oracle.FOUR_OVER_SIX)
    tq = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.dequantize(R)
    tdq = time.perf_counter() - t0
    nel = kv.size
    out["kv_round_trip"] = {
        "sample": "K of heads 0-5 of the KV workload, [110880, 128] bf16 (a quarter of one tensor)",
        "quantize_s": round(tq, 3), "quantize_GBps": round(nel * (2 + 9 / 16) / tq / 1e9, 3),
        "dequantize_s": round(tdq, 3), "dequantize_GBps_fp32_out": round(nel * (9 / 16 + 4) / tdq / 1e9, 3),
        "note": "algorithmic bytes per second (bf16 in / packed out; packed in / fp32 out), all host cores"}
    if gpu is None:
        return out, None

    def same(p, ref):
        codes, scales, alpha = p
        return bool(np.array_equal(codes, ref.codes) and np.array_equal(scales, ref.scales)
                    and alpha.view(np.uint32) == np.float32(ref.alpha).view(np.uint32))

    err = float(np.linalg.norm(gpu["y32"].astype(np.float64) - C) / np.linalg.norm(C))
    parity = {"workload": "QKV input set 0 (seed 2), full size, against the CPU oracle",
              "activation_codes_scales_alpha_bit_exact": same(gpu["a"], A),
              "weight_codes_scales_alpha_bit_exact": same(gpu["w"], W),
              "linear_fp32_rel_frobenius": err, "rel_frobenius_bound": 1e-5,
              "linear_bf16_equals_rne_of_fp32": bool(np.array_equal(gpu["y16"], oracle.bf16_rne(gpu["y32"])))}
    parity["pass"] = (parity["activation_codes_scales_alpha_bit_exact"] and
                      parity["weight_codes_scales_alpha_bit_exact"] and err <= 1e-5 and
                      parity["linear_bf16_equals_rne_of_fp32"])
    return out, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--parts", default="qkv,kv,extra,cpu",
                    help="comma list of qkv (the step), kv, extra, cpu")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-kv", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    parts = set(args.parts.split(","))
    if args.no_cpu:
        parts.discard("cpu")
    if args.no_extra:
        parts.discard("extra")
    if args.no_kv:
        parts.discard("kv")
    if args.copy_calibration:
        import torch
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the NVFP4 path here is built and timed on a single MI355X "
              "(multi-GPU sharding is a design note, not a measured run)", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_w4a4_quantized_04_amd as nv
    import workloads

    assert torch.cuda.is_available()
    m, k, n = 2640, 3072, 9216
    flops = 2.0 * m * n * k
    result = {
        "metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "nvfp4 operands, f16 mfma (exact), f32 accumulate, bf16 out",
        "data": "synthetic (seeded normals shaped like a 5B video DiT's QKV projection)",
        "config": {"workload": "qkv_projection_x2640x3072_w9216x3072_bf16out",
                   "m": m, "k": k, "n": n, "rule": "four-over-six", "weight_blocks": "16x16",
                   "act_blocks": "1x16", "input_sets": 4, "seeds": [2, 102, 202, 302],
                   "rotation_MB": None},
    }
    if "qkv" in parts:
        log("[bench] preparing QKV projection inputs")
        sets = linear_sets(nv, workloads, m, k, n, 4, 2)
        log("[bench] timing the fused linear")
        ms, dist = bench_linear(nv, sets, args.steps, args.warmup)
        value = flops / (ms * 1e-3) / 1e12
        log(f"[bench] linear {ms:.4f} ms/step, {value:.1f} TFLOP/s")
        result["step_ms_events"] = dist
        result["config"]["rotation_MB"] = round(sum(
            t.numel() * t.element_size() for st in sets for t in (st[0], st[1].codes, st[1].scales, st[2], st[3]))
            / 1e6, 1)

        def step(i):
            x, w, y, ws = sets[i % len(sets)]
            nv.linear(x, w, torch.bfloat16, out=y, workspace=ws)

        log("[bench] clock levels and power under load (untimed)")
        result["gpu_state"] = gpu_state_under_load(step)
        log("[bench] timing the GEMM kernel alone")
        gms = bench_gemm_kernel(nv, sets, max(50, args.steps // 2))
        achieved = flops / (gms * 1e-3) / 1e12
        result["value"] = round(value, 2)
        result["ms_per_step"] = round(ms, 5)
        result["roofline"] = {
            "bound": "mfma", "achieved": round(achieved, 1), "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": gemm_traffic(),
            "kernel": "k_gemm_nvfp4", "kernel_ms": round(gms, 5), "algorithmic_flops_per_launch": flops,
            "frac_of_fp4_mfma_peak": round(achieved / FP4_MFMA_PEAK_TFLOPS, 4)}
        # context: the same peak scaled to the shader clock read under load
        # (the published peak assumes 2.4 GHz)
        mhz = sclk_mhz(result.get("gpu_state"))
        if mhz:
            peak_clk = FP16_MFMA_PEAK_TFLOPS * mhz / PEAK_SCLK_MHZ
            result["roofline"]["sclk_mhz_under_load"] = mhz
            result["roofline"]["peak_at_that_sclk"] = round(peak_clk, 1)
            result["roofline"]["frac_at_that_sclk"] = round(achieved / peak_clk, 4)
        del sets
        torch.cuda.empty_cache()
    if "kv" in parts:
        log("[bench] KV cache quantize/dequantize")
        result["kv"] = bench_kv(nv, workloads, 30)
        torch.cuda.empty_cache()
    if "extra" in parts:
        log("[bench] FFN and training shapes")
        result["extra"] = bench_extra(nv, workloads, 20)
        torch.cuda.empty_cache()
    if "cpu" in parts:
        log("[bench] CPU oracle baseline (and full-size parity of the first QKV set)")
        gpu = gpu_outputs_for_parity(nv, workloads)
        result["cpu_baseline"], result["parity"] = cpu_baseline(workloads, m, k, n, gpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
