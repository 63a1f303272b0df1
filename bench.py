#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one gdn_prefill_fwd on the 32K-token workload (B=1, T=32768, H=32,
d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 gates, state and y) with every input
and its record workspace already resident in HBM; the single-kernel form
(no workspace) is timed the same way as `prefill_32k_fused`.  The JSON line carries that step's roofline (its
algorithmic flops and bytes over the median step time, against the bf16 MFMA
and HBM peaks), the 4K-context prefill (B=2, T=4096, H=16) measured the same
way, the decode step (256 sequences x 32 heads, fp32 128x128 states updated in
place), decode verify, the full layer (B=1, T=16384, hidden 2048, H=16) and
its decode step, the backward of the 32K prefill, and the fp64 oracle timed on
the host cores on a bounded sample of the same workload.

Timing: HIP events recorded on torch's current stream, which is the stream the
library launches on, around every timed step; a 512 MiB buffer is written
before each timed step (outside the events) so that no step finds its inputs
in the 256 MB Infinity Cache; the reported time is the median over the timed
steps.  The region of all timed steps is bracketed by device synchronisations.
`ms_back_to_back` is a second region of as many steps run back to back with
no flush in between (inputs may then sit in the Infinity Cache).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s at T=32K (MFMA % peak); decode state GB/s (HBM % peak)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def prefill_alg(B, T, H, Dk, Dv, C, has_s0=False):
    """Algorithmic bytes and flops of one prefill (what the method must move and
    compute, whatever the kernel).  Bytes per token-head: bf16 q, k, v, y and
    fp32 alpha, beta = 2 (2 Dk + 2 Dv) + 8 (1032 at d = 128); plus the final
    state written (and the initial state read, if given).  The outputs y here
    are fp32, so the bytes with y at 4 bytes are returned too.  Flops per
    token-head, triangle-exact: (3C - 1) Dk + 2 C Dv + 6 Dk Dv + C^2 / 3; with
    full C x C tiles: 2 C (3 Dk + 2 Dv) + 6 Dk Dv + C^2 / 3.
    Returns (bytes, bytes with fp32 y, F_alg, F_tile)."""
    tok = B * T * H
    st = B * H * Dk * Dv * 4 * (2 if has_s0 else 1)
    b_bf16_y = tok * (2 * (2 * Dk + 2 * Dv) + 8) + st
    b_fp32_y = tok * (2 * (2 * Dk + Dv) + 4 * Dv + 8) + st
    f_alg = (3 * C - 1) * Dk + 2 * C * Dv + 6 * Dk * Dv + C * C / 3.0
    f_tile = 2 * C * (3 * Dk + 2 * Dv) + 6 * Dk * Dv + C * C / 3.0
    return b_bf16_y, b_fp32_y, tok * f_alg, tok * f_tile


def decode_alg(N, H, Dk, Dv, in_bytes=2):
    """State read + written once, q/k/v/alpha/beta read, y (fp32) written."""
    per = 8 * Dk * Dv + (2 * Dk + Dv) * in_bytes + 8 + 4 * Dv
    return N * H * per, N * H * 8 * Dk * Dv


def verify_alg(N, T, H, Dk, Dv, in_bytes=2):
    """States read once, the T snapshots written once, q/k/v/alpha/beta read and
    y (fp32) written once per token."""
    return N * H * Dk * Dv * 4 * (1 + T) + N * T * H * ((2 * Dk + Dv) * in_bytes + 8 + 4 * Dv)


def layer_decode_alg(N, hidden, H, Dk, Dv, conv_k):
    """One layer-decode step: the four weight matrices (bf16) and x read once,
    the conv history (fp32) and the states read and written once, out (fp32)
    written once; gate and norm vectors are negligible."""
    nqkv = H * (2 * Dk + Dv)
    weights = 2 * hidden * (nqkv + H * Dv + 2 * H) + 2 * H * Dv * hidden
    return (weights + N * hidden * 2 + 2 * N * (conv_k - 1) * nqkv * 4 + 2 * N * H * Dk * Dv * 4
            + N * hidden * 4)


def bwd_flops(B, T, H, Dk, Dv, C):
    """Flops of the chunked reverse mode, per (sequence, head, chunk) summed
    over its four kernels: the Gram blocks and inverse of the preparation, the
    two state passes (K S, the triangular C x C products, the state updates)
    and the chunk gradients (K S, Q S, K dS', three triangular products, dP and
    dA, the three C x Dk outer-product sums over Dv, and the four C x C by C x
    Dk products of dQ and dK).  Triangular products count the 16 x 16 blocks
    on and below the diagonal."""
    nb = C // 16
    tri = nb * (nb + 1) // 2 * 256            # entries of the lower blocks
    prep = 2 * tri * Dk + C ** 3 / 6.0
    fwd = 2 * C * Dk * Dv + tri * Dv
    adj = 3 * C * Dk * Dv + 2 * tri * Dv
    chunk = 6 * C * Dk * Dv + 5 * tri * Dv + 4 * tri * Dk
    return 2.0 * B * H * (-(-T // C)) * (prep + fwd + adj + chunk)


def bwd_kernel_alg(B, T, H, Dk, Dv, C, in_bytes=2):
    """Algorithmic HBM bytes of each backward kernel: its inputs read once and
    its outputs written once, the workspace included (per-chunk records: T, P,
    Gamma o K K^T and the decay prefix; the state entering and the state
    gradient leaving every chunk; the chunk's U, V - e^G K S and dX)."""
    nc = -(-T // C)
    tok, ch = B * T * H, B * H * nc
    qk, v = tok * Dk * in_bytes, tok * Dv * in_bytes
    f32v = tok * Dv * 4
    cc = ch * C * C * 4
    g = ch * C * 4
    st = ch * Dk * Dv * 4
    cv = ch * C * Dv * 4
    return {
        "prep": 2 * qk + 8 * tok + ch * 4 * ((3 * C * C + C + 63) // 64 * 64),
        "state": qk + v + cc + g + 4 * tok + st + 2 * cv,
        "adjoint": 2 * qk + f32v + 2 * cc + g + 4 * tok + st + cv + f32v,
        "chunk": 2 * qk + f32v + 2 * st + 3 * cv + 2 * cc + g + 8 * tok + 2 * tok * Dk * 4 + 8 * tok,
    }


def layer_flops(B, T, hidden, H, Dk, Dv, C):
    M = B * T
    gemm = 2 * M * hidden * (H * (2 * Dk + Dv) + 2 * H + H * Dv) + 2 * M * (H * Dv) * hidden
    core = B * T * H * ((3 * C - 1) * Dk + 2 * C * Dv + 6 * Dk * Dv + C * C / 3.0)
    return gemm, core


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ["linear_attention_token_gated_amd/csrc/recurrence.hip",
                   "linear_attention_token_gated_amd/csrc/chunk_prep.hip",
                   "linear_attention_token_gated_amd/csrc/prep_layout.hpp",
                   "linear_attention_token_gated_amd/csrc/common.hpp"]
FUSED_SOURCES = ["linear_attention_token_gated_amd/csrc/prefill_fused.hip",
                 "linear_attention_token_gated_amd/csrc/common.hpp"]


DECODE_SOURCES = ["linear_attention_token_gated_amd/csrc/decode.hip"]


# counter keys: the kernels whose FETCH_SIZE + WRITE_SIZE add up to one launch
# of the workload, and the sources whose hash the stored counts were taken on
TRAFFIC_KERNELS = {
    "prefill_32k": (["gdn_chunk_prep_kernel", "gdn_recurrence_kernel"], PREFILL_SOURCES),
    "prefill_32k_fused": (["gdn_prefill_fused_kernel"], FUSED_SOURCES),
    "decode_256x32": (["gdn_decode_kernel"], DECODE_SOURCES),
}


def measured_traffic(key="prefill_32k", sources=None):
    """HBM bytes of one launch of a workload from the committed rocprofv3
    counter runs (FETCH_SIZE + WRITE_SIZE, each scaled by its reading for a
    copy of known size), if they were taken on the current kernel source;
    else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            t = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha") != source_sha(sources or TRAFFIC_KERNELS[key][1]):
        return None
    return t.get("hbm_bytes_per_launch")


class Flush:
    """A 512 MiB device buffer written before every timed step: twice the
    256 MB Infinity Cache, so no step finds its inputs left in it by the
    previous one."""

    def __init__(self, torch, nbytes=512 << 20):
        self.buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.fill_(1.0)


def time_steps(fns, steps, warmup, torch, flush=None):
    """A step calls every function of `fns` in order on torch's current stream
    (the stream the library launches on).  `warmup` untimed steps, then
    `steps` timed ones, each preceded by `flush` (outside the timed events) and
    bracketed by HIP events, with an event between consecutive functions.
    Then `steps` more steps back to back, without the flush, between two
    events.  Each region is bracketed by device synchronisations.  Returns
    (per-step ms list, per-function ms lists, ms of the back-to-back region)."""
    if callable(fns):
        fns = [fns]
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for ev in evs:
        if flush is not None:
            flush()
        ev[0].record(stream)
        for i, fn in enumerate(fns):
            fn()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        for fn in fns:
            fn()
    t1.record(stream)
    torch.cuda.synchronize()
    per_step = [ev[0].elapsed_time(ev[-1]) for ev in evs]
    per_fn = [[ev[i].elapsed_time(ev[i + 1]) for ev in evs] for i in range(len(fns))]
    return per_step, per_fn, t0.elapsed_time(t1)


def median(x):
    return float(np.median(np.asarray(x, dtype=np.float64)))


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def prefill_setup(cfg, torch, gdn, wl, fused=False):
    """The prefill of a workload: with the record workspace (per-chunk
    preparation, then the recurrence), or with fused=True the single-kernel
    form that takes none."""
    inp = wl.prefill_config_inputs(cfg)
    t = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "alpha", "beta", "S0")}
    y = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    sT = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), dtype=torch.float32, device="cuda")
    ws = None if fused else torch.empty(max(1, gdn.prefill_workspace_bytes(
        cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk, cfg.dtype)), dtype=torch.uint8, device="cuda")
    fn = lambda: gdn.prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["S0"], chunk=cfg.chunk, y=y,
                             final_state=sT, workspace=ws, fused=fused)
    return inp, fn


def prefill_report(cfg, per_step, region_ms, steps, peak_tflops):
    ms = median(per_step)
    b8, b32, f_alg, f_tile = prefill_alg(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk,
                                         has_s0=cfg.s0_std is not None)
    t = ms * 1e-3
    return {"workload": cfg.name, "ms_per_step": round(ms, 4), "ms_mean": round(float(np.mean(per_step)), 4),
            "ms_min": round(float(np.min(per_step)), 4), "ms_back_to_back": round(region_ms / steps, 4),
            "tokens_per_s": cfg.B * cfg.T / t,
            "flops_alg": f_alg, "tflops_alg": f_alg / t / 1e12, "mfma_frac": f_alg / t / 1e12 / peak_tflops,
            "mfma_frac_tile": f_tile / t / 1e12 / peak_tflops,
            "alg_bytes": b8, "hbm_GBps": b8 / t / 1e9, "hbm_frac": b8 / t / 1e9 / HBM_PEAK_GBPS,
            "alg_bytes_fp32_y": b32, "hbm_frac_fp32_y": b32 / t / 1e9 / HBM_PEAK_GBPS}


def bench_simple(fn, args, torch, flush, steps=None, warmup=None):
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    per, _, region = time_steps(fn, steps, warmup, torch, flush)
    return median(per), region / steps, steps


def bench_decode(args, torch, gdn, wl, flush):
    cfg = wl.DECODE_256
    inp = wl.decode_config_inputs(cfg)
    q, k, v, al, be, S = (to_dev(inp[n], torch) for n in ("q", "k", "v", "alpha", "beta", "S"))
    y = torch.empty((cfg.N, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    fn = lambda: gdn.decode_step(q, k, v, al, be, S, y=y)   # in place: each step is a valid next step
    ms, hot, _ = bench_simple(fn, args, torch, flush)
    b, _ = decode_alg(cfg.N, cfg.H, cfg.Dk, cfg.Dv)
    state = 8 * cfg.N * cfg.H * cfg.Dk * cfg.Dv
    return {"workload": cfg.name, "ms_per_step": round(ms, 4), "ms_back_to_back": round(hot, 4),
            "GBps": b / (ms * 1e-3) / 1e9, "state_GBps": state / (ms * 1e-3) / 1e9,
            "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "alg_bytes_per_launch": b,
            "traffic": measured_traffic("decode_256x32", DECODE_SOURCES)}


def bench_layer(args, torch, gdn, wl, flush, peak):
    cfg = wl.LAYER_16K
    inp = wl.layer_config_inputs(cfg)
    names = ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate", "norm_gamma", "W_o")
    params = {n: to_dev(inp[n], torch) for n in names}
    x = to_dev(inp["x"], torch)
    out = torch.empty((cfg.B, cfg.T, cfg.hidden), dtype=torch.float32, device="cuda")
    sT = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.layer_workspace_bytes(cfg.B, cfg.T, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv, cfg.conv_k,
                                               cfg.chunk), dtype=torch.uint8, device="cuda")
    fn = lambda: gdn.layer_fwd(x, params, cfg.H, cfg.Dk, cfg.Dv, chunk=cfg.chunk, out=out, final_state=sT,
                               workspace=ws)
    ms, hot, steps = bench_simple(fn, args, torch, flush, max(1, min(args.steps, 10)), max(1, min(args.warmup, 2)))
    gemm_f, core_f = layer_flops(cfg.B, cfg.T, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk)
    t = ms * 1e-3
    return {"workload": cfg.name, "ms_per_step": round(ms, 4), "ms_back_to_back": round(hot, 4),
            "tokens_per_s": cfg.B * cfg.T / t, "gemm_tflops_alg": gemm_f / 1e12, "core_tflops_alg": core_f / 1e12,
            "tflops_achieved": (gemm_f + core_f) / t / 1e12,
            "mfma_frac": (gemm_f + core_f) / t / 1e12 / peak}


def bench_verify(args, torch, gdn, wl, flush):
    cfg = wl.VERIFY_256x4
    inp = wl.prefill_config_inputs(cfg)
    q, k, v, al, be, S = (to_dev(inp[n], torch) for n in ("q", "k", "v", "alpha", "beta", "S0"))
    y = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    so = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv), dtype=torch.float32, device="cuda")
    fn = lambda: gdn.decode_verify(q, k, v, al, be, S, states_out=so, y=y)
    ms, hot, _ = bench_simple(fn, args, torch, flush)
    b = verify_alg(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv)
    return {"workload": cfg.name, "ms_per_step": round(ms, 4), "alg_bytes_per_step": b,
            "GBps": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def bench_layer_decode(args, torch, gdn, wl, flush):
    cfg = wl.LAYER_DECODE_256
    inp, cs0, S0 = wl.layer_decode_config_inputs(cfg)
    names = ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate", "norm_gamma", "W_o")
    params = {n: to_dev(inp[n], torch) for n in names}
    x = to_dev(inp["x"], torch)[:, 0].contiguous()
    cs, S = to_dev(cs0, torch), to_dev(S0, torch)
    out = torch.empty((cfg.B, cfg.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.layer_decode_workspace_bytes(cfg.B, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv),
                     dtype=torch.uint8, device="cuda")
    # in place: each step is a valid next step of the same sequences
    fn = lambda: gdn.layer_decode_step(x, params, cfg.H, cfg.Dk, cfg.Dv, cs, S, out=out, workspace=ws)
    ms, hot, _ = bench_simple(fn, args, torch, flush)
    b = layer_decode_alg(cfg.B, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv, cfg.conv_k)
    return {"workload": cfg.name, "ms_per_step": round(ms, 4), "tokens_per_s": cfg.B / (ms * 1e-3),
            "alg_bytes_per_step": b, "GBps": b / (ms * 1e-3) / 1e9,
            "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def bench_bwd(args, torch, gdn, wl, flush, fwd_ms, peak):
    cfg = wl.PREFILL_32K
    inp = wl.bwd_config_inputs(cfg)
    t = {n: to_dev(inp[n], torch) for n in ("q", "k", "v", "alpha", "beta", "dy", "S0", "dST")}
    out = {n: torch.empty(shp, dtype=torch.float32, device="cuda") for n, shp in
           (("dq", (cfg.B, cfg.T, cfg.H, cfg.Dk)), ("dk", (cfg.B, cfg.T, cfg.H, cfg.Dk)),
            ("dv", (cfg.B, cfg.T, cfg.H, cfg.Dv)), ("dalpha", (cfg.B, cfg.T, cfg.H)),
            ("dbeta", (cfg.B, cfg.T, cfg.H)), ("dinitial_state", (cfg.B, cfg.H, cfg.Dk, cfg.Dv)))}
    ws = torch.empty(gdn.prefill_bwd_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: gdn.prefill_bwd(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["dy"], t["S0"], t["dST"],
                                 chunk=cfg.chunk, out=out, workspace=ws)
    ms, hot, steps = bench_simple(fn, args, torch, flush, max(1, min(args.steps, 10)), max(1, min(args.warmup, 2)))
    f = bwd_flops(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk)
    tf = f / (ms * 1e-3) / 1e12
    return {"workload": cfg.name + ", gradients of every input from dy and dS_T",
            "ms_per_call": round(ms, 4), "tokens_per_s": cfg.B * cfg.T / (ms * 1e-3),
            "bwd_over_fwd": ms / fwd_ms, "flops_alg_per_call": f, "tflops_achieved": tf,
            "peak_tflops": peak, "frac": tf / peak,
            "alg_bytes_per_kernel": bwd_kernel_alg(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk),
            "note": "bf16 inputs: every product of the four kernels runs on bf16 MFMA (fp32 operands as hi/lo "
                    "bf16 pairs), so frac is against the bf16 dense peak"}


def cpu_baseline(wl, sample_T):
    """The oracle, untouched, on the first sample_T tokens of every head of
    the 32K workload (all host threads), plus single-thread runs of the tiny
    workload and of a sample of the 4K workload."""
    import oracle

    def rate(cfg, T, nthreads):
        inp = wl.prefill_config_inputs(cfg)
        sl = slice(0, T)
        args = [wl.widen(inp[n][:, sl]) for n in ("q", "k", "v", "alpha", "beta")]
        s0 = wl.widen(inp["S0"])
        t0 = time.perf_counter()
        oracle.gdn_recurrence(*args, s0, nthreads=nthreads)
        dt = time.perf_counter() - t0
        return cfg.B * T / dt, dt, oracle.last_threads_used

    v, dt, cores = rate(wl.PREFILL_32K, sample_T, 0)
    tiny, _, _ = rate(wl.TINY, wl.TINY.T, 1)
    t4 = min(512, wl.PREFILL_4K.T)
    one4k, dt4, _ = rate(wl.PREFILL_4K, t4, 1)
    return {"value": v, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 sequential recurrence on the first {sample_T} tokens of all "
                      f"{wl.PREFILL_32K.B * wl.PREFILL_32K.H} (batch, head) sequences of the 32K workload "
                      f"({dt:.1f} s)",
            "one_thread": {"tiny_tokens_per_s": tiny,
                           "4k_tokens_per_s": one4k,
                           "4k_sample": f"first {t4} tokens of all {wl.PREFILL_4K.B * wl.PREFILL_4K.H} sequences "
                                        f"({dt4:.1f} s)"}}


def device_info(torch):
    """Name, CU count, the peak engine clock HIP reports and, where readable,
    the current engine clock level from sysfs."""
    import ctypes
    import glob
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "peak_clock_mhz": None, "sclk_now_mhz": None}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, torch.cuda.current_device()) == 0:  # ClockRate, kHz
            info["peak_clock_mhz"] = v.value / 1000.0
    except OSError:
        pass
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if line.strip().endswith("*"):
                    info["sclk_now_mhz"] = float(line.split(":")[1].strip().rstrip("*").strip().lower()
                                                 .replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            continue
        if info["sclk_now_mhz"] is not None:
            break
    return info


def pmc_summarize(fetch_csv, write_csv):
    """Turn two rocprofv3 counter runs of `bench.py --pmc-run` (FETCH_SIZE,
    then WRITE_SIZE, csv counter collections) into profiles/traffic.json: per
    workload kernel, HBM bytes per launch, each counter scaled by its reading
    for the 1 GiB copy of known size that --pmc-run ends with."""
    import csv

    def load(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name", counter) != counter:
                continue
            name = r["Kernel_Name"]
            val = float(r["Counter_Value"])
            rows.setdefault(name, []).append(val)
        return rows

    fr, wr = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = [n for n in fr if "copyBuffer" in n]
    assert copy, "no calibration copy in the counter run"
    gib = float(1 << 30)
    f_fac = max(fr[copy[0]]) * 1024 / gib
    w_fac = max(wr[copy[0]]) * 1024 / gib
    out = {"calibration": {"kernel": copy[0] + " (torch copy_ of 1 GiB fp32)", "bytes_read": 1 << 30,
                           "bytes_written": 1 << 30, "fetch_factor": f_fac, "write_factor": w_fac}}
    for key, (needles, sources) in TRAFFIC_KERNELS.items():
        names = [next((n for n in fr if nd in n), None) for nd in needles]
        if None in names:
            continue
        # the largest dispatch of each kernel is the workload's (smaller ones are other shapes)
        fk = sum(max(fr[n]) for n in names)
        wk = sum(max(wr.get(n, [0.0])) for n in names)
        rd, wb = fk * 1024 / f_fac, wk * 1024 / w_fac
        out[key] = {"kernels": names, "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk, "hbm_read_bytes": rd,
                    "hbm_write_bytes": wb, "hbm_bytes_per_launch": rd + wb, "source_sha": source_sha(sources)}
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(out, f, indent=1)
    for key, t in out.items():
        if key != "calibration":
            print(f"| {key} | {t['FETCH_SIZE_KiB']:.0f} | {t['WRITE_SIZE_KiB']:.0f} | "
                  f"{t['hbm_read_bytes'] / 1e6:.1f} MB | {t['hbm_write_bytes'] / 1e6:.1f} MB | "
                  f"{t['hbm_bytes_per_launch'] / 1e6:.1f} MB |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768)
    ap.add_argument("--skip-layer", action="store_true")
    ap.add_argument("--only-prefill", action="store_true", help="the 32K and 4K prefill objects only")
    ap.add_argument("--pmc-run", action="store_true",
                    help="for hardware-counter passes: each workload twice and a 1 GiB device copy of known size "
                         "(the copy calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two --pmc-run counter collections")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
        return

    import torch
    import linear_attention_token_gated_amd as gdn
    from linear_attention_token_gated_amd import workloads as wl

    gdn.lib()
    dev = device_info(torch)
    clock = dev["peak_clock_mhz"] or 2400.0
    peak_from_clock = dev["cus"] * 4096 * clock * 1e6 / 1e12          # bf16 dense: 4096 flop/clk per CU

    if args.pmc_run:
        pargs = argparse.Namespace(steps=1, warmup=1)
        for cfg in (wl.PREFILL_32K, wl.PREFILL_4K):
            for fused in (False, True):
                _, fn = prefill_setup(cfg, torch, gdn, wl, fused)
                fn(); fn()
                del fn
                torch.cuda.synchronize()
        bench_decode(pargs, torch, gdn, wl, None)
        bench_layer(pargs, torch, gdn, wl, None, BF16_PEAK_TFLOPS)
        bench_layer_decode(pargs, torch, gdn, wl, None)
        bench_verify(pargs, torch, gdn, wl, None)
        bench_bwd(pargs, torch, gdn, wl, None, 1.0, BF16_PEAK_TFLOPS)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_run": "done", "copy_bytes_read": src.numel() * 4,
                          "copy_bytes_written": dst.numel() * 4}))
        return

    flush = Flush(torch)
    cfg = wl.PREFILL_32K
    inp, fn = prefill_setup(cfg, torch, gdn, wl)
    per, _, region = time_steps(fn, args.steps, args.warmup, torch, flush)
    head = prefill_report(cfg, per, region, args.steps, BF16_PEAK_TFLOPS)
    print(f"prefill 32K: {head['ms_per_step']} ms", file=sys.stderr, flush=True)
    _, fn4 = prefill_setup(wl.PREFILL_4K, torch, gdn, wl)
    per4, _, region4 = time_steps(fn4, args.steps, args.warmup, torch, flush)
    p4k = prefill_report(wl.PREFILL_4K, per4, region4, args.steps, BF16_PEAK_TFLOPS)
    del fn4
    _, fnf = prefill_setup(cfg, torch, gdn, wl, fused=True)
    perf, _, regionf = time_steps(fnf, args.steps, args.warmup, torch, flush)
    pfused = prefill_report(cfg, perf, regionf, args.steps, BF16_PEAK_TFLOPS)
    pfused["form"] = "one fused kernel, no workspace (q, k, v read once)"
    pfused["traffic"] = measured_traffic("prefill_32k_fused")
    del fnf
    print(f"prefill 32K fused: {pfused['ms_per_step']} ms", file=sys.stderr, flush=True)
    traffic = measured_traffic("prefill_32k")
    head["form"] = "per-chunk records (preparation kernel), then the recurrence"
    ms_step = head["ms_per_step"]

    extra = {}
    if not args.only_prefill:
        extra["decode"] = bench_decode(args, torch, gdn, wl, flush)
        print(f"decode: {extra['decode']['ms_per_step']} ms", file=sys.stderr, flush=True)
        extra["layer"] = None if args.skip_layer else bench_layer(args, torch, gdn, wl, flush, BF16_PEAK_TFLOPS)
        extra["layer_decode"] = bench_layer_decode(args, torch, gdn, wl, flush)
        extra["verify"] = bench_verify(args, torch, gdn, wl, flush)
        extra["bwd"] = bench_bwd(args, torch, gdn, wl, flush, ms_step, BF16_PEAK_TFLOPS)
        print(f"bwd: {extra['bwd']['ms_per_call']} ms", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, min(args.cpu_sample_tokens, cfg.T))

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "Dk": cfg.Dk, "Dv": cfg.Dv,
                   "chunk": cfg.chunk, "qkv": "bf16", "alpha_beta_state_y": "fp32", "initial_state": "none"},
        "roofline": {"bound": "mfma", "achieved": head["tflops_alg"], "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": head["mfma_frac"], "traffic": traffic,
                     "scope": "whole prefill step (every kernel gdn_prefill_fwd launches)",
                     "flops_alg_per_step": head["flops_alg"],
                     "frac_full_tile_flops": head["mfma_frac_tile"],
                     "peak_from_clock_tflops": peak_from_clock,
                     "alg_bytes_per_step": head["alg_bytes"],
                     "traffic_over_alg_bytes": (traffic / head["alg_bytes"]) if traffic else None,
                     "hbm": {"achieved_GBps": head["hbm_GBps"], "peak": HBM_PEAK_GBPS,
                             "frac": head["hbm_frac"], "frac_with_fp32_y": head["hbm_frac_fp32_y"]}},
        "prefill_32k": head,
        "prefill_4k": p4k,
        "prefill_32k_fused": pfused,
        **extra,
        "cpu_baseline": cpu,
        "device": dev,
        "timing": {"protocol": "HIP events on the launch stream around each step; a 512 MiB buffer written "
                               "before every timed step (outside the events); median over the timed steps",
                   "mall_flush_bytes": 512 << 20},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
