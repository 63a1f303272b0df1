#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunked prefill on the 32K-token workload (B=1, T=32768,
H=32, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 gates, state and y) with every
input already resident in HBM: gdn_prefill_prepare (the per-chunk
preparation kernel) then gdn_prefill_recurrence (the state recurrence
kernel), which together are exactly gdn_prefill_fwd.  The line printed also
carries the decode step (256 sequences x 32 heads, fp32 128x128 states
updated in place), the full layer (B=1, T=16384, hidden 2048, H=16) and the
backward of the 32K prefill (every input gradient from dy and dS_T)
measured the same way, the roofline of the recurrence kernel (the larger part
of the step) with the preparation kernel beside it, and the fp64 oracle timed
on the host cores on a bounded sample of the same workload.

Timing: HIP events recorded on the stream the kernels are launched on
(torch's current stream), around every launch of the timed region (each of
the two prefill kernels has its own pair); the region itself is bracketed by
device synchronisations.
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


def prefill_alg(B, T, H, Dk, Dv, C, in_bytes=2, has_s0=False):
    """Algorithmic bytes and flops of one prefill call (what the method must
    move and compute, independent of the kernel): q, k, v read once, alpha and
    beta read once, y (fp32) written once, final state written once."""
    tok = B * T * H
    bytes_ = tok * ((2 * Dk + Dv) * in_bytes + 8 + 4 * Dv) + B * H * Dk * Dv * 4 * (2 if has_s0 else 1)
    f_alg = (3 * C - 1) * Dk + 2 * C * Dv + 6 * Dk * Dv + C * C / 3.0     # per token-head
    return bytes_, tok * f_alg


def record_bytes(C):
    """Bytes of one per-chunk record of the preparation kernel: T' and P as
    bf16 hi/lo 16x16 blocks (C/16 (C/16 + 1) / 2 of each, 1 KB per block),
    then the decay vectors (2C + 16 floats)."""
    nb = C // 16
    return 2 * (nb * (nb + 1) // 2) * 1024 + (2 * C + 16) * 4


def prep_alg(B, T, H, Dk, C, in_bytes=2):
    """Preparation kernel: q, k, alpha, beta read once, one record written per
    (sequence, head, chunk)."""
    return B * T * H * (2 * Dk * in_bytes + 8) + B * H * (-(-T // C)) * record_bytes(C)


def recurrence_alg(B, T, H, Dk, Dv, C, in_bytes=2, has_s0=False):
    """Recurrence kernel: q, k, v and the records read once, y (fp32) and the
    final state written once."""
    tok = B * T * H
    return (tok * ((2 * Dk + Dv) * in_bytes + 4 * Dv) + B * H * (-(-T // C)) * record_bytes(C)
            + B * H * Dk * Dv * 4 * (2 if has_s0 else 1))


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


DECODE_SOURCES = ["linear_attention_token_gated_amd/csrc/decode.hip"]


def measured_traffic(key="prefill_32k", sources=PREFILL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, each scaled by its reading for a copy of known
    size), if they were taken on the current kernel source; else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            t = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha") != source_sha(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def time_launches(fns, steps, warmup, torch):
    """A step calls every function of `fns` in order.  Run `warmup` steps,
    then `steps` steps with a HIP event pair around each call on the current
    stream.  Returns (total ms of the bracketed region, per function a list of
    per-call ms)."""
    if callable(fns):
        fns = [fns]
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for step in ev:
        for fn, (a, b) in zip(fns, step):
            a.record(stream)
            fn()
            b.record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    per = [[step[i][0].elapsed_time(step[i][1]) for step in ev] for i in range(len(fns))]
    return t_all0.elapsed_time(t_all1), (per[0] if len(fns) == 1 else per)


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bench_prefill(args, torch, gdn, wl):
    cfg = wl.PREFILL_32K
    inp = wl.prefill_config_inputs(cfg)
    q, k, v = (to_dev(inp[n], torch) for n in ("q", "k", "v"))
    al, be = to_dev(inp["alpha"], torch), to_dev(inp["beta"], torch)
    y = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    sT = torch.empty((cfg.B, cfg.H, cfg.Dk, cfg.Dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk, "bf16"),
                     dtype=torch.uint8, device="cuda")
    prep = lambda: gdn.prefill_prepare(q, k, al, be, ws, chunk=cfg.chunk)
    rec = lambda: gdn.prefill_recurrence(q, k, v, ws, None, chunk=cfg.chunk, y=y, final_state=sT)
    total_ms, (per_prep, per_rec) = time_launches([prep, rec], args.steps, args.warmup, torch)
    return cfg, inp, total_ms, per_prep, per_rec


def bench_decode(args, torch, gdn, wl):
    cfg = wl.DECODE_256
    inp = wl.decode_config_inputs(cfg)
    q, k, v = (to_dev(inp[n], torch) for n in ("q", "k", "v"))
    al, be, S = (to_dev(inp[n], torch) for n in ("alpha", "beta", "S"))
    y = torch.empty((cfg.N, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    fn = lambda: gdn.decode_step(q, k, v, al, be, S, y=y)   # in place: each step is a valid next step
    total_ms, per = time_launches(fn, args.steps, args.warmup, torch)
    return cfg, total_ms, per


def bench_layer(args, torch, gdn, wl):
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
    steps = max(1, min(args.steps, 10))
    total_ms, per = time_launches(fn, steps, max(1, min(args.warmup, 2)), torch)
    return cfg, total_ms, per, steps


def bench_verify(args, torch, gdn, wl):
    cfg = wl.VERIFY_256x4
    inp = wl.prefill_config_inputs(cfg)
    q, k, v, al, be, S = (to_dev(inp[n], torch) for n in ("q", "k", "v", "alpha", "beta", "S0"))
    y = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    so = torch.empty((cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv), dtype=torch.float32, device="cuda")
    fn = lambda: gdn.decode_verify(q, k, v, al, be, S, states_out=so, y=y)
    total_ms, per = time_launches(fn, args.steps, args.warmup, torch)
    return cfg, total_ms, per


def bench_layer_decode(args, torch, gdn, wl):
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
    total_ms, per = time_launches(fn, args.steps, args.warmup, torch)
    return cfg, total_ms, per


def bench_bwd(args, torch, gdn, wl):
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
    steps = max(1, min(args.steps, 10))
    total_ms, per = time_launches(fn, steps, max(1, min(args.warmup, 2)), torch)
    return cfg, total_ms, per, steps


def cpu_baseline(inp, cfg, wl, sample_T):
    """The oracle, untouched, on the first sample_T tokens of every head."""
    import oracle
    sl = slice(0, sample_T)
    args = [wl.widen(inp[n][:, sl]) for n in ("q", "k", "v", "alpha", "beta")]
    t0 = time.perf_counter()
    oracle.gdn_recurrence(*args, None)
    dt = time.perf_counter() - t0
    return {"value": cfg.B * sample_T / dt, "unit": "tokens/s", "cores": oracle.last_threads_used,
            "kind": "oracle",
            "sample": f"fp64 sequential recurrence on the first {sample_T} tokens of all {cfg.B * cfg.H} "
                      f"(batch, head) sequences of the 32K workload ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768)
    ap.add_argument("--skip-layer", action="store_true")
    ap.add_argument("--pmc-run", action="store_true",
                    help="for hardware-counter passes: two prefill launches, two decode steps, two layer "
                         "calls and a 1 GiB device copy of known size (the copy calibrates FETCH_SIZE / "
                         "WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import linear_attention_token_gated_amd as gdn
    from linear_attention_token_gated_amd import workloads as wl

    gdn.lib()
    props = torch.cuda.get_device_properties(0)

    if args.pmc_run:
        pargs = argparse.Namespace(steps=1, warmup=1)
        bench_prefill(pargs, torch, gdn, wl)
        bench_decode(pargs, torch, gdn, wl)
        bench_layer(pargs, torch, gdn, wl)
        bench_layer_decode(pargs, torch, gdn, wl)
        bench_verify(pargs, torch, gdn, wl)
        bench_bwd(pargs, torch, gdn, wl)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_run": "done", "copy_bytes_read": src.numel() * 4,
                          "copy_bytes_written": dst.numel() * 4}))
        return

    cfg, inp, p_total, p_prep, p_rec = bench_prefill(args, torch, gdn, wl)
    alg_bytes, alg_flops = prefill_alg(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk)
    ms_step = p_total / args.steps
    ms_prep, ms_rec = float(np.mean(p_prep)), float(np.mean(p_rec))
    tok_s = cfg.B * cfg.T / (ms_step * 1e-3)
    rec_bytes = recurrence_alg(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk)
    prep_bytes = prep_alg(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.chunk)
    achieved_gbps = rec_bytes / (ms_rec * 1e-3) / 1e9
    traffic = measured_traffic("prefill_32k_recurrence")

    d_cfg, d_total, d_per = bench_decode(args, torch, gdn, wl)
    d_bytes, _ = decode_alg(d_cfg.N, d_cfg.H, d_cfg.Dk, d_cfg.Dv)
    d_state = 8 * d_cfg.N * d_cfg.H * d_cfg.Dk * d_cfg.Dv
    d_ms = float(np.mean(d_per))

    layer = None
    if not args.skip_layer:
        l_cfg, l_total, l_per, l_steps = bench_layer(args, torch, gdn, wl)
        gemm_f, core_f = layer_flops(l_cfg.B, l_cfg.T, l_cfg.hidden, l_cfg.H, l_cfg.Dk, l_cfg.Dv, l_cfg.chunk)
        l_ms = l_total / l_steps
        layer = {"workload": l_cfg.name, "ms_per_step": round(l_ms, 4),
                 "tokens_per_s": l_cfg.B * l_cfg.T / (l_ms * 1e-3),
                 "gemm_tflops_alg": gemm_f / 1e12, "core_tflops_alg": core_f / 1e12,
                 "tflops_achieved": (gemm_f + core_f) / (l_ms * 1e-3) / 1e12,
                 "note": "core runs on fp32 q/k/v (two kernels, bf16 MFMA with hi/lo operands); projections on hipBLASLt, bf16 operands, fp32 accumulation"}

    ld_cfg, ld_total, ld_per = bench_layer_decode(args, torch, gdn, wl)
    ld_ms = float(np.mean(ld_per))
    ld_bytes = layer_decode_alg(ld_cfg.B, ld_cfg.hidden, ld_cfg.H, ld_cfg.Dk, ld_cfg.Dv, ld_cfg.conv_k)
    layer_decode = {"workload": ld_cfg.name, "ms_per_step": round(ld_ms, 4),
                    "tokens_per_s": ld_cfg.B / (ld_ms * 1e-3), "alg_bytes_per_step": ld_bytes,
                    "GBps": ld_bytes / (ld_ms * 1e-3) / 1e9,
                    "hbm_frac": ld_bytes / (ld_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    v_cfg, v_total, v_per = bench_verify(args, torch, gdn, wl)
    v_ms = float(np.mean(v_per))
    v_bytes = verify_alg(v_cfg.B, v_cfg.T, v_cfg.H, v_cfg.Dk, v_cfg.Dv)
    verify = {"workload": v_cfg.name, "ms_per_step": round(v_ms, 4), "alg_bytes_per_step": v_bytes,
              "GBps": v_bytes / (v_ms * 1e-3) / 1e9, "hbm_frac": v_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    b_cfg, b_total, b_per, b_steps = bench_bwd(args, torch, gdn, wl)
    b_ms = float(np.mean(b_per))
    b_flops = bwd_flops(b_cfg.B, b_cfg.T, b_cfg.H, b_cfg.Dk, b_cfg.Dv, b_cfg.chunk)
    bwd = {"workload": b_cfg.name + ", gradients of every input from dy and dS_T",
           "ms_per_call": round(b_ms, 4), "tokens_per_s": b_cfg.B * b_cfg.T / (b_ms * 1e-3),
           "bwd_over_fwd": b_ms / ms_step, "flops_alg_per_call": b_flops,
           "tflops_achieved": b_flops / (b_ms * 1e-3) / 1e12, "peak_tflops": FP32_PEAK_TFLOPS,
           "frac": b_flops / (b_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS,
           "alg_bytes_per_kernel": bwd_kernel_alg(b_cfg.B, b_cfg.T, b_cfg.H, b_cfg.Dk, b_cfg.Dv, b_cfg.chunk),
           "note": "four kernels: preparation (Gram on bf16 MFMA), state pass and adjoint state pass (bf16 MFMA, "
                   "hi/lo operands), chunk gradients (fp32 MFMA); frac is against the fp32 MFMA peak"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, cfg, wl, min(args.cpu_sample_tokens, cfg.T))

    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "Dk": cfg.Dk, "Dv": cfg.Dv,
                   "chunk": cfg.chunk, "qkv": "bf16", "alpha_beta_state_y": "fp32",
                   "initial_state": "none"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "kernel": "gdn_recurrence_kernel<C=64, Dk=128>",
                     "ms_per_launch": round(ms_rec, 4),
                     "alg_bytes_per_launch": rec_bytes},
        "prep_kernel": {"kernel": "gdn_chunk_prep_kernel<C=64, Dk=128>", "ms_per_launch": round(ms_prep, 4),
                        "alg_bytes_per_launch": prep_bytes,
                        "achieved_GBps": prep_bytes / (ms_prep * 1e-3) / 1e9,
                        "hbm_frac": prep_bytes / (ms_prep * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                        "traffic": measured_traffic("prefill_32k_prep")},
        "step_hbm": {"alg_bytes_per_step": alg_bytes, "achieved_GBps": alg_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "mfma": {"flops_alg_per_step": alg_flops,
                 "tflops_achieved": alg_flops / (ms_step * 1e-3) / 1e12,
                 "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": alg_flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "decode": {"workload": d_cfg.name, "ms_per_step": round(d_ms, 4),
                   "GBps": d_bytes / (d_ms * 1e-3) / 1e9,
                   "state_GBps": d_state / (d_ms * 1e-3) / 1e9,
                   "hbm_frac": d_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                   "alg_bytes_per_launch": d_bytes,
                   "traffic": measured_traffic("decode_256x32", DECODE_SOURCES)},
        "layer": layer,
        "layer_decode": layer_decode,
        "verify": verify,
        "bwd": bwd,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
