#!/usr/bin/env python3
"""Benchmark of the Mesa-layer forward (and decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

One step is one ``mesa_forward`` call (chunk states, every CG iteration and
the output contraction) over the layer-sized workload: B=8, H=16, T=4096,
d=128, chunk 64, bf16 q/k/v, fp32 arithmetic, fixed 30 CG iterations, seeded
synthetic inputs already resident in device memory.  Prints ONE JSON line.

Besides the headline it measures, in the same run and reported in the same
line: the dynamic-stopping forward (4x16x8192, fp32, tol 1e-4, cap 30) and
1024 recurrent decode steps over 256 x 16 heads (d=128, states from
4096-token prefixes).  Per-kernel average durations come from HIP events
recorded by the library around each launch on the stream it runs on.
The CPU baseline is the fp64 oracle timed on a bounded sample of the same
headline workload on this host's cores.
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

PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_BF16_MFMA_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cg_h2_layer_bf16_d128_T4096_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "cg_h2_layer_bf16_d128_T4096_mfma.json")
KERNEL_SOURCES = ["test_regression_amd/csrc/cg_output.hip", "test_regression_amd/csrc/cg_output_bf16.hip",
                  "test_regression_amd/csrc/cg_output_kernels.h", "test_regression_amd/csrc/cg_h2.h",
                  "test_regression_amd/csrc/cg_core.h", "test_regression_amd/csrc/persistent.h",
                  "test_regression_amd/csrc/mesa_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_per_token_head(d, C, k):
    """Algorithmic flops of one forward token-head: chunk states, k CG matvecs
    (state term 2d^2, causal intra-chunk term 2(C+1)d, vector work 11d) and the
    output contraction."""
    states = 4 * d * d
    cg = k * (2 * d * d + 2 * (C + 1) * d + 11 * d)
    output = 2 * d * d + 2 * (C + 1) * d
    return states, cg, output


def h2_cg_mfma_flops(d, C, key_planes, wave_iters):
    """MFMA flops one launch of the forward CG kernel (d >= 32) issues, from
    its structure.  Wave w of a chunk owns tokens 16w..16w+15 and runs as many
    matvecs as the largest iteration count among them (`wave_iters`: a
    [n_chunks, C/16] integer array; k everywhere for a fixed count).  A matvec
    of wave w issues 16x16x32 fp16 MFMAs: three per 32-feature step and
    16-row block for the state term (hi.hi, hi.lo, lo.hi of the two-part
    splits), and (1 + key planes) per causal key block and feature step for
    the scores and per row block and 32-key step for the apply (keys stored
    as bf16 are one exact fp16 plane, fp32 keys two).  At d = 128, 64-token
    chunks and bf16 keys, waves 2 and 3 start from the mid-chunk state, so
    their causal key blocks start at block 2; that state is formed once per
    chunk, shared out among three waves (four MFMAs per 32-feature step and
    row block).  Per chunk the
    output adds the scores and apply of the solution over the keys from the
    chunk start, and the G_c term: three fp16 MFMAs per feature step and row
    block when a wave splits at most two of G_c's row blocks (64-token
    chunks at d = 128), else 16x16x4 fp32 MFMAs.  Returns (fp16 flops, fp32
    flops)."""
    import numpy as np
    NT, NQ, NW = d // 16, d // 32, C // 16
    np_ = 1 + key_planes
    mid = d == 128 and C == 64 and key_planes == 1
    gl = (NT + NW - 1) // NW <= 2
    per_iter = np.zeros(NW, np.int64)
    out16 = 4 * NQ * NT if mid else 0
    for w in range(NW):
        kb0 = 2 if mid and w >= 2 else 0
        nb = w + 1 - kb0
        per_iter[w] = 3 * NT * NQ + np_ * NQ * nb + np_ * NT * ((nb + 1) // 2)
        out16 += np_ * NQ * (w + 1) + np_ * NT * ((w + 2) // 2)
        if gl:
            out16 += 3 * NQ * NT
    wave_iters = np.asarray(wave_iters, np.int64)
    n_chunks = wave_iters.shape[0]
    f16 = 2 * 16 * 16 * 32 * (int((wave_iters * per_iter[None, :]).sum()) + n_chunks * out16)
    fp32 = 0 if gl else 2 * 16 * 16 * 4 * (NW * NT * NT * 4) * n_chunks
    return f16, fp32


def h2_adjoint_mfma_flops(d, C, key_planes, k, n_chunks):
    """MFMA flops one launch of the adjoint kernel (d >= 32) issues at a fixed
    iteration count k: k CG matvecs and H x, each as a matvec of the forward
    CG kernel (h2_cg_mfma_flops); the right side G^T g with the (S^G)^T term
    and the value scores on 16x16x4 fp32 MFMAs, and its apply through K^T on
    (1 + key planes) fp16 products per row block and 32-key step.
    Returns (fp16 flops, fp32 flops)."""
    NT, NQ, NW = d // 16, d // 32, C // 16
    np_ = 1 + key_planes
    per_iter, rhs16, rhs32 = 0, 0, 0
    for w in range(NW):
        nbo, ns = w + 1, (w + 2) // 2
        per_iter += 3 * NT * NQ + np_ * NQ * nbo + np_ * NT * ns
        rhs16 += np_ * NT * ns
        rhs32 += 4 * NT * NT + 4 * NT * nbo
    f16 = 2 * 16 * 16 * 32 * ((k + 1) * per_iter + rhs16) * n_chunks
    fp32 = 2 * 16 * 16 * 4 * rhs32 * n_chunks
    return f16, fp32


def mixed_roofline(bf16_flops, fp32_flops, ms, alg_flops, bf16_peak, fp32_peak):
    """Roofline of a kernel whose MFMA work is split between bf16 and fp32
    instructions: the shortest time is bf16/peak_bf16 + fp32/peak_fp32, the
    effective peak is the issued flops over that time, and the fraction is
    that time over the measured one."""
    t_min = bf16_flops / (bf16_peak * 1e12) + fp32_flops / (fp32_peak * 1e12)
    issued = bf16_flops + fp32_flops
    t = ms * 1e-3
    return dict(achieved=round(issued / t / 1e12, 2), peak=round(issued / t_min / 1e12, 1),
                frac=round(t_min / t, 4), issued_flops_per_launch=issued,
                issued_bf16_flops=bf16_flops, issued_fp32_flops=fp32_flops,
                algorithmic_tflops=round(alg_flops / t / 1e12, 2))


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_counters(path):
    """A committed rocprofv3 summary of the CG/output kernel, only if it was
    taken on the current kernel source."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


def measured_traffic():
    """HBM bytes per launch of the CG/output kernel (FETCH_SIZE + WRITE_SIZE)."""
    t = committed_counters(TRAFFIC_FILE)
    return t.get("bytes_per_launch") if t else None


def measured_mfma_busy():
    """Fraction of SIMD cycles the MFMA unit was busy during the CG/output kernel."""
    t = committed_counters(MFMA_FILE)
    return t.get("mfma_busy_frac") if t else None


def to_dev(torch, x, dtype, dev):
    import numpy as np
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def timed_forward(torch, mesa, t, w, steps, warmup):
    """Warmup, then `steps` timed calls bracketed by device synchronisation."""
    B, H, T, d = t["q"].shape
    out = torch.empty((B, H, T, d), dtype=torch.float32, device=t["q"].device)
    iters = torch.empty((B, H, T), dtype=torch.int32, device=t["q"].device)
    ws = torch.empty(mesa.mesa_forward_workspace_bytes(B, H, T, d, d, w.chunk), dtype=torch.uint8,
                     device=t["q"].device)

    def step():
        mesa.mesa_forward(t["q"], t["k"], t["v"], t["gamma"], t["lam"], w.max_iters, w.tol, w.chunk,
                          out=out, iters=iters, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mesa.profile_reset()
    mesa.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mesa.profile_enable(False)
    k1 = mesa.profile_read(mesa.KERNEL_CHUNK_STATES)
    k2 = mesa.profile_read(mesa.KERNEL_CG_OUTPUT)
    mesa.profile_reset()
    return (t1 - t0), k1, k2, out, iters


def headline(torch, mesa, inputs, args, dev, peaks):
    w = inputs.WORKLOADS["layer_bf16_d128_T4096_k30"]
    log(f"[bench] generating {w.name}")
    x = inputs.forward_inputs(w)
    t = {n: to_dev(torch, x[n], w.dtype if n in ("q", "k", "v") else "f32", dev) for n in x}
    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    el, k1, k2, _, _ = timed_forward(torch, mesa, t, w, args.steps, args.warmup)
    n_tok = w.B * w.H * w.T
    fs, fcg, fo = flops_per_token_head(w.d, w.chunk, w.max_iters)
    ms_step = 1e3 * el / args.steps
    k2_ms = k2[0] / max(k2[1], 1)
    k1_ms = k1[0] / max(k1[1], 1)
    k2_flops = (fcg + fo) * n_tok
    # chunk-state kernel: reads k, v (bf16) and gamma once; writes each chunk's
    # S^H (packed upper 16x16-block triangle, d(d+16)/2 floats) and S^G (d*d)
    k1_bytes = n_tok * (2 * w.d * 2 + 4) + w.B * w.H * (w.T // w.chunk) * (w.d * (w.d + 16) // 2 + w.d * w.d) * 4
    achieved = k2_flops / (k2_ms * 1e-3) / 1e12
    traffic = measured_traffic()
    # The CG kernel's products run on fp16 MFMAs over two-part splits: its
    # roofline is the algorithmic flops at the fp16 (= bf16) MFMA peak; the
    # issued work (three products per state product) is reported beside it.
    import numpy as np
    n_chunks = w.B * w.H * (w.T // w.chunk)
    bf, fp = h2_cg_mfma_flops(w.d, w.chunk, 1, np.full((n_chunks, w.chunk // 16), w.max_iters))
    rl = mixed_roofline(bf, fp, k2_ms, k2_flops, PEAK_BF16_MFMA_TFLOPS, PEAK_FP32_MFMA_TFLOPS)
    rlm = mixed_roofline(bf, fp, k2_ms, k2_flops, peaks["mfma_bf16_tflops"], peaks["mfma_f32_tflops"])
    res = dict(
        w=w, x=x, n_tok=n_tok, ms_step=ms_step, value=n_tok * args.steps / el,
        tflops=(fs + fcg + fo) * n_tok / (ms_step * 1e-3) / 1e12,
        # The kernel's contractions issue on fp16 MFMAs (2500 TFLOP/s, the
        # bf16 figure), so its roofline is the method's algorithmic flops
        # against that peak; the split products multiply the issued work,
        # which is reported as a secondary fraction against its own bound.
        roofline=dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s",
                      frac=round(achieved / PEAK_BF16_MFMA_TFLOPS, 4), traffic=traffic,
                      kernel="cg_h2_kernel<128,64,bf16> (fp16 MFMA on two-part splits)",
                      basis="algorithmic flops of the CG iterations and the output contraction "
                            f"({fcg + fo} per token-head) per launch / average launch time / the fp16 "
                            "(= bf16) MFMA peak the kernel's products issue at",
                      algorithmic_flops_per_launch=k2_flops, avg_launch_ms=round(k2_ms, 4),
                      frac_measured_peak=round(achieved / peaks["mfma_bf16_tflops"], 4),
                      algorithmic_over_fp32_peak=round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
                      mfma_busy_frac=measured_mfma_busy(),
                      issued=dict(achieved=rl["achieved"], peak=rl["peak"], frac=rl["frac"],
                                  flops_per_launch=rl["issued_flops_per_launch"], fp16_flops=bf, fp32_flops=fp,
                                  basis="issued MFMA work (split products) over its shortest time at the "
                                        "fp16 and fp32 MFMA peaks",
                                  peak_measured=rlm["peak"], frac_measured=rlm["frac"])),
        kernels={
            "cg_h2_kernel": dict(avg_ms=round(k2_ms, 4), launches=k2[1],
                                    algorithmic_tflops=round(achieved, 2)),
            "chunk_states_kernel": dict(avg_ms=round(k1_ms, 4), launches=k1[1],
                                        gbs=round(k1_bytes / (k1_ms * 1e-3) / 1e9, 1),
                                        hbm_frac=round(k1_bytes / (k1_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)),
        })
    del t
    return res


def backward(torch, mesa, h, dev, peaks, steps=5, warmup=2):
    """Training step of the layer on the headline workload: mesa_forward_train
    then mesa_backward with a seeded dL/d(out), timed separately."""
    w, x = h["w"], h["x"]
    t = {n: to_dev(torch, x[n], w.dtype if n in ("q", "k", "v") else "f32", dev) for n in x}
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 9)
    gout = torch.randn((w.B, w.H, w.T, w.d), generator=g, device=dev)
    n_tok = w.B * w.H * w.T
    fws = torch.empty(mesa.mesa_forward_workspace_bytes(w.B, w.H, w.T, w.d, w.d, w.chunk), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(mesa.mesa_backward_workspace_bytes(w.B, w.H, w.T, w.d, w.d, w.chunk), dtype=torch.uint8,
                      device=dev)

    def fwd():
        return mesa.mesa_forward_train(t["q"], t["k"], t["v"], t["gamma"], t["lam"], w.max_iters, w.tol, w.chunk,
                                       workspace=fws)

    def bwd(out, xs):
        return mesa.mesa_backward(t["k"], t["v"], t["gamma"], t["lam"], xs, out, gout, w.max_iters, w.tol,
                                  w.chunk, workspace=bws)
    log(f"[bench] backward: {steps} training steps after {warmup} warmup")
    for _ in range(warmup):
        out, _, xs = fwd()
        bwd(out, xs)
    torch.cuda.synchronize()
    ids = {"chunk_states_kernel": mesa.KERNEL_CHUNK_STATES, "bwd_adjoint_kernel": mesa.KERNEL_BWD_ADJOINT,
           "bwd_states_kernel": mesa.KERNEL_BWD_STATES, "bwd_kv_kernel": mesa.KERNEL_BWD_KV,
           "bwd_gate_kernel": mesa.KERNEL_BWD_GATE}
    f_el = b_el = 0.0
    kt = {n: [0.0, 0] for n in ids}
    for _ in range(steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out, _, xs = fwd()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        mesa.profile_reset()
        mesa.profile_enable(True)
        bwd(out, xs)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        mesa.profile_enable(False)
        for n, i in ids.items():
            ms, c = mesa.profile_read(i)
            kt[n][0] += ms
            kt[n][1] += c
        mesa.profile_reset()
        f_el += t1 - t0
        b_el += t2 - t1
    d, C, k = w.d, w.chunk, w.max_iters
    # adjoint kernel per token-head: G^T g and H x (each 2d^2 + 2(C+1)d), the k-step CG
    adj_flops = n_tok * (k * (2 * d * d + 2 * (C + 1) * d + 11 * d) + 2 * (2 * d * d + 2 * (C + 1) * d))
    adj_ms = kt["bwd_adjoint_kernel"][0] / max(kt["bwd_adjoint_kernel"][1], 1)
    achieved = adj_flops / (adj_ms * 1e-3) / 1e12
    bf, fp = h2_adjoint_mfma_flops(d, C, 1 if w.dtype == "bf16" else 2, k, w.B * w.H * (w.T // C))
    rl = mixed_roofline(bf, fp, adj_ms, adj_flops, PEAK_BF16_MFMA_TFLOPS, PEAK_FP32_MFMA_TFLOPS)
    rlm = mixed_roofline(bf, fp, adj_ms, adj_flops, peaks["mfma_bf16_tflops"], peaks["mfma_f32_tflops"])
    kernels = {n: {"avg_ms": round(v[0] / max(v[1], 1), 4), "launches": v[1]} for n, v in kt.items()}
    del t, gout, fws, bws
    return {"workload": w.name, "grad_out": "N(0,1), seeded",
            "forward_train_ms": round(1e3 * f_el / steps, 4), "backward_ms": round(1e3 * b_el / steps, 4),
            "train_step_tokens_per_s": round(n_tok * steps / (f_el + b_el), 1),
            "kernels": kernels,
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_MFMA_TFLOPS, 4),
                         "kernel": "bwd_adjoint_h2_kernel<128,64,bf16> (fp16 MFMA on two-part splits)",
                         "basis": "algorithmic flops per launch / average launch time / the fp16 (= bf16) MFMA "
                                  "peak",
                         "algorithmic_flops_per_launch": adj_flops, "avg_launch_ms": round(adj_ms, 4),
                         "algorithmic_over_fp32_peak": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
                         "issued": {"achieved": rl["achieved"], "peak": rl["peak"], "frac": rl["frac"],
                                    "fp16_flops": bf, "fp32_flops": fp,
                                    "basis": "issued MFMA work: fp16 split products at 2500 TFLOP/s, the "
                                             "right side's fp32 products at 157.3",
                                    "peak_measured": rlm["peak"], "frac_measured": rlm["frac"]}}}


def dynamic(torch, mesa, inputs, dev):
    w = inputs.WORKLOADS["dynamic_f32_d128_T8192_tol1e-4"]
    log(f"[bench] generating {w.name}")
    x = inputs.forward_inputs(w)
    t = {n: to_dev(torch, x[n], "f32", dev) for n in x}
    del x
    steps = 5
    el, k1, k2, _, iters = timed_forward(torch, mesa, t, w, steps, 2)
    n_tok = w.B * w.H * w.T
    it = iters.to(torch.float64)
    mean_it = float(it.mean())
    fs, _, fo = flops_per_token_head(w.d, w.chunk, 0)
    per_it = 2 * w.d * w.d + 2 * (w.chunk + 1) * w.d + 11 * w.d
    useful = n_tok * (fs + fo) + float(it.sum()) * per_it
    k2_useful = n_tok * fo + float(it.sum()) * per_it
    ms = 1e3 * el / steps
    k2_ms = k2[0] / max(k2[1], 1)
    k1_ms = k1[0] / max(k1[1], 1)
    wave_iters = iters.view(-1, w.chunk // 16, 16).amax(dim=-1).cpu().numpy()
    f16, f32 = h2_cg_mfma_flops(w.d, w.chunk, 2, wave_iters)
    issued = f16 + f32
    t_min = f16 / (PEAK_BF16_MFMA_TFLOPS * 1e12) + f32 / (PEAK_FP32_MFMA_TFLOPS * 1e12)
    hist = torch.bincount(iters.flatten().to(torch.int64), minlength=w.max_iters + 1).cpu().tolist()
    ach = k2_useful / (k2_ms * 1e-3) / 1e12
    del t
    return {"workload": w.name, "tokens_per_s": round(n_tok / (ms * 1e-3), 1), "ms_per_call": round(ms, 3),
            "iters_mean": round(mean_it, 3), "iters_min": int(iters.min()), "iters_max": int(iters.max()),
            "iters_histogram": {str(i): c for i, c in enumerate(hist) if c},
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2),
            "kernels": {"cg_h2_kernel": {"avg_ms": round(k2_ms, 4), "launches": k2[1]},
                        "chunk_states_kernel": {"avg_ms": round(k1_ms, 4), "launches": k1[1]}},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_MFMA_TFLOPS, 4),
                         "kernel": "cg_h2_kernel<128,64,float> (fp16 MFMA on two-part splits of the fp32 "
                                   "keys, state and vectors)",
                         "basis": "useful flops (each token's own iteration count) per launch / average "
                                  "launch time / the fp16 MFMA peak",
                         "useful_flops_per_launch": k2_useful,
                         "useful_over_fp32_peak": round(ach / PEAK_FP32_MFMA_TFLOPS, 4),
                         "issued_flops_per_launch": issued, "issued_fp16_flops": f16, "issued_fp32_flops": f32,
                         "issued_over_useful": round(issued / k2_useful, 4),
                         "issued_frac": round(t_min / (k2_ms * 1e-3), 4),
                         "avg_launch_ms": round(k2_ms, 4)}}


def small_workload(torch, mesa, inputs, dev, name, steps=20, warmup=3):
    """A launch-latency-sized forward workload, timed like the headline."""
    w = inputs.WORKLOADS[name]
    x = inputs.forward_inputs(w)
    t = {n: to_dev(torch, x[n], w.dtype if n in ("q", "k", "v") else "f32", dev) for n in x}
    el, k1, k2, _, _ = timed_forward(torch, mesa, t, w, steps, warmup)
    n_tok = w.B * w.H * w.T
    fs, fcg, fo = flops_per_token_head(w.d, w.chunk, w.max_iters)
    ms = 1e3 * el / steps
    return {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "qkv_storage": w.dtype,
            "cg_iters": w.max_iters, "tokens_per_s": round(n_tok / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
            "algorithmic_tflops": round((fs + fcg + fo) * n_tok / (ms * 1e-3) / 1e12, 3),
            "kernels": {"chunk_states_kernel_ms": round(k1[0] / max(k1[1], 1), 4),
                        "cg_kernel_ms": round(k2[0] / max(k2[1], 1), 4)},
            "note": "launch-latency-sized: reported, not graded on a roofline"}


def decode(torch, mesa, inputs, dev, steps=1024, warmup=8, warm_start=True):
    """1024 decode steps over 256 x 16 heads; states built on the device from
    seeded 4096-token prefixes by the forward path with zero CG iterations.
    The cold-start run is the measured line; the same steps are then run
    again from the same states with the warm-started solve, on these i.i.d.
    queries and on queries that overlap their neighbours (each the sum of 4
    consecutive Gaussian rows, as a short causal convolution would mix them)."""
    w = inputs.WORKLOADS["decode_f32_d128_N256_prefix4096"]
    N, H, d, P = w.B, w.H, w.d, w.T
    gen = inputs.DecodeDeviceStream(torch, w, dev)
    log(f"[bench] decode: building {N}x{H} prefix states of {P} tokens")
    SH0 = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    SG0 = torch.empty_like(SH0)
    lam = torch.from_numpy(inputs.decode_lambda(w)).to(dev)
    for n0, pk, pv, pg in gen.prefix_batches(64):   # 64 sequences at a time: 2 GiB prefix buffers
        nb = pk.shape[0]
        mesa.mesa_forward(pk, pk, pv, pg, lam, 0, 0.0, w.chunk, return_iters=False,
                          final_H=SH0[n0:n0 + nb], final_G=SG0[n0:n0 + nb], return_final=True)
        del pk, pv, pg
    S = steps + warmup
    q, k, v, ga = gen.steps(S)
    out = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    its = torch.empty((S, N, H), dtype=torch.int32, device=dev)

    def run(qs, mode):
        """All S steps from the prefix states; mode None = mesa_decode_step, else the warm entry."""
        SH, SG = SH0.clone(), SG0.clone()
        SX = torch.zeros((N, H, d), dtype=torch.float32, device=dev)

        def step(s):
            if mode is None:
                mesa.mesa_decode_step(qs[s], k[s], v[s], ga[s], lam, SH, SG, w.max_iters, w.tol,
                                      out=out, iters=its[s])
            else:
                mesa.mesa_decode_step_warm(qs[s], k[s], v[s], ga[s], lam, SH, SG, SX, w.max_iters, w.tol,
                                           mode, out=out, iters=its[s])
        for s in range(warmup):
            step(s)
        torch.cuda.synchronize()
        mesa.profile_reset()
        mesa.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(warmup, S):
            step(s)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        mesa.profile_enable(False)
        kd = mesa.profile_read(mesa.KERNEL_DECODE)
        mesa.profile_reset()
        del SH, SG, SX
        return el, kd[0] / max(kd[1], 1), its[warmup:].to(torch.float64)

    el, kd_ms, itf = run(q, None)
    nh = N * H
    # per head-step: read + write H and G (fp32 d x d each), q, k, v, gamma, out, iters
    bytes_hs = 4 * 4 * d * d + 3 * 4 * d + 4 + 4 * d + 4
    gbs = bytes_hs * nh / (kd_ms * 1e-3) / 1e9
    hist = torch.bincount(itf.flatten().to(torch.int64), minlength=w.max_iters + 1).cpu().tolist()
    res = {"workload": w.name, "head_steps_per_s": round(steps * nh / el, 1),
           "ms_per_step": round(1e3 * el / steps, 4),
           "iters_mean": round(float(itf.mean()), 3), "iters_max": int(itf.max()),
           "iters_histogram": {str(i): c for i, c in enumerate(hist) if c},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "decode_kernel<128,float>",
                        "bytes_per_launch": bytes_hs * nh, "avg_launch_ms": round(kd_ms, 4)}}
    q4 = gen.windowed_queries(S, 4)
    warm = {}
    for qname, qs in ((("iid", q), ("window4", q4)) if warm_start else ()):
        warm[qname] = {}
        for mname, mode in (("cold", None), ("previous", mesa.MESA_WARM_PREVIOUS),
                            ("projected", mesa.MESA_WARM_PROJECTED)):
            if qname == "iid" and mode is None:
                el_m, itf_m = el, itf
            else:
                log(f"[bench] decode warm start: queries {qname}, start {mname}")
                el_m, _, itf_m = run(qs, mode)
            warm[qname][mname] = {"iters_mean": round(float(itf_m.mean()), 3),
                                  "ms_per_step": round(1e3 * el_m / steps, 4),
                                  "head_steps_per_s": round(steps * nh / el_m, 1)}
    if warm_start:
        res["warm_start"] = warm
    del q, q4, k, v, ga
    return res


def qk_preprocess(torch, mesa, inputs, dev, steps=20, warmup=3, W=4):
    """The q/k pre-processing pass at the headline layer's shape: raw q and k
    (bf16, 8 x 16 x 4096, d=128) -> causal width-4 convolution + L2
    normalisation -> bf16, two launches per step.  HBM-bound."""
    w = inputs.WORKLOADS["layer_bf16_d128_T4096_k30"]
    B, H, T, d = w.B, w.H, w.T, w.d
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 77)
    xq = torch.randn((B, H, T, d), generator=g, device=dev).to(torch.bfloat16)
    xk = torch.randn((B, H, T, d), generator=g, device=dev).to(torch.bfloat16)
    wq = torch.randn((H, W, d), generator=g, device=dev) / W ** 0.5
    wk = torch.randn((H, W, d), generator=g, device=dev) / W ** 0.5
    yq = torch.empty_like(xq)
    yk = torch.empty_like(xk)

    def step():
        mesa.mesa_qk_preprocess(xq, wq, out=yq)
        mesa.mesa_qk_preprocess(xk, wk, out=yk)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mesa.profile_reset()
    mesa.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    mesa.profile_enable(False)
    kp = mesa.profile_read(mesa.KERNEL_QK_PREPROCESS)
    mesa.profile_reset()
    k_ms = kp[0] / max(kp[1], 1)
    per_launch = B * H * T * d * (2 + 2) + H * W * d * 4     # read x, write y (bf16), weights
    gbs = per_launch / (k_ms * 1e-3) / 1e9
    del xq, xk, yq, yk
    return {"workload": f"qk_preprocess_bf16_d128_T4096_W{W}", "B": B, "H": H, "T": T, "width": W,
            "tokens_per_s": round(B * H * T * steps / el, 1), "ms_per_step_q_and_k": round(1e3 * el / steps, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "qk_preprocess_kernel<128,bf16,bf16>",
                         "bytes_per_launch": per_launch, "avg_launch_ms": round(k_ms, 4)}}


def hawk(torch, mesa, dev, steps=20, warmup=3, c=8.0):
    """The Hawk layer's recurrence at the width of the headline layer
    (8 sequences x 4096 tokens x 2048 channels, bf16 inputs, fp32 output).
    HBM-bound; at this width the scan is one pass (each input read once)."""
    B, T, D = 8, 4096, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    x, ga, gx = (torch.randn((B, T, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    s = (0.9 + 0.099 * torch.rand(D, generator=g, device=dev)) ** (1.0 / c)
    lam = torch.log(s / (1 - s))
    h0 = torch.randn((B, D), generator=g, device=dev)
    y = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    ws = torch.empty(mesa.lib().mesa_hawk_workspace_bytes(B, T, D), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        mesa.mesa_hawk_scan(x, ga, gx, lam, c, h0, out=y, workspace=ws)
    torch.cuda.synchronize()
    mesa.profile_reset()
    mesa.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        mesa.mesa_hawk_scan(x, ga, gx, lam, c, h0, out=y, workspace=ws)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    mesa.profile_enable(False)
    kh = mesa.profile_read(mesa.KERNEL_HAWK)
    mesa.profile_reset()
    k_ms = kh[0] / max(kh[1], 1)
    per_call = B * T * D * (3 * 2 + 4) + D * 4 + 2 * B * D * 4    # x, ga, gx (bf16) + y (fp32); lam, h0
    gbs = per_call / (k_ms * 1e-3) / 1e9
    del x, ga, gx, y, ws
    return {"workload": f"hawk_bf16_B{B}_T{T}_D{D}", "tokens_per_s": round(B * T * steps / el, 1),
            "ms_per_call": round(1e3 * el / steps, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "hawk_stream_kernel<bf16,8,8> (one pass)",
                         "bytes_per_launch": per_call, "avg_launch_ms": round(k_ms, 4)}}


def measured_peaks(torch, mesa, dev):
    """Attainable rates on this GPU from known-work probe kernels: fp32 and
    bf16 MFMA register-resident loops (1024 workgroups x 4 waves) and a 1 GiB
    streaming copy; each timed with events on the stream it runs on."""
    sink = torch.empty(1024 * 256, dtype=torch.float32, device=dev)
    res = {}

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    for dt, it in (("f32", 2000), ("bf16", 2000)):
        flops = [0]

        def run(dt=dt, it=it):
            flops[0] = mesa.probe_mfma(dt, 1024, it, sink)
        ms = timed(run)
        res[f"mfma_{dt}_tflops"] = round(flops[0] / (ms * 1e-3) / 1e12, 1)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = timed(lambda: mesa.probe_copy(src, dst))
    res["copy_gbs"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    del src, dst, sink
    return res


def host_facts():
    """The host the oracle is timed on: logical CPUs, the CPUs this process
    may run on, the CPU model and OMP_NUM_THREADS."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"nproc": os.cpu_count(), "cpus_allowed": affinity, "cpu_model": model,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(x, w, heads=16):
    """The fp64 oracle, as it stands, on `heads` heads x all T tokens of the
    headline workload (one OpenMP thread per head), and on one head alone
    (one thread) for a per-core figure."""
    import numpy as np
    import oracle
    from test_regression_amd import inputs
    heads = min(heads, w.B * w.H)
    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:heads] if heads == w.B * w.H else \
        [(i % w.B, (5 * i) % w.H) for i in range(heads)]
    q = np.stack([inputs.as_f64(x["q"][b, h], w.dtype) for b, h in sel])[None]
    k = np.stack([inputs.as_f64(x["k"][b, h], w.dtype) for b, h in sel])[None]
    v = np.stack([inputs.as_f64(x["v"][b, h], w.dtype) for b, h in sel])[None]
    g = np.stack([x["gamma"][b, h] for b, h in sel])[None].astype(np.float64)
    lam = np.stack([x["lam"][h] for _, h in sel]).astype(np.float64)
    threads = min(oracle.max_threads(), heads)
    t0 = time.perf_counter()
    oracle.forward(q, k, v, g, lam, w.max_iters, w.tol)
    el = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.forward(q[:, :1], k[:, :1], v[:, :1], g[:, :1], lam[:1], w.max_iters, w.tol)
    el1 = time.perf_counter() - t0
    n = heads * w.T
    orc_flops = (8 + 2 * w.max_iters) * w.d * w.d + 11 * w.max_iters * w.d
    return {"value": round(n / el, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"all {w.B * w.H} heads" if heads == w.B * w.H else
                       f"{heads} of {w.B * w.H} heads (b, h) = {sel[:3]}...") +
                      f", all {w.T} tokens, k={w.max_iters}; {n} token-heads in {el:.1f} s",
            "seconds": round(el, 2), "host": host_facts(),
            "oracle_gflops": round(n * orc_flops / el / 1e9, 2),
            "one_thread": {"value": round(w.T / el1, 2), "unit": "tokens/s", "sample": f"head {sel[0]}, all "
                           f"{w.T} tokens, one OpenMP thread", "seconds": round(el1, 2),
                           "oracle_gflops": round(w.T * orc_flops / el1 / 1e9, 3)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="skip the dynamic-stopping and decode measurements")
    ap.add_argument("--decode-steps", type=int, default=1024, help="timed decode steps (1024 is the workload)")
    ap.add_argument("--no-warm-start", action="store_true", help="skip the warm-started decode runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=128)
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="also run one device-to-device copy of this many GiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the Mesa layer's heads are independent; sharding is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from test_regression_amd import inputs, mesa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    mesa.lib()
    log("[bench] measuring attainable peaks")
    peaks = measured_peaks(torch, mesa, dev)
    h = headline(torch, mesa, inputs, args, dev, peaks)
    torch.cuda.empty_cache()
    if args.copy_probe_gib > 0:
        n = int(args.copy_probe_gib * (1 << 30)) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {4 * n} bytes read, {4 * n} bytes written")
        del a, b
    extra = {}
    if not args.no_extra:
        extra["small_workloads"] = [small_workload(torch, mesa, inputs, dev, n)
                                    for n in ("tiny_f32_d16_T256", "mid_bf16_d64_T2048")]
        torch.cuda.empty_cache()
        extra["backward"] = backward(torch, mesa, h, dev, peaks)
        torch.cuda.empty_cache()
        extra["dynamic"] = dynamic(torch, mesa, inputs, dev)
        torch.cuda.empty_cache()
        extra["decode"] = decode(torch, mesa, inputs, dev, steps=args.decode_steps,
                                 warm_start=not args.no_warm_start)
        torch.cuda.empty_cache()
        extra["qk_preprocess"] = qk_preprocess(torch, mesa, inputs, dev)
        torch.cuda.empty_cache()
        extra["hawk"] = hawk(torch, mesa, dev)
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on {args.cpu_heads} heads")
        cpu = cpu_baseline(h["x"], h["w"], args.cpu_heads)
    w = h["w"]
    line = {
        "metric": "Mesa-layer fwd tokens/sec (B·H·T) at d=128, k=30 CG; % of MFMA/HBM roofline",
        "value": round(h["value"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(h["ms_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "arithmetic": "fp32 vectors and accumulation; matvec products on fp16 MFMAs over two-part splits "
                      "(hi + lo to 22 bits, three products hi.hi + hi.lo + lo.hi; bf16 keys exact in one part)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d_k": w.d, "d_v": w.d,
                   "chunk": w.chunk, "qkv_storage": w.dtype, "cg_iters": w.max_iters, "tol": w.tol,
                   "seed": w.seed},
        "tflops": round(h["tflops"], 2),
        "roofline": h["roofline"],
        "cpu_baseline": cpu,
        "kernels": h["kernels"],
    }
    line["measured_peaks"] = peaks
    for sec in ("decode", "qk_preprocess", "hawk"):
        if sec in extra:
            d = extra[sec]["roofline"]
            d["peak_measured"] = peaks["copy_gbs"]
            d["frac_measured"] = round(d["achieved"] / peaks["copy_gbs"], 4)
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
