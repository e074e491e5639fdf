"""Benchmark: one Klein-9B-shaped 1024^2 denoiser step (8 double + 24 single blocks) on one
MI355X through the C ABI.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --probe dominant|attention|copy|bandwidth   # bare launches, for counter runs
    python bench.py --per-config               # one JSON line per traced workload: ms per
                                               # block, LN+modulate and RMSNorm+RoPE GB/s

Prints ONE JSON line: step throughput (algorithmic TFLOP/s, whole step), ms per step, the
roofline of the dominant kernel (timed live with HIP events on the stream it runs on), and
the fp64 oracle's throughput on a bounded sample of the same workload on the host cores.
Inputs are synthetic (seeded N(0, 0.02) weights, N(0, 1) activations) and already resident
in HBM when the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published); dense fp16 is the same
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
METRIC = "Klein-9B 1024² denoiser step ms + TFLOP/s (% of bf16 MFMA peak)"


# ------------------------------------------------------------------------------------
# algorithmic FLOPs (2 M N K per linear, 4 L^2 D per attention)
# ------------------------------------------------------------------------------------
def block_flops(kind: str, D: int, H: int, n_img: int, n_txt: int, B: int = 1) -> float:
    L = n_img + n_txt
    attn = 4.0 * L * L * D * B
    if kind == "double":
        per_tok = 2.0 * (3 * D * D + D * D + 2 * H * D + H * D)
        return per_tok * L * B + attn
    per_tok = 2.0 * ((3 * D + 2 * H) * D + (D + H) * D)
    return per_tok * L * B + attn


def step_flops(wl) -> float:
    D, H, B = wl.dim, wl.mlp_hidden, wl.batch
    f = wl.n_double * block_flops("double", D, H, wl.n_img, wl.n_txt, B)
    f += wl.n_single * block_flops("single", D, H, wl.n_img, wl.n_txt, B)
    f += 2.0 * B * (wl.n_img * wl.in_channels * D + wl.n_txt * wl.context_dim * D)   # stems
    f += 2.0 * B * wl.n_img * D * wl.in_channels                                      # proj_out
    f += 2.0 * B * (256 * D + D * D + 17 * D * D)                                     # temb + mods
    return f


def split_mfma_flops(wl) -> float:
    """MFMA work of a step with FLUX_PRECISION_SPLIT: the products that read the LayerNorm
    outputs (QKV, MLP-in, linear1) or the SwiGLU outputs (MLP-out, linear2's MLP columns) run
    twice (hi and lo planes)."""
    D, H, B, L = wl.dim, wl.mlp_hidden, wl.batch, wl.seq
    extra_double = 2.0 * L * B * (3 * D * D + 2 * H * D + H * D)
    extra_single = 2.0 * L * B * ((3 * D + 2 * H) * D + H * D)
    extra_head = 2.0 * B * wl.n_img * D * wl.in_channels  # in both precisions
    return step_flops(wl) + wl.n_double * extra_double + wl.n_single * extra_single + extra_head


# ------------------------------------------------------------------------------------
# device-resident synthetic weights (seeded, generated on the GPU for speed)
# ------------------------------------------------------------------------------------
def device_weights(specs: dict, seed: int, dtype):
    import torch
    g = torch.Generator(device="cuda")
    out = {}
    for i, (name, (shape, kind)) in enumerate(sorted(specs.items())):
        g.manual_seed(seed * 100003 + i)
        if kind == "g":
            out[name] = 1.0 + 0.02 * torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        else:
            out[name] = (0.02 * torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)).to(dtype)
    return out


class Events:
    """HIP events on a given stream."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record(self.stream)

    def stop_ms(self):
        import torch
        self.b.record(self.stream)
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


# ------------------------------------------------------------------------------------
# HBM traffic of the dominant kernel from committed rocprofv3 counter runs.  The summary
# records a hash of the GEMM sources it was taken with; once those sources change the
# figure no longer describes the kernel and is reported as null.
# ------------------------------------------------------------------------------------
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_swiglu_4608x24576x4096_hbm_counters.md")
KERNEL_SOURCES = ("diffusion_transformer_mmdit_amd/csrc/gemm.hip",
                  "diffusion_transformer_mmdit_amd/csrc/kernels.h",
                  "diffusion_transformer_mmdit_amd/csrc/common.h")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when absent or stale."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch",
                                                             "kernel_source_sha256"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------------------------
# dominant kernel: the MFMA GEMM with the fused SwiGLU epilogue at the single-block MLP-in
# shape (the largest launch of the step), with binary16 operands in the headline precision
# (FLUX_PRECISION_F16, the mode that meets the fp64 parity bars at bf16's MFMA rate).  Its
# launches inside the timed steps are bracketed by HIP events on the step's stream
# (libflux's timing hook); the probe mode launches it alone, exactly as the step does, for
# the counter runs.
# ------------------------------------------------------------------------------------
DOMINANT_KERNEL = ("gemm_bf16_lds_kernel<256,256,64,2,3,16,1,4,2,EpiSwiGLU<_Float16>,_Float16> "
                   "(single-block linear1 MLP part, binary16 operands)")


def to_headline_precision(F, w: dict) -> dict:
    """Device weights of FLUX_PRECISION_F16: the block linears in binary16, the rest as given."""
    import torch
    return {k: (v.to(torch.float16) if F.is_block_linear(k) else v) for k, v in w.items()}


def dominant_shape(wl):
    return wl.batch * wl.seq, 2 * wl.mlp_hidden, wl.dim


def dominant_probe(F, wl):
    import torch
    D, H = wl.dim, wl.mlp_hidden
    m, n, k = dominant_shape(wl)
    x = (torch.randn((m, k), device="cuda")).to(torch.float16)
    w = (0.02 * torch.randn((n, k), device="cuda")).to(torch.float16)
    y = torch.empty((m, D + H), device="cuda", dtype=torch.float16)
    cfg = F.make_cfg(D, wl.heads, H, precision=F.FLUX_PRECISION_F16)
    s = torch.cuda.current_stream()
    # the same split-K scratch the step gives its linear layers
    lnb = F.flux_linear_workspace_size()
    lws = torch.empty(lnb, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        F.flux_linear(cfg, F.FLUX_EPI_SWIGLU, m, n, k, x, k, w, k, y[:, D:], D + H, 0,
                      workspace=lws, workspace_bytes=lnb, stream=s)
    torch.cuda.synchronize()


def dominant_roofline(wl, launches: int, mean_us: float) -> dict:
    m, n, k = dominant_shape(wl)
    flops = 2.0 * m * n * k
    achieved = flops / (mean_us * 1e-6) / 1e12
    algo_bytes = 2 * (m * k + n * k + m * (n // 2))   # A, W once; binary16 h once
    return {
        "kernel": DOMINANT_KERNEL,
        "shape": [m, n, k],
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": PEAK_BF16_TFLOPS,
        "peak_of": "dense fp16 MFMA (2.5 PFLOP/s, as bf16)",
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
        "algorithmic_bytes_per_launch": algo_bytes,
        "avg_launch_us": round(mean_us, 1),
        "launches_timed": launches,
        "timed": "inside the timed steps: HIP event pair around each launch on the step's stream",
        "algorithmic_flops_per_launch": flops,
    }


# Every timing-hook site of the step: (site name, what it launches, its shape and
# algorithmic FLOP per launch at the workload).  The double block runs each linear of its
# two streams as one launch (image rows, then text rows), so those sites time both streams.
def site_table(F, wl):
    D, H, L = wl.dim, wl.mlp_hidden, wl.seq
    lin = lambda m, n, k: (2.0 * m * n * k, [m, n, k])
    att = (4.0 * L * L * D * wl.batch, [wl.batch, wl.heads, L, L])
    return [
        ("single_qkv", F.FLUX_SITE_SINGLE_QKV, "linear1 q|k|v, V^T epilogue", wl.n_single,
         *lin(L, 3 * D, D)),
        ("single_mlp_in", F.FLUX_SITE_SINGLE_MLP_IN, "linear1 gate|up, SwiGLU epilogue",
         wl.n_single, *lin(L, 2 * H, D)),
        ("single_attention", F.FLUX_SITE_SINGLE_ATTENTION, "flash joint attention (+ merge)",
         wl.n_single, *att),
        ("single_linear2", F.FLUX_SITE_SINGLE_LINEAR2, "linear2, gated-residual epilogue",
         wl.n_single, *lin(L, D, D + H)),
        ("double_qkv", F.FLUX_SITE_DOUBLE_QKV, "image + text QKV (one launch), V^T epilogue",
         wl.n_double, *lin(L, 3 * D, D)),
        ("double_attention", F.FLUX_SITE_DOUBLE_ATTENTION, "flash joint attention (+ merge)",
         wl.n_double, *att),
        ("double_out", F.FLUX_SITE_DOUBLE_OUT, "image + text out-proj (one launch), "
         "gated-residual epilogue", wl.n_double, *lin(L, D, D)),
        ("double_mlp_in", F.FLUX_SITE_DOUBLE_MLP_IN, "image + text MLP-in (one launch), SwiGLU "
         "epilogue", wl.n_double, *lin(L, 2 * H, D)),
        ("double_mlp_out", F.FLUX_SITE_DOUBLE_MLP_OUT, "image + text MLP-out (one launch), "
         "gated-residual epilogue", wl.n_double, *lin(L, D, H)),
    ]


def site_rooflines(F, wl, step, steps: int) -> list:
    """One timed pass of `steps` steps per site, the site's launches bracketed by HIP events
    on the step's stream (libflux's timing hook); TFLOP/s from the algorithmic FLOPs."""
    import torch
    out = []
    for name, site, what, per_step, flops, shape in site_table(F, wl):
        F.flux_timing_begin(site, per_step * steps)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        n, us = F.flux_timing_end()
        tf = flops / (us * 1e-6) / 1e12
        out.append({"site": name, "launch": what, "shape": shape, "launches_timed": n,
                    "avg_launch_us": round(us, 1), "algorithmic_flops_per_launch": flops,
                    "achieved_tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
    return out


def attention_probe(F, wl):
    """The joint attention at the step's shape (L x heads, bf16) through flux_attention,
    launched 3 times: the MFMA / VALU counter runs of the attention kernel use it."""
    import torch
    D, L = wl.dim, wl.seq
    qkv = torch.randn((wl.batch, L, 3 * D), device="cuda").to(torch.bfloat16)
    o = torch.empty((wl.batch, L, D), device="cuda", dtype=torch.bfloat16)
    cfg = F.make_cfg(D, wl.heads, wl.mlp_hidden)
    s = torch.cuda.current_stream()
    nb = F.flux_attention_workspace_size(cfg, wl.batch, L)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        F.flux_attention(cfg, wl.batch, L, qkv, qkv[..., D:], qkv[..., 2 * D:], 3 * D, o, D, ws,
                         nb, s)
    torch.cuda.synchronize()


def copy_probe(mib: int = 1024):
    """A plain 1 GiB device copy: the reference that scales the HBM byte counters."""
    import torch
    a = torch.full((mib << 20,), 1, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on one double block and one single block of the workload
# ------------------------------------------------------------------------------------
def cpu_baseline(wl, flops_step: float):
    import numpy as np
    import flux_synth as fs
    from oracle import flux_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("internal_api") == "openblas"] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    D, H = wl.dim, wl.mlp_hidden
    times = {}
    for kind in ("double", "single"):
        inp = fs.block_inputs(fs.workload(wl.name, kind=kind), kind=kind)
        fn = O.double_block if kind == "double" else O.single_block
        t0 = time.perf_counter()
        fn(inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"], inp["txt_ids"])
        times[kind] = time.perf_counter() - t0
        del inp
    est = wl.n_double * times["double"] + wl.n_single * times["single"]
    sample_flops = block_flops("double", D, H, wl.n_img, wl.n_txt) + \
        block_flops("single", D, H, wl.n_img, wl.n_txt)
    return {
        "value": round(flops_step / est / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"one double block ({times['double']:.1f} s) + one single block "
                   f"({times['single']:.1f} s) of the same workload in fp64 numpy; step time "
                   f"estimated as {wl.n_double} x double + {wl.n_single} x single = {est:.1f} s "
                   f"(sample {sample_flops / 1e12:.2f} TFLOP)"),
        "est_step_s": round(est, 2),
    }


# ------------------------------------------------------------------------------------
# per-workload block timings and bandwidth-kernel rates
# ------------------------------------------------------------------------------------
PER_CONFIG = ("tiny_single_f32", "klein4b_single_512", "klein9b_double_1024",
              "klein9b_step_1024", "dev_pair_2048", "klein9b_generate_1024", "klein9b_edit_1024",
              "klein9b_fp8_linear_1024")
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# editing cells (reference images, output side in pixels) of the pages' K/V cache table
EDIT_CELLS = ((1, 512), (1, 1024), (2, 1024), (4, 1024))


def _time_ms(fn, s, warmup=3, reps=10):
    import torch
    for _ in range(warmup):
        fn()
    ev = Events(s)
    torch.cuda.synchronize()
    ev.start()
    for _ in range(reps):
        fn()
    return ev.stop_ms() / reps


def _time_rotating_ms(fns, s, rounds=3):
    """Mean duration of one call when consecutive calls use different buffer sets: `fns` are
    the same kernel call on len(fns) disjoint sets of operands, together larger than the
    256 MB MALL, so a set's last use lies several hundred MB of other traffic back and every
    call streams its operands from HBM.  Timed back to back between two events on `s`."""
    for fn in fns:
        fn()
    ev = Events(s)
    import torch
    torch.cuda.synchronize()
    ev.start()
    for _ in range(rounds):
        for fn in fns:
            fn()
    return ev.stop_ms() / (rounds * len(fns))


def _sets_for(nbytes: int, floor_mb: int = 768) -> int:
    """Buffer sets so that the others' traffic between two uses of one set is > floor_mb."""
    return max(2, -(-floor_mb * (1 << 20) // nbytes) + 1)


def generate_line(F, fs, wl) -> dict:
    """Sampling loop at the step's shapes: a 4-step distilled generation and guided steps
    (one batch-2 forward each), against the plain step; all on device-resident inputs."""
    import torch
    dtype = torch.bfloat16
    # the benchmark's precision (binary16 block linears: the mode that meets the fp64 bars)
    w = to_headline_precision(F, device_weights(fs.step_weight_specs(wl), wl.seed, dtype))
    mw = F.ModelWeights(w, wl.n_double, wl.n_single)
    cfg = F.make_cfg(wl.dim, wl.heads, wl.mlp_hidden, in_channels=wl.in_channels,
                     context_dim=wl.context_dim, n_double=wl.n_double, n_single=wl.n_single,
                     precision=F.FLUX_PRECISION_F16)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    lat = 2 * wl.grid
    C = wl.in_channels // 4
    noise = torch.randn((1, C, lat, lat), generator=g, device="cuda")
    ctx = torch.randn((1, wl.n_txt, wl.context_dim), generator=g, device="cuda").to(dtype)
    unc = torch.randn((1, wl.n_txt, wl.context_dim), generator=g, device="cuda").to(dtype)
    out = torch.empty_like(noise)
    s = torch.cuda.current_stream()
    res = {"workload": wl.name, "dtype": wl.dtype, "precision": "FLUX_PRECISION_F16",
           "latent": [1, C, lat, lat], "n_txt": wl.n_txt}
    # the plain step on the same shapes
    x = torch.randn((1, wl.n_img, wl.in_channels), generator=g, device="cuda").to(dtype)
    t = torch.rand((1,), generator=g, device="cuda")
    img_ids = torch.from_numpy(fs.image_ids(wl.n_img)).cuda()
    txt_ids = torch.from_numpy(fs.text_ids(wl.n_txt)).cuda()
    vout = torch.empty((1, wl.n_img, wl.in_channels), device="cuda")
    nb = F.flux_denoiser_step_workspace_size(cfg, 1, wl.n_img, wl.n_txt)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    step_ms = _time_ms(lambda: F.flux_denoiser_step(cfg, mw, t, None, 1, wl.n_img, wl.n_txt, x, ctx,
                                                    img_ids, txt_ids, vout, ws, nb, s), s)
    del ws
    res["step_ms"] = round(step_ms, 3)
    fl = step_flops(wl)
    for guided, n, key in ((False, 4, "generate_4step"), (True, 4, "guided_4step")):
        nb = F.flux_denoise_workspace_size(cfg, 1, lat, lat, wl.n_txt, guided)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        fn = lambda: F.flux_denoise(cfg, mw, n, None, 4.0, 1, lat, lat, wl.n_txt, noise, ctx,
                                    unc if guided else None, out, ws, nb, s)
        ms = _time_ms(fn, s, warmup=1, reps=3)
        flops = n * (2 if guided else 1) * fl
        res[f"{key}_ms"] = round(ms, 3)
        res[f"{key}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        # time outside the n (or 2n batch rows of) denoiser steps: packing, ids, updates
        res[f"{key}_ms_per_step"] = round(ms / n, 3)
        del ws
    res["sampler_overhead_ms"] = round(res["generate_4step_ms"] - 4 * step_ms, 3)
    del w, mw
    return res


def edit_line(F, fs, wl) -> dict:
    """4-step generations conditioned on 1024^2 reference latents: the reference K/V cache
    filled once (extract, then cached steps) against filled before every step (the
    references recomputed each step); the cached steps' single-block attention (joint
    sequence + reference keys) timed with the library's event hook."""
    import torch
    dtype = torch.bfloat16
    w = to_headline_precision(F, device_weights(fs.step_weight_specs(wl), wl.seed, dtype))
    mw = F.ModelWeights(w, wl.n_double, wl.n_single)
    cfg = F.make_cfg(wl.dim, wl.heads, wl.mlp_hidden, in_channels=wl.in_channels,
                     context_dim=wl.context_dim, n_double=wl.n_double, n_single=wl.n_single,
                     precision=F.FLUX_PRECISION_F16)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    C = wl.in_channels // 4
    ctx = torch.randn((1, wl.n_txt, wl.context_dim), generator=g, device="cuda").to(dtype)
    s = torch.cuda.current_stream()
    res = {"workload": wl.name, "dtype": wl.dtype, "precision": "FLUX_PRECISION_F16", "n_steps": 4,
           "reference_side": 1024, "cells": []}
    for n_refs, side in EDIT_CELLS:
        lat = side // 8                      # 8x VAE downsampling: latent side
        ref_lat = 1024 // 8
        noise = torch.randn((1, C, lat, lat), generator=g, device="cuda")
        refs = torch.randn((1, n_refs, C, ref_lat, ref_lat), generator=g, device="cuda")
        out = torch.empty_like(noise)
        nb = F.flux_denoise_refs_workspace_size(cfg, 1, lat, lat, wl.n_txt, n_refs, ref_lat,
                                                ref_lat)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        cell = {"refs": n_refs, "output": side}
        for use_cache, key in ((True, "cached"), (False, "recomputed")):
            fn = lambda: F.flux_denoise_refs(cfg, mw, 4, None, 1, lat, lat, wl.n_txt, noise, ctx,
                                             n_refs, ref_lat, ref_lat, refs, use_cache, out, ws,
                                             nb, s)
            if use_cache:
                fn()
                F.flux_timing_begin(F.FLUX_SITE_SINGLE_ATTENTION, 4 * wl.n_single)
                fn()
                n_att, att_us = F.flux_timing_end()
                Lq = wl.n_txt + (lat // 2) ** 2
                Lk = Lq + n_refs * (ref_lat // 2) ** 2
                cell["attention_us"] = round(att_us, 1)
                cell["attention_tflops"] = round(4.0 * Lq * Lk * wl.dim / (att_us * 1e-6) / 1e12,
                                                 1)
            cell[f"{key}_ms"] = round(_time_ms(fn, s, warmup=1, reps=2), 2)
        cell["speedup"] = round(cell["recomputed_ms"] / cell["cached_ms"], 3)
        res["cells"].append(cell)
        del ws, noise, refs, out
        torch.cuda.empty_cache()
    del w, mw
    return res


def fp8_line(F, fs, wl) -> dict:
    """The single block's linears in bf16 and in FP8 (E4M3, per-row x per-channel scales)
    on the same shapes and epilogues, and the per-row quantization of the activations."""
    import torch
    D, H, L = wl.dim, wl.mlp_hidden, wl.seq
    cfg = F.make_cfg(D, wl.heads, H)
    s = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    lnb = F.flux_linear_workspace_size()
    lws = torch.empty(lnb, dtype=torch.uint8, device="cuda")
    res = {"workload": wl.name, "tokens": L, "peak_fp8_tflops": PEAK_FP8_TFLOPS,
           "peak_bf16_tflops": PEAK_BF16_TFLOPS, "linears": []}
    shapes = (("mlp_in_swiglu", F.FLUX_EPI_SWIGLU, 2 * H, D),
              ("qkv_store", F.FLUX_EPI_STORE, 3 * D, D),
              ("linear2_gated_residual", F.FLUX_EPI_GATED_RESIDUAL, D, D + H))
    for name, epi, n, k in shapes:
        m = L
        x = torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16)
        w = (0.02 * torch.randn((n, k), generator=g, device="cuda")).to(torch.bfloat16)
        nout = n // 2 if epi == F.FLUX_EPI_SWIGLU else n
        ydt = F.FLUX_F32 if epi == F.FLUX_EPI_GATED_RESIDUAL else F.FLUX_BF16
        y = torch.empty((m, nout), device="cuda",
                        dtype=torch.float32 if ydt == F.FLUX_F32 else torch.bfloat16)
        r = torch.randn((m, nout), generator=g, device="cuda") if ydt == F.FLUX_F32 else None
        gt = torch.randn((1, nout), generator=g, device="cuda") if r is not None else None
        qa = torch.empty((m, k), dtype=torch.uint8, device="cuda")
        qw = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        sa = torch.empty(m, device="cuda")
        sw = torch.empty(n, device="cuda")
        F.flux_quantize_fp8_rows(n, k, w, F.FLUX_BF16, k, qw, k, sw, s)
        quant = lambda: F.flux_quantize_fp8_rows(m, k, x, F.FLUX_BF16, k, qa, k, sa, s)
        quant()
        kw = dict(resid=r, ldr=nout, gate=gt, rows_per_batch=m, workspace=lws,
                  workspace_bytes=lnb, stream=s)
        b16 = _time_ms(lambda: F.flux_linear(cfg, epi, m, n, k, x, k, w, k, y, nout, ydt, **kw), s)
        f8 = _time_ms(lambda: F.flux_linear_fp8(cfg, epi, m, n, k, qa, k, sa, qw, k, sw, y, nout,
                                                ydt, **kw), s)
        qms = _time_ms(quant, s)
        flops = 2.0 * m * n * k
        qbytes = m * k * 3 + m * 4
        res["linears"].append({
            "name": name, "shape": [m, n, k],
            "bf16_us": round(b16 * 1e3, 1), "bf16_tflops": round(flops / (b16 * 1e-3) / 1e12, 1),
            "fp8_us": round(f8 * 1e3, 1), "fp8_tflops": round(flops / (f8 * 1e-3) / 1e12, 1),
            "fp8_frac_of_peak": round(flops / (f8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "speedup": round(b16 / f8, 3),
            "quantize_activations_us": round(qms * 1e3, 1),
            "quantize_gbs": round(qbytes / (qms * 1e-3) / 1e9, 1),
            "speedup_incl_quantize": round(b16 / (f8 + qms), 3)})
        del x, w, y, r, qa, qw
    return res


def per_config_line(F, fs, name: str) -> dict:
    import torch
    wl = fs.workload(name)
    if wl.kind == "fp8":
        return fp8_line(F, fs, wl)
    if wl.kind == "generate":
        return generate_line(F, fs, wl)
    if wl.kind == "edit":
        return edit_line(F, fs, wl)
    dtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    fdt = F.FLUX_BF16 if wl.dtype == "bf16" else F.FLUX_F32
    D, H, B = wl.dim, wl.mlp_hidden, wl.batch
    Nt, Ni, L = wl.n_txt, wl.n_img, wl.seq
    # bf16 workloads in the benchmark's precision (binary16 block linears)
    prec = F.FLUX_PRECISION_F16 if wl.dtype == "bf16" else F.FLUX_PRECISION_BF16
    cfg = F.make_cfg(D, wl.heads, H, dtype=fdt, precision=prec)
    conv = (lambda w: to_headline_precision(F, w)) if prec == F.FLUX_PRECISION_F16 else (lambda w: w)
    s = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    img = torch.randn((B, Ni, D), generator=g, device="cuda").to(dtype)
    txt = torch.randn((B, Nt, D), generator=g, device="cuda").to(dtype)
    t = torch.rand((B,), generator=g, device="cuda")
    img_ids = torch.from_numpy(fs.image_ids(Ni)).cuda()
    txt_ids = torch.from_numpy(fs.text_ids(Nt)).cuda()
    img_o, txt_o = torch.empty_like(img), torch.empty_like(txt)
    kinds = {"single": ("single",), "double": ("double",), "step": ("double", "single"),
             "pair": ("double", "single")}[wl.kind]
    res = {"workload": name, "dtype": wl.dtype,
           "precision": "FLUX_PRECISION_F16" if prec == F.FLUX_PRECISION_F16 else "FLUX_PRECISION_BF16",
           "dim": D, "heads": wl.heads, "mlp_hidden": H, "n_txt": Nt, "n_img": Ni, "batch": B}
    for kind in kinds:
        if kind == "double":
            w = conv(device_weights(fs.double_block_weight_specs(D, H), wl.seed, dtype))
            nb = F.flux_double_block_workspace_size(cfg, B, Ni, Nt)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            bw = F.double_weights(w)
            fn = lambda: F.flux_double_block_fwd(cfg, bw, t, B, Ni, Nt, img, txt, img_ids, txt_ids,
                                                 img_o, txt_o, ws, nb, s)
        else:
            w = conv(device_weights(fs.single_block_weight_specs(D, H), wl.seed, dtype))
            nb = F.flux_single_block_workspace_size(cfg, B, Ni, Nt)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            bw = F.single_weights(w)
            fn = lambda: F.flux_single_block_fwd(cfg, bw, t, B, Ni, Nt, img, txt, img_ids, txt_ids,
                                                 img_o, txt_o, ws, nb, s)
        ms = _time_ms(fn, s)
        fl = block_flops(kind, D, H, Ni, Nt, B)
        res[f"{kind}_block_ms"] = round(ms, 4)
        res[f"{kind}_block_tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
        del w, ws, bw
    for kname, nbytes, fns in bandwidth_kernels(F, fs, wl, cfg, t, txt_ids, img_ids, g, dtype, s):
        bandwidth_entry(res, kname, nbytes, len(fns), _time_rotating_ms(fns, s),
                        _time_ms(fns[0], s))
        del fns
        if kname != "modulation_gemv":
            copy_reference(res, kname, nbytes, s)
    return res


def bandwidth_kernels(F, fs, wl, cfg, t, txt_ids, img_ids, g, dtype, s):
    """The HBM-bound kernels at the workload's shape, each as calls over several disjoint
    buffer sets that together exceed the MALL: [(name, algorithmic bytes per call, calls)].
    Yields one kernel at a time so only its sets are resident."""
    import torch
    D, B = wl.dim, wl.batch
    Nt, Ni, L = wl.n_txt, wl.n_img, wl.seq
    # LN + modulate over the joint sequence: fp32 residual in, model dtype out (as the step)
    sh = torch.randn((B, D), generator=g, device="cuda")
    sc = torch.randn((B, D), generator=g, device="cuda")
    esz = 2 if dtype == torch.bfloat16 else 4
    nbytes = B * L * D * (4 + esz)
    fns = []
    for _ in range(_sets_for(nbytes)):
        x32 = torch.randn((B * L, D), generator=g, device="cuda")
        # binary16 outputs under FLUX_PRECISION_F16 (the same bytes as bf16)
        y = torch.empty((B * L, D), device="cuda",
                        dtype=torch.float16 if cfg.precision == F.FLUX_PRECISION_F16 else dtype)
        fns.append(lambda x32=x32, y=y: F.flux_layernorm_modulate(cfg, B * L, L, x32, F.FLUX_F32,
                                                                  sh, sc, y, s))
    yield "ln_modulate", nbytes, fns
    del fns, x32, y
    # RMSNorm + RoPE on q and k in place, inside a [B, L, 3D] QKV buffer
    gam = torch.ones(128, device="cuda")
    nb = F.flux_qk_norm_rope_workspace_size(cfg, Nt, Ni)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    nbytes = 2 * 2 * B * L * D * esz
    fns = []
    for _ in range(_sets_for(nbytes)):
        qkv = torch.randn((B, L, 3 * D), generator=g, device="cuda").to(dtype)
        fns.append(lambda qkv=qkv: F.flux_qk_norm_rope(cfg, B, Nt, Ni, qkv, qkv[..., D:], 3 * D,
                                                       gam, gam, gam, gam, txt_ids, img_ids, ws,
                                                       nb, s))
    yield "qk_norm_rope", nbytes, fns
    del fns, qkv
    # modulation: timestep MLP + one modulation GEMV (the double block's image set, 6D x D);
    # weight reads dominate: (256 D + D^2 + 6 D^2) bf16
    if wl.dtype == "bf16":
        mout = torch.empty((B, 6 * D), device="cuda")
        mnb = F.flux_modulation_workspace_size(cfg, B)
        mws = torch.empty(max(mnb, 256), dtype=torch.uint8, device="cuda")
        nbytes = 2 * (256 * D + D * D + 6 * D * D)
        fns, keep = [], []
        for _ in range(_sets_for(nbytes)):
            tw = device_weights(fs.temb_weight_specs(D), wl.seed, dtype)
            wmod = (0.02 * torch.randn((6 * D, D), generator=g, device="cuda")).to(dtype)
            tws = F.temb_weights(tw)
            keep.append((tw, wmod, tws))
            fns.append(lambda tws=tws, wmod=wmod: F.flux_modulation(cfg, tws, wmod, 6 * D, t, B,
                                                                    mout, mws, mnb, s))
        yield "modulation_gemv", nbytes, fns
        del fns, keep


def bandwidth_probe(F, fs, name: str = "klein9b_step_1024"):
    """Each HBM-bound kernel of bandwidth_kernels, called twice over its buffer sets (every
    call after the first pass finds its operands evicted from the MALL): the HBM byte counter
    runs use it."""
    import torch
    wl = fs.workload(name)
    dtype = torch.bfloat16
    cfg = F.make_cfg(wl.dim, wl.heads, wl.mlp_hidden)
    s = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    t = torch.rand((wl.batch,), generator=g, device="cuda")
    img_ids = torch.from_numpy(fs.image_ids(wl.n_img)).cuda()
    txt_ids = torch.from_numpy(fs.text_ids(wl.n_txt)).cuda()
    for kname, nbytes, fns in bandwidth_kernels(F, fs, wl, cfg, t, txt_ids, img_ids, g, dtype, s):
        for _ in range(2):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        print(f"[bench] probe: {kname} ({nbytes} algorithmic bytes per call), 2 x {len(fns)} "
              "calls", file=sys.stderr, flush=True)
        del fns


def copy_reference(res: dict, name: str, nbytes: int, s):
    """A plain device copy with the same total traffic (nbytes / 2 read, nbytes / 2 written),
    timed the same way over rotating buffer sets: the rate HBM gives a read + write stream."""
    import torch
    half = (nbytes // 2 + 15) // 16 * 16
    fns = []
    for _ in range(_sets_for(nbytes)):
        a = torch.empty(half, dtype=torch.uint8, device="cuda")
        b = torch.empty(half, dtype=torch.uint8, device="cuda")
        fns.append(lambda a=a, b=b: b.copy_(a))
    ms = _time_rotating_ms(fns, s)
    res[f"{name}_copy_reference_gbs"] = round(2 * half / (ms * 1e-3) / 1e9, 1)
    res[f"{name}_pct_of_copy"] = round(100.0 * res[f"{name}_gbs"] / res[f"{name}_copy_reference_gbs"], 1)


def bandwidth_entry(res: dict, name: str, nbytes: int, sets: int, ms_cold: float,
                    ms_warm: float):
    """GB/s of an HBM-bound kernel from its algorithmic bytes: over rotating buffer sets
    larger than the MALL together (operands come from HBM: the HBM figure), and back to back
    on one set (operands may stay in the 256 MB MALL)."""
    gbs = nbytes / (ms_cold * 1e-3) / 1e9
    res[f"{name}_bytes"] = int(nbytes)
    res[f"{name}_buffer_sets"] = int(sets)
    res[f"{name}_us"] = round(ms_cold * 1e3, 2)
    res[f"{name}_gbs"] = round(gbs, 1)
    res[f"{name}_pct_hbm"] = round(100.0 * gbs / PEAK_HBM_GBS, 1)
    res[f"{name}_us_back_to_back"] = round(ms_warm * 1e3, 2)
    res[f"{name}_gbs_back_to_back"] = round(nbytes / (ms_warm * 1e-3) / 1e9, 1)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="klein9b_step_1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-config", action="store_true",
                    help="time the blocks and bandwidth kernels of every traced workload")
    ap.add_argument("--only", default=None, choices=PER_CONFIG,
                    help="with --per-config: just this workload")
    ap.add_argument("--probe", choices=("dominant", "attention", "copy", "bandwidth"),
                    default=None,
                    help="only launch the dominant kernel, the attention or a 1 GiB copy 3 "
                         "times (bandwidth: the HBM-bound kernels over rotating sets) and exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "path is not built", file=sys.stderr)
        return 2

    import torch
    import flux_synth as fs
    from diffusion_transformer_mmdit_amd import flux as F

    F.lib()
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 1
    if args.per_config:
        for name in PER_CONFIG if args.only is None else (args.only,):
            print(json.dumps(per_config_line(F, fs, name)), flush=True)
            torch.cuda.empty_cache()
        return 0
    wl = fs.workload(args.workload)
    assert wl.kind == "step"
    if args.probe == "dominant":
        dominant_probe(F, wl)
        print("[bench] probe: dominant kernel launched 3 times", file=sys.stderr, flush=True)
        return 0
    if args.probe == "attention":
        attention_probe(F, wl)
        print("[bench] probe: attention launched 3 times", file=sys.stderr, flush=True)
        return 0
    if args.probe == "bandwidth":
        bandwidth_probe(F, fs)
        return 0
    if args.probe == "copy":
        copy_probe()
        print("[bench] probe: 1 GiB copy launched 3 times", file=sys.stderr, flush=True)
        return 0
    dtype = torch.bfloat16
    print(f"[bench] {wl.name}: generating {fs.param_count(fs.step_weight_specs(wl)) / 1e9:.3f} B "
          "params on device", file=sys.stderr, flush=True)
    w = device_weights(fs.step_weight_specs(wl), wl.seed, dtype)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    x = torch.randn((wl.batch, wl.n_img, wl.in_channels), generator=g, device="cuda").to(dtype)
    ctx = torch.randn((wl.batch, wl.n_txt, wl.context_dim), generator=g, device="cuda").to(dtype)
    t = torch.rand((wl.batch,), generator=g, device="cuda")
    img_ids = torch.from_numpy(fs.image_ids(wl.n_img)).cuda()
    txt_ids = torch.from_numpy(fs.text_ids(wl.n_txt)).cuda()
    # the headline precision: binary16 operands of the block linears (FLUX_PRECISION_F16)
    cfg = F.make_cfg(wl.dim, wl.heads, wl.mlp_hidden, in_channels=wl.in_channels,
                     context_dim=wl.context_dim, n_double=wl.n_double, n_single=wl.n_single,
                     precision=F.FLUX_PRECISION_F16)
    w16 = to_headline_precision(F, w)
    mw = F.ModelWeights(w16, wl.n_double, wl.n_single)
    out = torch.empty((wl.batch, wl.n_img, wl.in_channels), device="cuda", dtype=torch.float32)
    nbytes = F.flux_denoiser_step_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()

    def step(stream=s):
        F.flux_denoiser_step(cfg, mw, t, None, wl.batch, wl.n_img, wl.n_txt, x, ctx, img_ids,
                             txt_ids, out, ws, nbytes, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    ev = Events(s)
    # events around every launch of the dominant kernel in the timed steps (created here)
    F.flux_timing_begin(F.FLUX_SITE_SINGLE_MLP_IN, wl.n_single * args.steps)
    torch.cuda.synchronize()
    ev.start()
    for _ in range(args.steps):
        step()
    total_ms = ev.stop_ms()
    torch.cuda.synchronize()
    launches, mean_us = F.flux_timing_end()
    ms = total_ms / args.steps
    flops = step_flops(wl)
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[bench] {ms:.2f} ms/step, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if not torch.isfinite(out).all():
        print("[bench] non-finite output", file=sys.stderr)
        return 1

    roof = dominant_roofline(wl, launches, mean_us)
    print(f"[bench] dominant kernel {roof['achieved']} TFLOP/s ({launches} launches, "
          f"{mean_us:.1f} us each)", file=sys.stderr, flush=True)
    # every GEMM epilogue and the attention, each timed the same way in passes of its own
    sites = site_rooflines(F, wl, step, args.steps)
    for r in sites:
        print(f"[bench]   {r['site']}: {r['avg_launch_us']} us, {r['achieved_tflops']} TFLOP/s "
              f"({100 * r['frac']:.1f}%)", file=sys.stderr, flush=True)
    # the same step captured once into a HIP graph and replayed (no host launch work between
    # kernels); the library enqueues only kernels, so the capture holds the whole step
    step()
    torch.cuda.synchronize()
    eager_out = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    graph_equal = bool(torch.equal(out, eager_out))
    ev.start()
    for _ in range(args.steps):
        graph.replay()
    ms_graph = ev.stop_ms() / args.steps
    torch.cuda.synchronize()
    del graph, eager_out
    graph_leg = {"steps": args.steps, "ms_per_step": round(ms_graph, 3),
                 "time_vs_eager": round(ms_graph / ms, 4), "bitwise_equal_to_eager": graph_equal}
    print(f"[bench] graph replay: {ms_graph:.2f} ms/step ({ms_graph / ms:.4f}x), output "
          f"{'bitwise equal' if graph_equal else 'DIFFERENT'}", file=sys.stderr, flush=True)
    del ws, w16
    torch.cuda.empty_cache()
    mw_bf16 = F.ModelWeights(w, wl.n_double, wl.n_single)

    def other_precision(precision):
        """The same step in another operand precision (bf16 weights), steps // 2 timed."""
        c = F.make_cfg(wl.dim, wl.heads, wl.mlp_hidden, in_channels=wl.in_channels,
                       context_dim=wl.context_dim, n_double=wl.n_double, n_single=wl.n_single,
                       precision=precision)
        nb = F.flux_denoiser_step_workspace_size(c, wl.batch, wl.n_img, wl.n_txt)
        wsp = torch.empty(nb, dtype=torch.uint8, device="cuda")

        def run():
            F.flux_denoiser_step(c, mw_bf16, t, None, wl.batch, wl.n_img, wl.n_txt, x, ctx,
                                 img_ids, txt_ids, out, wsp, nb, s)

        n = max(1, args.steps // 2)
        run()
        torch.cuda.synchronize()
        ev.start()
        for _ in range(n):
            run()
        m = ev.stop_ms() / n
        torch.cuda.synchronize()
        return n, m

    # every operand in bf16 (FLUX_PRECISION_BF16): misses the fp64 bars at this workload
    bf_steps, ms_bf = other_precision(F.FLUX_PRECISION_BF16)
    bf16 = {"precision": "FLUX_PRECISION_BF16", "steps": bf_steps, "ms_per_step": round(ms_bf, 3),
            "algorithmic_tflops": round(flops / (ms_bf * 1e-3) / 1e12, 2),
            "time_vs_headline": round(ms_bf / ms, 3), "meets_fp64_parity_bars": False}
    print(f"[bench] bf16 precision: {ms_bf:.2f} ms/step ({ms_bf / ms:.3f}x)", file=sys.stderr,
          flush=True)
    # the LayerNorm and SwiGLU outputs carried as bf16 hi + lo pairs (FLUX_PRECISION_SPLIT)
    split_steps, ms_split = other_precision(F.FLUX_PRECISION_SPLIT)
    split = {"precision": "FLUX_PRECISION_SPLIT", "steps": split_steps,
             "ms_per_step": round(ms_split, 3),
             "algorithmic_tflops": round(flops / (ms_split * 1e-3) / 1e12, 2),
             "mfma_tflop_per_step": round(split_mfma_flops(wl) / 1e12, 3),
             "time_vs_headline": round(ms_split / ms, 3), "meets_fp64_parity_bars": True}
    print(f"[bench] split precision: {ms_split:.2f} ms/step ({ms_split / ms:.2f}x)",
          file=sys.stderr, flush=True)
    del w, mw, mw_bf16
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on one double + one single block", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(wl, flops)

    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "pct_of_16bit_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16+bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations, resident in HBM)",
        "config": {"workload": wl.name, "dim": wl.dim, "heads": wl.heads,
                   "mlp_hidden": wl.mlp_hidden, "n_img": wl.n_img, "n_txt": wl.n_txt,
                   "in_channels": wl.in_channels, "context_dim": wl.context_dim,
                   "n_double": wl.n_double, "n_single": wl.n_single, "global_batch": wl.batch,
                   "seq_len": wl.seq, "algorithmic_tflop_per_step": round(flops / 1e12, 3),
                   "precision": "FLUX_PRECISION_F16 (block linears: binary16 operands and "
                                "weights; attention, embedders, modulation and head: bf16; "
                                "fp32 accumulation); meets the fp64 parity bars",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "kernels": sites,
        "graph_replay": graph_leg,
        "precision_bf16": bf16,
        "precision_split": split,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
