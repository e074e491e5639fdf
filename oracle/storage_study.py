"""Which bf16 rounding points decide the error of a bf16 denoiser step, and what binary16
storage at some of them does instead?  (CPU study)

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: it composes the oracle's own blocks.

    python oracle/storage_study.py [--dim 4096] [--n-img 1024] [--n-txt 128]
                                   [--n-double 8] [--n-single 24] [--variants v1,v2,...]

Runs one denoiser step of the Klein-9B topology ([TRACE] section 3: stems, 8 double-stream
blocks, 24 single-stream blocks, final LayerNorm + modulate and projection) on the seeded
synthetic inputs, once in exact fp64 and once per variant of the oracle's bf16 storage
mode, and prints each variant's max-abs and normalised L2 error against the exact step.
A variant rounds values to bf16 at a subset of oracle.STORAGE_POINTS:

    all        every point (what a plain bf16 pipeline stores)
    all-X      every point except X (X carried exactly)
    all-X+Y    every point except X and Y
    only-X     X alone
    f16-X+Y    X and Y rounded to IEEE binary16 instead, every other point to bf16 except the
               final LayerNorm output, kept exact (the library's binary16 operand mode, whose
               head carries that output as a bf16 hi + lo pair)
    f16all-X+Y the same with the final LayerNorm output rounded like the other points
    none       no point (the exact step: error 0, a self-check)

The weights are generated one block at a time and every variant advances through that
block before the next is generated, so each block's weights are made once.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import flux_synth as fs  # noqa: E402
from oracle import flux_oracle as O  # noqa: E402

DEFAULT_VARIANTS = ("all", "all-final", "all-ln", "all-ln+final", "all-qkv", "all-rope",
                    "all-p", "all-o", "all-mlp", "only-final", "only-ln", "all-ln+o+mlp+final")


def variant_storage(name: str):
    """{point: bf16_storage} for a variant name (see the module docstring)."""
    if name == "none":
        return {}
    if name == "all":
        return {p: O.bf16_storage for p in O.STORAGE_POINTS}
    kind, _, pts = name.partition("-")
    pts = pts.split("+")
    if any(p not in O.STORAGE_POINTS for p in pts):
        raise ValueError(f"unknown point in variant {name!r}")
    if kind in ("f16", "f16all"):
        st = {p: (O.f16_storage if p in pts else O.bf16_storage) for p in O.STORAGE_POINTS}
        if kind == "f16" and "final" not in pts:
            del st["final"]
        return st
    if kind == "all":
        return {p: O.bf16_storage for p in O.STORAGE_POINTS if p not in pts}
    if kind == "only":
        return {p: O.bf16_storage for p in pts}
    raise ValueError(f"unknown variant {name!r}")


def errors(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--dim", type=int, default=4096)
    ap.add_argument("--n-img", type=int, default=1024)
    ap.add_argument("--n-txt", type=int, default=128)
    ap.add_argument("--context-dim", type=int, default=1536)
    ap.add_argument("--n-double", type=int, default=8)
    ap.add_argument("--n-single", type=int, default=24)
    ap.add_argument("--variants", default=",".join(DEFAULT_VARIANTS))
    args = ap.parse_args(argv)
    D = args.dim
    wl = fs.workload("klein9b_step_1024", dim=D, heads=D // O.HEAD_DIM, mlp_hidden=3 * D,
                     n_img=args.n_img, n_txt=args.n_txt, context_dim=args.context_dim,
                     n_double=args.n_double, n_single=args.n_single)
    inp = fs.step_inputs(wl, with_weights=False)
    w = fs.LazyWeights(fs.step_weight_specs(wl), wl.seed, wl.dtype)
    names = ["none"] + [v for v in args.variants.split(",") if v and v != "none"]
    stores = {n: variant_storage(n) for n in names}
    t0 = time.time()
    print(f"[study] D {D}, {wl.n_txt} + {wl.n_img} tokens, {wl.n_double} + {wl.n_single} "
          f"blocks, seed {wl.seed}; variants {', '.join(names[1:])}", flush=True)

    # the step's structure, as oracle.denoiser_step, with every variant carried together
    mods = O.step_mods(inp["t"], w)
    img0 = O.linear(O.f64(inp["x"]), O.f64(w["img_in"]))
    txt0 = O.linear(O.f64(inp["ctx"]), O.f64(w["txt_in"]))
    state = {n: (img0, txt0) for n in names}
    for i in range(wl.n_double):
        wb = O._Prefixed(w, f"double.{i}.")
        for n in names:
            img, txt = state[n]
            state[n] = O.double_block(img, txt, None, wb, inp["img_ids"], inp["txt_ids"],
                                      mods=mods["double"], storage=stores[n])
        print(f"[study] double block {i} done at {time.time() - t0:.0f} s", flush=True)
    for i in range(wl.n_single):
        wb = O._Prefixed(w, f"single.{i}.")
        for n in names:
            img, txt = state[n]
            state[n] = O.single_block(img, txt, None, wb, inp["img_ids"], inp["txt_ids"],
                                      mods=mods["single"], storage=stores[n])
        print(f"[study] single block {i} done at {time.time() - t0:.0f} s", flush=True)
    shift_f, scale_f = mods["final"]
    out = {}
    for n in names:
        st = O._storage_at(stores[n], "final")
        out[n] = O.linear(st(O.layernorm_modulate(state[n][0], shift_f, scale_f)),
                          O.f64(w["proj_out"]))
    ref = out["none"]
    print(f"[study] output rms {np.sqrt(np.mean(ref ** 2)):.4g}; errors against the exact "
          f"step ({time.time() - t0:.0f} s):", flush=True)
    print(f"| variant | rounded points | max-abs | nL2 |")
    print(f"|---|---|---|---|")
    for n in names[1:]:
        ma, nl = errors(out[n], ref)
        pts = ", ".join(p + (" (f16)" if stores[n][p] is O.f16_storage else "")
                        for p in O.STORAGE_POINTS if p in stores[n]) or "-"
        print(f"| {n} | {pts} | {ma:.3e} | {nl:.3e} |", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
