"""Write the fp64 oracle output of one full Klein-9B 1024² denoiser step.

    python tests/golden/make_step_golden.py [--workload klein9b_step_1024] [--storage bf16]

Calls only oracle/ (the fp64 definition) and the seeded input generator: the weights are
generated block by block (flux_synth.LazyWeights), the step runs in fp64 on the host (about
ten minutes), and the whole output [n_img, in_channels] is written to
tests/golden/<workload>.npy (float64, no pickle) with its provenance in
tests/golden/<workload>.meta.txt, for the GPU test that runs the same step through
flux_denoiser_step.  With --storage bf16 the step is the oracle's bf16 storage mode (the
definition with values rounded to bf16 where a bf16 pipeline stores them) and the files are
tests/golden/<workload>_bf16_storage.*.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import flux_synth as fs  # noqa: E402
from oracle import flux_oracle as O  # noqa: E402


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="klein9b_step_1024")
    ap.add_argument("--storage", choices=("fp64", "bf16"), default="fp64")
    args = ap.parse_args(argv)
    wl = fs.workload(args.workload)
    assert wl.kind == "step" and wl.batch == 1
    inp = fs.step_inputs(wl, with_weights=False)
    w = fs.LazyWeights(fs.step_weight_specs(wl), wl.seed, wl.dtype)
    t0 = time.time()

    def progress(kind, i):
        print(f"[golden] {kind} block {i} done at {time.time() - t0:.0f} s", flush=True)

    storage = O.bf16_storage if args.storage == "bf16" else None
    out = O.denoiser_step(inp["x"], inp["ctx"], inp["t"], w, inp["img_ids"], inp["txt_ids"],
                          wl.n_double, wl.n_single, on_block=progress, storage=storage)
    suffix = "_bf16_storage" if storage else ""
    what = "fp64 oracle, bf16 storage mode," if storage else "fp64 oracle"
    base = os.path.join(HERE, f"{wl.name}{suffix}")
    np.save(base + ".npy", np.ascontiguousarray(out[0], dtype=np.float64), allow_pickle=False)
    with open(base + ".meta.txt", "w") as f:
        f.write(f"{what} output of one {wl.name} denoiser step (flux_synth seed {wl.seed},"
                f" t = {float(inp['t'][0]):.9g})\n")
        f.write(f"array: {os.path.basename(base)}.npy, float64 [{wl.n_img}, {wl.in_channels}]"
                f" (image tokens x output channels, batch item 0)\n")
        f.write("written by tests/golden/make_step_golden.py (oracle/ + flux_synth only)\n")
        f.write(f"output rms: {np.sqrt(np.mean(out[0] ** 2)):.17g}\n")
    print(f"[golden] wrote {base}.npy in {time.time() - t0:.0f} s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
