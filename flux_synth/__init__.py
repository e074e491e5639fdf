"""Seeded synthetic inputs for the FLUX.2-style MMDiT denoiser forward.

This module is shared by the fp64 oracle's tests and by the HIP path's tests and
benchmark.  It produces *data only*: shapes, seeded random values, bf16 rounding of
those values and integer position ids.  It holds none of the method's arithmetic
(no normalisation, attention, RoPE, modulation or projection).

Value recipe (the workloads' stated distributions):
  * linear weights     ~ N(0, 0.02)   (std 0.02)
  * QK-norm scales     = 1 + N(0, 0.02), stored fp32 (a jittered ones-init, so the
                         per-channel multiply is exercised without shrinking q, k)
  * activations        ~ N(0, 1)
  * timestep t         = 0.5 for the tiny configuration, else U[0, 1)
  * image ids          (0, row, col, 0) on a sqrt(N_img) x sqrt(N_img) grid, row-major
  * text ids           (0, 0, 0, i)
For bf16 workloads every floating value is rounded to bf16 (round to nearest even)
here, so both sides read the exact same numbers; the arrays are returned as float32
holding bf16-representable values (``to_bf16_bits`` gives the raw 16-bit patterns).

Every tensor has its own random stream, keyed by (seed, tensor name), so a tensor's
values do not depend on which other tensors were drawn or in what order.  That lets a
consumer generate one block's weights at a time (streaming) and still match a
consumer that generated everything at once.
"""
from __future__ import annotations

import math
import os
import zlib
from collections.abc import Mapping
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "rng_for", "normal", "uniform",
    "round_to_bf16", "to_bf16_bits", "image_ids", "text_ids",
    "temb_weight_specs", "double_block_weight_specs", "single_block_weight_specs",
    "step_weight_specs", "make_weights", "block_inputs", "step_inputs",
    "param_count",
]


# ----------------------------------------------------------------------------------
# Workload shapes
# ----------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload (B = batch, D = hidden, H = MLP hidden)."""
    name: str
    dim: int
    heads: int
    mlp_hidden: int
    n_img: int
    n_txt: int
    dtype: str = "bf16"          # "bf16" or "f32": storage / compute type
    batch: int = 1
    in_channels: int = 128
    context_dim: int = 0         # text input projection width (step only)
    n_double: int = 0            # double-stream blocks (step only)
    n_single: int = 0            # single-stream blocks (step only)
    t_fixed: float | None = None # fixed timestep, else drawn U[0,1)
    seed: int = 1000
    kind: str = "single"  # "single", "double", "pair", "step", "generate", "edit" or "fp8"

    @property
    def seq(self) -> int:
        return self.n_txt + self.n_img

    @property
    def grid(self) -> int:
        g = int(round(math.sqrt(self.n_img)))
        if g * g != self.n_img:
            raise ValueError(f"n_img={self.n_img} is not a square grid")
        return g


WORKLOADS: dict[str, Workload] = {
    # Tiny single-stream block, fp32: D 256 (2 heads x 128), MLP 768, 8x8 image grid +
    # 16 text tokens, t = 0.5.
    "tiny_single_f32": Workload("tiny_single_f32", 256, 2, 768, 64, 16, dtype="f32",
                                t_fixed=0.5, seed=1001, kind="single"),
    # Klein-4B-shaped single-stream block at 512^2.
    "klein4b_single_512": Workload("klein4b_single_512", 3072, 24, 9216, 1024, 512,
                                   seed=1002, kind="single"),
    # Klein-9B-shaped double-stream block at 1024^2.
    "klein9b_double_1024": Workload("klein9b_double_1024", 4096, 32, 12288, 4096, 512,
                                    seed=1003, kind="double"),
    # Full Klein-9B-shaped denoiser step at 1024^2: 8 double + 24 single blocks,
    # image packed width 128, text width 12288.
    "klein9b_step_1024": Workload("klein9b_step_1024", 4096, 32, 12288, 4096, 512,
                                  in_channels=128, context_dim=12288, n_double=8,
                                  n_single=24, seed=1004, kind="step"),
    # Klein-9B generation at 1024^2: the step's model sampled from a 32 x 128 x 128 noise
    # latent (4 distilled steps, or guided steps as one batch-2 forward each).
    "klein9b_generate_1024": Workload("klein9b_generate_1024", 4096, 32, 12288, 4096, 512,
                                      in_channels=128, context_dim=12288, n_double=8,
                                      n_single=24, seed=1006, kind="generate"),
    # Klein-9B editing with reference images: the generation above conditioned on 1024^2
    # reference latents (64 x 64 tokens each) through the reference K/V cache.
    "klein9b_edit_1024": Workload("klein9b_edit_1024", 4096, 32, 12288, 4096, 512,
                                  in_channels=128, context_dim=12288, n_double=8, n_single=24,
                                  seed=1007, kind="edit"),
    # The Klein-9B single block's linear layers at 1024^2 (4608 tokens) in FP8 (E4M3) against
    # bf16: MLP-in + SwiGLU, the q|k|v projection shape, linear2 + gated residual.
    "klein9b_fp8_linear_1024": Workload("klein9b_fp8_linear_1024", 4096, 32, 12288, 4096, 512,
                                        seed=1008, kind="fp8"),
    # FLUX.2-dev-shaped long-sequence block pair at 2048^2 (one double + one single).
    "dev_pair_2048": Workload("dev_pair_2048", 6144, 48, 18432, 16384, 512,
                              seed=1005, kind="pair"),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. smaller n_img)."""
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


# ----------------------------------------------------------------------------------
# Random streams and bf16 rounding
# ----------------------------------------------------------------------------------
def rng_for(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for one named tensor of one seeded workload."""
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), key])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    return (to_bf16_bits(x).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 values, round to nearest even.

    Inputs here are finite (Gaussian / uniform draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0,
           dtype: str = "bf16") -> np.ndarray:
    """Seeded N(mean, std^2) draws for tensor `name`, rounded per `dtype` (float32 out)."""
    x = rng_for(seed, name).standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return _finish(x, dtype)


def uniform(seed: int, name: str, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Seeded U[lo, hi) draws (float32, not rounded to bf16)."""
    x = rng_for(seed, name).random(size=tuple(shape), dtype=np.float32)
    return (np.float32(lo) + x * np.float32(hi - lo)).astype(np.float32)


# ----------------------------------------------------------------------------------
# Position ids (integer inputs)
# ----------------------------------------------------------------------------------
def image_ids(n_img: int) -> np.ndarray:
    """[n_img, 4] int32 ids (0, row, col, 0) on a square grid, row-major."""
    g = int(round(math.sqrt(n_img)))
    if g * g != n_img:
        raise ValueError(f"n_img={n_img} is not a square grid")
    ids = np.zeros((n_img, 4), dtype=np.int32)
    r, c = np.divmod(np.arange(n_img, dtype=np.int32), g)
    ids[:, 1] = r
    ids[:, 2] = c
    return ids


def text_ids(n_txt: int) -> np.ndarray:
    """[n_txt, 4] int32 ids (0, 0, 0, i)."""
    ids = np.zeros((n_txt, 4), dtype=np.int32)
    ids[:, 3] = np.arange(n_txt, dtype=np.int32)
    return ids


# ----------------------------------------------------------------------------------
# Weight manifests: name -> (shape, kind).  kind "w" = linear weight N(0,0.02),
# "g" = QK-norm scale 1+N(0,0.02) (always fp32).  Linear weights are [out, in].
# ----------------------------------------------------------------------------------
HEAD_DIM = 128
TEMB_CHANNELS = 256


def temb_weight_specs(D: int) -> dict:
    return {"temb.w1": ((D, TEMB_CHANNELS), "w"), "temb.w2": ((D, D), "w")}


def _stream_specs(prefix: str, D: int, H: int) -> dict:
    return {
        f"{prefix}.qkv": ((3 * D, D), "w"),
        f"{prefix}.out": ((D, D), "w"),
        f"{prefix}.mlp_in": ((2 * H, D), "w"),
        f"{prefix}.mlp_out": ((D, H), "w"),
        f"{prefix}.q_norm": ((HEAD_DIM,), "g"),
        f"{prefix}.k_norm": ((HEAD_DIM,), "g"),
    }


def double_block_weight_specs(D: int, H: int, prefix: str = "", with_mod: bool = True) -> dict:
    s = {}
    if with_mod:
        s.update(temb_weight_specs(D))
        s["mod_img"] = ((6 * D, D), "w")
        s["mod_txt"] = ((6 * D, D), "w")
    s.update(_stream_specs(prefix + "img", D, H))
    s.update(_stream_specs(prefix + "txt", D, H))
    return s


def single_block_weight_specs(D: int, H: int, prefix: str = "", with_mod: bool = True) -> dict:
    s = {}
    if with_mod:
        s.update(temb_weight_specs(D))
        s["mod"] = ((3 * D, D), "w")
    s[prefix + "linear1"] = ((3 * D + 2 * H, D), "w")
    s[prefix + "linear2"] = ((D, D + H), "w")
    s[prefix + "q_norm"] = ((HEAD_DIM,), "g")
    s[prefix + "k_norm"] = ((HEAD_DIM,), "g")
    return s


def step_weight_specs(wl: Workload) -> dict:
    D, H = wl.dim, wl.mlp_hidden
    s = {
        "img_in": ((D, wl.in_channels), "w"),
        "txt_in": ((D, wl.context_dim), "w"),
    }
    s.update(temb_weight_specs(D))
    s["mod_dimg"] = ((6 * D, D), "w")
    s["mod_dtxt"] = ((6 * D, D), "w")
    s["mod_single"] = ((3 * D, D), "w")
    s["mod_final"] = ((2 * D, D), "w")
    s["proj_out"] = ((wl.in_channels, D), "w")
    for i in range(wl.n_double):
        s.update(double_block_weight_specs(D, H, prefix=f"double.{i}.", with_mod=False))
    for i in range(wl.n_single):
        s.update(single_block_weight_specs(D, H, prefix=f"single.{i}.", with_mod=False))
    return s


def param_count(specs: dict) -> int:
    return int(sum(int(np.prod(shape)) for shape, _ in specs.values()))


def _make_one(seed: int, name: str, shape, kind: str, dtype: str) -> np.ndarray:
    if kind == "w":
        return normal(seed, name, shape, std=0.02, dtype=dtype)
    if kind == "g":
        return normal(seed, name, shape, std=0.02, mean=1.0, dtype="f32")
    raise ValueError(kind)


def make_weights(specs: dict, seed: int, dtype: str, names=None,
                 threads: int | None = None) -> dict:
    """Generate the named weights (all of `specs`, or the subset `names`)."""
    names = list(specs) if names is None else list(names)
    threads = threads or min(16, os.cpu_count() or 1)

    def one(n):
        shape, kind = specs[n]
        return n, _make_one(seed, n, shape, kind, dtype)

    if threads <= 1 or len(names) <= 1:
        return dict(one(n) for n in names)
    with ThreadPoolExecutor(threads) as ex:
        return dict(ex.map(one, names))


class LazyWeights(Mapping):
    """Step weights generated on first use, one block at a time.

    Names "double.{i}.*" / "single.{i}.*" form one group per block: the first access to a
    name of a block generates the whole block and drops the previously generated block;
    other names are generated once and kept.  Values equal make_weights(specs, ...)[name]
    (each tensor has its own named random stream), so a consumer that walks the blocks in
    order holds one block's weights at a time.
    """

    def __init__(self, specs: dict, seed: int, dtype: str, threads: int | None = None):
        self._specs, self._seed, self._dtype, self._threads = specs, seed, dtype, threads
        self._groups: dict[str, list] = {}
        for n in specs:
            self._groups.setdefault(self._group(n), []).append(n)
        self._block_key, self._block = None, {}
        self._kept: dict = {}

    @staticmethod
    def _group(name: str) -> str:
        parts = name.split(".")
        return ".".join(parts[:2]) if parts[0] in ("double", "single") and len(parts) > 2 else name

    def __getitem__(self, name):
        g = self._group(name)
        if g == name:
            if name not in self._kept:
                self._kept[name] = make_weights(self._specs, self._seed, self._dtype, [name])[name]
            return self._kept[name]
        if g != self._block_key:
            self._block = {}
            self._block = make_weights(self._specs, self._seed, self._dtype, self._groups[g],
                                       threads=self._threads)
            self._block_key = g
        return self._block[name]

    def __iter__(self):
        return iter(self._specs)

    def __len__(self):
        return len(self._specs)

    def groups(self) -> list:
        """Group keys in the order the step uses them (globals, then blocks)."""
        return list(self._groups)

    def group_names(self, group: str) -> list:
        """Tensor names of one group."""
        return list(self._groups[group])


# ----------------------------------------------------------------------------------
# Whole-input bundles
# ----------------------------------------------------------------------------------
def _timestep(wl: Workload) -> np.ndarray:
    if wl.t_fixed is not None:
        return np.full((wl.batch,), wl.t_fixed, dtype=np.float32)
    return uniform(wl.seed, "t", (wl.batch,))


def block_inputs(wl: Workload, kind: str | None = None, with_weights: bool = True) -> dict:
    """Inputs of one block: activations, ids, t and (optionally) weights.

    kind: "single" or "double" (defaults to the workload's kind).
    """
    kind = kind or wl.kind
    B, D, H = wl.batch, wl.dim, wl.mlp_hidden
    out = {
        "img": normal(wl.seed, "x_img", (B, wl.n_img, D), dtype=wl.dtype),
        "txt": normal(wl.seed, "x_txt", (B, wl.n_txt, D), dtype=wl.dtype),
        "img_ids": image_ids(wl.n_img),
        "txt_ids": text_ids(wl.n_txt),
        "t": _timestep(wl),
    }
    if with_weights:
        if kind == "double":
            specs = double_block_weight_specs(D, H)
        elif kind == "single":
            specs = single_block_weight_specs(D, H)
        else:
            raise ValueError(kind)
        out["weights"] = make_weights(specs, wl.seed, wl.dtype)
    return out


def step_inputs(wl: Workload, with_weights: bool = True) -> dict:
    """Inputs of one denoiser step: packed latent tokens, text condition, ids, t."""
    B = wl.batch
    out = {
        "x": normal(wl.seed, "x_latent", (B, wl.n_img, wl.in_channels), dtype=wl.dtype),
        "ctx": normal(wl.seed, "ctx", (B, wl.n_txt, wl.context_dim), dtype=wl.dtype),
        "img_ids": image_ids(wl.n_img),
        "txt_ids": text_ids(wl.n_txt),
        "t": _timestep(wl),
    }
    if with_weights:
        out["weights"] = make_weights(step_weight_specs(wl), wl.seed, wl.dtype)
    return out


def sample_inputs(wl: Workload, latent_h: int, latent_w: int, with_uncond: bool = False,
                  with_weights: bool = True) -> dict:
    """Inputs of a sampling run: fp32 noise latent [B, in_channels / 4, latent_h, latent_w],
    text condition (and an unconditional one for guidance) in the workload dtype."""
    B = wl.batch
    out = {
        "noise": normal(wl.seed, "noise", (B, wl.in_channels // 4, latent_h, latent_w),
                        dtype="f32"),
        "ctx": normal(wl.seed, "ctx", (B, wl.n_txt, wl.context_dim), dtype=wl.dtype),
    }
    if with_uncond:
        out["ctx_uncond"] = normal(wl.seed, "ctx_uncond", (B, wl.n_txt, wl.context_dim),
                                   dtype=wl.dtype)
    if with_weights:
        out["weights"] = make_weights(step_weight_specs(wl), wl.seed, wl.dtype)
    return out
