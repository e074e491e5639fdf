"""Helpers for the GPU parity tests: upload seeded inputs, call the C ABI through the
binding, compare with the oracle.  Imported only by tests marked `gpu` (and smoke)."""
from __future__ import annotations

import numpy as np

import flux_synth as fs

# Parity bar for bf16 storage with fp32 accumulation: max-abs error and normalised L2
# error of the output against the fp64 oracle.
MAX_ABS = 3e-2
NL2 = 1e-2
# fp32 workloads (tiny configuration): fp32 storage and arithmetic everywhere; the
# oracle sees the same fp32 inputs, so only fp32 rounding of ~1e3-term sums remains.
MAX_ABS_F32 = 1e-4
NL2_F32 = 1e-5


def torch():
    import torch as _t
    return _t


def dt(dtype: str):
    t = torch()
    return {"bf16": t.bfloat16, "f16": t.float16}.get(dtype, t.float32)


def dev(a, dtype: str | None = None):
    """numpy -> device tensor; float arrays become bf16 / fp32 per `dtype`."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a)).to("cuda")
    if dtype is not None:
        x = x.to(dt(dtype))
    return x


def upload_weights(w: dict, dtype: str) -> dict:
    """Linear weights in `dtype`; QK-norm scales always fp32."""
    out = {}
    for k, v in w.items():
        out[k] = dev(v, "f32" if k.endswith("_norm") else dtype)
    return out


def for_precision(w_dev: dict, precision: int) -> dict:
    """The device weights a precision mode takes: under FLUX_PRECISION_F16 the block
    linears converted to binary16 (exact for the bf16 values in binary16's normal range),
    the rest unchanged."""
    from diffusion_transformer_mmdit_amd import flux as F
    if precision != F.FLUX_PRECISION_F16:
        return w_dev
    t = torch()
    return {k: (v.to(t.float16) if F.is_block_linear(k) else v) for k, v in w_dev.items()}


def host(x) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def workspace(nbytes: int):
    t = torch()
    return t.empty(max(int(nbytes), 256), dtype=t.uint8, device="cuda")


def cfg_for(wl: fs.Workload, precision: int = 0):
    from diffusion_transformer_mmdit_amd import flux as F
    return F.make_cfg(wl.dim, wl.heads, wl.mlp_hidden,
                      dtype=F.FLUX_BF16 if wl.dtype == "bf16" else F.FLUX_F32,
                      in_channels=wl.in_channels, context_dim=wl.context_dim,
                      n_double=wl.n_double, n_single=wl.n_single, precision=precision)


def errors(got, ref) -> tuple[float, float]:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = got - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(ref))
    nl2 = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    return max_abs, nl2


def assert_close(got, ref, dtype: str = "bf16", what: str = "", max_abs=None, nl2=None):
    ma_bar = max_abs if max_abs is not None else (MAX_ABS if dtype == "bf16" else MAX_ABS_F32)
    nl_bar = nl2 if nl2 is not None else (NL2 if dtype == "bf16" else NL2_F32)
    ma, nl = errors(got, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} (bar {ma_bar:.0e}) nL2={nl:.3e} (bar {nl_bar:.0e})",
          flush=True)
    assert np.isfinite(np.asarray(got)).all(), f"{what}: non-finite output"
    assert ma <= ma_bar, f"{what}: max-abs {ma:.3e} > {ma_bar:.0e}"
    assert nl <= nl_bar, f"{what}: nL2 {nl:.3e} > {nl_bar:.0e}"
    return ma, nl


# Operation-level parity for bf16-STORED intermediates (q/k/v, LN output, SwiGLU output,
# ...): these can be much larger than 1 in magnitude, and bf16 storage alone moves a value
# by up to half an ulp, i.e. 2^-8 of its magnitude.  Each element must lie within that
# rounding bound of the exact value plus 2e-3 of the output RMS (fp32 accumulation and
# near-zero values), and the normalised L2 error must meet the block bar (1e-2).
def assert_op_close(got, ref, what: str = "", rtol: float = 2.0 ** -8, atol_rms: float = 2e-3,
                    nl2: float = NL2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rtol * np.abs(ref) + atol_rms * rms
    excess = np.abs(got - ref) - bound
    ma, nl = errors(got, ref)
    worst = float(excess.max()) if excess.size else 0.0
    print(f"[parity] {what}: max_abs={ma:.3e} nL2={nl:.3e} (bar {nl2:.0e}); worst element "
          f"excess over {rtol:.2e}|ref| + {atol_rms:.0e} rms = {worst:.2e}", flush=True)
    assert worst <= 0, f"{what}: element error exceeds the bf16 rounding bound by {worst:.3e}"
    assert nl <= nl2, f"{what}: nL2 {nl:.3e} > {nl2:.0e}"
    return ma, nl


def stream():
    return torch().cuda.current_stream()


# ------------------------------------------------------------------------------------
# Block runners through the C ABI
# ------------------------------------------------------------------------------------
def run_double_block(wl: fs.Workload, inp: dict, w_dev: dict | None = None, precision: int = 0):
    from diffusion_transformer_mmdit_amd import flux as F
    t = torch()
    cfg = cfg_for(wl, precision)
    w_dev = for_precision(w_dev or upload_weights(inp["weights"], wl.dtype), precision)
    img, txt = dev(inp["img"], wl.dtype), dev(inp["txt"], wl.dtype)
    img_out, txt_out = t.empty_like(img), t.empty_like(txt)
    nbytes = F.flux_double_block_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
    ws = workspace(nbytes)
    F.flux_double_block_fwd(cfg, F.double_weights(w_dev), dev(inp["t"]), wl.batch, wl.n_img,
                            wl.n_txt, img, txt, dev(inp["img_ids"]), dev(inp["txt_ids"]), img_out,
                            txt_out, ws, nbytes, stream())
    t.cuda.synchronize()
    return img_out, txt_out


def run_single_block(wl: fs.Workload, inp: dict, w_dev: dict | None = None, precision: int = 0):
    from diffusion_transformer_mmdit_amd import flux as F
    t = torch()
    cfg = cfg_for(wl, precision)
    w_dev = for_precision(w_dev or upload_weights(inp["weights"], wl.dtype), precision)
    img, txt = dev(inp["img"], wl.dtype), dev(inp["txt"], wl.dtype)
    img_out, txt_out = t.empty_like(img), t.empty_like(txt)
    nbytes = F.flux_single_block_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
    ws = workspace(nbytes)
    F.flux_single_block_fwd(cfg, F.single_weights(w_dev), dev(inp["t"]), wl.batch, wl.n_img,
                            wl.n_txt, img, txt, dev(inp["img_ids"]), dev(inp["txt_ids"]), img_out,
                            txt_out, ws, nbytes, stream())
    t.cuda.synchronize()
    return img_out, txt_out


def run_step(wl: fs.Workload, inp: dict, w_dev: dict | None = None, precision: int = 0):
    from diffusion_transformer_mmdit_amd import flux as F
    t = torch()
    cfg = cfg_for(wl, precision)
    w_dev = for_precision(w_dev or upload_weights(inp["weights"], wl.dtype), precision)
    mw = F.ModelWeights(w_dev, wl.n_double, wl.n_single)
    out = t.empty((wl.batch, wl.n_img, wl.in_channels), dtype=t.float32, device="cuda")
    nbytes = F.flux_denoiser_step_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
    ws = workspace(nbytes)
    F.flux_denoiser_step(cfg, mw, dev(inp["t"]), None, wl.batch, wl.n_img, wl.n_txt,
                         dev(inp["x"], wl.dtype), dev(inp["ctx"], wl.dtype), dev(inp["img_ids"]),
                         dev(inp["txt_ids"]), out, ws, nbytes, stream())
    t.cuda.synchronize()
    return out
