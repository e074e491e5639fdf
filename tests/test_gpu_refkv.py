"""Reference-image K/V cache through the C ABI: the filled cache (every block's reference K
after RMSNorm + RoPE and V) and the cached step against the oracle's literal extract step
over [txt, ref, img], sampling with references against the oracle's loop, and at the
Klein-9B 1024^2 size with one 1024^2 reference the properties that hold at any size
(filling the cache once or before every step gives the same latent, bit for bit;
repeated runs agree)."""
import numpy as np
import pytest

import flux_synth as fs
from oracle import flux_oracle as O
from tests import flux_gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_mmdit_amd import flux as F
    F.lib()


def F_():
    from diffusion_transformer_mmdit_amd import flux as F
    return F


def cache_views(wl, cache, B, Nr):
    """(k [B, Nr, D], vt [B, D, Nr]) device views of every block's slot."""
    D, es = wl.dim, 2 if wl.dtype == "bf16" else 4
    pitch = (Nr + 63) // 64 * 64
    a256 = lambda b: (b + 255) // 256 * 256
    qk_b, vt_b = a256(B * Nr * 2 * D * es), a256(B * D * pitch * es)
    dt = G.dt(wl.dtype)
    out = []
    for l in range(wl.n_double + wl.n_single):
        base = l * (qk_b + vt_b)
        qk = cache[base:base + B * Nr * 2 * D * es].view(dt).view(B, Nr, 2 * D)
        vt = cache[base + qk_b:base + qk_b + B * D * pitch * es].view(dt).view(B, D, pitch)
        out.append((qk[:, :, D:], vt[:, :, :Nr]))
    return out


def run_fill_and_cached(wl, inp, ref, rid, w_dev=None, precision=0):
    F, t = F_(), G.torch()
    cfg = G.cfg_for(wl, precision)
    w_dev = G.for_precision(w_dev or G.upload_weights(inp["weights"], wl.dtype), precision)
    mw = F.ModelWeights(w_dev, wl.n_double, wl.n_single)
    B, Nr = wl.batch, ref.shape[1]
    cb = F.flux_ref_cache_size(cfg, B, Nr)
    cache = t.empty(cb, dtype=t.uint8, device="cuda")
    fb = F.flux_ref_cache_fill_workspace_size(cfg, B, Nr)
    fws = G.workspace(fb)
    F.flux_ref_cache_fill(cfg, mw, B, Nr, G.dev(ref, wl.dtype), G.dev(rid), cache, cb, fws, fb,
                          G.stream())
    out = t.empty((B, wl.n_img, wl.in_channels), device="cuda")
    nb = F.flux_denoiser_step_workspace_size(cfg, B, wl.n_img, wl.n_txt)
    ws = G.workspace(nb)
    F.flux_denoiser_step_cached(cfg, mw, G.dev(inp["t"]), B, wl.n_img, wl.n_txt, Nr,
                                G.dev(inp["x"], wl.dtype), G.dev(inp["ctx"], wl.dtype),
                                G.dev(inp["img_ids"]), G.dev(inp["txt_ids"]), cache, cb, out, ws,
                                nb, G.stream())
    t.cuda.synchronize()
    return out, cache


def tiny_fp32(batch=1):
    return fs.workload("tiny_single_f32", kind="step", in_channels=32, context_dim=48,
                       n_double=1, n_single=2, n_img=16, n_txt=5, batch=batch)


def small_bf16(batch=1):
    return fs.workload("tiny_single_f32", dtype="bf16", kind="step", dim=512, heads=4,
                       mlp_hidden=1536, in_channels=128, context_dim=64, n_double=2, n_single=2,
                       n_img=64, n_txt=24, t_fixed=None, batch=batch, seed=1012)


def check_against_oracle(wl, R, gh, gw, what, precision=0):
    inp = fs.step_inputs(wl)
    Nr = R * gh * gw
    ref = fs.normal(wl.seed, "ref_tokens", (wl.batch, Nr, wl.in_channels), dtype=wl.dtype)
    rid = O.reference_ids(R, gh, gw)
    print(f"[refkv] {what}: batch {wl.batch}, {Nr} reference tokens", flush=True)
    out, cache = run_fill_and_cached(wl, inp, ref, rid, precision=precision)
    ref_out, ref_cache = O.step_extract(inp["x"], ref, inp["ctx"], inp["t"], inp["weights"],
                                        inp["img_ids"], rid, inp["txt_ids"], wl.n_double,
                                        wl.n_single)
    G.assert_close(G.host(out), ref_out, wl.dtype, f"{what}: cached step vs oracle extract step")
    for l, ((k, vt), (rk, rv)) in enumerate(zip(cache_views(wl, cache, wl.batch, Nr), ref_cache)):
        B = wl.batch
        rk = rk.reshape(B, Nr, -1)
        rv = rv.reshape(B, Nr, -1).transpose(0, 2, 1)
        if wl.dtype == "bf16":
            # Element-wise bound.  K is stored twice in bf16 (after the projection and after
            # RMSNorm + RoPE: 2^-8 of |k|), V once.  Both also carry the bf16 LayerNorm
            # output's rounding through the projection (a sum over the row, so its size is
            # relative to the row's RMS, not to the element: 2^-9/sqrt(3) = 1.1e-3 of the RMS
            # per element) and the reference rows' own pipeline error from earlier blocks.
            # Together that is a standard deviation of about 3e-3 of the RMS (the oracle's
            # bf16 storage mode: nL2 2.9e-3 on these inputs), and the largest of a slot's
            # up to ~70k values lies about 4.5 deviations out: hence 5 x 3e-3 of the RMS.
            G.assert_op_close(G.host(k), rk, f"{what}: block {l} cached K", rtol=2.0 ** -8,
                              atol_rms=1.5e-2)
            G.assert_op_close(G.host(vt), rv, f"{what}: block {l} cached V", rtol=2.0 ** -8,
                              atol_rms=1.5e-2)
        else:
            G.assert_close(G.host(k), rk, "f32", f"{what}: block {l} cached K")
            G.assert_close(G.host(vt), rv, "f32", f"{what}: block {l} cached V")


@pytest.mark.parametrize("batch", [1, 2])
def test_tiny_fp32_cache_and_cached_step(batch):
    check_against_oracle(tiny_fp32(batch), 1, 3, 4, "tiny fp32")


@pytest.mark.parametrize("batch", [1, 2])
def test_small_bf16_cache_and_cached_step(batch):
    # two 5 x 7 references: 70 reference tokens, a partial second extra key tile
    check_against_oracle(small_bf16(batch), 2, 5, 7, "small bf16")


@pytest.mark.parametrize("precision", [1, 2])
def test_klein9b_width_cache_and_cached_step_precise_modes(precision):
    """The reference cache and the cached step at the Klein-9B width (D 4096, 32 heads,
    MLP 12288; 2 + 2 blocks): one 6 x 8 reference (48 tokens, a partial extra key tile).  In
    FLUX_PRECISION_SPLIT: with bf16 LayerNorm outputs the reference rows' own pipeline error
    grows with the width (the linears' gain 0.02 sqrt(D) > 1), and at D 4096 the cached K of
    the third block exceeded the element-wise bound above by 2e-3 while the cached step met
    3e-2 / 1e-2 (2.1e-2 / 4.1e-3).  Also in FLUX_PRECISION_F16 (binary16 LayerNorm outputs)."""
    from tests.test_gpu_sampler import klein9b_width
    check_against_oracle(klein9b_width(seed=1014), 1, 6, 8, f"Klein-9B width (p{precision})",
                         precision=precision)


def run_denoise_refs(wl, inp, refs, n_steps, use_cache, sigmas=None, w_dev=None, lat=None):
    F, t = F_(), G.torch()
    cfg = G.cfg_for(wl)
    w_dev = w_dev or G.upload_weights(inp["weights"], wl.dtype)
    mw = F.ModelWeights(w_dev, wl.n_double, wl.n_single)
    B, C, H, W = lat or inp["noise"].shape
    R, Hr, Wr = refs.shape[1], refs.shape[3], refs.shape[4]
    noise = inp["noise_dev"] if "noise_dev" in inp else G.dev(inp["noise"], "f32")
    ctx = inp["ctx_dev"] if "ctx_dev" in inp else G.dev(inp["ctx"], wl.dtype)
    rd = refs if not isinstance(refs, np.ndarray) else G.dev(refs, "f32")
    out = t.empty((B, C, H, W), device="cuda")
    nb = F.flux_denoise_refs_workspace_size(cfg, B, H, W, wl.n_txt, R, Hr, Wr)
    ws = G.workspace(nb)
    F.flux_denoise_refs(cfg, mw, n_steps, sigmas, B, H, W, wl.n_txt, noise, ctx, R, Hr, Wr, rd,
                        use_cache, out, ws, nb, G.stream())
    t.cuda.synchronize()
    return out


def test_small_bf16_sampling_with_references():
    wl = small_bf16()
    inp = fs.sample_inputs(wl, 12, 16)
    refs = fs.normal(wl.seed, "refs", (1, 2, 32, 10, 14), dtype="f32")
    w_dev = G.upload_weights(inp["weights"], wl.dtype)
    print("[refkv] small bf16 sampling, 3 steps, 2 references", flush=True)
    a = run_denoise_refs(wl, inp, refs, 3, True, w_dev=w_dev)
    b = run_denoise_refs(wl, inp, refs, 3, False, w_dev=w_dev)
    assert G.torch().equal(a, b)
    ref = O.denoise_with_refs(inp["noise"], refs, inp["ctx"], inp["weights"], O.uniform_sigmas(3),
                              2, 2, model_input=O.bf16_storage)
    G.assert_close(G.host(a), ref, "bf16", "small bf16 sampling with references")


def test_klein9b_sampling_with_a_reference_cache_equals_refill():
    from tests.test_gpu_sampler import klein9b_device_weights
    wl = fs.workload("klein9b_step_1024")
    t = G.torch()
    g = t.Generator(device="cuda")
    g.manual_seed(wl.seed + 2)
    inp = {"noise_dev": t.randn((1, 32, 128, 128), generator=g, device="cuda"),
           "ctx_dev": t.randn((1, wl.n_txt, wl.context_dim), generator=g,
                              device="cuda").to(t.bfloat16)}
    refs = t.randn((1, 1, 32, 128, 128), generator=g, device="cuda")
    w = klein9b_device_weights(wl, zero_proj_out=False)
    print("[refkv] Klein-9B 1024^2 + one 1024^2 reference, 4 steps, cached vs refilled",
          flush=True)
    a = run_denoise_refs(wl, inp, refs, 4, True, w_dev=w, lat=(1, 32, 128, 128))
    b = run_denoise_refs(wl, inp, refs, 4, False, w_dev=w, lat=(1, 32, 128, 128))
    c = run_denoise_refs(wl, inp, refs, 4, True, w_dev=w, lat=(1, 32, 128, 128))
    assert t.isfinite(a).all()
    assert t.equal(a, b) and t.equal(a, c)
    del w
