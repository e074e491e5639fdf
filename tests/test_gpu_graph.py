"""HIP graph capture through the C ABI: a double block, a single block, a denoiser step and a
guided two-step sampling loop are captured with torch.cuda.graph (the library enqueues only
kernels and device-to-device copies on the caller's stream, and allocates nothing) and
replayed several times, with unrelated work and synchronisations between the replays and the
outputs poisoned before each; every replay must equal the eager result bit for bit."""
import pytest

import flux_synth as fs
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


def small_bf16(**kw):
    base = dict(dtype="bf16", dim=512, heads=4, mlp_hidden=1536, in_channels=128,
                context_dim=64, n_double=2, n_single=2, n_img=64, n_txt=24, t_fixed=None,
                seed=3100)
    base.update(kw)
    return fs.workload("tiny_single_f32", **base)


def check_replays(call, outs, what, replays=3):
    """Eager call, capture, then replays against the eager outputs."""
    t = G.torch()
    call()  # eager (also the first launch of every kernel instance, outside the capture)
    t.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        call()
    for r in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        t.cuda.synchronize()
        print(f"[graph] {what}: replay {r}", flush=True)
        g.replay()
        # unrelated eager work on the same device between replays
        x = t.randn((256, 256), device="cuda")
        (x @ x).sum().item()
        t.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert t.equal(o, e), f"{what}: replay {r} differs from the eager result"
    del g


@pytest.mark.parametrize("kind", ["double", "single"])
def test_block_graph_replays(kind):
    F, t = F_(), G.torch()
    wl = small_bf16(kind=kind, batch=1)
    inp = fs.block_inputs(wl, kind=kind)
    cfg = G.cfg_for(wl)
    w_dev = G.upload_weights(inp["weights"], wl.dtype)
    img, txt = G.dev(inp["img"], wl.dtype), G.dev(inp["txt"], wl.dtype)
    tt, img_ids, txt_ids = G.dev(inp["t"]), G.dev(inp["img_ids"]), G.dev(inp["txt_ids"])
    img_o, txt_o = t.empty_like(img), t.empty_like(txt)
    if kind == "double":
        nb = F.flux_double_block_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
        bw, fwd = F.double_weights(w_dev), F.flux_double_block_fwd
    else:
        nb = F.flux_single_block_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
        bw, fwd = F.single_weights(w_dev), F.flux_single_block_fwd
    ws = G.workspace(nb)
    check_replays(lambda: fwd(cfg, bw, tt, wl.batch, wl.n_img, wl.n_txt, img, txt, img_ids,
                              txt_ids, img_o, txt_o, ws, nb, G.stream()),
                  [img_o, txt_o], f"bf16 {kind} block")


def test_step_graph_replays():
    F, t = F_(), G.torch()
    wl = small_bf16(kind="step", batch=1)
    inp = fs.step_inputs(wl)
    cfg = G.cfg_for(wl)
    w_dev = G.upload_weights(inp["weights"], wl.dtype)
    mw = F.ModelWeights(w_dev, wl.n_double, wl.n_single)
    x, ctx = G.dev(inp["x"], wl.dtype), G.dev(inp["ctx"], wl.dtype)
    tt, img_ids, txt_ids = G.dev(inp["t"]), G.dev(inp["img_ids"]), G.dev(inp["txt_ids"])
    out = t.empty((wl.batch, wl.n_img, wl.in_channels), dtype=t.float32, device="cuda")
    nb = F.flux_denoiser_step_workspace_size(cfg, wl.batch, wl.n_img, wl.n_txt)
    ws = G.workspace(nb)
    check_replays(lambda: F.flux_denoiser_step(cfg, mw, tt, None, wl.batch, wl.n_img, wl.n_txt,
                                               x, ctx, img_ids, txt_ids, out, ws, nb,
                                               G.stream()),
                  [out], "bf16 denoiser step")


def test_guided_sampling_graph_replays():
    # the guided loop copies both conditions into one batch-2 context (device copies)
    F, t = F_(), G.torch()
    wl = small_bf16(kind="step", batch=1, n_img=60)
    inp = fs.sample_inputs(wl, 12, 20, with_uncond=True)
    cfg = G.cfg_for(wl)
    w_dev = G.upload_weights(inp["weights"], wl.dtype)
    mw = F.ModelWeights(w_dev, wl.n_double, wl.n_single)
    noise = G.dev(inp["noise"], "f32")
    ctx, unc = G.dev(inp["ctx"], wl.dtype), G.dev(inp["ctx_uncond"], wl.dtype)
    B, C, H, W = inp["noise"].shape
    out = t.empty((B, C, H, W), device="cuda")
    nb = F.flux_denoise_workspace_size(cfg, B, H, W, wl.n_txt, True)
    ws = G.workspace(nb)
    check_replays(lambda: F.flux_denoise(cfg, mw, 2, None, 3.5, B, H, W, wl.n_txt, noise, ctx,
                                         unc, out, ws, nb, G.stream()),
                  [out], "bf16 guided 2-step sampling")
