"""The C-ABI library: it loads, exports every entry point include/flux.h declares, and its
host-side validation rejects bad arguments before anything is enqueued (CPU only).

The validation tests pass fake device addresses: every one of them must be rejected by the
library's argument checks before any HIP call, so they are only run where no GPU is
present (on a GPU the same paths are exercised with real buffers by the GPU tests)."""
import ctypes
import os
import re

import pytest

from diffusion_transformer_mmdit_amd import flux as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flux.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(flux_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


def test_header_declares_the_three_block_entry_points():
    names = declared_functions()
    for n in ("flux_double_block_fwd", "flux_single_block_fwd", "flux_denoiser_step"):
        assert n in names
    assert len(names) >= 15


def test_library_exports_every_declared_symbol():
    lib = F.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    # and the binding wraps every one of them under the same name
    assert sorted(F.EXPORTED) == declared_functions()
    for n in declared_functions():
        assert callable(getattr(F, n))


def test_version_and_empty_error():
    assert "gfx950" in F.flux_version()
    assert isinstance(F.flux_last_error(), str)


def cfg9b():
    return F.make_cfg(4096, 32, 12288, in_channels=128, context_dim=12288, n_double=8,
                      n_single=24)


def test_workspace_sizes_are_positive_and_reject_bad_configs():
    c = cfg9b()
    for fn in (F.flux_double_block_workspace_size, F.flux_single_block_workspace_size,
               F.flux_denoiser_step_workspace_size):
        n = fn(c, 1, 4096, 512)
        assert 100 << 20 < n < 4 << 30
        assert fn(c, 2, 4096, 512) > n
    bad = cfg9b()
    bad.dim = 4000
    assert F.flux_double_block_workspace_size(bad, 1, 4096, 512) == 0
    assert "dim" in F.flux_last_error()
    bad = cfg9b()
    bad.axes_dim[0] = 30
    assert F.flux_single_block_workspace_size(bad, 1, 64, 16) == 0
    assert "axes_dim" in F.flux_last_error()
    assert F.flux_denoiser_step_workspace_size(c, 0, 64, 16) == 0


FAKE = 1 << 40          # a 256-byte aligned fake device address (never dereferenced)


def fake_double_weights():
    w = F.flux_double_weights()
    w.temb = F.flux_temb_weights(FAKE, FAKE)
    w.mod_img = w.mod_txt = FAKE
    w.img = F.flux_stream_weights(*([FAKE] * 6))
    w.txt = F.flux_stream_weights(*([FAKE] * 6))
    return w


def call_double(cfg, w, ws_bytes=None, **over):
    a = dict(t=FAKE, batch=1, n_img=64, n_txt=16, img=FAKE, txt=FAKE, img_ids=FAKE, txt_ids=FAKE,
             img_out=FAKE, txt_out=FAKE, ws=FAKE)
    a.update(over)
    nb = ws_bytes if ws_bytes is not None else F.flux_double_block_workspace_size(cfg, 1, 64, 16)
    L = F.lib()
    return L.flux_double_block_fwd(ctypes.byref(cfg), ctypes.byref(w), a["t"], a["batch"],
                                   a["n_img"], a["n_txt"], a["img"], a["txt"], a["img_ids"],
                                   a["txt_ids"], a["img_out"], a["txt_out"], a["ws"], nb, None)


@pytest.mark.skipif(not no_gpu(), reason="fake-pointer validation tests run only without a GPU")
def test_double_block_validation_errors():
    c = F.make_cfg(256, 2, 768)
    w = fake_double_weights()
    assert call_double(c, w, img=0) == F.FLUX_EINVAL
    assert call_double(c, w, img=FAKE + 2) == F.FLUX_EALIGN
    assert call_double(c, w, ws=0) == F.FLUX_EWORKSPACE
    assert call_double(c, w, ws=FAKE + 16) == F.FLUX_EWORKSPACE
    assert call_double(c, w, ws_bytes=1024) == F.FLUX_EWORKSPACE
    assert call_double(c, w, batch=0) == F.FLUX_EINVAL
    assert call_double(c, w, n_img=0) == F.FLUX_EINVAL
    w2 = fake_double_weights()
    w2.img.q_norm = 0
    assert call_double(c, w2) == F.FLUX_EINVAL
    assert "img.q_norm" in F.flux_last_error()
    bad = F.make_cfg(256, 2, 768, dtype=7)
    assert call_double(bad, w) == F.FLUX_EDTYPE
    bad = F.make_cfg(256, 2, 768, head_dim=64)
    assert call_double(bad, w) == F.FLUX_ESHAPE
    bad = F.make_cfg(256, 2, 770)
    assert call_double(bad, w) == F.FLUX_ESHAPE
    L = F.lib()
    assert L.flux_double_block_fwd(None, ctypes.byref(w), FAKE, 1, 64, 16, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, 1 << 30, None) == F.FLUX_EINVAL


@pytest.mark.skipif(not no_gpu(), reason="fake-pointer validation tests run only without a GPU")
def test_step_and_op_validation_errors():
    c = F.make_cfg(256, 2, 768, in_channels=128, context_dim=384, n_double=1, n_single=1)
    mw = F.flux_model_weights()
    L = F.lib()
    nb = F.flux_denoiser_step_workspace_size(c, 1, 64, 16)
    # guidance is not supported (no guidance embedder)
    st = L.flux_denoiser_step(ctypes.byref(c), ctypes.byref(mw), FAKE, FAKE, 1, 64, 16, FAKE,
                              FAKE, FAKE, FAKE, FAKE, FAKE, nb, None)
    assert st == F.FLUX_EINVAL and "guidance" in F.flux_last_error()
    # missing weights
    st = L.flux_denoiser_step(ctypes.byref(c), ctypes.byref(mw), FAKE, None, 1, 64, 16, FAKE, FAKE,
                              FAKE, FAKE, FAKE, FAKE, nb, None)
    assert st == F.FLUX_EINVAL
    # linear: k must be a multiple of 8; bad epilogue
    assert L.flux_linear(ctypes.byref(c), 0, 8, 8, 12, FAKE, 12, FAKE, 12, FAKE, 8, 0, None, 0,
                         None, 1, None, 0, None) == F.FLUX_ESHAPE
    assert L.flux_linear(ctypes.byref(c), 9, 8, 8, 16, FAKE, 16, FAKE, 16, FAKE, 8, 0, None, 0,
                         None, 1, None, 0, None) == F.FLUX_EINVAL
    assert L.flux_linear(ctypes.byref(c), 2, 8, 8, 16, FAKE, 16, FAKE, 16, FAKE, 8, 0, None, 0,
                         None, 1, None, 0, None) == F.FLUX_EINVAL
    # split-K workspace smaller than flux_linear_workspace_size()
    assert L.flux_linear(ctypes.byref(c), 0, 8, 8, 16, FAKE, 16, FAKE, 16, FAKE, 8, 0, None, 0,
                         None, 1, FAKE, 1024, None) == F.FLUX_EWORKSPACE
    # attention: leading dimension smaller than dim
    assert L.flux_attention(ctypes.byref(c), 1, 10, FAKE, FAKE, FAKE, 128, FAKE, 256, FAKE,
                            1 << 20, None) == F.FLUX_EALIGN
    # attention: workspace too small
    assert L.flux_attention(ctypes.byref(c), 1, 10, FAKE, FAKE, FAKE, 256, FAKE, 256, FAKE,
                            16, None) == F.FLUX_EWORKSPACE
    # layernorm: bad x dtype
    assert L.flux_layernorm_modulate(ctypes.byref(c), 4, 4, FAKE, 5, FAKE, FAKE, FAKE,
                                     None) == F.FLUX_EDTYPE


def test_sampler_validation_errors():
    L = F.lib()
    c = F.make_cfg(256, 2, 768, in_channels=32, context_dim=48, n_double=1, n_single=1)
    mw = F.flux_model_weights()
    args = lambda n, sig, h, w, nt, unc, ws=FAKE, nb=1 << 30: (
        ctypes.byref(c), ctypes.byref(mw), n, sig, ctypes.c_float(2.0), 1, h, w, nt, FAKE, FAKE,
        unc, FAKE, ws, nb, None)
    assert L.flux_denoise(*args(0, None, 8, 8, 5, None)) == F.FLUX_EINVAL
    assert L.flux_denoise(*args(4, None, 7, 8, 5, None)) == F.FLUX_ESHAPE
    up = (ctypes.c_float * 3)(1.0, 0.5, 0.5)
    assert L.flux_denoise(*args(2, ctypes.cast(up, ctypes.c_void_p), 8, 8, 5, None)) == F.FLUX_EINVAL
    assert "decrease" in F.flux_last_error()
    nan = (ctypes.c_float * 2)(1.0, float("nan"))
    assert L.flux_denoise(*args(1, ctypes.cast(nan, ctypes.c_void_p), 8, 8, 5, None)) == F.FLUX_EINVAL
    # missing weights are reported before anything is enqueued
    assert L.flux_denoise(*args(2, None, 8, 8, 5, None)) == F.FLUX_EINVAL
    # workspace queries: 0 for bad shapes, guided needs more than unguided
    assert F.flux_denoise_workspace_size(c, 1, 7, 8, 5, False) == 0
    assert F.flux_denoise_workspace_size(c, 0, 8, 8, 5, False) == 0
    a = F.flux_denoise_workspace_size(c, 1, 8, 8, 5, False)
    b = F.flux_denoise_workspace_size(c, 1, 8, 8, 5, True)
    assert 0 < a < b
    # binding: wrong number of levels
    with pytest.raises(F.FluxError):
        F.flux_denoise(c, mw, 2, [1.0, 0.0], 1.0, 1, 8, 8, 5, FAKE, FAKE, None, FAKE, FAKE, 1 << 30)
    # packing and ids
    assert L.flux_pack_latents(1, 4, 6, 5, FAKE, FAKE, None) == F.FLUX_ESHAPE
    assert L.flux_pack_latents(1, 4, 6, 6, None, FAKE, None) == F.FLUX_EINVAL
    assert L.flux_unpack_latents(1, 4, 6, 6, FAKE + 4, FAKE, None) == F.FLUX_EALIGN
    assert L.flux_unpack_latents(0, 4, 6, 6, FAKE, FAKE, None) == F.FLUX_EINVAL
    assert L.flux_generation_ids(0, 4, 2, FAKE, FAKE, None) == F.FLUX_EINVAL
    assert L.flux_generation_ids(4, 4, 2, FAKE, None, None) == F.FLUX_EINVAL


def test_fp8_validation_errors():
    L = F.lib()
    c = F.make_cfg(256, 2, 768)
    args = lambda epi, m, n, k, lda, ldw, sa=FAKE, ydt=0: (
        ctypes.byref(c), epi, m, n, k, FAKE, lda, sa, FAKE, ldw, FAKE, FAKE, n, ydt, None, 0,
        None, 1, None, 0, None)
    assert L.flux_linear_fp8(*args(0, 8, 8, 100, 128, 128)) == F.FLUX_ESHAPE     # k % 128
    assert L.flux_linear_fp8(*args(0, 8, 8, 128, 136, 128)) == F.FLUX_EALIGN     # lda % 16
    assert L.flux_linear_fp8(*args(0, 8, 8, 128, 128, 128, sa=None)) == F.FLUX_EINVAL
    assert L.flux_linear_fp8(*args(7, 8, 8, 128, 128, 128)) == F.FLUX_EINVAL     # epilogue
    assert L.flux_linear_fp8(*args(0, 8, 8, 128, 128, 128, ydt=9)) == F.FLUX_EDTYPE
    assert L.flux_linear_fp8(*args(2, 8, 8, 128, 128, 128)) == F.FLUX_EINVAL     # no resid
    assert L.flux_quantize_fp8_rows(0, 8, FAKE, 0, 8, FAKE, 8, FAKE, None) == F.FLUX_EINVAL
    assert L.flux_quantize_fp8_rows(4, 8, FAKE, 5, 8, FAKE, 8, FAKE, None) == F.FLUX_EDTYPE
    assert L.flux_quantize_fp8_rows(4, 8, FAKE, 0, 4, FAKE, 8, FAKE, None) == F.FLUX_ESHAPE


def test_timing_hook_validation():
    L = F.lib()
    n, us = ctypes.c_int(7), ctypes.c_double(1.0)
    # unknown site, capacity out of range, NULL outputs: rejected before any HIP call
    assert L.flux_timing_begin(0, 4) == F.FLUX_EINVAL
    assert L.flux_timing_begin(10, 4) == F.FLUX_EINVAL
    assert L.flux_timing_begin(F.FLUX_SITE_SINGLE_MLP_IN, 0) == F.FLUX_EINVAL
    assert L.flux_timing_begin(F.FLUX_SITE_SINGLE_MLP_IN, (1 << 16) + 1) == F.FLUX_EINVAL
    assert L.flux_timing_end(None, None) == F.FLUX_EINVAL
    # not armed: nothing was timed
    assert L.flux_timing_end(ctypes.byref(n), ctypes.byref(us)) == F.FLUX_OK
    assert (n.value, us.value) == (0, 0.0)


def test_binding_raises_when_library_missing(tmp_path, monkeypatch):
    monkeypatch.setattr(F, "_lib", None)
    with pytest.raises(F.FluxError):
        F.lib(str(tmp_path / "nope.so"))
    monkeypatch.setattr(F, "_lib", None)


def test_weight_structures_keep_their_tensors_alive():
    """The C structures hold raw pointers: the binding's builders keep the tensors they point
    to alive for as long as the structure exists (a temporary dict must not leave them
    dangling)."""
    import gc
    import weakref
    import numpy as np
    import torch
    import flux_synth as fs
    wl = fs.workload("tiny_single_f32", kind="step", in_channels=32, context_dim=48, n_double=1,
                     n_single=1, n_img=16, n_txt=5)
    inp = fs.step_inputs(wl)

    def fresh():
        return {k: torch.from_numpy(v.astype(np.float32)) for k, v in inp["weights"].items()}

    w = fresh()
    probe = weakref.ref(w["proj_out"])
    mw = F.ModelWeights(w, wl.n_double, wl.n_single)
    del w
    gc.collect()
    assert probe() is not None, "ModelWeights let its tensors be freed"
    del mw
    gc.collect()
    assert probe() is None
    for kind, build in (("double", F.double_weights), ("single", F.single_weights)):
        bw = fs.block_inputs(fs.workload("tiny_single_f32", kind=kind), kind=kind)["weights"]
        w = {k: torch.from_numpy(v.astype(np.float32)) for k, v in bw.items()}
        probe = weakref.ref(next(iter(w.values())))
        s = build(w)
        del w
        gc.collect()
        assert probe() is not None, f"{kind}_weights let its tensors be freed"
        del s


def test_status_codes_match_the_header():
    """The binding's status constants are the header's flux_status values (0 = OK, errors
    negative)."""
    src = open(HEADER).read()
    vals = dict((n, int(v)) for n, v in re.findall(r"(FLUX_E?[A-Z]+)\s*=\s*(-?\d+)\s*,?\s*/\*", src)
                if n.startswith(("FLUX_E", "FLUX_OK")))
    vals["FLUX_OK"] = int(re.search(r"FLUX_OK\s*=\s*(-?\d+)", src).group(1))
    for name in ("FLUX_OK", "FLUX_EINVAL", "FLUX_ESHAPE", "FLUX_EDTYPE", "FLUX_EALIGN",
                 "FLUX_EWORKSPACE", "FLUX_EHIP"):
        assert getattr(F, name) == vals[name], name
        assert name == "FLUX_OK" or vals[name] < 0


def test_precision_constants_match_the_header():
    src = open(HEADER).read()
    for name in ("FLUX_BF16", "FLUX_F32", "FLUX_F16", "FLUX_PRECISION_BF16",
                 "FLUX_PRECISION_SPLIT", "FLUX_PRECISION_F16"):
        m = re.search(name + r"\s*=\s*(\d+)", src)
        assert m and getattr(F, name) == int(m.group(1)), name


def test_binary16_precision_workspace_and_rejections():
    """FLUX_PRECISION_F16 stores 2-byte operands like bf16 (same workspaces); it needs the bf16
    workload, and an unknown precision is refused."""
    c = cfg9b()
    c16 = cfg9b()
    c16.precision = F.FLUX_PRECISION_F16
    for fn in (F.flux_double_block_workspace_size, F.flux_single_block_workspace_size,
               F.flux_denoiser_step_workspace_size):
        assert fn(c16, 1, 4096, 512) == fn(c, 1, 4096, 512) > 0
    bad = F.make_cfg(256, 2, 768, dtype=F.FLUX_F32, precision=F.FLUX_PRECISION_F16)
    assert F.flux_single_block_workspace_size(bad, 1, 64, 16) == 0
    assert "FLUX_PRECISION_F16" in F.flux_last_error()
    bad = F.make_cfg(256, 2, 768, precision=3)
    assert F.flux_double_block_workspace_size(bad, 1, 64, 16) == 0
    assert "precision" in F.flux_last_error()


def test_block_linear_names_are_the_block_weights():
    """The weights FLUX_PRECISION_F16 takes in binary16 are exactly the block linears of the
    step's weight set: every double / single block matrix except the modulation and the norm
    scales, and none of the embedders, modulation or head."""
    import flux_synth as fs
    wl = fs.workload("klein9b_step_1024", n_double=2, n_single=2)
    names = set(fs.step_weight_specs(wl))
    got = {n for n in names if F.is_block_linear(n)}
    want = {f"double.{i}.{s}.{m}" for i in range(2) for s in ("img", "txt")
            for m in ("qkv", "out", "mlp_in", "mlp_out")}
    want |= {f"single.{i}.{m}" for i in range(2) for m in ("linear1", "linear2")}
    assert got == want
