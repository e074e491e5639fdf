"""Block-level parity with the fp64 oracle through the C ABI (double-stream block,
single-stream block), identities that must hold bitwise, and determinism."""
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


def oracle_block(kind, inp):
    fn = O.double_block if kind == "double" else O.single_block
    return fn(inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"], inp["txt_ids"])


def run(kind, wl, inp, precision=0):
    return (G.run_double_block if kind == "double" else G.run_single_block)(wl, inp,
                                                                              precision=precision)


def check_block(kind, wl, inp, what, precision=0):
    img, txt = run(kind, wl, inp, precision)
    ref_img, ref_txt = oracle_block(kind, inp)
    G.assert_close(G.host(img), ref_img, wl.dtype, f"{what} img")
    if wl.n_txt:
        G.assert_close(G.host(txt), ref_txt, wl.dtype, f"{what} txt")
    # the block's own contribution (output - input) must match too, not just the residual
    d_got = G.host(img) - inp["img"].astype(np.float64)
    d_ref = ref_img - inp["img"].astype(np.float64)
    ma, nl = G.errors(d_got, d_ref)
    rel_bar = 2e-2 if wl.dtype == "bf16" else 1e-4
    # the output is stored in the workload dtype, so the update inherits the output's
    # rounding (half an ulp: 2^-9 of |x| for bf16, 2^-24 for fp32) relative to its own norm
    unit = 2.0 ** -9 if wl.dtype == "bf16" else 2.0 ** -24
    floor = np.linalg.norm(inp["img"].astype(np.float64)) * unit / max(np.linalg.norm(d_ref), 1e-30)
    print(f"[parity] {what} img update: nL2={nl:.3e} (bar {rel_bar:.0e} + 2 x rounding floor "
          f"{floor:.1e})", flush=True)
    assert nl <= rel_bar + 2 * floor, (nl, floor)


# ------------------------------------------------------------------------------------
# tiny configurations (fp32: the tiny single-stream workload; bf16 variants)
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["single", "double"])
def test_tiny_fp32_block(kind):
    wl = fs.workload("tiny_single_f32")
    inp = fs.block_inputs(wl, kind=kind)
    check_block(kind, wl, inp, f"tiny fp32 {kind}")


@pytest.mark.parametrize("precision", [0, 1, 2])
@pytest.mark.parametrize("kind", ["single", "double"])
# (1, 64): a one-token text stream; (300, 289): both streams' products in one launch with
# several tiles each and ragged last tiles in both
@pytest.mark.parametrize("n_txt,n_img,batch", [(16, 64, 1), (5, 36, 2), (0, 49, 1), (130, 196, 1),
                                               (1, 64, 1), (300, 289, 1)])
def test_small_bf16_block(kind, n_txt, n_img, batch, precision):
    wl = fs.workload("tiny_single_f32", dtype="bf16", n_txt=n_txt, n_img=n_img, batch=batch,
                     t_fixed=None, seed=2000 + n_img)
    inp = fs.block_inputs(wl, kind=kind)
    check_block(kind, wl, inp, f"bf16 {kind} Nt={n_txt} Ni={n_img} B={batch} p{precision}",
                precision)


def test_tiny_fp32_single_batch_and_text_free():
    wl = fs.workload("tiny_single_f32", n_txt=0, batch=2, t_fixed=None)
    inp = fs.block_inputs(wl, kind="single")
    check_block("single", wl, inp, "tiny fp32 single B=2 Nt=0")


# ------------------------------------------------------------------------------------
# workload shapes
# ------------------------------------------------------------------------------------
def test_klein4b_single_block_512():
    wl = fs.workload("klein4b_single_512")
    inp = fs.block_inputs(wl)
    check_block("single", wl, inp, "Klein-4B single 512^2")


def test_klein9b_double_block_1024():
    wl = fs.workload("klein9b_double_1024")
    inp = fs.block_inputs(wl)
    check_block("double", wl, inp, "Klein-9B double 1024^2")


@pytest.mark.parametrize("precision", [1, 2])
@pytest.mark.parametrize("kind,name", [("single", "klein4b_single_512"),
                                       ("double", "klein9b_double_1024")])
def test_precise_modes_block_full_shape(kind, name, precision):
    """FLUX_PRECISION_SPLIT (LayerNorm and SwiGLU outputs as bf16 hi + lo pairs: the hi / lo
    products take other K extents, 2D, 2H, D + 2H, and the SwiGLU epilogue writes two planes)
    and FLUX_PRECISION_F16 (binary16 operands of every block linear) at the Klein-4B single /
    Klein-9B double block shapes."""
    wl = fs.workload(name)
    inp = fs.block_inputs(wl, kind=kind)
    check_block(kind, wl, inp, f"{name} {kind} (precision {precision})", precision=precision)


def test_klein9b_single_block_1024():
    """The Klein-9B single-stream block at its real shape (D 4096, 32 heads, MLP 12288,
    512 + 4096 tokens): the whole output element by element against the oracle.  The step's
    24 single blocks take about three quarters of its time; this runs the dominant GEMM
    (linear1's MLP part, 4608 x 24576 x 4096, 1728 tiles over 256 CUs: a partial last
    round) with its real operands."""
    wl = fs.workload("klein9b_double_1024", kind="single", seed=1009)
    inp = fs.block_inputs(wl, kind="single")
    check_block("single", wl, inp, "Klein-9B single 1024^2")


def _sample(n, k, seed):
    if n == 0:
        return np.array([], dtype=np.int64)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(n), size=min(k, n), replace=False)
    return np.unique(np.concatenate([[0, n - 1], mid])).astype(np.int64)


@pytest.mark.parametrize("precision", [0, 2])
@pytest.mark.parametrize("kind", ["double", "single"])
def test_dev_pair_block_2048_sampled_rows(kind, precision):
    """FLUX.2-dev shapes at 2048² (D 6144, 48 heads, 512 + 16384 tokens): the whole block
    on the GPU, the oracle at sampled output rows (keys and values from every token); bf16
    operands and binary16 block-linear operands."""
    wl = fs.workload("dev_pair_2048")
    inp = fs.block_inputs(wl, kind=kind)
    img, txt = run(kind, wl, inp, precision)
    ri, rt = _sample(wl.n_img, 40, 11), _sample(wl.n_txt, 10, 12)
    fn = O.double_block_rows if kind == "double" else O.single_block_rows
    ref_img, ref_txt = fn(inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"],
                          inp["txt_ids"], ri, rt)
    got_img, got_txt = G.host(img)[:, ri], G.host(txt)[:, rt]
    G.assert_close(got_img, ref_img, wl.dtype, f"dev {kind} 2048^2 img rows p{precision}")
    G.assert_close(got_txt, ref_txt, wl.dtype, f"dev {kind} 2048^2 txt rows p{precision}")
    # the block's own update at those rows, against the rounding floor of the output
    d_got = got_img - inp["img"][:, ri].astype(np.float64)
    d_ref = ref_img - inp["img"][:, ri].astype(np.float64)
    _, nl = G.errors(d_got, d_ref)
    floor = np.linalg.norm(inp["img"][:, ri].astype(np.float64)) * 2.0 ** -9 / np.linalg.norm(d_ref)
    print(f"[parity] dev {kind} img update at sampled rows p{precision}: nL2={nl:.3e} "
          f"(floor {floor:.1e})",
          flush=True)
    assert nl <= 2e-2 + 2 * floor, (nl, floor)


# ------------------------------------------------------------------------------------
# identities and determinism
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("kind,dtype", [("single", "bf16"), ("double", "bf16"), ("double", "f32")])
def test_zero_gate_block_is_bitwise_identity(kind, dtype):
    wl = fs.workload("tiny_single_f32", dtype=dtype, n_txt=16, n_img=64)
    inp = fs.block_inputs(wl, kind=kind)
    w = dict(inp["weights"])
    D = wl.dim
    names = ["mod"] if kind == "single" else ["mod_img", "mod_txt"]
    chunks = [2] if kind == "single" else [2, 5]
    for nm in names:
        m = w[nm].copy()
        for c in chunks:
            m[c * D:(c + 1) * D] = 0
        w[nm] = m
    inp = dict(inp, weights=w)
    img, txt = run(kind, wl, inp)
    assert np.array_equal(G.host(img), inp["img"].astype(np.float64))
    assert np.array_equal(G.host(txt), inp["txt"].astype(np.float64))


@pytest.mark.parametrize("precision", [0, 2])
@pytest.mark.parametrize("kind", ["single", "double"])
def test_block_is_deterministic(kind, precision):
    wl = fs.workload("tiny_single_f32", dtype="bf16", n_txt=64, n_img=256, t_fixed=None,
                     dim=512, heads=4, mlp_hidden=1536)
    inp = fs.block_inputs(wl, kind=kind)
    wd = G.upload_weights(inp["weights"], "bf16")
    fn = G.run_double_block if kind == "double" else G.run_single_block
    a = fn(wl, inp, wd, precision=precision)
    b = fn(wl, inp, wd, precision=precision)
    assert G.torch().equal(a[0], b[0]) and G.torch().equal(a[1], b[1])


def test_timing_hook_times_only_the_armed_site():
    """The measurement hook brackets exactly the armed site's launches (one per block of its
    kind, none from the other kind) and refuses more launches than it was armed for."""
    from diffusion_transformer_mmdit_amd import flux as F
    wl = fs.workload("tiny_single_f32", dtype="bf16", n_txt=64, n_img=256, t_fixed=None,
                     dim=512, heads=4, mlp_hidden=1536)
    single = fs.block_inputs(wl, kind="single")
    double = fs.block_inputs(wl, kind="double")
    ws_single = G.upload_weights(single["weights"], "bf16")
    ws_double = G.upload_weights(double["weights"], "bf16")
    for site in (F.FLUX_SITE_SINGLE_QKV, F.FLUX_SITE_SINGLE_MLP_IN, F.FLUX_SITE_SINGLE_ATTENTION,
                 F.FLUX_SITE_SINGLE_LINEAR2):
        F.flux_timing_begin(site, 4)
        G.run_single_block(wl, single, ws_single)
        G.run_double_block(wl, double, ws_double)
        G.run_single_block(wl, single, ws_single)
        n, us = F.flux_timing_end()
        assert n == 2 and 0.0 < us < 1e5, (site, n, us)
    # double-block sites: each linear (both streams in one launch) and the joint attention, one
    # each per double block, none from a single block
    for site in (F.FLUX_SITE_DOUBLE_QKV, F.FLUX_SITE_DOUBLE_ATTENTION, F.FLUX_SITE_DOUBLE_OUT,
                 F.FLUX_SITE_DOUBLE_MLP_IN, F.FLUX_SITE_DOUBLE_MLP_OUT):
        F.flux_timing_begin(site, 4)
        G.run_double_block(wl, double, ws_double)
        G.run_single_block(wl, single, ws_single)
        G.run_double_block(wl, double, ws_double)
        G.run_double_block(wl, double, ws_double)
        n, us = F.flux_timing_end()
        assert n == 3 and 0.0 < us < 1e5, (site, n, us)
    # capacity exceeded: an error, and the hook is disarmed afterwards
    F.flux_timing_begin(F.FLUX_SITE_SINGLE_MLP_IN, 1)
    G.run_single_block(wl, single, ws_single)
    G.run_single_block(wl, single, ws_single)
    with pytest.raises(F.FluxError):
        F.flux_timing_end()
    G.run_single_block(wl, single, ws_single)
    assert F.flux_timing_end() == (0, 0.0)
    # the timed launches still compute the same result
    F.flux_timing_begin(F.FLUX_SITE_SINGLE_MLP_IN, 1)
    a = G.run_single_block(wl, single, ws_single)
    F.flux_timing_end()
    b = G.run_single_block(wl, single, ws_single)
    assert G.torch().equal(a[0], b[0]) and G.torch().equal(a[1], b[1])
