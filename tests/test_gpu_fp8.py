"""FP8 (E4M3) linear layer through the C ABI: per-row quantization bit-exact against the
oracle (codes and scales), and the fp8 product with each epilogue against the oracle's
exact product of the dequantized operands, at sizes that span several tiles with ragged
edges and at the Klein-9B single-block MLP-in shape (4608 x 24576 x 4096) on sampled rows.

Error bar of the product: the MFMA adds exact fp8 products into fp32, so the result may
differ from the exact sum by a few fp32 roundings of the running sums; the bar is 2^-16
of sum_k |a_k w_k| (about 256 roundings of the largest possible running sum), plus the
rounding of a bf16 output (8 significant bits: up to 2^-8 of |y|)."""
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


@pytest.mark.parametrize("rows,cols,dtype", [(64, 4096, "bf16"), (77, 264, "f32"),
                                             (5, 100, "f32"), (3, 4096, "f32"),
                                             (4608, 4096, "bf16")])
def test_quantize_rows_bit_exact(rows, cols, dtype):
    F, t = F_(), G.torch()
    print(f"[fp8] quantize {rows} x {cols} {dtype}", flush=True)
    x = fs.normal(31, "q", (rows, cols), dtype=dtype) * 3.0
    x = fs.round_to_bf16(x) if dtype == "bf16" else x.astype(np.float32)
    if rows == 3:
        x[1] = 0.0                    # all-zero row: scale 1, codes 0
        x[2, 7] = 1e6                 # one huge value: the rest quantize to tiny codes
    xd = G.dev(x, dtype)
    q = t.empty((rows, cols), dtype=t.uint8, device="cuda")
    sc = t.empty(rows, dtype=t.float32, device="cuda")
    F.flux_quantize_fp8_rows(rows, cols, xd, F.FLUX_BF16 if dtype == "bf16" else F.FLUX_F32,
                             cols, q, cols, sc, G.stream())
    t.cuda.synchronize()
    rq, rs = O.quantize_rows_fp8(x)
    assert np.array_equal(sc.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def product_bound(qa, sa, qw, sw):
    A = np.abs(O.fp8_decode(qa)) * sa[:, None].astype(np.float64)
    W = np.abs(O.fp8_decode(qw)) * sw[:, None].astype(np.float64)
    return 2.0 ** -16 * (A @ W.T)


def quantized(seed, name, rows, cols, scale=1.0):
    x = fs.normal(seed, name, (rows, cols), dtype="f32") * scale
    return O.quantize_rows_fp8(fs.round_to_bf16(x))


def run_fp8(epi, m, n, k, qa, sa, qw, sw, ydt, resid=None, gate=None, split=True):
    F, t = F_(), G.torch()
    cfg = F.make_cfg(256, 2, 768)
    nout = n // 2 if epi == F.FLUX_EPI_SWIGLU else n
    y = t.empty((m, nout), dtype=t.float32 if ydt == "f32" else t.bfloat16, device="cuda")
    ws = nb = None
    if split:
        nb = F.flux_linear_workspace_size()
        ws = G.workspace(nb)
    F.flux_linear_fp8(cfg, epi, m, n, k, G.dev(qa), k, G.dev(sa), G.dev(qw), k, G.dev(sw), y,
                      nout, F.FLUX_F32 if ydt == "f32" else F.FLUX_BF16,
                      resid=None if resid is None else G.dev(resid, ydt), ldr=nout,
                      gate=None if gate is None else G.dev(gate), rows_per_batch=m,
                      workspace=ws, workspace_bytes=nb or 0, stream=G.stream())
    t.cuda.synchronize()
    return G.host(y)


def check(got, ref, bound, ydt, what):
    err = np.abs(got - ref)
    bar = bound + (2.0 ** -8 * (np.abs(ref) + bound) if ydt == "bf16" else 0.0)
    worst = float((err - bar).max())
    ma, nl = G.errors(got, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} nL2={nl:.3e}; worst element excess over the "
          f"bar = {worst:.2e}", flush=True)
    assert np.isfinite(got).all()
    assert worst <= 0, f"{what}: error exceeds the bar by {worst:.3e}"


@pytest.mark.parametrize("m,n,k,ydt", [(300, 200, 256, "f32"), (512, 384, 1024, "bf16"),
                                       (1100, 700, 2048, "f32"), (4608, 4096, 4096, "bf16")])
def test_linear_fp8_store(m, n, k, ydt):
    F = F_()
    print(f"[fp8] store {m} x {n} x {k} -> {ydt}", flush=True)
    qa, sa = quantized(41, "a", m, k)
    qw, sw = quantized(42, "w", n, k, 0.02)
    got = run_fp8(F.FLUX_EPI_STORE, m, n, k, qa, sa, qw, sw, ydt)
    rows = np.arange(m) if m <= 1100 else np.random.default_rng(0).choice(m, 24, replace=False)
    ref = O.linear_fp8(qa[rows], sa[rows], qw, sw)
    check(got[rows], ref, product_bound(qa[rows], sa[rows], qw, sw), ydt,
          f"fp8 store {m}x{n}x{k}")


def test_linear_fp8_gated_residual():
    F = F_()
    m, n, k = 520, 640, 1024
    qa, sa = quantized(43, "a", m, k)
    qw, sw = quantized(44, "w", n, k, 0.02)
    resid = fs.normal(45, "r", (m, n), dtype="f32")
    gate = fs.normal(46, "g", (1, n), dtype="f32")
    got = run_fp8(F.FLUX_EPI_GATED_RESIDUAL, m, n, k, qa, sa, qw, sw, "f32", resid, gate)
    ref = resid + gate * O.linear_fp8(qa, sa, qw, sw)
    bound = np.abs(gate) * product_bound(qa, sa, qw, sw) + 2.0 ** -22 * np.abs(ref)
    check(got, ref, bound, "f32", "fp8 gated residual")


@pytest.mark.parametrize("m,n_half,k", [(320, 512, 512), (4608, 12288, 4096)])
def test_linear_fp8_swiglu(m, n_half, k):
    F = F_()
    print(f"[fp8] SwiGLU {m} x 2*{n_half} x {k}", flush=True)
    qa, sa = quantized(47, "a", m, k)
    qw, sw = quantized(48, "w", 2 * n_half, k, 0.02)
    got = run_fp8(F.FLUX_EPI_SWIGLU, m, 2 * n_half, k, qa, sa, qw, sw, "bf16")
    rows = np.arange(m) if m <= 512 else np.random.default_rng(1).choice(m, 16, replace=False)
    u = O.linear_fp8(qa[rows], sa[rows], qw, sw)
    ref = O.swiglu(u)
    # silu(g) u: the product error of each half, amplified by at most |silu'| <= 1.1 and
    # the other factor
    bg = product_bound(qa[rows], sa[rows], qw[:n_half], sw[:n_half])
    bu = product_bound(qa[rows], sa[rows], qw[n_half:], sw[n_half:])
    g, up = u[:, :n_half], u[:, n_half:]
    bound = 1.1 * bg * (np.abs(up) + bu) + np.abs(O.silu(g)) * bu + 2.0 ** -20 * np.abs(ref)
    check(got[rows], ref, bound, "bf16", f"fp8 SwiGLU {m}x{2 * n_half}x{k}")
