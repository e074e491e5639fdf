"""flux_linear_noalloc (the linear layer with the library's fixed split-K scratch, for
callers that cannot allocate) against flux_linear with a caller workspace: two calls in a
row through the C ABI, the second on a smaller input, both on shapes whose last partial
round of tiles is split along K (so the fixed scratch is written and read)."""
import numpy as np
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


def _run(noalloc: bool, epi_name: str, m: int, n: int, k: int, seed: int, precision: int = 0):
    from diffusion_transformer_mmdit_amd import flux as F
    t = G.torch()
    cfg = F.make_cfg(256, 2, 768, precision=precision)
    # operands: bf16, or binary16 under FLUX_PRECISION_F16 (the SwiGLU output too)
    op = "f16" if precision == F.FLUX_PRECISION_F16 else "bf16"
    x = G.dev(fs.normal(seed, "x", (m, k), dtype="bf16"), op)
    w = G.dev(fs.normal(seed, "w", (n, k), std=0.02, dtype="bf16"), op)
    epi = getattr(F, f"FLUX_EPI_{epi_name}")
    kw = {}
    if epi_name == "GATED_RESIDUAL":
        rpb = m // 2
        r = G.dev(fs.normal(seed, "r", (m, n), dtype="bf16"), "bf16")
        gate = G.dev(fs.normal(seed, "gate", (2, n), std=0.5, dtype="f32"))
        y = t.empty((m, n), dtype=t.bfloat16, device="cuda")
        kw = dict(resid=r, ldr=n, gate=gate, rows_per_batch=rpb)
        ldy, y_dt = n, F.FLUX_BF16
    elif epi_name == "SWIGLU":
        y = t.empty((m, n // 2), dtype=G.dt(op), device="cuda")
        ldy, y_dt = n // 2, F.FLUX_BF16
    else:
        y = t.empty((m, n), dtype=t.float32, device="cuda")
        ldy, y_dt = n, F.FLUX_F32
    y.fill_(float("nan"))
    print(f"[no-alloc] {'noalloc' if noalloc else 'workspace'} {epi_name} {m}x{n}x{k} {op}",
          flush=True)
    if noalloc:
        F.flux_linear_noalloc(cfg, epi, m, n, k, x, k, w, k, y, ldy, y_dt, stream=G.stream(), **kw)
    else:
        nb = F.flux_linear_workspace_size()
        ws = G.workspace(nb)
        ws.fill_(0xFF)
        F.flux_linear(cfg, epi, m, n, k, x, k, w, k, y, ldy, y_dt, workspace=ws,
                      workspace_bytes=nb, stream=G.stream(), **kw)
    t.cuda.synchronize()
    return G.host(y)


# first call: 4608 x 4096 x 16384 (288 tiles of 256 x 256: 32 tail tiles split 8 ways, the
# whole 64 MiB scratch); second call, smaller: 1536 x 3072 x 12288 (72 tiles, all in one
# partial round, split 3 ways) and a SwiGLU launch at a Klein-4B shape
CASES = [("GATED_RESIDUAL", 4608, 4096, 16384), ("STORE", 1536, 3072, 12288),
         ("SWIGLU", 1536, 2 * 9216, 3072)]


@pytest.mark.parametrize("precision", [0, 2])
def test_linear_noalloc_matches_linear_with_workspace_on_calls_in_a_row(precision):
    for epi_name, m, n, k in CASES:
        seed = m + n + k
        got = _run(True, epi_name, m, n, k, seed, precision)
        ref = _run(False, epi_name, m, n, k, seed, precision)
        assert np.isfinite(got).all()
        ma, nl = G.errors(got, ref)
        print(f"[parity] flux_linear_noalloc {epi_name} {m}x{n}x{k} vs flux_linear: "
              f"max_abs={ma:.3e} nL2={nl:.3e} (same kernels and split plan: expected 0)",
              flush=True)
        # the same kernels with the same tile and split plan: identical bits
        assert np.array_equal(got, ref), (ma, nl)
