"""Parity of each hot-path operation (one kernel each) with the fp64 oracle, through the
C ABI.  Small cases span several tiles and ragged tails; the full-size cases use the
block shapes and compare sampled outputs that the oracle computes one by one."""
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


def F():
    from diffusion_transformer_mmdit_amd import flux
    return flux


def cfg(D, dtype="bf16", H=None, precision=0):
    f = F()
    return f.make_cfg(D, D // 128, H or 3 * D, dtype=f.FLUX_BF16 if dtype == "bf16" else f.FLUX_F32,
                      precision=precision)


# binary16 storage (FLUX_PRECISION_F16) moves a value by at most half an ulp: 2^-11 of its
# magnitude in the normal range
F16_HALF_ULP = 2.0 ** -11


# ------------------------------------------------------------------------------------
# a0: RoPE position table (integer, bit-exact)
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_txt,n_img", [(16, 64), (512, 1024), (512, 4096), (0, 16384), (7, 9)])
def test_rope_positions_bit_exact(n_txt, n_img):
    t = G.torch()
    txt_ids, img_ids = fs.text_ids(n_txt), fs.image_ids(n_img)
    pos = t.empty((n_txt + n_img, 64), dtype=t.int32, device="cuda")
    F().flux_rope_positions(cfg(256), G.dev(txt_ids) if n_txt else None, G.dev(img_ids), n_txt,
                            n_img, pos, G.stream())
    t.cuda.synchronize()
    ref = O.rope_positions(txt_ids, img_ids)
    assert np.array_equal(pos.cpu().numpy().astype(np.int64), ref)


def test_rope_positions_random_ids_bit_exact():
    t = G.torch()
    rng = np.random.default_rng(3)
    txt_ids = rng.integers(-1000, 100000, size=(37, 4)).astype(np.int32)
    img_ids = rng.integers(-1000, 100000, size=(101, 4)).astype(np.int32)
    pos = t.empty((138, 64), dtype=t.int32, device="cuda")
    F().flux_rope_positions(cfg(256), G.dev(txt_ids), G.dev(img_ids), 37, 101, pos, G.stream())
    t.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy().astype(np.int64), O.rope_positions(txt_ids, img_ids))


# ------------------------------------------------------------------------------------
# a1/a2: timestep embedding + modulation
# ------------------------------------------------------------------------------------
# x of batch x D floats is staged in LDS up to 64 KB (the last three cases: 48 KB with fp32
# weights, 48 KB with bf16, 80 KB through the kernel that reads x from the caches)
@pytest.mark.parametrize("D,dtype,batch,n_chunks", [(256, "f32", 1, 3), (256, "bf16", 3, 6),
                                                    (3072, "bf16", 1, 3), (4096, "bf16", 2, 6),
                                                    (3072, "f32", 4, 2), (6144, "bf16", 2, 2),
                                                    (4096, "bf16", 5, 3)])
def test_modulation(D, dtype, batch, n_chunks):
    t = G.torch()
    seed = 77 + D
    specs = fs.temb_weight_specs(D)
    specs["mod"] = ((n_chunks * D, D), "w")
    w = fs.make_weights(specs, seed, dtype)
    tt = fs.uniform(seed, "t", (batch,))
    wd = G.upload_weights(w, dtype)
    c = cfg(D, dtype)
    out = t.empty((batch, n_chunks * D), dtype=t.float32, device="cuda")
    nb = F().flux_modulation_workspace_size(c, batch)
    ws = G.workspace(nb)
    F().flux_modulation(c, F().temb_weights(wd), wd["mod"], n_chunks * D, G.dev(tt), batch, out,
                        ws, nb, G.stream())
    t.cuda.synchronize()
    ref = np.concatenate(O.modulation(O.conditioning(tt, w), w["mod"].astype(np.float64), n_chunks),
                         axis=-1)
    # modulation vectors feed every block; hold them to a tighter bar than the outputs
    G.assert_close(G.host(out), ref, dtype, f"modulation D={D}", max_abs=1e-3 if dtype == "bf16" else 1e-5,
                   nl2=1e-3 if dtype == "bf16" else 1e-5)


# ------------------------------------------------------------------------------------
# a3: LayerNorm + modulate
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("D,rows,rpb,x_dtype,y_dtype", [
    (256, 80, 80, "f32", "f32"), (256, 77, 7, "bf16", "bf16"), (3072, 1536, 1536, "bf16", "bf16"),
    (4096, 4608, 4608, "f32", "bf16"), (6144, 333, 111, "bf16", "bf16"),
    # fp32 residual rows at every width of the per-item kernel: items of a row count that is
    # not a multiple of 4, a last item cut short (rows not a multiple of rows_per_batch),
    # rows_per_batch beyond rows, and items of fewer rows than a workgroup's 4 waves
    (3072, 150, 75, "f32", "bf16"), (4096, 70, 30, "f32", "bf16"), (4096, 9, 100, "f32", "f32"),
    (4096, 9, 1, "f32", "bf16"), (3072, 10, 3, "f32", "bf16"),
    (6144, 222, 37, "f32", "bf16"), (6144, 75, 25, "f32", "f32"), (8192, 37, 37, "f32", "f32")])
def test_layernorm_modulate(D, rows, rpb, x_dtype, y_dtype):
    t = G.torch()
    seed = 11 + rows
    B = -(-rows // rpb)
    # scale / shift before rounding, so both sides read the same representable values
    x = fs.normal(seed, "x", (rows, D), std=2.0, mean=0.5, dtype=x_dtype)
    shift = fs.normal(seed, "shift", (B, D), std=0.3, dtype="f32")
    scale = fs.normal(seed, "scale", (B, D), std=0.3, dtype="f32")
    y = t.empty((rows, D), dtype=G.dt(y_dtype), device="cuda")
    f = F()
    f.flux_layernorm_modulate(cfg(D, y_dtype), rows, rpb, G.dev(x, x_dtype),
                              f.FLUX_BF16 if x_dtype == "bf16" else f.FLUX_F32, G.dev(shift),
                              G.dev(scale), y, G.stream())
    t.cuda.synchronize()
    # row r takes item r // rpb: pad the last item to whole rows for the oracle, then drop the pad
    xp = np.zeros((B * rpb, D), np.float64)
    xp[:rows] = x.astype(np.float64)
    xp[rows:] = 1.0 + np.arange(D) / D  # any row with non-zero variance
    ref = O.layernorm_modulate(xp.reshape(B, rpb, D), shift.astype(np.float64),
                               scale.astype(np.float64)).reshape(B * rpb, D)[:rows]
    if y_dtype == "bf16":
        G.assert_op_close(G.host(y), ref, f"LN+mod D={D} rows={rows}")
    else:
        G.assert_close(G.host(y), ref, "f32", f"LN+mod D={D} rows={rows}")


@pytest.mark.parametrize("D,rows,rpb,x_dtype", [
    (256, 77, 7, "bf16"), (6144, 333, 111, "bf16"), (4096, 4608, 4608, "f32"),
    (3072, 150, 75, "f32"), (6144, 222, 37, "f32"), (8192, 37, 37, "f32"), (4096, 9, 1, "f32")])
def test_layernorm_modulate_f16_output(D, rows, rpb, x_dtype):
    """FLUX_PRECISION_F16: the same LayerNorm + modulate stored in binary16 (every kernel
    variant: fp32 rows per item, the split fp32 kernel at 6144 / 8192, bf16 rows)."""
    t = G.torch()
    seed = 11 + rows
    B = -(-rows // rpb)
    x = fs.normal(seed, "x", (rows, D), std=2.0, mean=0.5, dtype=x_dtype)
    shift = fs.normal(seed, "shift", (B, D), std=0.3, dtype="f32")
    scale = fs.normal(seed, "scale", (B, D), std=0.3, dtype="f32")
    y = t.empty((rows, D), dtype=t.float16, device="cuda")
    f = F()
    f.flux_layernorm_modulate(cfg(D, precision=f.FLUX_PRECISION_F16), rows, rpb, G.dev(x, x_dtype),
                              f.FLUX_BF16 if x_dtype == "bf16" else f.FLUX_F32, G.dev(shift),
                              G.dev(scale), y, G.stream())
    t.cuda.synchronize()
    xp = np.zeros((B * rpb, D), np.float64)
    xp[:rows] = x.astype(np.float64)
    xp[rows:] = 1.0 + np.arange(D) / D
    ref = O.layernorm_modulate(xp.reshape(B, rpb, D), shift.astype(np.float64),
                               scale.astype(np.float64)).reshape(B * rpb, D)[:rows]
    G.assert_op_close(G.host(y), ref, f"LN+mod D={D} rows={rows} -> binary16",
                      rtol=F16_HALF_ULP, atol_rms=1e-4, nl2=1e-3)


# ------------------------------------------------------------------------------------
# a5: QK RMSNorm + RoPE (in place)
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("D,n_txt,n_img,batch,dtype", [
    (256, 16, 64, 1, "f32"), (256, 5, 36, 2, "bf16"), (3072, 512, 1024, 1, "bf16"),
    (4096, 512, 4096, 1, "bf16"),
    # head counts whose last chunk per thread is partial (12, 20 heads), and 48 heads
    # (the per-(token, head) kernel)
    (1536, 7, 36, 2, "bf16"), (2560, 3, 49, 1, "f32"), (6144, 7, 25, 1, "bf16")])
def test_qk_norm_rope(D, n_txt, n_img, batch, dtype):
    t = G.torch()
    seed = 5 + D + n_img
    L, h = n_txt + n_img, D // 128
    ld = 3 * D
    buf = fs.normal(seed, "qkv", (batch, L, ld), std=1.7, dtype=dtype)
    g = {k: fs.normal(seed, k, (128,), std=0.02, mean=1.0, dtype="f32")
         for k in ("qt", "kt", "qi", "ki")}
    txt_ids, img_ids = fs.text_ids(n_txt), fs.image_ids(n_img)
    xb = G.dev(buf, dtype)
    c = cfg(D, dtype)
    nb = F().flux_qk_norm_rope_workspace_size(c, n_txt, n_img)
    ws = G.workspace(nb)
    F().flux_qk_norm_rope(c, batch, n_txt, n_img, xb, xb[..., D:], ld, G.dev(g["qt"]), G.dev(g["kt"]),
                          G.dev(g["qi"]), G.dev(g["ki"]), G.dev(txt_ids) if n_txt else None,
                          G.dev(img_ids), ws, nb, G.stream())
    t.cuda.synchronize()
    got = G.host(xb)
    pos = O.rope_positions(txt_ids, img_ids)
    b64 = buf.astype(np.float64)
    for sl, gq, gk in ((slice(0, n_txt), "qt", "kt"), (slice(n_txt, L), "qi", "ki")):
        q = b64[:, sl, :D].reshape(batch, -1, h, 128)
        k = b64[:, sl, D:2 * D].reshape(batch, -1, h, 128)
        qn = O.rms_norm(q, g[gq].astype(np.float64))
        kn = O.rms_norm(k, g[gk].astype(np.float64))
        b64[:, sl, :D] = qn.reshape(batch, -1, D)
        b64[:, sl, D:2 * D] = kn.reshape(batch, -1, D)
    q = O.apply_rope(b64[..., :D].reshape(batch, L, h, 128), pos).reshape(batch, L, D)
    k = O.apply_rope(b64[..., D:2 * D].reshape(batch, L, h, 128), pos).reshape(batch, L, D)
    check = G.assert_op_close if dtype == "bf16" else (lambda a, b, w: G.assert_close(a, b, "f32", w))
    check(got[..., :D], q, f"RMS+RoPE q D={D} L={L}")
    check(got[..., D:2 * D], k, f"RMS+RoPE k D={D} L={L}")
    # v columns untouched
    assert np.array_equal(got[..., 2 * D:], buf[..., 2 * D:].astype(np.float64))


# ------------------------------------------------------------------------------------
# a4/a7/a8/a9: linear layers with their epilogues
# ------------------------------------------------------------------------------------
LIN_CASES = [  # m, n, k, dtype
    (80, 768, 256, "f32"), (77, 200, 136, "bf16"), (300, 390, 520, "bf16"),
    (1536, 3072, 3072, "bf16"), (4096, 12288, 4096, "bf16"), (512, 4096, 12288, "bf16"),
    # 1, 2, 3 and 5 K slices of 64: every branch of the peeled K loop, ragged M and N tails
    (300, 520, 64, "bf16"), (600, 1100, 128, "bf16"), (513, 700, 192, "bf16"),
    (1030, 2050, 320, "bf16"),
    # the same short K loops on 256 x 256 tiles (two A and three W stages), which the tile
    # choice takes only for products of several rounds
    (8192, 8192, 64, "bf16"), (8192, 8192, 128, "bf16"), (8192, 8192, 192, "bf16")]


def _sample_rows(m, k=64, seed=0):
    """First and last rows, k random rows, and two rows of every 256-row band (so every
    output tile of the large-tile kernels is checked at some row)."""
    rng = np.random.default_rng(seed)
    bands = np.arange(0, m, 256)
    per_band = np.concatenate([np.minimum(bands + rng.integers(0, 256, size=len(bands)), m - 1)
                               for _ in range(2)])
    return np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, size=k), per_band]))


def _lin_ws(use_ws):
    """Split-K scratch (None: the kernels never split along K)."""
    if not use_ws:
        return None, 0
    nb = F().flux_linear_workspace_size()
    return G.workspace(nb), nb


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("m,n,k,dtype", LIN_CASES)
def test_linear_store(m, n, k, dtype, use_ws):
    t = G.torch()
    seed = m + n + k
    x = fs.normal(seed, "x", (m, k), dtype=dtype)
    w = fs.normal(seed, "w", (n, k), std=0.02, dtype=dtype)
    f = F()
    for y_dtype in ("f32", dtype):
        y = t.empty((m, n), dtype=G.dt(y_dtype), device="cuda")
        ws, nb = _lin_ws(use_ws)
        f.flux_linear(cfg(256, dtype), f.FLUX_EPI_STORE, m, n, k, G.dev(x, dtype), k, G.dev(w, dtype),
                      k, y, n, f.FLUX_F32 if y_dtype == "f32" else f.FLUX_BF16, workspace=ws,
                      workspace_bytes=nb, stream=G.stream())
        t.cuda.synchronize()
        rows = _sample_rows(m) if m * n * k > 2e9 else np.arange(m)
        ref = O.linear(x[rows].astype(np.float64), w.astype(np.float64))
        if y_dtype == "bf16":
            G.assert_op_close(G.host(y)[rows], ref, f"linear {m}x{n}x{k} -> bf16")
        else:
            G.assert_close(G.host(y)[rows], ref, dtype, f"linear {m}x{n}x{k} -> f32")


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("m,n,k,dtype", LIN_CASES + [(4608, 12288, 4096, "bf16")])
def test_linear_swiglu(m, n, k, dtype, use_ws):
    t = G.torch()
    seed = 3 * m + n + k
    n2 = 2 * n
    x = fs.normal(seed, "x", (m, k), dtype=dtype)
    w = fs.normal(seed, "w", (n2, k), std=0.02, dtype=dtype)
    f = F()
    y = t.empty((m, n), dtype=G.dt(dtype), device="cuda")
    ws, nb = _lin_ws(use_ws)
    f.flux_linear(cfg(256, dtype), f.FLUX_EPI_SWIGLU, m, n2, k, G.dev(x, dtype), k, G.dev(w, dtype), k,
                  y, n, 0, workspace=ws, workspace_bytes=nb, stream=G.stream())
    t.cuda.synchronize()
    rows = _sample_rows(m) if m * n2 * k > 2e9 else np.arange(m)
    ref = O.swiglu(O.linear(x[rows].astype(np.float64), w.astype(np.float64)))
    if dtype == "bf16":
        G.assert_op_close(G.host(y)[rows], ref, f"linear+SwiGLU {m}x{n2}x{k}")
    else:
        G.assert_close(G.host(y)[rows], ref, dtype, f"linear+SwiGLU {m}x{n2}x{k}")


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("m,n,k,dtype", LIN_CASES + [(4608, 4096, 16384, "bf16")])
def test_linear_gated_residual(m, n, k, dtype, use_ws):
    t = G.torch()
    seed = 5 * m + n + k
    rpb = m // 2 if m % 2 == 0 else m
    B = m // rpb
    x = fs.normal(seed, "x", (m, k), dtype=dtype)
    w = fs.normal(seed, "w", (n, k), std=0.02, dtype=dtype)
    r = fs.normal(seed, "r", (m, n), dtype=dtype)
    gate = fs.normal(seed, "gate", (B, n), std=0.5, dtype="f32")
    f = F()
    rd = G.dev(r, dtype)
    f.flux_linear(cfg(256, dtype), f.FLUX_EPI_GATED_RESIDUAL, m, n, k, G.dev(x, dtype), k,
                  G.dev(w, dtype), k, rd, n, f.FLUX_BF16 if dtype == "bf16" else f.FLUX_F32,
                  resid=rd, ldr=n, gate=G.dev(gate), rows_per_batch=rpb, workspace=_lin_ws(use_ws)[0],
                  workspace_bytes=_lin_ws(use_ws)[1], stream=G.stream())
    t.cuda.synchronize()
    rows = _sample_rows(m) if m * n * k > 2e9 else np.arange(m)
    ref = r[rows].astype(np.float64) + gate[rows // rpb].astype(np.float64) * O.linear(
        x[rows].astype(np.float64), w.astype(np.float64))
    if dtype == "bf16":
        G.assert_op_close(G.host(rd)[rows], ref, f"linear+gated residual {m}x{n}x{k} (in place)")
    else:
        G.assert_close(G.host(rd)[rows], ref, dtype, f"linear+gated residual {m}x{n}x{k} (in place)")


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("m,n,k", [(77, 200, 136), (300, 390, 520), (1030, 2050, 320),
                                   (513, 700, 192), (8192, 8192, 128), (4608, 12288, 4096)])
def test_linear_f16_operands(m, n, k, use_ws):
    """FLUX_PRECISION_F16 linears: binary16 x and W (fp16 MFMA, fp32 accumulation) with each
    epilogue, against the exact product of the same binary16 operands: a store to fp32 (only
    accumulation error remains) and to bf16, SwiGLU to binary16, a gated residual into bf16.
    The small shapes take the generic kernel, the others the large-tile one (whole rounds and
    a split-K tail)."""
    t = G.torch()
    f = F()
    seed = 7 * m + n + k
    x = fs.normal(seed, "x", (m, k), dtype="f32").astype(np.float16)
    w = fs.normal(seed, "w", (n, k), std=0.02, dtype="f32").astype(np.float16)
    xd, wd = G.dev(x), G.dev(w)
    c = cfg(256, precision=f.FLUX_PRECISION_F16)
    ws, nb = _lin_ws(use_ws)
    rows = _sample_rows(m) if m * n * k > 2e9 else np.arange(m)
    acc = O.linear(x[rows].astype(np.float64), w.astype(np.float64))
    for ydt, yt in ((f.FLUX_F32, t.float32), (f.FLUX_BF16, t.bfloat16)):
        y = t.empty((m, n), dtype=yt, device="cuda")
        f.flux_linear(c, f.FLUX_EPI_STORE, m, n, k, xd, k, wd, k, y, n, ydt, workspace=ws,
                      workspace_bytes=nb, stream=G.stream())
        t.cuda.synchronize()
        if ydt == f.FLUX_F32:
            # fp32 accumulation only (the MFMA sums of exact products: within 2^-16 of
            # sum |x w| per element, ~0.6e-3 of the RMS here; measured nL2 ~1e-5)
            G.assert_op_close(G.host(y)[rows], acc, f"f16 linear {m}x{n}x{k} -> f32",
                              rtol=2.0 ** -16, atol_rms=1e-3, nl2=1e-4)
        else:
            G.assert_op_close(G.host(y)[rows], acc, f"f16 linear {m}x{n}x{k} -> bf16")
    ys = t.empty((m, n // 2), dtype=t.float16, device="cuda")
    f.flux_linear(c, f.FLUX_EPI_SWIGLU, m, n, k, xd, k, wd, k, ys, n // 2, 0, workspace=ws,
                  workspace_bytes=nb, stream=G.stream())
    rpb = m // 2 if m % 2 == 0 else m
    r = fs.normal(seed, "r", (m, n), dtype="bf16")
    gate = fs.normal(seed, "gate", (m // rpb, n), std=0.5, dtype="f32")
    rd = G.dev(r, "bf16")
    f.flux_linear(c, f.FLUX_EPI_GATED_RESIDUAL, m, n, k, xd, k, wd, k, rd, n, f.FLUX_BF16,
                  resid=rd, ldr=n, gate=G.dev(gate), rows_per_batch=rpb, workspace=ws,
                  workspace_bytes=nb, stream=G.stream())
    t.cuda.synchronize()
    G.assert_op_close(G.host(ys)[rows], O.swiglu(acc), f"f16 linear+SwiGLU {m}x{n}x{k} -> binary16",
                      rtol=F16_HALF_ULP, atol_rms=1e-4, nl2=1e-3)
    ref = r[rows].astype(np.float64) + gate[rows // rpb].astype(np.float64) * acc
    G.assert_op_close(G.host(rd)[rows], ref, f"f16 linear+gated residual {m}x{n}x{k}")


# ------------------------------------------------------------------------------------
# a6: joint attention
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("seq,heads,batch,dtype,n_q", [
    (80, 2, 1, "f32", None), (80, 2, 1, "bf16", None), (200, 3, 2, "bf16", None),
    (1, 1, 1, "bf16", None), (1536, 24, 1, "bf16", 96), (4608, 32, 1, "bf16", 48),
    # query blocks of a partial last round split along the keys and merged: 2-wave blocks
    # with 2 key ranges, 4-wave blocks with 4 ranges and a ragged last tile, batch 2
    (600, 3, 1, "bf16", None), (1100, 64, 1, "bf16", 64), (700, 6, 2, "bf16", None),
    # key ranges of 1, 2 and 3 tiles, whole or with a ragged last tile (the pipelined key
    # loop's last steps), and 256 4-wave units: the smallest grid that takes 4-wave blocks,
    # its partial round split in 2
    (64, 2, 1, "bf16", None), (128, 1, 1, "bf16", None), (150, 2, 1, "bf16", None),
    (192, 1, 1, "bf16", None), (1024, 32, 1, "bf16", 48),
    # 264 4-wave units (more than CUs, fewer than slots): 256 whole, 8 split 5 ways
    (1300, 24, 1, "bf16", 64)])
def test_attention(seq, heads, batch, dtype, n_q):
    t = G.torch()
    seed = seq + heads
    D = heads * 128
    ld = 3 * D
    # q, k after RMSNorm have unit RMS per head; scale like the block's inputs
    qkv = fs.normal(seed, "qkv", (batch, seq, ld), dtype=dtype)
    xb = G.dev(qkv, dtype)
    o = t.empty((batch, seq, D), dtype=G.dt(dtype), device="cuda")
    f = F()
    c = cfg(D, dtype)
    nb = f.flux_attention_workspace_size(c, batch, seq)
    ws = G.workspace(nb)
    f.flux_attention(c, batch, seq, xb, xb[..., D:], xb[..., 2 * D:], ld, o, D, ws, nb, G.stream())
    t.cuda.synchronize()
    got = G.host(o)
    q = qkv[..., :D].astype(np.float64).reshape(batch, seq, heads, 128)
    k = qkv[..., D:2 * D].astype(np.float64).reshape(batch, seq, heads, 128)
    v = qkv[..., 2 * D:].astype(np.float64).reshape(batch, seq, heads, 128)
    rows = np.arange(seq) if n_q is None else _sample_rows(seq, n_q, seed)
    ref = np.empty((batch, len(rows), heads, 128))
    for b in range(batch):
        for h in range(heads):
            p = O.attention_weights(q[b, rows, h], k[b, :, h])
            ref[b, :, h] = p @ v[b, :, h]
    G.assert_close(got[:, rows], ref.reshape(batch, len(rows), D), dtype, f"attention L={seq} h={heads}")


@pytest.mark.parametrize("seq,heads,batch,n_q", [
    (80, 2, 1, None), (200, 3, 2, None), (1100, 64, 1, 64), (1300, 24, 1, 64),
    (4608, 32, 1, 48)])
def test_attention_f16_output(seq, heads, batch, n_q):
    """FLUX_PRECISION_F16: O stored in binary16 (whole units, and units split along the keys
    whose merge writes O).  Against the oracle at the block bars, and against the bf16 O of
    the same kernel: both round the same fp32 value, so they differ by at most the sum of the
    two unit roundoffs (2^-8 + 2^-11 of |O|, plus half binary16's subnormal spacing)."""
    t = G.torch()
    f = F()
    seed = seq + heads
    D = heads * 128
    ld = 3 * D
    qkv = fs.normal(seed, "qkv", (batch, seq, ld), dtype="bf16")
    xb = G.dev(qkv, "bf16")
    outs = {}
    for prec, odt in ((f.FLUX_PRECISION_BF16, t.bfloat16), (f.FLUX_PRECISION_F16, t.float16)):
        c = cfg(D, precision=prec)
        o = t.empty((batch, seq, D), dtype=odt, device="cuda")
        nb = f.flux_attention_workspace_size(c, batch, seq)
        ws = G.workspace(nb)
        f.flux_attention(c, batch, seq, xb, xb[..., D:], xb[..., 2 * D:], ld, o, D, ws, nb,
                         G.stream())
        t.cuda.synchronize()
        outs[prec] = G.host(o)
    got, got_bf = outs[f.FLUX_PRECISION_F16], outs[f.FLUX_PRECISION_BF16]
    bound = (2.0 ** -8 + 2.0 ** -11) * (1 + 2.0 ** -11) * np.abs(got) + 2.0 ** -25
    assert (np.abs(got - got_bf) <= bound).all(), float((np.abs(got - got_bf) - bound).max())
    q = qkv[..., :D].astype(np.float64).reshape(batch, seq, heads, 128)
    k = qkv[..., D:2 * D].astype(np.float64).reshape(batch, seq, heads, 128)
    v = qkv[..., 2 * D:].astype(np.float64).reshape(batch, seq, heads, 128)
    rows = np.arange(seq) if n_q is None else _sample_rows(seq, n_q, seed)
    ref = np.empty((batch, len(rows), heads, 128))
    for b in range(batch):
        for h in range(heads):
            ref[b, :, h] = O.attention_weights(q[b, rows, h], k[b, :, h]) @ v[b, :, h]
    G.assert_close(got[:, rows], ref.reshape(batch, len(rows), D), "bf16",
                   f"attention L={seq} h={heads} -> binary16")


def test_attention_equal_scores_give_mean():
    # q = 0 -> uniform weights -> every output row is the mean of V (exact up to rounding)
    t = G.torch()
    seq, heads = 333, 2
    D = heads * 128
    v = fs.normal(9, "v", (1, seq, D), dtype="bf16")
    q = np.zeros_like(v)
    k = fs.normal(9, "k", (1, seq, D), dtype="bf16")
    o = t.empty((1, seq, D), dtype=t.bfloat16, device="cuda")
    nb = F().flux_attention_workspace_size(cfg(D), 1, seq)
    ws = G.workspace(nb)
    F().flux_attention(cfg(D), 1, seq, G.dev(q, "bf16"), G.dev(k, "bf16"), G.dev(v, "bf16"), D, o, D,
                       ws, nb, G.stream())
    t.cuda.synchronize()
    ref = np.broadcast_to(v.astype(np.float64).mean(axis=1, keepdims=True), (1, seq, D))
    G.assert_close(G.host(o), ref, "bf16", "attention equal scores", max_abs=1e-2, nl2=1e-2)


@pytest.mark.parametrize("seq,heads,beta", [(640, 2, 2.0), (640, 2, 4.0), (1100, 64, 4.0),
                                            (4608, 32, 4.0)])
def test_attention_scores_far_above_first_tile(seq, heads, beta):
    # Every query meets a few keys late in the sequence whose scores exceed those of its
    # first key tile by ~2^6 (beta 2: the kept first-tile maximum still serves, p ~ 2^60) or
    # by ~2^7 and more (beta 4: the fp32 row sum overflows with the first tile's maximum and
    # the range is recomputed with a running one).  1100 x 64 heads takes the key-split
    # path; 4608 x 32 is the Klein-9B shape.
    t = G.torch()
    D = heads * 128
    seed = 31 + seq
    q = fs.normal(seed, "q", (1, seq, D), std=0.1, mean=beta)  # bf16-exact values
    k = fs.normal(seed, "k", (1, seq, D))
    k[:, [seq // 2, seq - 5]] = beta
    v = fs.normal(seed, "v", (1, seq, D))
    o = t.empty((1, seq, D), dtype=t.bfloat16, device="cuda")
    nb = F().flux_attention_workspace_size(cfg(D), 1, seq)
    ws = G.workspace(nb)
    F().flux_attention(cfg(D), 1, seq, G.dev(q, "bf16"), G.dev(k, "bf16"), G.dev(v, "bf16"), D,
                       o, D, ws, nb, G.stream())
    t.cuda.synchronize()
    got = G.host(o)
    rows = _sample_rows(seq, 48, seed)
    qh = q.astype(np.float64).reshape(1, seq, heads, 128)
    kh = k.astype(np.float64).reshape(1, seq, heads, 128)
    vh = v.astype(np.float64).reshape(1, seq, heads, 128)
    ref = np.empty((1, len(rows), heads, 128))
    for h in range(heads):
        p = O.attention_weights(qh[0, rows, h], kh[0, :, h])
        ref[0, :, h] = p @ vh[0, :, h]
    assert np.isfinite(got).all()
    G.assert_close(got[:, rows], ref.reshape(1, len(rows), D), "bf16",
                   f"attention L={seq} h={heads} late scores beta={beta}")
