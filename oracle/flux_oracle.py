"""fp64 CPU oracle for the FLUX.2-style MMDiT denoiser forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The product path
(the HIP library and its Python binding) never imports it and shares no code with it.

It is the plain definition of the forward pass, written out in float64 with numpy; the
only library primitive used as a step is the matrix product.  There is no blocking,
fusion or reordering beyond what the definitions state.  Inputs are the same values the
GPU reads (bf16-rounded for bf16 workloads), converted exactly to float64.

Sources ("pages") cited below:
  [TRACE]   "FLUX.2 Klein 9B Base 宏观架构" (flux-vis shape trace of FLUX2-KLEIN-9B-BASE-FULL)
  [DIFF]    "Diffusers 中 Flux2Transformer2DModel 全面解析：架构、配置与源码级原理" (trdm.cn)
  [KLEIN]   "FLUX.2 [klein]" research note (zhao9797.github.io), section 模型架构
  [SDPA]    "Transformer架构解析FLUX.2-klein-base-9b-nvfp4…" (kwkr.cn), section 2 (核心引擎：
            自注意力机制如何工作), the scaled dot-product attention formula

Readings of points the pages leave open (each also listed in the design doc):
  * sinusoid: 128 frequencies f_k = 10000^(-k/128), layout [cos | sin], argument 1000*t
  * MLPEmbedder: Linear(256->D), SiLU, Linear(D->D); modulation: Linear(SiLU(temb))
  * chunk order: (shift, scale, gate) for attention then MLP; final layer (shift, scale)
  * LayerNorm: no affine, biased variance, eps inside the square root; modulate as
    (1 + scale) * x_hat + shift
  * RoPE: adjacent pairs (2p, 2p+1); axis a owns dims [32a, 32a+32); pair j of an axis
    rotates by pos * theta^(-2j/32)
  * single block: linear1 output order [q | k | v | gate | up]; linear2 input [attn | mlp]
  * joint sequence order: text tokens first, then image tokens
  * no biases anywhere
  * sampling: latent 2x2 patches -> token channels in (c, ph, pw) order, patches row-major;
    noise levels on the uniform grid 1 - i/n; Euler step x += (sigma_next - sigma) v with
    v taken at sigma; guidance v_u + g (v_c - v_u)
  * reference K/V cache: reference image j has ids (1 + j, r, c, 0); all reference tokens
    attend to all reference tokens (one segment); the fixed reference timestep is 0
  * FP8 linear: OCP E4M3, per-row (activation) and per-output-channel (weight) scales
    amax / 448 (values multiplied by 448 / amax), round to nearest even with saturation

Parity pins for every function live in tests/test_oracle_pins.py and, for the sampling
loop, the reference K/V cache and the FP8 linear, tests/test_oracle_sampler.py,
tests/test_oracle_refkv.py and tests/test_oracle_fp8.py (closed forms, invariants, brute force and an
independent library routine); none is "parity unpinned".
"""
from __future__ import annotations

from typing import Mapping, Sequence

import numpy as np

# Hyper-parameters fixed by the pages.
HEAD_DIM = 128                  # [DIFF] config table: attention_head_dim 128
EPS = 1e-6                      # [DIFF] config table: eps 1e-6 for LayerNorm / RMSNorm
ROPE_THETA = 2000.0             # [DIFF] config table rope_theta; [KLEIN] RoPE theta=2000
AXES_DIM = (32, 32, 32, 32)     # [DIFF] axes_dims_rope; [KLEIN] axes_dim [32,32,32,32]
TIME_FACTOR = 1000.0            # [DIFF] 时间步缩放: forward multiplies timestep by 1000
TEMB_CHANNELS = 256             # [DIFF] timestep_guidance_channels 256; [KLEIN] 256-dim sinusoid
MAX_PERIOD = 10000.0            # reading: the usual sinusoid period (pages give none)


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------------
def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x).  [DIFF] 激活函数与 FFN (SwiGLU); [KLEIN] MLPEmbedder."""
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W stored [out, in] (bias-free linear layer)."""
    return np.matmul(x, w.T)


# ----------------------------------------------------------------------------------
# Conditioning: timestep embedding and modulation
# ----------------------------------------------------------------------------------
def bf16_storage(x) -> np.ndarray:
    """Value of x after it is computed in fp32 and stored as bf16 (round to nearest, ties
    to even, at each step: fp64 -> fp32 -> bf16), returned as float64.

    Used only through the `storage` argument of the blocks and the step, which applies it
    where a bf16 pipeline stores an intermediate (GEMM operands, attention probabilities
    and outputs); the definition itself (storage=None) keeps every value in fp64.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def f16_storage(x) -> np.ndarray:
    """Value of x after it is computed in fp32 and stored as IEEE binary16 (round to nearest,
    ties to even, at each step: fp64 -> fp32 -> binary16; beyond 65504 it overflows to inf),
    returned as float64.  Used only through the `storage` argument, like bf16_storage.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    with np.errstate(over="ignore"):
        return x32.astype(np.float16).astype(np.float64)


def _keep(x):
    return x


# Where a bf16 pipeline stores a value that a later product reads.  `storage` arguments
# take one callable (applied at every point) or a mapping {point: callable} (points it
# omits keep fp64), so the effect of each rounding point can be measured on its own.
STORAGE_POINTS = (
    "ln",    # LayerNorm + modulate outputs (the inputs of QKV / MLP-in / linear1 / proj_out)
    "qkv",   # q, k, v as the QKV projection produces them
    "rope",  # q and k after RMSNorm + RoPE (the score product's operands)
    "p",     # unnormalised attention probabilities (the PV product's operand)
    "o",     # attention output (the out-projection's input)
    "mlp",   # SwiGLU output (the MLP-out / linear2 input)
    "final", # the step's final LayerNorm + modulate output (the output projection's input)
)


def _storage_at(storage, point: str):
    """The rounding `storage` applies at `point` (identity when none)."""
    if storage is None:
        return _keep
    if isinstance(storage, Mapping):
        if any(k not in STORAGE_POINTS for k in storage):
            raise ValueError(f"unknown storage point in {sorted(storage)}")
        return storage.get(point) or _keep
    return storage


def _p_storage(storage):
    """attention()'s `storage`: None keeps the exact softmax."""
    if storage is None:
        return None
    if isinstance(storage, Mapping):
        return storage.get("p")
    return storage


def timestep_embedding(t) -> np.ndarray:
    """256-channel sinusoid of 1000*t.  [DIFF] 时间步缩放; [KLEIN] 条件注入.

    t: [B] floats in [0, 1] (the pipeline passes t/1000 and the model multiplies by
    1000, so the model sees tau = 1000 t).  Returns [B, 256] = [cos(tau f) | sin(tau f)]
    with f_k = MAX_PERIOD^(-k/128), k = 0..127.
    """
    tau = TIME_FACTOR * f64(t).reshape(-1)
    half = TEMB_CHANNELS // 2
    k = np.arange(half, dtype=np.float64)
    freqs = MAX_PERIOD ** (-k / half)
    arg = tau[:, None] * freqs[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def mlp_embedder(e: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """temb = W2 silu(W1 e).  [KLEIN] 条件注入 (sinusoid -> MLPEmbedder)."""
    return linear(silu(linear(e, w1)), w2)


def modulation(temb: np.ndarray, w_mod: np.ndarray, n_chunks: int) -> list:
    """Modulation vectors m = W_mod silu(temb), split into n_chunks [B, D] pieces.

    [DIFF] 双流块: each stream has shift/scale/gate for attention and for the MLP
    (Flux2Modulation.split(temb_mod, 2)); 单流块: one set (mod_param_sets = 1).
    """
    m = linear(silu(temb), w_mod)
    return np.split(m, n_chunks, axis=-1)


def conditioning(t, w: Mapping) -> np.ndarray:
    return mlp_embedder(timestep_embedding(t), f64(w["temb.w1"]), f64(w["temb.w2"]))


# ----------------------------------------------------------------------------------
# Normalisations
# ----------------------------------------------------------------------------------
def layernorm_modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray,
                       eps: float = EPS) -> np.ndarray:
    """(1 + scale) * (x - mean) / sqrt(var + eps) + shift over the last axis.

    [DIFF] 双流块 / 单流块 (AdaLN modulation of the pre-norm), config eps 1e-6.
    x: [B, N, D]; shift, scale: [B, D].  Biased variance, no affine parameters.
    """
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    xhat = (x - mu) / np.sqrt(var + eps)
    return (1.0 + scale[:, None, :]) * xhat + shift[:, None, :]


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float = EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis (one head's 128 dims).

    [DIFF] 双流块 (norm_q / norm_k after projection); 并行化支持 (QK-Norm acts on the
    full head_dim).
    """
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * gamma


# ----------------------------------------------------------------------------------
# Rotary position embedding over 4 id axes
# ----------------------------------------------------------------------------------
def _ids2d(ids) -> np.ndarray:
    """[DIFF] 位置 id 的维度: 2-D ids are used as is, 3-D ids take [0]."""
    a = np.asarray(ids)
    if a.ndim == 3:
        a = a[0]
    if a.ndim != 2 or a.shape[1] != len(AXES_DIM):
        raise ValueError(f"ids must be [N, {len(AXES_DIM)}], got {a.shape}")
    return a


def rope_positions(txt_ids, img_ids) -> np.ndarray:
    """Integer position of every rotation pair: [L, 64] int64.

    The joint ids are cat(txt_ids, img_ids) (text first); pair p belongs to the axis
    whose dims contain 2p, and takes that axis' id.  [DIFF] 位置 id 的维度 (per-axis
    1-D RoPE, concatenated); [KLEIN] axes_dim [32,32,32,32].
    """
    ids = np.concatenate([_ids2d(txt_ids), _ids2d(img_ids)], axis=0).astype(np.int64)
    cols = []
    for a, d in enumerate(AXES_DIM):
        cols.extend([a] * (d // 2))
    return ids[:, np.array(cols, dtype=np.int64)]


def rope_frequencies() -> np.ndarray:
    """omega for each of the 64 pairs: axis-local pair j of an axis with d dims has
    omega = theta^(-2j/d).  [DIFF] rope_theta 2000; [KLEIN] RoPE theta=2000."""
    out = []
    for d in AXES_DIM:
        j = np.arange(d // 2, dtype=np.float64)
        out.append(ROPE_THETA ** (-2.0 * j / d))
    return np.concatenate(out)


def apply_rope(x: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (2p, 2p+1) of each head by phi = pos[:, p] * omega_p.

    x: [B, L, h, 128]; pos: [L, 64] integer.  (x_{2p}, x_{2p+1}) ->
    (x_{2p} cos phi - x_{2p+1} sin phi, x_{2p} sin phi + x_{2p+1} cos phi).
    """
    phi = pos.astype(np.float64) * rope_frequencies()[None, :]     # [L, 64]
    c = np.cos(phi)[None, :, None, :]
    s = np.sin(phi)[None, :, None, :]
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ----------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------
def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Exact max-subtracted softmax along the last axis."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_weights(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d_k)) for one head: q [Lq, d], k [Lk, d] -> [Lq, Lk].

    [SDPA] the scaled dot-product attention formula (scores scaled by 1/sqrt(d_k),
    softmax over the key axis)."""
    return softmax_rows(np.matmul(q, k.T) / np.sqrt(q.shape[-1]))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, storage=None) -> np.ndarray:
    """Multi-head attention over the full joint sequence, no mask.

    q, k, v: [B, L, h, d] -> [B, L, h*d] (heads concatenated in head order).
    [TRACE] Joint multi-head attention (separate QKV, shared attention); [SDPA].
    With `storage`, the unnormalised probabilities exp(s - max) are stored through it and
    normalised by the sum of the stored values.
    """
    B, L, h, d = q.shape
    out = np.empty((B, L, h, d), dtype=np.float64)
    for b in range(B):
        for head in range(h):
            if storage is None:
                p = attention_weights(q[b, :, head, :], k[b, :, head, :])
                out[b, :, head, :] = np.matmul(p, v[b, :, head, :])
            else:
                sc = np.matmul(q[b, :, head, :], k[b, :, head, :].T) / np.sqrt(d)
                e = storage(np.exp(sc - sc.max(axis=-1, keepdims=True)))
                out[b, :, head, :] = np.matmul(e, v[b, :, head, :]) / e.sum(axis=-1, keepdims=True)
    return out.reshape(B, L, h * d)


def swiglu(u: np.ndarray) -> np.ndarray:
    """silu(gate) * up with u = [gate | up] along the last axis.

    [DIFF] 激活函数与 FFN: the gate linear is fused into the preceding linear
    (linear_in -> 2x width), SwiGLU halves it, then linear_out."""
    H = u.shape[-1] // 2
    return silu(u[..., :H]) * u[..., H:]


def _heads(x: np.ndarray) -> np.ndarray:
    B, N, D = x.shape
    return x.reshape(B, N, D // HEAD_DIM, HEAD_DIM)


# ----------------------------------------------------------------------------------
# Blocks
# ----------------------------------------------------------------------------------
def double_block_mods(t, w: Mapping) -> dict:
    temb = conditioning(t, w)
    return {"img": modulation(temb, f64(w["mod_img"]), 6),
            "txt": modulation(temb, f64(w["mod_txt"]), 6)}


def double_block(img, txt, t, w: Mapping, img_ids, txt_ids, mods: dict | None = None,
                 storage=None):
    """Double-stream block.  Returns (img_out, txt_out), float64.

    [TRACE] section 4 (Double-stream block: modulate image + text streams, joint
    multi-head attention with separate QKV, per-stream MLP, residual update);
    [DIFF] 双流块 Flux2TransformerBlock.
    img: [B, N_img, D]; txt: [B, N_txt, D]; w keys "img.qkv", "img.out", "img.mlp_in",
    "img.mlp_out", "img.q_norm", "img.k_norm" and the same for "txt."; mods: per stream
    the six [B, D] chunks (shift1, scale1, gate1, shift2, scale2, gate2), computed from
    t with "temb.*", "mod_img", "mod_txt" when not given.  `storage` (e.g. bf16_storage)
    is applied where a bf16 pipeline stores a value: the normalised-and-modulated inputs
    of the linears, q / k / v, q and k after RMSNorm + RoPE, the attention probabilities
    and output, and the SwiGLU output; the residual stream is not rounded.
    """
    st_ln, st_qkv, st_rope = (_storage_at(storage, p) for p in ("ln", "qkv", "rope"))
    st_o, st_mlp = _storage_at(storage, "o"), _storage_at(storage, "mlp")
    streams = {"txt": f64(txt), "img": f64(img)}
    if mods is None:
        mods = double_block_mods(t, w)
    qs, ks, vs = {}, {}, {}
    for s in ("txt", "img"):
        shift1, scale1 = mods[s][0], mods[s][1]
        a = st_ln(layernorm_modulate(streams[s], shift1, scale1))
        q, k, v = (st_qkv(y) for y in np.split(linear(a, f64(w[f"{s}.qkv"])), 3, axis=-1))
        qs[s] = rms_norm(_heads(q), f64(w[f"{s}.q_norm"]))
        ks[s] = rms_norm(_heads(k), f64(w[f"{s}.k_norm"]))
        vs[s] = _heads(v)
    pos = rope_positions(txt_ids, img_ids)
    q = st_rope(apply_rope(np.concatenate([qs["txt"], qs["img"]], axis=1), pos))
    k = st_rope(apply_rope(np.concatenate([ks["txt"], ks["img"]], axis=1), pos))
    v = np.concatenate([vs["txt"], vs["img"]], axis=1)
    o = st_o(attention(q, k, v, _p_storage(storage)))
    n_txt = streams["txt"].shape[1]
    o_s = {"txt": o[:, :n_txt], "img": o[:, n_txt:]}
    out = {}
    for s in ("txt", "img"):
        _, _, gate1, shift2, scale2, gate2 = mods[s]
        x = streams[s] + gate1[:, None, :] * linear(o_s[s], f64(w[f"{s}.out"]))
        u = linear(st_ln(layernorm_modulate(x, shift2, scale2)), f64(w[f"{s}.mlp_in"]))
        x = x + gate2[:, None, :] * linear(st_mlp(swiglu(u)), f64(w[f"{s}.mlp_out"]))
        out[s] = x
    return out["img"], out["txt"]


def single_block_mods(t, w: Mapping) -> list:
    return modulation(conditioning(t, w), f64(w["mod"]), 3)


def single_block(img, txt, t, w: Mapping, img_ids, txt_ids, mods: Sequence | None = None,
                 storage=None):
    """Single-stream (parallel) block.  Returns (img_out, txt_out), float64.

    [TRACE] section 4 (merge image + text sequence, attention + gated MLP);
    [DIFF] 单流块 Flux2SingleTransformerBlock: cat the streams, one modulation set,
    fused to_qkv_mlp_proj (D -> 3D + 2H), attention and SwiGLU in parallel, fused
    to_out ((D + H) -> D), gated residual.
    w keys "linear1" [3D+2H, D], "linear2" [D, D+H], "q_norm", "k_norm" (and "temb.*",
    "mod" when mods is not given); mods = (shift, scale, gate), each [B, D].  `storage`
    as for double_block (the linear1 MLP part feeds SwiGLU unrounded).
    """
    st_ln, st_qkv, st_rope = (_storage_at(storage, p) for p in ("ln", "qkv", "rope"))
    st_o, st_mlp = _storage_at(storage, "o"), _storage_at(storage, "mlp")
    txt = f64(txt)
    img = f64(img)
    n_txt = txt.shape[1]
    x = np.concatenate([txt, img], axis=1)
    D = x.shape[-1]
    if mods is None:
        mods = single_block_mods(t, w)
    shift, scale, gate = mods
    y = linear(st_ln(layernorm_modulate(x, shift, scale)), f64(w["linear1"]))
    q, k, v, u = (st_qkv(y[..., :D]), st_qkv(y[..., D:2 * D]), st_qkv(y[..., 2 * D:3 * D]),
                  y[..., 3 * D:])
    pos = rope_positions(txt_ids, img_ids)
    q = st_rope(apply_rope(rms_norm(_heads(q), f64(w["q_norm"])), pos))
    k = st_rope(apply_rope(rms_norm(_heads(k), f64(w["k_norm"])), pos))
    o = st_o(attention(q, k, _heads(v), _p_storage(storage)))
    x = x + gate[:, None, :] * linear(np.concatenate([o, st_mlp(swiglu(u))], axis=-1),
                                      f64(w["linear2"]))
    return x[:, n_txt:], x[:, :n_txt]


# ----------------------------------------------------------------------------------
# Blocks evaluated at a subset of output rows (large workloads)
#
# Every step of a block except the attention's mixing over keys acts on one token at a
# time, so the outputs of selected rows need only the keys and values of all tokens and
# everything else for the selected rows.  These functions compute exactly that, with the
# same steps as double_block / single_block; tests pin them to those on small inputs.
# ----------------------------------------------------------------------------------
def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """attention() for a subset of queries: q [B, R, h, d] (already rotated), k and v
    [B, L, h, d] -> [B, R, h*d]."""
    B, R, h, d = q.shape
    out = np.empty((B, R, h, d), dtype=np.float64)
    for b in range(B):
        for head in range(h):
            p = attention_weights(q[b, :, head, :], k[b, :, head, :])
            out[b, :, head, :] = np.matmul(p, v[b, :, head, :])
    return out.reshape(B, R, h * d)


def double_block_rows(img, txt, t, w: Mapping, img_ids, txt_ids, rows_img, rows_txt,
                      mods: dict | None = None):
    """double_block() outputs at image rows `rows_img` and text rows `rows_txt` only.

    Returns (img_out [B, len(rows_img), D], txt_out [B, len(rows_txt), D]), float64."""
    streams = {"txt": f64(txt), "img": f64(img)}
    rows = {"txt": np.asarray(rows_txt, dtype=np.int64), "img": np.asarray(rows_img, dtype=np.int64)}
    if mods is None:
        mods = double_block_mods(t, w)
    D = streams["img"].shape[-1]
    n_txt = streams["txt"].shape[1]
    pos = rope_positions(txt_ids, img_ids)
    qs, ks, vs = {}, {}, {}
    for s in ("txt", "img"):
        shift1, scale1 = mods[s][0], mods[s][1]
        wqkv = f64(w[f"{s}.qkv"])
        a = layernorm_modulate(streams[s], shift1, scale1)
        kv = linear(a, wqkv[D:])                                 # keys, values: all tokens
        ks[s] = rms_norm(_heads(kv[..., :D]), f64(w[f"{s}.k_norm"]))
        vs[s] = _heads(kv[..., D:])
        q = linear(a[:, rows[s]], wqkv[:D])                      # queries: selected rows
        qs[s] = rms_norm(_heads(q), f64(w[f"{s}.q_norm"]))
    k = apply_rope(np.concatenate([ks["txt"], ks["img"]], axis=1), pos)
    v = np.concatenate([vs["txt"], vs["img"]], axis=1)
    out = {}
    for s, off in (("txt", 0), ("img", n_txt)):
        q = apply_rope(qs[s], pos[rows[s] + off])
        o = attention_rows(q, k, v)
        _, _, gate1, shift2, scale2, gate2 = mods[s]
        x = streams[s][:, rows[s]] + gate1[:, None, :] * linear(o, f64(w[f"{s}.out"]))
        u = linear(layernorm_modulate(x, shift2, scale2), f64(w[f"{s}.mlp_in"]))
        out[s] = x + gate2[:, None, :] * linear(swiglu(u), f64(w[f"{s}.mlp_out"]))
    return out["img"], out["txt"]


def single_block_rows(img, txt, t, w: Mapping, img_ids, txt_ids, rows_img, rows_txt,
                      mods: Sequence | None = None):
    """single_block() outputs at image rows `rows_img` and text rows `rows_txt` only.

    Returns (img_out [B, len(rows_img), D], txt_out [B, len(rows_txt), D]), float64."""
    txt = f64(txt)
    img = f64(img)
    n_txt = txt.shape[1]
    x = np.concatenate([txt, img], axis=1)
    D = x.shape[-1]
    if mods is None:
        mods = single_block_mods(t, w)
    shift, scale, gate = mods
    w1 = f64(w["linear1"])
    a = layernorm_modulate(x, shift, scale)
    kv = linear(a, w1[D:3 * D])                                  # keys, values: all tokens
    pos = rope_positions(txt_ids, img_ids)
    k = apply_rope(rms_norm(_heads(kv[..., :D]), f64(w["k_norm"])), pos)
    v = _heads(kv[..., D:])
    sel = np.concatenate([np.asarray(rows_txt, dtype=np.int64),
                          n_txt + np.asarray(rows_img, dtype=np.int64)])
    y = linear(a[:, sel], w1[np.r_[0:D, 3 * D:w1.shape[0]]])     # q and [gate | up]
    q = apply_rope(rms_norm(_heads(y[..., :D]), f64(w["q_norm"])), pos[sel])
    o = attention_rows(q, k, v)
    out = x[:, sel] + gate[:, None, :] * linear(np.concatenate([o, swiglu(y[..., D:])], axis=-1),
                                                f64(w["linear2"]))
    nt = len(rows_txt)
    return out[:, nt:], out[:, :nt]


# ----------------------------------------------------------------------------------
# Denoiser step
# ----------------------------------------------------------------------------------
class _Prefixed(Mapping):
    """Read-only view of the keys of `w` that start with `prefix` (prefix removed)."""

    def __init__(self, w: Mapping, prefix: str):
        self._w, self._p = w, prefix

    def __getitem__(self, k):
        return self._w[self._p + k]

    def __iter__(self):
        return (k[len(self._p):] for k in self._w if k.startswith(self._p))

    def __len__(self):
        return sum(1 for _ in self)


def step_mods(t, w: Mapping) -> dict:
    """Model-level modulation shared by all blocks of a kind.

    [DIFF] 双流块 (temb_mod_img / temb_mod_txt are passed into every double block);
    单流块 (mod_param_sets = 1, declared at model level)."""
    temb = conditioning(t, w)
    return {
        "double": {"img": modulation(temb, f64(w["mod_dimg"]), 6),
                   "txt": modulation(temb, f64(w["mod_dtxt"]), 6)},
        "single": modulation(temb, f64(w["mod_single"]), 3),
        "final": modulation(temb, f64(w["mod_final"]), 2),
    }


def denoiser_step(x, ctx, t, w: Mapping, img_ids, txt_ids, n_double: int, n_single: int,
                  on_block=None, storage=None):
    """One denoiser forward: [B, N_img, in_ch] -> [B, N_img, in_ch], float64.

    [TRACE] section 3 (packed image tokens width 128 -> hidden; text condition joint dim;
    Double-stream block x8; Single-stream block x24; Project / Unpack keeping the noisy
    image tokens -> [1, 4096, 128]); [DIFF] 前向传播输入输出约定.
    Block weights are read as "double.{i}.<key>" and "single.{i}.<key>" so `w` may be a
    lazy mapping that materialises one block at a time.  `on_block(kind, i)` is called
    after each block (progress reporting).  `storage` as for the blocks, plus the final
    LayerNorm+modulate output; the residual stream and the output are not rounded.
    """
    st_final = _storage_at(storage, "final")
    mods = step_mods(t, w)
    img = linear(f64(x), f64(w["img_in"]))
    txt = linear(f64(ctx), f64(w["txt_in"]))
    for i in range(n_double):
        img, txt = double_block(img, txt, None, _Prefixed(w, f"double.{i}."),
                                img_ids, txt_ids, mods=mods["double"], storage=storage)
        if on_block:
            on_block("double", i)
    for i in range(n_single):
        img, txt = single_block(img, txt, None, _Prefixed(w, f"single.{i}."),
                                img_ids, txt_ids, mods=mods["single"], storage=storage)
        if on_block:
            on_block("single", i)
    shift_f, scale_f = mods["final"]
    return linear(st_final(layernorm_modulate(img, shift_f, scale_f)), f64(w["proj_out"]))


# ----------------------------------------------------------------------------------
# Sampling loop around the denoiser step
#
# [KLEIN] 训练方法: latent rectified flow / flow matching; the distilled model samples in
# 4 steps with guidance folded into its weights, the base model in 50 steps with the two
# forwards of classifier-free guidance.  [DIFF] Flux2 管线 call chain: the VAE latent is
# packed into tokens with their 4-D ids, a flow-matching Euler scheduler calls the
# transformer once per step.  [KLEIN] Visual tokenizer / VAE: 32-channel latent, 2x2
# patchify -> in_channels 128 (32 x 2 x 2).
# ----------------------------------------------------------------------------------
def pack_latents(z) -> np.ndarray:
    """[B, C, H, W] latent -> [B, (H/2)(W/2), 4C] tokens: one token per 2x2 patch, patches
    in row-major order of the (H/2) x (W/2) grid, channel index 4c + 2 ph + pw (reading:
    the pages give only the 32 x 2 x 2 product; this is that factor order)."""
    z = f64(z)
    B, C, H, W = z.shape
    if H % 2 or W % 2:
        raise ValueError("latent height and width must be even")
    p = z.reshape(B, C, H // 2, 2, W // 2, 2)          # b, c, r, ph, col, pw
    return p.transpose(0, 2, 4, 1, 3, 5).reshape(B, (H // 2) * (W // 2), 4 * C)


def unpack_latents(x, H: int, W: int) -> np.ndarray:
    """Inverse of pack_latents: [B, (H/2)(W/2), 4C] -> [B, C, H, W]."""
    x = f64(x)
    B, N, C4 = x.shape
    if H % 2 or W % 2 or N != (H // 2) * (W // 2) or C4 % 4:
        raise ValueError("token count / channels do not match the latent shape")
    p = x.reshape(B, H // 2, W // 2, C4 // 4, 2, 2)     # b, r, col, c, ph, pw
    return p.transpose(0, 3, 1, 4, 2, 5).reshape(B, C4 // 4, H, W)


def generation_ids(grid_h: int, grid_w: int, n_txt: int):
    """(img_ids [grid_h * grid_w, 4], txt_ids [n_txt, 4]) int32: image token (r, c) of the
    packed grid has id (0, r, c, 0) in row-major order, text token i has (0, 0, 0, i).
    [DIFF] 位置 id (4-D (T, H, W, L) ids shared by the batch); the tiny shape example's
    (0, row, col, 0) image ids on an 8 x 8 grid."""
    img = np.zeros((grid_h * grid_w, 4), dtype=np.int32)
    for r in range(grid_h):
        img[r * grid_w:(r + 1) * grid_w, 1] = r
        img[r * grid_w:(r + 1) * grid_w, 2] = np.arange(grid_w)
    txt = np.zeros((n_txt, 4), dtype=np.int32)
    txt[:, 3] = np.arange(n_txt)
    return img, txt


def uniform_sigmas(n_steps: int) -> np.ndarray:
    """n_steps + 1 noise levels 1 - i / n_steps (fp32), from pure noise (t = 1) to data
    (t = 0).  Reading: the pages name the flow-matching Euler scheduler but neither its
    schedule nor a shift; this is the plain uniform grid."""
    if n_steps <= 0:
        raise ValueError("n_steps must be > 0")
    return (1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps).astype(np.float32)


def cfg_combine(v_cond, v_uncond, scale: float) -> np.ndarray:
    """v_u + scale (v_c - v_u).  Reading: the pages say the base model needs the two
    forwards of classifier-free guidance (and that distillation removes them) but not how
    they are combined; this is the standard combination."""
    v_u = f64(v_uncond)
    return v_u + float(scale) * (f64(v_cond) - v_u)


def denoise(noise, ctx, w: Mapping, sigmas, n_double: int, n_single: int, ctx_uncond=None,
            guidance: float = 1.0, model_input=None, storage=None, on_step=None) -> np.ndarray:
    """Rectified-flow Euler sampling: [B, C, H, W] noise latent -> [B, C, H, W] latent.

    x_0 = pack(noise); for i < n: v_i = velocity of the denoiser step at x_i, t = sigma_i;
    x_{i+1} = x_i + (sigma_{i+1} - sigma_i) v_i; result unpack(x_n).  With ctx_uncond the
    velocity is cfg_combine(step(ctx), step(ctx_uncond), guidance).  Position ids are
    generation_ids of the packed grid and the text length.  `model_input(x)` maps the
    state to the values the step reads (e.g. bf16 rounding for a bf16 model; default:
    the state itself); `storage` is passed to the step.  `on_step(i)` reports progress.
    """
    sig = np.asarray(sigmas, dtype=np.float32).astype(np.float64)
    noise = f64(noise)
    B, C, H, W = noise.shape
    img_ids, txt_ids = generation_ids(H // 2, W // 2, np.shape(ctx)[1])
    feed = model_input or (lambda a: a)
    x = pack_latents(noise)
    for i in range(len(sig) - 1):
        t = np.full((B,), sig[i], dtype=np.float32)
        xi = feed(x)
        v = denoiser_step(xi, ctx, t, w, img_ids, txt_ids, n_double, n_single, storage=storage)
        if ctx_uncond is not None:
            vu = denoiser_step(xi, ctx_uncond, t, w, img_ids, txt_ids, n_double, n_single,
                               storage=storage)
            v = cfg_combine(v, vu, guidance)
        x = x + (sig[i + 1] - sig[i]) * v
        if on_step:
            on_step(i)
    return unpack_latents(x, H, W)


# ----------------------------------------------------------------------------------
# Reference-image K/V cache
#
# [DIFF] 参考图 KV 缓存机制: a per-layer cache (Flux2KVLayerCache) keeps the reference
# tokens' K and V after RoPE, for every double and single block.  Extract mode (first
# denoising step): sequence [txt, ref, img]; reference tokens attend only to reference
# tokens, text and image tokens attend to every token; reference tokens are modulated at a
# fixed timestep (ref_fixed_timestep, default 0.0), placed by position beside the image
# modulation; the reference K/V are stored.  Cached mode (later steps): sequence
# [txt, img]; the cached reference K/V are inserted between the text and image keys.
# [KLEIN] Infra (KV 缓存): step 0 extracts, later steps reuse the reference K/V.
# Reading: reference image j (0-based) has ids (1 + j, r, c, 0) on its own packed grid.
# ----------------------------------------------------------------------------------
def attention_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed=None,
                     storage=None) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v per head, each query over the keys `allowed[q, :]` marks
    (all keys when None).  q [B, Lq, h, d], k and v [B, Lk, h, d] -> [B, Lq, h*d].
    `storage` as for attention()."""
    B, Lq, h, d = q.shape
    out = np.empty((B, Lq, h, d), dtype=np.float64)
    for b in range(B):
        for head in range(h):
            sc = np.matmul(q[b, :, head, :], k[b, :, head, :].T) / np.sqrt(d)
            if allowed is not None:
                sc = np.where(allowed, sc, -np.inf)
            e = np.exp(sc - sc.max(axis=-1, keepdims=True))
            if storage is not None:
                e = storage(e)
            out[b, :, head, :] = np.matmul(e, v[b, :, head, :]) / e.sum(axis=-1, keepdims=True)
    return out.reshape(B, Lq, h * d)


def reference_ids(n_refs: int, grid_h: int, grid_w: int) -> np.ndarray:
    """[n_refs * grid_h * grid_w, 4] int32: token (r, c) of reference j -> (1 + j, r, c, 0)."""
    img, _ = generation_ids(grid_h, grid_w, 0)
    out = np.concatenate([img] * n_refs) if n_refs else np.zeros((0, 4), np.int32)
    out[:, 0] = np.repeat(np.arange(1, n_refs + 1, dtype=np.int32), grid_h * grid_w)
    return out


def _ln_rows(x, segments, shift_idx, scale_idx):
    """LayerNorm + modulate where consecutive row segments [(n_rows, mods), ...] use their own
    modulation set."""
    parts, r0 = [], 0
    for n, m in segments:
        parts.append(layernorm_modulate(x[:, r0:r0 + n], m[shift_idx], m[scale_idx]))
        r0 += n
    return np.concatenate(parts, axis=1)


def _gate_rows(y, segments, gate_idx):
    parts, r0 = [], 0
    for n, m in segments:
        parts.append(m[gate_idx][:, None, :] * y[:, r0:r0 + n])
        r0 += n
    return np.concatenate(parts, axis=1)


def step_extract(x, ref_x, ctx, t, w: Mapping, img_ids, ref_ids, txt_ids, n_double: int,
                 n_single: int, t_ref: float = 0.0, storage=None):
    """Extract-mode denoiser step over [txt, ref, img] -> (out [B, N_img, in_ch], cache).

    cache[l] = (K, V) of the reference tokens at block l (double blocks first, then single
    blocks): K after RMSNorm + RoPE and V, each [B, N_ref, h, 128].  `storage` as for
    denoiser_step.
    """
    st = storage or _keep
    B = np.shape(x)[0]
    mods = step_mods(t, w)
    mods_r = step_mods(np.full((B,), t_ref, dtype=np.float32), w)
    txt = linear(f64(ctx), f64(w["txt_in"]))
    ref = linear(f64(ref_x), f64(w["img_in"]))
    img = linear(f64(x), f64(w["img_in"]))
    Nt, Nr, Ni = txt.shape[1], ref.shape[1], img.shape[1]
    L = Nt + Nr + Ni
    pos = rope_positions(txt_ids, np.concatenate([_ids2d(ref_ids), _ids2d(img_ids)]))
    allowed = np.ones((L, L), dtype=bool)
    allowed[Nt:Nt + Nr, :] = False
    allowed[Nt:Nt + Nr, Nt:Nt + Nr] = True
    cache = []
    for i in range(n_double):
        wd = _Prefixed(w, f"double.{i}.")
        # text stream alone; image stream = [ref ; img] rows with per-segment modulation
        seg = {"txt": [(Nt, mods["double"]["txt"])],
               "img": [(Nr, mods_r["double"]["img"]), (Ni, mods["double"]["img"])]}
        xs = {"txt": txt, "img": np.concatenate([ref, img], axis=1)}
        qs, ks, vs = {}, {}, {}
        for s in ("txt", "img"):
            a = st(_ln_rows(xs[s], seg[s], 0, 1))
            q, k, v = (st(y) for y in np.split(linear(a, f64(wd[f"{s}.qkv"])), 3, axis=-1))
            qs[s] = rms_norm(_heads(q), f64(wd[f"{s}.q_norm"]))
            ks[s] = rms_norm(_heads(k), f64(wd[f"{s}.k_norm"]))
            vs[s] = _heads(v)
        q = st(apply_rope(np.concatenate([qs["txt"], qs["img"]], axis=1), pos))
        k = st(apply_rope(np.concatenate([ks["txt"], ks["img"]], axis=1), pos))
        v = np.concatenate([vs["txt"], vs["img"]], axis=1)
        cache.append((k[:, Nt:Nt + Nr], v[:, Nt:Nt + Nr]))
        o = st(attention_masked(q, k, v, allowed, storage))
        o_s = {"txt": o[:, :Nt], "img": o[:, Nt:]}
        for s in ("txt", "img"):
            xx = xs[s] + _gate_rows(linear(o_s[s], f64(wd[f"{s}.out"])), seg[s], 2)
            u = linear(st(_ln_rows(xx, seg[s], 3, 4)), f64(wd[f"{s}.mlp_in"]))
            xs[s] = xx + _gate_rows(linear(st(swiglu(u)), f64(wd[f"{s}.mlp_out"])), seg[s], 5)
        txt, ref, img = xs["txt"], xs["img"][:, :Nr], xs["img"][:, Nr:]
    seg = [(Nt, mods["single"]), (Nr, mods_r["single"]), (Ni, mods["single"])]
    h = np.concatenate([txt, ref, img], axis=1)
    D = h.shape[-1]
    for i in range(n_single):
        ws = _Prefixed(w, f"single.{i}.")
        y = linear(st(_ln_rows(h, seg, 0, 1)), f64(ws["linear1"]))
        q, k, v, u = st(y[..., :D]), st(y[..., D:2 * D]), st(y[..., 2 * D:3 * D]), y[..., 3 * D:]
        q = st(apply_rope(rms_norm(_heads(q), f64(ws["q_norm"])), pos))
        k = st(apply_rope(rms_norm(_heads(k), f64(ws["k_norm"])), pos))
        v = _heads(v)
        cache.append((k[:, Nt:Nt + Nr], v[:, Nt:Nt + Nr]))
        o = st(attention_masked(q, k, v, allowed, storage))
        h = h + _gate_rows(linear(np.concatenate([o, st(swiglu(u))], axis=-1),
                                  f64(ws["linear2"])), seg, 2)
    shift_f, scale_f = mods["final"]
    out = linear(st(layernorm_modulate(h[:, Nt + Nr:], shift_f, scale_f)), f64(w["proj_out"]))
    return out, cache


def step_cached(x, ctx, t, w: Mapping, img_ids, txt_ids, cache, n_double: int, n_single: int,
                storage=None) -> np.ndarray:
    """Cached-mode denoiser step over [txt, img]: at block l the keys and values are
    [txt ; cached reference ; img] (cache[l] as returned by step_extract)."""
    st = storage or _keep
    mods = step_mods(t, w)
    txt = linear(f64(ctx), f64(w["txt_in"]))
    img = linear(f64(x), f64(w["img_in"]))
    Nt = txt.shape[1]
    pos = rope_positions(txt_ids, img_ids)

    def inject(kv, l):
        return tuple(np.concatenate([a[:, :Nt], f64(c), a[:, Nt:]], axis=1)
                     for a, c in zip(kv, cache[l]))

    for i in range(n_double):
        wd = _Prefixed(w, f"double.{i}.")
        xs = {"txt": txt, "img": img}
        qs, ks, vs = {}, {}, {}
        for s in ("txt", "img"):
            m = mods["double"][s]
            a = st(layernorm_modulate(xs[s], m[0], m[1]))
            q, k, v = (st(y) for y in np.split(linear(a, f64(wd[f"{s}.qkv"])), 3, axis=-1))
            qs[s] = rms_norm(_heads(q), f64(wd[f"{s}.q_norm"]))
            ks[s] = rms_norm(_heads(k), f64(wd[f"{s}.k_norm"]))
            vs[s] = _heads(v)
        q = st(apply_rope(np.concatenate([qs["txt"], qs["img"]], axis=1), pos))
        k = st(apply_rope(np.concatenate([ks["txt"], ks["img"]], axis=1), pos))
        v = np.concatenate([vs["txt"], vs["img"]], axis=1)
        k, v = inject((k, v), i)
        o = st(attention_masked(q, k, v, None, storage))
        o_s = {"txt": o[:, :Nt], "img": o[:, Nt:]}
        for s in ("txt", "img"):
            _, _, g1, s2, c2, g2 = mods["double"][s]
            xx = xs[s] + g1[:, None, :] * linear(o_s[s], f64(wd[f"{s}.out"]))
            u = linear(st(layernorm_modulate(xx, s2, c2)), f64(wd[f"{s}.mlp_in"]))
            xs[s] = xx + g2[:, None, :] * linear(st(swiglu(u)), f64(wd[f"{s}.mlp_out"]))
        txt, img = xs["txt"], xs["img"]
    shift, scale, gate = mods["single"]
    h = np.concatenate([txt, img], axis=1)
    D = h.shape[-1]
    for i in range(n_single):
        ws = _Prefixed(w, f"single.{i}.")
        y = linear(st(layernorm_modulate(h, shift, scale)), f64(ws["linear1"]))
        q, k, v, u = st(y[..., :D]), st(y[..., D:2 * D]), st(y[..., 2 * D:3 * D]), y[..., 3 * D:]
        q = st(apply_rope(rms_norm(_heads(q), f64(ws["q_norm"])), pos))
        k = st(apply_rope(rms_norm(_heads(k), f64(ws["k_norm"])), pos))
        k, v = inject((k, _heads(v)), n_double + i)
        o = st(attention_masked(q, k, v, None, storage))
        h = h + gate[:, None, :] * linear(np.concatenate([o, st(swiglu(u))], axis=-1),
                                          f64(ws["linear2"]))
    shift_f, scale_f = mods["final"]
    return linear(st(layernorm_modulate(h[:, Nt:], shift_f, scale_f)), f64(w["proj_out"]))


def denoise_with_refs(noise, refs, ctx, w: Mapping, sigmas, n_double: int, n_single: int,
                      use_cache: bool = True, model_input=None, on_step=None) -> np.ndarray:
    """denoise() conditioned on reference latents refs [B, R, C, Hr, Wr]: the first step
    runs in extract mode, later steps in cached mode (use_cache) or again in extract mode
    (every step recomputes the references).  Reference j has ids (1 + j, r, c, 0)."""
    sig = np.asarray(sigmas, dtype=np.float32).astype(np.float64)
    noise = f64(noise)
    refs = f64(refs)
    B, C, H, W = noise.shape
    R, Hr, Wr = refs.shape[1], refs.shape[3], refs.shape[4]
    ref_x = np.concatenate([pack_latents(refs[:, j]) for j in range(R)], axis=1)
    ref_ids = reference_ids(R, Hr // 2, Wr // 2)
    img_ids, txt_ids = generation_ids(H // 2, W // 2, np.shape(ctx)[1])
    feed = model_input or (lambda a: a)
    rin = feed(ref_x)
    x = pack_latents(noise)
    cache = None
    for i in range(len(sig) - 1):
        t = np.full((B,), sig[i], dtype=np.float32)
        if cache is None or not use_cache:
            v, cache = step_extract(feed(x), rin, ctx, t, w, img_ids, ref_ids, txt_ids,
                                    n_double, n_single)
        else:
            v = step_cached(feed(x), ctx, t, w, img_ids, txt_ids, cache, n_double, n_single)
        x = x + (sig[i + 1] - sig[i]) * v
        if on_step:
            on_step(i)
    return unpack_latents(x, H, W)


# ----------------------------------------------------------------------------------
# FP8 (E4M3) linear layer
#
# [KLEIN] Infra (量化): the pages report FP8 versions of the models and their speed-ups but
# give no recipe.  Reading: OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
# bits; largest finite 448, no infinities, S.1111.111 is NaN); values are scaled into
# range per activation row and per weight row (output channel) by amax / 448, rounded to
# nearest even with saturation at 448; the layer is y = s_a[m] s_w[n] sum_k qa[m, k] qw[n, k]
# with fp32 accumulation of the exact fp8 products.
# ----------------------------------------------------------------------------------
FP8_MAX = 448.0


def fp8_decode(code) -> np.ndarray:
    """E4M3 byte -> float64 (NaN for the NaN codes)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * val)


def fp8_encode(x) -> np.ndarray:
    """float -> E4M3 byte, round to nearest (ties to even mantissa), magnitudes past 448
    saturate to 448; NaN -> 0x7F.  Works on the exact value of x (x in float64): the
    magnitude is written as n * 2^(e-3) in its binade e (e >= -6; below 2^-6 the subnormal
    spacing 2^-9 is the binade -6 spacing), n rounded to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), FP8_MAX)
    with np.errstate(divide="ignore"):
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
    # guard log2 rounding at binade edges
    e = np.where((np.exp2(e) > a) & (e > -6) & (a > 0), e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    q = a / np.exp2(e) * 8.0                       # in [8, 16) for normals, [0, 8) below
    n = np.floor(q)
    r = q - n
    n = n + ((r > 0.5) | ((r == 0.5) & (n % 2 == 1)))
    e = np.where(n == 16, e + 1, e)
    n = np.where(n == 16, 8, n)
    code = np.where((e == -6) & (n < 8), n, (e + 7) * 8 + (n - 8)).astype(np.int64)
    code = np.where(a == 0, 0, np.minimum(code, 0x7E))
    return np.where(nan, 0x7F, sign | code).astype(np.uint8)


def quantize_rows_fp8(x):
    """Per-row E4M3 quantization: dequantization scale s = amax(|row|) / 448 and
    quantization multiplier r = 448 / amax (both fp32, correctly rounded; s = r = 1 for an
    all-zero row), q = encode(fp32(x * r)).  Returns (q uint8, s float32)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1.0)).astype(np.float32)
    s = np.where(pos, safe / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    r = np.where(pos, np.float32(FP8_MAX) / safe, np.float32(1.0)).astype(np.float32)
    q = fp8_encode((x32 * r[..., None]).astype(np.float32).astype(np.float64))
    return q, s


def linear_fp8(qa, sa, qw, sw) -> np.ndarray:
    """y[m, n] = sa[m] sw[n] sum_k dec(qa[m, k]) dec(qw[n, k]), exactly (float64)."""
    return (fp8_decode(qa) * f64(sa)[..., None]) @ (fp8_decode(qw) * f64(sw)[..., None]).T
