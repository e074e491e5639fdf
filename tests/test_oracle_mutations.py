"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation replaces one oracle function with a subtly wrong variant for the duration
of one check; the pins of tests/test_oracle_pins.py are then run and at least one of
them must fail.  This shows the pins are strong enough that the oracle cannot be wrong
in these ways and still pass.
"""
import inspect

import numpy as np
import pytest

import tests.test_oracle_pins as pins
from oracle import flux_oracle as O

PIN_FUNCS = [f for n, f in inspect.getmembers(pins, inspect.isfunction)
             if n.startswith("test_") and "manifest" not in n]


def _mut_rope_sign(x, pos):
    phi = pos.astype(np.float64) * O.rope_frequencies()[None, :]
    c, s = np.cos(phi)[None, :, None, :], np.sin(phi)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _mut_rope_halves(x, pos):
    # rotate (i, i + 64) pairs instead of adjacent pairs
    phi = pos.astype(np.float64) * O.rope_frequencies()[None, :]
    c, s = np.cos(phi)[None, :, None, :], np.sin(phi)[None, :, None, :]
    a, b = x[..., :64], x[..., 64:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _mut_freq():
    return np.concatenate([O.ROPE_THETA ** (-np.arange(d // 2) / d) for d in O.AXES_DIM])


def _mut_positions(txt_ids, img_ids):
    return _orig["rope_positions"](img_ids, txt_ids) if len(txt_ids) == len(img_ids) else \
        np.concatenate([O._ids2d(img_ids), O._ids2d(txt_ids)])[:, np.repeat(np.arange(4), 16)]


def _mut_ln_unbiased(x, shift, scale, eps=O.EPS):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).sum(-1, keepdims=True) / max(x.shape[-1] - 1, 1)
    return (1 + scale[:, None, :]) * (x - mu) / np.sqrt(var + eps) + shift[:, None, :]


def _mut_ln_eps_out(x, shift, scale, eps=O.EPS):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (1 + scale[:, None, :]) * (x - mu) / (np.sqrt(var) + eps) + shift[:, None, :]


def _mut_ln_no_one(x, shift, scale, eps=O.EPS):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return scale[:, None, :] * (x - mu) / np.sqrt(var + eps) + shift[:, None, :]


def _mut_rms_sum(x, gamma, eps=O.EPS):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps) * gamma


def _mut_attn_scale(q, k):
    return O.softmax_rows(q @ k.T / q.shape[-1])


def _mut_attn_transposed(q, k):
    s = q @ k.T / np.sqrt(q.shape[-1])
    e = np.exp(s - s.max(0, keepdims=True))
    return e / e.sum(0, keepdims=True)


def _mut_swiglu(u):
    H = u.shape[-1] // 2
    return O.silu(u[..., H:]) * u[..., :H]


def _mut_temb_sin_cos(t):
    e = _orig["timestep_embedding"](t)
    return np.concatenate([e[:, 128:], e[:, :128]], axis=1)


def _mut_temb_no_scale(t):
    return _orig["timestep_embedding"](np.asarray(t, dtype=np.float64) / 1000.0)


def _mut_silu(x):
    return x / (1.0 + np.exp(x))


def _mut_mod_reversed(temb, w_mod, n):
    return _orig["modulation"](temb, w_mod, n)[::-1]


def _mut_single_qk_swap(img, txt, t, w, img_ids, txt_ids, mods=None):
    D = np.asarray(txt).shape[-1]
    w2 = dict(w)
    l1 = np.asarray(w["linear1"], dtype=np.float64).copy()
    l1[:D], l1[D:2 * D] = l1[D:2 * D].copy(), l1[:D].copy()
    w2["linear1"] = l1
    return _orig["single_block"](img, txt, t, w2, img_ids, txt_ids, mods)


def _mut_single_concat(img, txt, t, w, img_ids, txt_ids, mods=None):
    D = np.asarray(txt).shape[-1]
    w2 = dict(w)
    l2 = np.asarray(w["linear2"], dtype=np.float64)
    w2["linear2"] = np.concatenate([l2[:, -D:], l2[:, :-D]], axis=1)
    return _orig["single_block"](img, txt, t, w2, img_ids, txt_ids, mods)


_orig = {}

MUTATIONS = {
    "rope_rotation_sign": ("apply_rope", _mut_rope_sign),
    "rope_half_split_pairs": ("apply_rope", _mut_rope_halves),
    "rope_frequency_exponent": ("rope_frequencies", _mut_freq),
    "rope_image_ids_first": ("rope_positions", _mut_positions),
    "layernorm_unbiased_variance": ("layernorm_modulate", _mut_ln_unbiased),
    "layernorm_eps_outside_root": ("layernorm_modulate", _mut_ln_eps_out),
    "modulate_without_one_plus": ("layernorm_modulate", _mut_ln_no_one),
    "rmsnorm_sum_not_mean": ("rms_norm", _mut_rms_sum),
    "attention_scale_1_over_d": ("attention_weights", _mut_attn_scale),
    "softmax_over_query_axis": ("attention_weights", _mut_attn_transposed),
    "swiglu_halves_swapped": ("swiglu", _mut_swiglu),
    "sinusoid_sin_first": ("timestep_embedding", _mut_temb_sin_cos),
    "sinusoid_missing_x1000": ("timestep_embedding", _mut_temb_no_scale),
    "silu_sign": ("silu", _mut_silu),
    "modulation_chunks_reversed": ("modulation", _mut_mod_reversed),
    "single_q_k_split_swapped": ("single_block", _mut_single_qk_swap),
    "single_concat_mlp_first": ("single_block", _mut_single_concat),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    _orig.clear()
    _orig.update({k: getattr(O, k) for k in ("rope_positions", "timestep_embedding",
                                             "modulation", "single_block")})
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for f in PIN_FUNCS:
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, ValueError, IndexError):
            failed.append(f.__name__)
        if failed:
            break
    assert failed, f"no pin caught mutation {name}"


# ----------------------------------------------------------------------------------
# Sampling loop: each planted mistake must fail a pin of tests/test_oracle_sampler.py
# ----------------------------------------------------------------------------------
import tests.test_oracle_sampler as spins  # noqa: E402


def _sampler_pins():
    out = []
    for n, f in inspect.getmembers(spins, inspect.isfunction):
        if not n.startswith("test_"):
            continue
        if "shape" in inspect.signature(f).parameters:
            out.append(lambda f=f: f((2, 8, 6, 10)))
        else:
            out.append(f)
    return out


def _mut_pack_channels_last(z):
    z = np.asarray(z, dtype=np.float64)
    B, C, H, W = z.shape
    p = z.reshape(B, C, H // 2, 2, W // 2, 2)
    return p.transpose(0, 2, 4, 3, 5, 1).reshape(B, (H // 2) * (W // 2), 4 * C)


def _mut_pack_column_major(z):
    z = np.asarray(z, dtype=np.float64)
    B, C, H, W = z.shape
    p = z.reshape(B, C, H // 2, 2, W // 2, 2)
    return p.transpose(0, 4, 2, 1, 3, 5).reshape(B, (H // 2) * (W // 2), 4 * C)


def _mut_ids_transposed(gh, gw, n_txt):
    img, txt = _sorig["generation_ids"](gh, gw, n_txt)
    return img[:, [0, 2, 1, 3]], txt


def _mut_sigmas_reversed(n):
    return _sorig["uniform_sigmas"](n)[::-1].copy()


def _mut_cfg_swapped(v_cond, v_uncond, scale):
    return _sorig["cfg_combine"](v_uncond, v_cond, scale)


def _denoise_variant(noise, ctx, w, sigmas, n_double, n_single, ctx_uncond=None, guidance=1.0,
                     model_input=None, storage=None, on_step=None, t_next=False, flip=False,
                     restart=False):
    sig = np.asarray(sigmas, dtype=np.float32).astype(np.float64)
    noise = np.asarray(noise, dtype=np.float64)
    B, C, H, W = noise.shape
    img_ids, txt_ids = O.generation_ids(H // 2, W // 2, np.shape(ctx)[1])
    x0 = O.pack_latents(noise)
    x = x0
    for i in range(len(sig) - 1):
        t = np.full((B,), sig[i + 1] if t_next else sig[i], dtype=np.float32)
        src = x0 if restart else x
        v = O.denoiser_step(src, ctx, t, w, img_ids, txt_ids, n_double, n_single)
        if ctx_uncond is not None:
            v = O.cfg_combine(v, O.denoiser_step(src, ctx_uncond, t, w, img_ids, txt_ids,
                                                 n_double, n_single), guidance)
        d = (sig[i] - sig[i + 1]) if flip else (sig[i + 1] - sig[i])
        x = src + d * v
    return O.unpack_latents(x, H, W)


_sorig = {}

SAMPLER_MUTATIONS = {
    "pack_channel_factor_last": ("pack_latents", _mut_pack_channels_last),
    "pack_patches_column_major": ("pack_latents", _mut_pack_column_major),
    "ids_rows_and_columns_swapped": ("generation_ids", _mut_ids_transposed),
    "sigmas_increasing": ("uniform_sigmas", _mut_sigmas_reversed),
    "cfg_branches_swapped": ("cfg_combine", _mut_cfg_swapped),
    "euler_velocity_at_next_level": ("denoise", lambda *a, **k: _denoise_variant(*a, t_next=True, **k)),
    "euler_step_sign_flipped": ("denoise", lambda *a, **k: _denoise_variant(*a, flip=True, **k)),
    "euler_restarts_from_noise": ("denoise", lambda *a, **k: _denoise_variant(*a, restart=True, **k)),
}


@pytest.mark.parametrize("name", sorted(SAMPLER_MUTATIONS))
def test_sampler_mutation_is_caught(name, monkeypatch):
    attr, fn = SAMPLER_MUTATIONS[name]
    _sorig.clear()
    _sorig.update({k: getattr(O, k) for k in ("generation_ids", "uniform_sigmas", "cfg_combine")})
    monkeypatch.setattr(O, attr, fn)
    failed = False
    for f in _sampler_pins():
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, ValueError, IndexError):
            failed = True
            break
    assert failed, f"no pin caught mutation {name}"


# ----------------------------------------------------------------------------------
# Reference K/V cache: each planted mistake must fail a pin of tests/test_oracle_refkv.py
# ----------------------------------------------------------------------------------
import tests.test_oracle_refkv as rpins  # noqa: E402

_rorig = {}


def _mut_mask_ignored(q, k, v, allowed=None, storage=None):
    return _rorig["attention_masked"](q, k, v, None, storage)


def _mut_ref_ids_same_plane(n_refs, gh, gw):
    ids = _rorig["reference_ids"](n_refs, gh, gw)
    ids[:, 0] -= 1
    return ids


def _mut_ln_rows_first_set(x, segments, shift_idx, scale_idx):
    m0 = segments[0][1]
    return O.layernorm_modulate(x, m0[shift_idx], m0[scale_idx])


def _mut_gate_rows_last_set(y, segments, gate_idx):
    return segments[-1][1][gate_idx][:, None, :] * y


REFKV_MUTATIONS = {
    "reference_queries_see_every_key": ("attention_masked", _mut_mask_ignored),
    "reference_ids_on_the_image_plane": ("reference_ids", _mut_ref_ids_same_plane),
    "one_modulation_set_for_all_rows": ("_ln_rows", _mut_ln_rows_first_set),
    "one_gate_set_for_all_rows": ("_gate_rows", _mut_gate_rows_last_set),
}


@pytest.mark.parametrize("name", sorted(REFKV_MUTATIONS))
def test_refkv_mutation_is_caught(name, monkeypatch):
    attr, fn = REFKV_MUTATIONS[name]
    _rorig.clear()
    _rorig.update({k: getattr(O, k) for k in ("attention_masked", "reference_ids")})
    monkeypatch.setattr(O, attr, fn)
    failed = False
    for n, f in inspect.getmembers(rpins, inspect.isfunction):
        if not n.startswith("test_"):
            continue
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, ValueError, IndexError):
            failed = True
            break
    assert failed, f"no pin caught mutation {name}"


# ----------------------------------------------------------------------------------
# Storage rounding: each planted mistake must fail a pin of tests/test_oracle_storage.py
# ----------------------------------------------------------------------------------
import tests.test_oracle_storage as stpins  # noqa: E402

_orig_bf16 = O.bf16_storage


def _mut_f16_truncates(x):
    x16 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16)
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    up = np.abs(x16.astype(np.float32)) > np.abs(x32)
    x16 = np.where(up, np.nextafter(x16, np.float16(0)), x16)
    return x16.astype(np.float64)


def _mut_f16_is_bf16(x):
    return _orig_bf16(x)


def _mut_bf16_truncates(x):
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _storage_pins():
    pins = [stpins.test_f16_storage_matches_torch_conversion,
            stpins.test_bf16_storage_matches_torch_conversion,
            stpins.test_f16_storage_is_eight_times_finer_than_bf16]
    for x, want in ((1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9), (65520.0, np.inf)):
        pins.append(lambda x=x, want=want: stpins.test_f16_storage_worked_values(x, want))
    for x, want in ((1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6), (1.0 / 3.0, 0.333984375)):
        pins.append(lambda x=x, want=want: stpins.test_bf16_storage_worked_values(x, want))
    return pins


STORAGE_MUTATIONS = {
    "f16_storage_truncates": ("f16_storage", _mut_f16_truncates),
    "f16_storage_is_bf16": ("f16_storage", _mut_f16_is_bf16),
    "bf16_storage_truncates": ("bf16_storage", _mut_bf16_truncates),
}


@pytest.mark.parametrize("name", sorted(STORAGE_MUTATIONS))
def test_storage_mutation_is_caught(name, monkeypatch):
    attr, fn = STORAGE_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for f in _storage_pins():
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, ValueError):
            failed.append(getattr(f, "__name__", "pin"))
            break
    assert failed, f"no pin caught mutation {name}"
