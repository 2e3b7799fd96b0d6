"""Planted mistakes in the oracle must each be caught by at least one pin.

Each mutant below replaces one function of the oracle (on the CPU, inside this
process only) with a plausible wrong variant: a dropped term, a wrong sign or
index, a transposed operand.  The test passes when some pin in ALL_PINS
rejects the mutant; this shows the pins constrain every step of the oracle.
"""
import math

import numpy as np
import pytest

import oracle.reference as R
from oracle_pins import ALL_PINS


def _rope_sign(x, positions, base):
    x = R._f64(x)
    D = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[..., None] * R.rope_inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _rope_half_split(x, positions, base):
    x = R._f64(x)
    D = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[..., None] * R.rope_inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _inv_freq_wrong(D, base):
    return np.power(float(base), -np.arange(D // 2, dtype=np.float64) / D)


_orig_rope = R.rope


def _rope_pos_plus_one(x, positions, base):
    return _orig_rope(x, np.asarray(positions) + 1, base)


def _norm_sum(x, eps=1e-6):
    x = R._f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _norm_eps_outside(x, eps=1e-6):
    x = R._f64(x)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)


def _rope_qknorm_no_k_norm(q, k, base=10000.0, pos_offset=0):
    q, k = R._f64(q), R._f64(k)
    pos = (pos_offset + np.arange(q.shape[1]))[None, :, None]
    return R.qk_norm(R.rope(q, pos, base)), R.rope(k, pos, base)


def _rope_qknorm_norm_q_before_no_rope(q, k, base=10000.0, pos_offset=0):
    q, k = R._f64(q), R._f64(k)
    pos = (pos_offset + np.arange(q.shape[1]))[None, :, None]
    return R.qk_norm(q), R.qk_norm(R.rope(k, pos, base))


def _mask_off_by_one(T, W):
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return ((i - j) >= 0) & ((i - j) <= W)


def _mask_anti_causal(T, W):
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return ((j - i) >= 0) & ((j - i) < W)


def _core_variant(kind):
    def core(qn, kn, v, W, return_probs=False):
        qn, kn, v = R._f64(qn), R._f64(kn), R._f64(v)
        B, T, H, D = qn.shape
        Hkv = kn.shape[2]
        G = H // Hkv
        vis = R.band_mask(T, W)
        out = np.empty((B, T, H, D))
        probs = np.empty((B, H, T, T)) if return_probs else None
        for b in range(B):
            for h in range(H):
                g = (h % Hkv) if kind == "gqa_mod" else h // G
                S = qn[b, :, h, :] @ kn[b, :, g, :].T
                if kind == "transposed":
                    S = S.T
                if kind != "no_scale":
                    S = S / math.sqrt(D)
                S = np.where(vis, S, -np.inf)
                ax = 0 if kind == "softmax_axis" else 1
                E = np.exp(S - np.max(np.where(np.isfinite(S), S, -1e300), axis=ax,
                                      keepdims=True))
                E = np.where(vis, E, 0.0)
                P = E / np.maximum(E.sum(axis=ax, keepdims=True), 1e-300)
                out[b, :, h, :] = P @ v[b, :, g, :]
                if return_probs:
                    probs[b, h] = P
        return (out, probs) if return_probs else out
    return core


_orig_decode = R.attn_decode


def _decode_raw_append(q, k_new, v_new, k_cache, v_cache, seqlens, window, base=10000.0, **kw):
    # appends the raw key instead of the rotated, normalised one
    o, kc, vc = _orig_decode(q, k_new, v_new, k_cache, v_cache, seqlens, window, base, **kw)
    k_new = R._f64(k_new)
    for b, L in enumerate(np.asarray(R._f64(seqlens), dtype=np.int64)):
        kc[b, L - 1] = k_new[b]
    return o, kc, vc


def _decode_window_plus_one(q, k_new, v_new, k_cache, v_cache, seqlens, window, base=10000.0, **kw):
    return _orig_decode(q, k_new, v_new, k_cache, v_cache, seqlens, window + 1, base, **kw)


_orig_prefill = R.attn_prefill


def _prefill_local_mask(q, k, v, k_cache, v_cache, window, base=10000.0, pos_offset=0, ve=None,
                        ve_gate=None):
    # masks with the chunk-local query index t instead of the position P + t
    qf, kf, vf = R._f64(q), R._f64(k), R.value_gate(v, ve, ve_gate)
    kc, vc = R._f64(k_cache).copy(), R._f64(v_cache).copy()
    B, T, H, D = qf.shape
    G = H // kf.shape[2]
    P = int(pos_offset)
    qn, kn = R.rope_qknorm(qf, kf, base, P)
    kc[:, P:P + T] = kn
    vc[:, P:P + T] = vf
    i = np.arange(T)[:, None]
    j = np.arange(P + T)[None, :]
    vis = (i - j >= 0) & (i - j < window)
    o = np.empty((B, T, H, D))
    for b in range(B):
        for h in range(H):
            S = np.where(vis, qn[b, :, h] @ kc[b, :P + T, h // G].T / math.sqrt(D), -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            o[b, :, h] = (E / E.sum(axis=1, keepdims=True)) @ vc[b, :P + T, h // G]
    return o, kc, vc


def _shifted_prefill(q, k, v, k_cache, v_cache, window, base, P):
    qf, kf = R._f64(q), R._f64(k)
    T = qf.shape[1]
    qn0, kn0 = R.rope_qknorm(qf, kf, base, 0)
    kc, vc = R._f64(k_cache).copy(), R._f64(v_cache).copy()
    kc[:, P:P + T] = kn0
    vc[:, P:P + T] = R._f64(v)
    B, _, H, D = qf.shape
    G = H // kf.shape[2]
    i = P + np.arange(T)[:, None]
    j = np.arange(P + T)[None, :]
    vis = (i - j >= 0) & (i - j < window)
    o = np.empty((B, T, H, D))
    for b in range(B):
        for h in range(H):
            S = np.where(vis, qn0[b, :, h] @ kc[b, :P + T, h // G].T / math.sqrt(D), -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            o[b, :, h] = (E / E.sum(axis=1, keepdims=True)) @ vc[b, :P + T, h // G]
    return o, kc, vc


def _shifted_prefill_entry(q, k, v, k_cache, v_cache, window, base=10000.0, pos_offset=0, ve=None,
                           ve_gate=None):
    # rotates the chunk as if it started at position 0
    return _shifted_prefill(q, k, R.value_gate(v, ve, ve_gate), k_cache, v_cache, window, base,
                            int(pos_offset))


def _prefill_window_plus_one(q, k, v, k_cache, v_cache, window, base=10000.0, pos_offset=0, **kw):
    return _orig_prefill(q, k, v, k_cache, v_cache, window + 1, base, pos_offset, **kw)


def _prefill_no_v_append(q, k, v, k_cache, v_cache, window, base=10000.0, pos_offset=0, **kw):
    o, kc, _ = _orig_prefill(q, k, v, k_cache, v_cache, window, base, pos_offset, **kw)
    return o, kc, R._f64(v_cache).copy()


_orig_decode_shared = R.attn_decode_shared


def _decode_shared_row_off_by_one(q, k_new, v_new, k_prompt, v_prompt, k_cache, v_cache, seqlens,
                                  window, base=10000.0, **kw):
    # reads the samples' own rows one row late (position p from row p - Lp + 1)
    kc = np.roll(R._f64(k_cache), -1, axis=1)
    vc = np.roll(R._f64(v_cache), -1, axis=1)
    return _orig_decode_shared(q, k_new, v_new, k_prompt, v_prompt, kc, vc, seqlens, window, base, **kw)


def _value_gate_on_v(v, ve, gate):
    # scales v by the gate instead of adding the gated embedding
    v = R._f64(v)
    return v if ve is None else v * R._f64(gate)[..., None] + R._f64(ve)


def _value_gate_dropped(v, ve, gate):
    return R._f64(v)


MUTANTS = {
    "rope_sign": ("rope", _rope_sign),
    "rope_half_split": ("rope", _rope_half_split),
    "rope_inv_freq": ("rope_inv_freq", _inv_freq_wrong),
    "rope_pos_plus_one": ("rope", _rope_pos_plus_one),
    "norm_sum_not_mean": ("qk_norm", _norm_sum),
    "norm_eps_outside_sqrt": ("qk_norm", _norm_eps_outside),
    "no_k_norm": ("rope_qknorm", _rope_qknorm_no_k_norm),
    "no_q_rope": ("rope_qknorm", _rope_qknorm_norm_q_before_no_rope),
    "mask_off_by_one": ("band_mask", _mask_off_by_one),
    "mask_anti_causal": ("band_mask", _mask_anti_causal),
    "core_no_scale": ("attention_core", _core_variant("no_scale")),
    "core_gqa_mod": ("attention_core", _core_variant("gqa_mod")),
    "core_transposed": ("attention_core", _core_variant("transposed")),
    "core_softmax_axis": ("attention_core", _core_variant("softmax_axis")),
    "decode_raw_append": ("attn_decode", _decode_raw_append),
    "decode_window_plus_one": ("attn_decode", _decode_window_plus_one),
    "prefill_local_mask": ("attn_prefill", _prefill_local_mask),
    "prefill_rope_from_zero": ("attn_prefill", _shifted_prefill_entry),
    "prefill_window_plus_one": ("attn_prefill", _prefill_window_plus_one),
    "prefill_no_v_append": ("attn_prefill", _prefill_no_v_append),
    "decode_shared_row_off_by_one": ("attn_decode_shared", _decode_shared_row_off_by_one),
    "value_gate_on_v": ("value_gate", _value_gate_on_v),
    "value_gate_dropped": ("value_gate", _value_gate_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(R)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
