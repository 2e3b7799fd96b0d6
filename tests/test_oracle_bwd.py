"""The fp64 backward oracle against its pins, and planted mistakes in it.

Each mutant replaces one function of oracle/backward.py (on the CPU, inside
this process only) with a plausible wrong variant: a dropped term, a wrong
sign, a transposed operand, a missing group sum. Some pin must reject it.
"""
import math

import numpy as np
import pytest

import oracle.backward as BW
import oracle.reference as R
from oracle_bwd_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_oracle_pin(pin):
    pin(BW)


def _rope_bwd_plus(dy, positions, base):
    return R.rope(dy, positions, base)        # rotates by +p*theta: the wrong sign


def _rope_bwd_skipped(dy, positions, base):
    return R._f64(dy)


def _norm_bwd_no_projection(x, dy, eps=1e-6):
    x, dy = R._f64(x), R._f64(dy)
    return dy / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _norm_bwd_sum(x, dy, eps=1e-6):
    x, dy = R._f64(x), R._f64(dy)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * np.sum(dy * y, axis=-1, keepdims=True))


def _core_variant(kind):
    def core(qn, kn, v, do, W):
        qn, kn, v, do = R._f64(qn), R._f64(kn), R._f64(v), R._f64(do)
        B, T, H, D = qn.shape
        G = H // kn.shape[2]
        vis = R.band_mask(T, W)
        sc = 1.0 / math.sqrt(D)
        dq, dk, dv = np.zeros_like(qn), np.zeros_like(kn), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                g = h // G
                S = np.where(vis, (qn[b, :, h] @ kn[b, :, g].T) * sc, -np.inf)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                dP = do[b, :, h] @ v[b, :, g].T
                if kind == "no_delta":
                    dS = P * dP
                else:
                    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
                if kind == "dv_not_transposed":
                    dv[b, :, g] += P @ do[b, :, h]
                elif kind == "gqa_not_summed":
                    dv[b, :, g] = P.T @ do[b, :, h]
                else:
                    dv[b, :, g] += P.T @ do[b, :, h]
                dq[b, :, h] = (dS @ kn[b, :, g]) * (1.0 if kind == "no_scale" else sc)
                if kind == "dk_not_transposed":
                    dk[b, :, g] += (dS @ qn[b, :, h]) * sc
                elif kind == "gqa_not_summed":
                    dk[b, :, g] = (dS.T @ qn[b, :, h]) * sc
                else:
                    dk[b, :, g] += (dS.T @ qn[b, :, h]) * sc
        return dq, dk, dv
    return core


def _bwd_norm_of_normalised(q, k, v, do, window, base=10000.0, pos_offset=0):
    # the norm's backward taken at the normalised rows instead of its input
    q, k = R._f64(q), R._f64(k)
    pos = (pos_offset + np.arange(q.shape[1]))[None, :, None]
    qn, kn = R.qk_norm(R.rope(q, pos, base)), R.qk_norm(R.rope(k, pos, base))
    dqn, dkn, dv = BW.attention_core_bwd(qn, kn, v, do, window)
    return (BW.rope_bwd(BW.qk_norm_bwd(qn, dqn), pos, base),
            BW.rope_bwd(BW.qk_norm_bwd(kn, dkn), pos, base), dv)


def _lse_log2(q, k, v, window, base=10000.0, pos_offset=0):
    o, lse = _orig_lse(q, k, v, window, base, pos_offset)
    return o, lse / math.log(2.0)


_orig_lse = BW.attn_fwd_lse

MUTANTS = {
    "rope_bwd_wrong_sign": ("rope_bwd", _rope_bwd_plus),
    "rope_bwd_skipped": ("rope_bwd", _rope_bwd_skipped),
    "norm_bwd_no_projection": ("qk_norm_bwd", _norm_bwd_no_projection),
    "norm_bwd_sum_not_mean": ("qk_norm_bwd", _norm_bwd_sum),
    "core_no_delta": ("attention_core_bwd", _core_variant("no_delta")),
    "core_dv_not_transposed": ("attention_core_bwd", _core_variant("dv_not_transposed")),
    "core_dk_not_transposed": ("attention_core_bwd", _core_variant("dk_not_transposed")),
    "core_no_scale": ("attention_core_bwd", _core_variant("no_scale")),
    "core_gqa_not_summed": ("attention_core_bwd", _core_variant("gqa_not_summed")),
    "bwd_norm_at_output": ("attn_bwd", _bwd_norm_of_normalised),
    "lse_in_log2": ("attn_fwd_lse", _lse_log2),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(BW, attr, fn)
    caught = []
    for pin in ALL_BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(BW)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
