"""The fp64 projection oracle (oracle/projection.py) against facts that do not
come from it, and planted mistakes in it.

Pins: scalar brute force (explicit loops over the input dimension, rotation
and norm written out with the math module) on a tiny case; identity weights
reduce it to oracle.rope_qknorm of x itself; zero weights give zero outputs
(the norm of a zero row is zero); v is linear in x and q', k' do not change
when x is scaled (QK-norm). Each mutant (a transposed weight, a head-major
reshape, the rotation skipped, the norm skipped on k, the norm applied to v)
must fail at least one pin.
"""
import math

import numpy as np
import pytest

import oracle.projection as PR
import oracle.reference as R


def _rng(s):
    return np.random.default_rng(s)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, f"{what}: {err:.3e}"


def pin_brute_force(M):
    r = _rng(1)
    B, T, C, H, Hkv, D = 1, 3, 8, 2, 2, 4  # square weights: a transposed one is caught on values
    x = r.standard_normal((B, T, C))
    wq, wk, wv = r.standard_normal((H * D, C)), r.standard_normal((Hkv * D, C)), r.standard_normal((Hkv * D, C))
    q, k, v = M.qkv_rope_qknorm(x, wq, wk, wv, H, Hkv, 100.0, 7)

    def proj(w, t, o):
        return sum(x[0, t, c] * w[o, c] for c in range(C))

    def rot_norm(row, p):
        out = [0.0] * D
        for i in range(D // 2):
            a = p * 100.0 ** (-(2.0 * i) / D)
            out[2 * i] = row[2 * i] * math.cos(a) - row[2 * i + 1] * math.sin(a)
            out[2 * i + 1] = row[2 * i] * math.sin(a) + row[2 * i + 1] * math.cos(a)
        rn = 1.0 / math.sqrt(sum(z * z for z in out) / D + 1e-6)
        return [z * rn for z in out]

    for t in range(T):
        for h in range(H):
            want = rot_norm([proj(wq, t, h * D + d) for d in range(D)], 7 + t)
            _close(q[0, t, h], want, 1e-12, f"q' t={t} h={h}")
        for g in range(Hkv):
            want = rot_norm([proj(wk, t, g * D + d) for d in range(D)], 7 + t)
            _close(k[0, t, g], want, 1e-12, f"k' t={t} g={g}")
            _close(v[0, t, g], [proj(wv, t, g * D + d) for d in range(D)], 1e-12, f"v t={t} g={g}")


def pin_identity_weights(M):
    r = _rng(2)
    H, D = 2, 8
    x = r.standard_normal((2, 5, H * D))
    eye = np.eye(H * D)
    q, k, v = M.qkv_rope_qknorm(x, eye, eye, eye, H, H, 1e4, 3)
    xq = x.reshape(2, 5, H, D)
    want_q, want_k = R.rope_qknorm(xq, xq, 1e4, 3)
    _close(q, want_q, 1e-13, "q' with identity weights")
    _close(k, want_k, 1e-13, "k' with identity weights")
    _close(v, xq, 0.0, "v with identity weights")


def pin_zero_weights(M):
    x = _rng(3).standard_normal((1, 4, 6))
    z = np.zeros((4, 6))
    q, k, v = M.qkv_rope_qknorm(x, z, z, z, 2, 2, 1e4, 0)
    for a in (q, k, v):
        _close(a, np.zeros_like(a), 0.0, "zero weights")


def pin_linear_and_scale_invariant(M):
    r = _rng(4)
    x = r.standard_normal((1, 6, 16))
    wq, wk, wv = r.standard_normal((16, 16)), r.standard_normal((8, 16)), r.standard_normal((8, 16))
    q1, k1, v1 = M.qkv_rope_qknorm(x, wq, wk, wv, 2, 1, 1e4, 0)
    q2, k2, v2 = M.qkv_rope_qknorm(3.0 * x, wq, wk, wv, 2, 1, 1e4, 0)
    _close(v2, 3.0 * v1, 1e-12, "v linear")
    _close(q2, q1, 1e-6, "q' scale invariant")
    _close(k2, k1, 1e-6, "k' scale invariant")


PINS = [pin_brute_force, pin_identity_weights, pin_zero_weights, pin_linear_and_scale_invariant]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_projection_pin(pin):
    pin(PR)


def _variant(kind):
    def f(x, w_q, w_k, w_v, H, Hkv, base=10000.0, pos_offset=0):
        x = R._f64(x)
        B, T, C = x.shape
        wq, wk, wv = R._f64(w_q), R._f64(w_k), R._f64(w_v)
        D = wq.shape[0] // H
        if kind == "transposed":
            q, k, v = x @ wq, x @ wk, x @ wv
        else:
            q, k, v = x @ wq.T, x @ wk.T, x @ wv.T
        if kind == "head_minor":
            q = q.reshape(B, T, D, H).transpose(0, 1, 3, 2)
            k = k.reshape(B, T, D, Hkv).transpose(0, 1, 3, 2)
            v = v.reshape(B, T, D, Hkv).transpose(0, 1, 3, 2)
        else:
            q, k, v = q.reshape(B, T, H, D), k.reshape(B, T, Hkv, D), v.reshape(B, T, Hkv, D)
        pos = (pos_offset + np.arange(T))[None, :, None]
        if kind == "no_rope":
            return R.qk_norm(q), R.qk_norm(k), v
        if kind == "no_k_norm":
            return R.qk_norm(R.rope(q, pos, base)), R.rope(k, pos, base), v
        if kind == "v_normed":
            qn, kn = R.rope_qknorm(q, k, base, pos_offset)
            return qn, kn, R.qk_norm(v)
        qn, kn = R.rope_qknorm(q, k, base, pos_offset)
        return qn, kn, v
    return f


MUTANTS = ["transposed", "head_minor", "no_rope", "no_k_norm", "v_normed"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_projection_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(PR, "qkv_rope_qknorm", _variant(kind))
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(PR)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every pin"
