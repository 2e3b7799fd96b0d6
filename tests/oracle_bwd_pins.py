"""Pins of the fp64 backward oracle (oracle/backward.py) against facts that do
not come from it.

Each ``pin_*`` takes the backward module and raises AssertionError when it
disagrees with central finite differences of the FORWARD oracle (the
definition of a gradient), a closed form, float64 autograd of a library
attention routine, or an identity the forward fixes. ``ALL_BWD_PINS`` runs on
the real module in ``test_oracle_bwd.py`` and on planted mutants there (every
mutant must fail at least one pin).

Sources (page title, section): "从文本到聊天模型" (onehacker.top) §6.5 (a
training step backpropagates the loss through the block); §5.4-5.6 (the
forward being differentiated); "Nanochat与nanoGPT对比：关键升级"
(lzwjava.github.io) §1 table and notes (QK-norm after RoPE, parameter-free
RMSNorm, GQA, sliding window).
"""
import math

import numpy as np
import torch

import oracle.reference as R


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _inputs(seed, B, T, H, Hkv, D, scale=2.5):
    r = _rng(seed)
    return (r.standard_normal((B, T, H, D)) * scale, r.standard_normal((B, T, Hkv, D)) * scale,
            r.standard_normal((B, T, Hkv, D)), r.standard_normal((B, T, H, D)))


def _fd_grads(q, k, v, do, W, base, off, h=1e-6):
    """Central differences of L = sum(o * dO), o the forward oracle's output."""
    def loss(q_, k_, v_):
        return float(np.sum(R.attn_fwd(q_, k_, v_, W, base, off) * do))
    grads = []
    for which in range(3):
        x = [q, k, v][which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = xp
            args_m[which] = xm
            g[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        grads.append(g)
    return grads


def pin_bwd_finite_differences_band_gqa(BW):
    """Every element of dq, dk, dv against central differences of the forward:
    a sliding window, two query heads per K/V head, positions from 5, base 100
    (large angles), inputs of RMS 2.5 (the norm's scale factor is not 1)."""
    q, k, v, do = _inputs(1, 1, 7, 4, 2, 4)
    dq, dk, dv = BW.attn_bwd(q, k, v, do, 3, 100.0, 5)
    fq, fk, fv = _fd_grads(q, k, v, do, 3, 100.0, 5)
    _close(dq, fq, 2e-7, "dq vs finite differences")
    _close(dk, fk, 2e-7, "dk vs finite differences")
    _close(dv, fv, 2e-7, "dv vs finite differences")


def pin_bwd_finite_differences_causal(BW):
    """The same over the full causal band, two sequences, one query head per
    K/V head, D = 8."""
    q, k, v, do = _inputs(2, 2, 5, 2, 2, 8, scale=0.7)
    dq, dk, dv = BW.attn_bwd(q, k, v, do, 64, 10000.0, 0)
    fq, fk, fv = _fd_grads(q, k, v, do, 64, 10000.0, 0)
    _close(dq, fq, 2e-7, "dq vs finite differences")
    _close(dk, fk, 2e-7, "dk vs finite differences")
    _close(dv, fv, 2e-7, "dv vs finite differences")


def pin_bwd_gqa_equals_repeated_mha(BW):
    """GQA gradients: dq as for MHA over K/V repeated G times along the heads;
    dk and dv the sums of the MHA gradients over each group of G heads."""
    q, k, v, do = _inputs(3, 2, 9, 6, 2, 8)
    dq, dk, dv = BW.attn_bwd(q, k, v, do, 4, 1e4, 2)
    G = 3
    mq, mk, mv = BW.attn_bwd(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), do, 4, 1e4, 2)
    _close(dq, mq, 1e-12, "dq")
    _close(dk, mk.reshape(2, 9, 2, G, 8).sum(axis=3), 1e-12, "dk group sums")
    _close(dv, mv.reshape(2, 9, 2, G, 8).sum(axis=3), 1e-12, "dv group sums")


def pin_bwd_window_one(BW):
    """W = 1: every query sees only itself, o = v (per group), so dq = dk = 0
    and dv of a K/V head is the sum of dO over its query heads."""
    q, k, v, do = _inputs(4, 1, 6, 4, 2, 8)
    dq, dk, dv = BW.attn_bwd(q, k, v, do, 1, 1e4, 0)
    _close(dq, np.zeros_like(dq), 1e-14, "dq")
    _close(dk, np.zeros_like(dk), 1e-14, "dk")
    _close(dv, do.reshape(1, 6, 2, 2, 8).sum(axis=3), 1e-14, "dv")


def pin_bwd_core_matches_autograd(BW):
    """Steps 1-4 (attention core with the band mask and GQA) against float64
    autograd of torch's scaled_dot_product_attention on the CPU."""
    r = _rng(5)
    B, T, H, Hkv, D, W = 2, 10, 4, 2, 16, 4
    qn = R.qk_norm(r.standard_normal((B, T, H, D)))
    kn = R.qk_norm(r.standard_normal((B, T, Hkv, D)))
    v = r.standard_normal((B, T, Hkv, D))
    do = r.standard_normal((B, T, H, D))
    dq, dk, dv = BW.attention_core_bwd(qn, kn, v, do, W)
    G = H // Hkv
    tq = torch.tensor(qn).permute(0, 2, 1, 3).requires_grad_(True)
    tk = torch.tensor(kn).permute(0, 2, 1, 3).requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_(True)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (i - j >= 0) & (i - j < W)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), attn_mask=mask,
        scale=1.0 / math.sqrt(D))
    o.backward(torch.tensor(do).permute(0, 2, 1, 3))
    _close(dq, tq.grad.permute(0, 2, 1, 3).numpy(), 1e-12, "dq'")
    _close(dk, tk.grad.permute(0, 2, 1, 3).numpy(), 1e-12, "dk'")
    _close(dv, tv.grad.permute(0, 2, 1, 3).numpy(), 1e-12, "dv")


def pin_norm_bwd_closed_form_d1(BW):
    """D = 1: y = x / sqrt(x^2 + eps), dy/dx = eps / (x^2 + eps)^(3/2)."""
    for x in (1e-3, 0.02, 0.5, -3.0):
        want = 1e-6 / (x * x + 1e-6) ** 1.5
        got = BW.qk_norm_bwd(np.array([x]), np.array([1.0]))[0]
        assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (x, got, want)


def pin_norm_bwd_finite_differences(BW):
    """dx = J^T dy of the RMSNorm, column by column against central differences."""
    r = _rng(6)
    x = r.standard_normal(6) * np.array([0.01, 1, 3, 0.2, 5, 1])
    dy = r.standard_normal(6)
    got = BW.qk_norm_bwd(x, dy)
    h = 1e-7
    fd = np.array([(np.dot(R.qk_norm(x + h * e), dy) - np.dot(R.qk_norm(x - h * e), dy)) / (2 * h)
                   for e in np.eye(6)])
    _close(got, fd, 1e-7, "norm bwd")


def pin_rope_bwd_inverts_rope(BW):
    """The gradient of a rotation is its transpose, which is its inverse:
    rope_bwd(rope(x, p), p) = x."""
    x = _rng(7).standard_normal((3, 5, 32))
    pos = np.arange(5)[None, :] * 37 + 11
    _close(BW.rope_bwd(R.rope(x, pos, 1e4), pos, 1e4), x, 1e-12, "rope_bwd o rope")


def pin_bwd_scale_orthogonality(BW):
    """The forward is unchanged when a q or k row is scaled (QK-norm), so each
    raw row is orthogonal to its gradient up to the epsilon:
    x . dx = r (x . dy) eps / (m + eps), about 1e-7 relative here."""
    q, k, v, do = _inputs(8, 1, 8, 2, 1, 16, scale=1.0)
    dq, dk, _ = BW.attn_bwd(q, k, v, do, 5, 1e4, 3)
    for x, g in ((q, dq), (k, dk)):
        dots = np.abs(np.sum(x * g, axis=-1))
        norms = np.linalg.norm(x, axis=-1) * np.linalg.norm(g, axis=-1) + 1e-300
        assert np.all(dots <= 1e-5 * norms + 1e-12), float(np.max(dots / norms))


def pin_lse_brute_force(BW):
    """lse[b,t,h] = ln sum_j exp(s_j) over the visible keys, evaluated with
    scalar loops and the math module; the output equals the forward's."""
    q, k, v, _ = _inputs(9, 1, 6, 2, 1, 4, scale=1.0)
    W, base, off = 4, 1e4, 2
    o, lse = BW.attn_fwd_lse(q, k, v, W, base, off)
    _close(o, R.attn_fwd(q, k, v, W, base, off), 1e-13, "o")
    qn, kn = R.rope_qknorm(q, k, base, off)
    for t in range(6):
        for h in range(2):
            tot = 0.0
            for j in range(6):
                if 0 <= t - j < W:
                    tot += math.exp(sum(qn[0, t, h, d] * kn[0, j, 0, d] for d in range(4)) / 2.0)
            assert abs(lse[0, t, h] - math.log(tot)) <= 1e-12, (t, h)


ALL_BWD_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
