"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` takes the oracle module and raises AssertionError when it
disagrees with a closed form, an invariant the pages fix, a textbook library
routine, or brute force.  ``ALL_PINS`` is run on the real oracle by
``test_oracle_pins.py`` and on planted mutants of it by
``test_oracle_mutants.py`` (every mutant must fail at least one pin).

Sources of the facts (page title, section):
  * "从文本到聊天模型" (onehacker.top) §5.4 (score, softmax, weighted sum of V;
    Q (B,T,H,D), K/V (B,T,Hkv,D)), §5.5 (causal mask), §5.6 (RoPE gives
    relative position), §10.2-10.4 (append new K/V, then attend).
  * "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io) §1 table + notes
    (RoPE as complex rotation, parameter-free RMSNorm, QK-norm after RoPE,
    GQA, SSSL window of a quarter context).
"""
import math

import numpy as np
import torch

from brute_ref import brute_attn

TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------- RoPE pins

def pin_rope_position_zero_identity(O):
    """RoPE at position 0 is the identity (a rotation by angle 0)."""
    x = _rng(1).standard_normal((3, 5, 16))
    _close(O.rope(x, 0, 10000.0), x, what="rope(x, 0)")


def pin_rope_d2_closed_form(O):
    """D=2 has theta_0 = base^0 = 1: (1, 0) at position p becomes (cos p, sin p)."""
    for p in (1, 2, 7, 100, 2047):
        got = O.rope(np.array([1.0, 0.0]), p, 10000.0)
        _close(got, [math.cos(p), math.sin(p)], what=f"D=2 p={p}")
        got = O.rope(np.array([0.0, 1.0]), p, 10000.0)
        _close(got, [-math.sin(p), math.cos(p)], what=f"D=2 e1 p={p}")


def pin_rope_frequency_closed_form(O):
    """D=4: the second pair turns by p * base^(-2/4)."""
    for base in (10000.0, 500.0):
        th1 = base ** -0.5
        for p in (3, 50):
            got = O.rope(np.array([0.0, 0.0, 1.0, 0.0]), p, base)
            _close(got, [0, 0, math.cos(p * th1), math.sin(p * th1)],
                   what=f"D=4 base={base} p={p}")


def pin_rope_complex_form(O):
    """Adjacent pairs as complex numbers z_i = x_2i + i x_2i+1, times e^{i p theta_i}."""
    D = 32
    x = _rng(2).standard_normal((4, 7, D))
    pos = np.arange(7)[None, :] * 13 + 5
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.array([10000.0 ** (-2.0 * i / D) for i in range(D // 2)])
    zr = z * np.exp(1j * pos[..., None] * theta)
    want = np.empty_like(x)
    want[..., 0::2] = zr.real
    want[..., 1::2] = zr.imag
    _close(O.rope(x, pos, 10000.0), want, tol=1e-11, what="complex form")


def pin_rope_preserves_pair_norms(O):
    D = 64
    x = _rng(3).standard_normal((6, D))
    y = O.rope(x, np.arange(6) * 311, 10000.0)
    _close(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
           tol=1e-12, what="pair norms")


def pin_rope_composition(O):
    """rope(rope(x, a), b) = rope(x, a + b)."""
    x = _rng(4).standard_normal((5, 32))
    a, b = np.arange(5) * 17, np.arange(5) * 5 + 3
    _close(O.rope(O.rope(x, a, 1e4), b, 1e4), O.rope(x, a + b, 1e4), tol=1e-11,
           what="composition")


def pin_rope_relative_position(O):
    """<rope(q, m), rope(k, n)> depends only on m - n (the §5.6 purpose of RoPE)."""
    r = _rng(5)
    q, k = r.standard_normal(64), r.standard_normal(64)
    base_dot = O.rope(q, 10, 1e4) @ O.rope(k, 3, 1e4)
    for s in (1, 40, 1000):
        _close(O.rope(q, 10 + s, 1e4) @ O.rope(k, 3 + s, 1e4), base_dot, tol=1e-10,
               what=f"shift {s}")


# --------------------------------------------------------------- norm pins

def pin_norm_hand_example(O):
    """x = (3, 4): mean of squares 12.5, so y = x / sqrt(12.5 + eps)."""
    _close(O.qk_norm(np.array([3.0, 4.0])),
           np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-6), what="norm (3,4)")


def pin_norm_unit_rms(O):
    """mean(y^2) = m / (m + eps) exactly, m = mean(x^2): unit RMS up to eps."""
    x = _rng(6).standard_normal((10, 128)) * np.array([[0.1], [1], [3], [10], [1e-2],
                                                        [5], [2], [7], [0.5], [100]])
    y = O.qk_norm(x)
    m = np.mean(x * x, axis=-1)
    _close(np.mean(y * y, axis=-1), m / (m + 1e-6), tol=1e-12, what="unit rms")


def pin_norm_commutes_with_rope(O):
    """Rotation keeps the RMS, so norm(rope(x)) = rope(norm(x))."""
    x = _rng(7).standard_normal((4, 6, 32)) * 3
    pos = np.arange(6)[None, :] * 100
    _close(O.qk_norm(O.rope(x, pos, 1e4)), O.rope(O.qk_norm(x), pos, 1e4),
           tol=1e-12, what="norm o rope")


# ---------------------------------------------------------- attention pins

def _small(seed, B=2, T=12, H=4, Hkv=2, D=8, scale=1.0):
    r = _rng(seed)
    return (r.standard_normal((B, T, H, D)) * scale,
            r.standard_normal((B, T, Hkv, D)) * scale,
            r.standard_normal((B, T, Hkv, D)))


def pin_brute_force(O):
    """Oracle = scalar loops on tiny shapes, including GQA, windows and offsets."""
    cases = [(1, 5, 2, 2, 4, 5, 0), (2, 6, 4, 2, 4, 2, 3), (1, 8, 3, 1, 6, 3, 0),
             (1, 7, 2, 1, 2, 1, 9), (1, 8, 4, 4, 8, 100, 1)]
    for n, (B, T, H, Hkv, D, W, off) in enumerate(cases):
        q, k, v = _small(100 + n, B, T, H, Hkv, D, scale=2.0)
        want = brute_attn(q.tolist(), k.tolist(), v.tolist(), W, 10000.0, off)
        _close(O.attn_fwd(q, k, v, W, 10000.0, off), np.array(want), tol=1e-11,
               what=f"brute case {n}")


def pin_core_matches_sdpa_float64(O):
    """The attention step equals torch SDPA (float64, CPU) with an explicit band
    mask, scale 1/sqrt(D), and enable_gqa (contiguous head groups)."""
    for (B, T, H, Hkv, D, W) in [(2, 33, 4, 4, 16, 33), (1, 40, 8, 2, 32, 7),
                                 (2, 17, 6, 3, 8, 1), (1, 64, 4, 1, 64, 16)]:
        r = _rng(T * 7 + W)
        qn = r.standard_normal((B, T, H, D))
        kn = r.standard_normal((B, T, Hkv, D))
        v = r.standard_normal((B, T, Hkv, D))
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        mask = torch.from_numpy(((i - j) >= 0) & ((i - j) < W))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qn).transpose(1, 2), torch.from_numpy(kn).transpose(1, 2),
            torch.from_numpy(v).transpose(1, 2), attn_mask=mask, scale=1.0 / math.sqrt(D),
            enable_gqa=(H != Hkv)).transpose(1, 2).numpy()
        _close(O.attention_core(qn, kn, v, W), ref, tol=1e-12, what=f"sdpa {B,T,H,Hkv,D,W}")


def pin_single_token_returns_v(O):
    """T = 1 (and row 0 in general): the only visible key is the query's own."""
    q, k, v = _small(8, B=2, T=1, H=4, Hkv=2, D=16)
    out = O.attn_fwd(q, k, v, 1)
    _close(out, np.repeat(v, 2, axis=2), what="T=1")
    q, k, v = _small(9, B=1, T=9, H=2, Hkv=2, D=16)
    _close(O.attn_fwd(q, k, v, 9)[:, 0], v[:, 0], what="row 0")


def pin_window_one_returns_v(O):
    """W = 1: each query sees only itself, so o[t, h] = v[t, h // G]."""
    q, k, v = _small(10, B=2, T=11, H=6, Hkv=3, D=8)
    _close(O.attn_fwd(q, k, v, 1), np.repeat(v, 2, axis=2), what="W=1")


def pin_constant_v(O):
    q, k, _ = _small(11, B=1, T=10, H=2, Hkv=2, D=8)
    v = np.broadcast_to(np.arange(8.0), (1, 10, 2, 8)).copy()
    _close(O.attn_fwd(q, k, v, 4), v, what="constant v")


def pin_probs_band_and_sum(O):
    """Softmax rows sum to 1, are positive exactly on the band 0 <= i-j < W."""
    q, k, v = _small(12, B=1, T=13, H=2, Hkv=1, D=8)
    for W in (1, 3, 13, 50):
        _, P = O.attn_fwd(q, k, v, W, return_probs=True)
        _close(P.sum(axis=-1), np.ones((1, 2, 13)), what="row sums")
        i = np.arange(13)[:, None]
        j = np.arange(13)[None, :]
        band = ((i - j) >= 0) & ((i - j) < W)
        assert np.all((P > 0) == band[None, None]), f"band support W={W}"


def pin_full_window_is_causal(O):
    """Any W >= T reproduces full causal attention."""
    q, k, v = _small(13, B=1, T=9, H=2, Hkv=2, D=8)
    a = O.attn_fwd(q, k, v, 9)
    _close(O.attn_fwd(q, k, v, 10), a, what="W=T+1")
    _close(O.attn_fwd(q, k, v, 1000), a, what="W=1000")


def pin_gqa_equals_repeated_mha(O):
    """GQA equals MHA on K/V repeated G times per head group."""
    q, k, v = _small(14, B=2, T=10, H=6, Hkv=2, D=8)
    a = O.attn_fwd(q, k, v, 4)
    b = O.attn_fwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 4)
    _close(a, b, what="gqa vs repeated mha")


def pin_linear_in_v(O):
    q, k, v1 = _small(15, B=1, T=10, H=2, Hkv=2, D=8)
    v2 = _rng(16).standard_normal(v1.shape)
    _close(O.attn_fwd(q, k, 2.0 * v1 - 3.0 * v2, 5),
           2.0 * O.attn_fwd(q, k, v1, 5) - 3.0 * O.attn_fwd(q, k, v2, 5),
           tol=1e-11, what="linearity")


def pin_batch_independence(O):
    q, k, v = _small(17, B=3, T=8, H=2, Hkv=1, D=8)
    a = O.attn_fwd(q, k, v, 3)
    perm = [2, 0, 1]
    _close(O.attn_fwd(q[perm], k[perm], v[perm], 3), a[perm], what="batch perm")


def pin_pos_offset_invariance(O):
    """A shift of every position leaves the output unchanged (relative positions)."""
    q, k, v = _small(18, B=1, T=12, H=2, Hkv=2, D=16, scale=3.0)
    a = O.attn_fwd(q, k, v, 5, 1e4, 0)
    _close(O.attn_fwd(q, k, v, 5, 1e4, 777), a, tol=1e-10, what="pos_offset")


def pin_q_and_k_scale_invariance(O):
    """QK-norm makes the output independent of the scale of q and of k rows
    (up to the eps term, which moves scores by about eps/mean(x^2))."""
    q, k, v = _small(19, B=1, T=10, H=2, Hkv=2, D=16)
    a = O.attn_fwd(q, k, v, 10)
    _close(O.attn_fwd(q * 37.0, k, v, 10), a, tol=1e-5, what="q scale")
    _close(O.attn_fwd(q, k * 20.0, v, 10), a, tol=1e-5, what="k scale")


def pin_rows_match_full(O):
    """The one-row-at-a-time evaluation equals the full evaluation."""
    q, k, v = _small(20, B=2, T=20, H=4, Hkv=2, D=16)
    full = O.attn_fwd(q, k, v, 6, 1e4, 3)
    rows = [(0, 0, 0), (1, 19, 3), (0, 7, 2), (1, 5, 1), (0, 19, 1)]
    got = O.attn_fwd_rows(q, k, v, rows, 6, 1e4, 3)
    _close(got, np.stack([full[b, t, h] for b, t, h in rows]), tol=1e-12, what="rows")


# ------------------------------------------------------------- decode pins

def _decode_case(seed, B=3, Tmax=12, H=4, Hkv=2, D=16):
    r = _rng(seed)
    return (r.standard_normal((B, H, D)), r.standard_normal((B, Hkv, D)),
            r.standard_normal((B, Hkv, D)), r.standard_normal((B, Tmax, Hkv, D)),
            r.standard_normal((B, Tmax, Hkv, D)))


def pin_decode_matches_prefill(O):
    """Decode of token L-1 over a cache holding the prefill's normalised, rotated
    keys and raw values equals row L-1 of the prefill (append, then attend)."""
    r = _rng(21)
    B, T, H, Hkv, D = 2, 11, 4, 2, 16
    q = r.standard_normal((B, T, H, D))
    k = r.standard_normal((B, T, Hkv, D))
    v = r.standard_normal((B, T, Hkv, D))
    for W in (3, 11):
        full = O.attn_fwd(q, k, v, W)
        _, kn = O.rope_qknorm(q, k)
        for L in (1, 4, 11):
            kc = np.where(np.arange(T)[None, :, None, None] < L - 1, kn, 9.0)
            vc = np.where(np.arange(T)[None, :, None, None] < L - 1, v, -9.0)
            o, kco, vco = O.attn_decode(q[:, L - 1], k[:, L - 1], v[:, L - 1], kc, vc,
                                        np.full(B, L), W)
            _close(o, full[:, L - 1], tol=1e-11, what=f"decode L={L} W={W}")
            _close(kco[:, L - 1], kn[:, L - 1], tol=1e-12, what="appended k")
            _close(vco[:, L - 1], v[:, L - 1], tol=0, what="appended v")


def pin_decode_first_token(O):
    """L = 1: the new token attends only to itself, o = v_new of its group."""
    q, kn, vn, kc, vc = _decode_case(22)
    o, _, _ = O.attn_decode(q, kn, vn, kc, vc, np.ones(3, dtype=int), 5)
    _close(o, np.repeat(vn, 2, axis=1), what="L=1")


def pin_decode_touches_only_row(O):
    q, kn, vn, kc, vc = _decode_case(23)
    L = np.array([5, 12, 1])
    _, kco, vco = O.attn_decode(q, kn, vn, kc, vc, L, 4)
    for b in range(3):
        keep = np.arange(12) != L[b] - 1
        _close(kco[b, keep], kc[b, keep], tol=0, what="k rows kept")
        _close(vco[b, keep], vc[b, keep], tol=0, what="v rows kept")


def pin_decode_brute(O):
    """Decode against scalar loops over the visible keys."""
    q, kn, vn, kc, vc = _decode_case(24, B=2, Tmax=9, H=4, Hkv=2, D=6)
    L = np.array([9, 6])
    W = 4
    o, _, _ = O.attn_decode(q, kn, vn, kc, vc, L, W)
    for b in range(2):
        p = L[b] - 1
        # rotate + normalise by hand (adjacent pairs, +p*theta, eps 1e-6)
        def rn(row):
            out = []
            for i in range(3):
                a = p * 10000.0 ** (-(2.0 * i) / 6)
                x, y = row[2 * i], row[2 * i + 1]
                out += [x * math.cos(a) - y * math.sin(a), x * math.sin(a) + y * math.cos(a)]
            r = 1.0 / math.sqrt(sum(z * z for z in out) / 6 + 1e-6)
            return [z * r for z in out]
        for h in range(4):
            g = h // 2
            qh = rn(list(q[b, h]))
            ss, vs = [], []
            for j in range(max(0, L[b] - W), L[b]):
                kj = rn(list(kn[b, g])) if j == p else list(kc[b, j, g])
                vj = list(vn[b, g]) if j == p else list(vc[b, j, g])
                ss.append(sum(a * c for a, c in zip(qh, kj)) / math.sqrt(6))
                vs.append(vj)
            mx = max(ss)
            ws = [math.exp(s - mx) for s in ss]
            want = [sum(w * vv[d] for w, vv in zip(ws, vs)) / sum(ws) for d in range(6)]
            _close(o[b, h], want, tol=1e-12, what=f"decode brute b={b} h={h}")


# ------------------------------------------------------------ prefill pins

def _prefill_case(seed, B=2, T=13, H=4, Hkv=2, D=8):
    r = _rng(seed)
    return (r.standard_normal((B, T, H, D)), r.standard_normal((B, T, Hkv, D)),
            r.standard_normal((B, T, Hkv, D)))


def pin_prefill_chunks_match_fwd(O):
    """Causality makes chunking invisible: prefilling a sequence chunk by chunk
    into one cache gives the rows of the whole-sequence forward, and leaves the
    normalised, rotated keys and the raw values in the cache."""
    q, k, v = _prefill_case(31)
    T = q.shape[1]
    _, kn = O.rope_qknorm(q, k)
    for W in (1, 3, 5, T):
        full = O.attn_fwd(q, k, v, W)
        for cuts in ((0, T), (0, 4, T), (0, 1, 7, 8, T)):
            kc = np.full((2, T + 3, 2, 8), 5.0)
            vc = np.full((2, T + 3, 2, 8), -5.0)
            for a, b in zip(cuts[:-1], cuts[1:]):
                o, kc, vc = O.attn_prefill(q[:, a:b], k[:, a:b], v[:, a:b], kc, vc, W,
                                           pos_offset=a)
                _close(o, full[:, a:b], tol=1e-11, what=f"chunk {a}:{b} W={W}")
            _close(kc[:, :T], kn, tol=1e-12, what="cached keys")
            _close(vc[:, :T], v, tol=0, what="cached values")


def pin_prefill_then_decode(O):
    """A prefill of T-1 tokens followed by a decode step of token T-1 gives the
    last row of the whole-sequence forward."""
    q, k, v = _prefill_case(32, T=10)
    T = q.shape[1]
    for W in (4, T):
        full = O.attn_fwd(q, k, v, W)
        kc = np.zeros((2, T, 2, 8))
        vc = np.zeros((2, T, 2, 8))
        _, kc, vc = O.attn_prefill(q[:, :T - 1], k[:, :T - 1], v[:, :T - 1], kc, vc, W)
        o, _, _ = O.attn_decode(q[:, T - 1], k[:, T - 1], v[:, T - 1], kc, vc,
                                np.full(2, T), W)
        _close(o, full[:, T - 1], tol=1e-11, what=f"prefill+decode W={W}")


def pin_prefill_touches_only_chunk_rows(O):
    q, k, v = _prefill_case(33, T=5)
    r = _rng(34)
    kc0 = r.standard_normal((2, 12, 2, 8))
    vc0 = r.standard_normal((2, 12, 2, 8))
    _, kc, vc = O.attn_prefill(q, k, v, kc0, vc0, 4, pos_offset=6)
    keep = (np.arange(12) < 6) | (np.arange(12) >= 11)
    _close(kc[:, keep], kc0[:, keep], tol=0, what="k rows kept")
    _close(vc[:, keep], vc0[:, keep], tol=0, what="v rows kept")


def pin_prefill_brute(O):
    """Chunk at offset P over a cache whose earlier rows are arbitrary (used as
    stored), against scalar loops over the visible (query, key) pairs."""
    q, k, v = _prefill_case(35, B=1, T=4, H=2, Hkv=1, D=6)
    r = _rng(36)
    P, W, Tmax = 5, 6, 10
    kc0 = r.standard_normal((1, Tmax, 1, 6))
    vc0 = r.standard_normal((1, Tmax, 1, 6))
    o, _, _ = O.attn_prefill(q, k, v, kc0, vc0, W, pos_offset=P)

    def rn(row, p):
        out = []
        for i in range(3):
            a = p * 10000.0 ** (-(2.0 * i) / 6)
            x, y = row[2 * i], row[2 * i + 1]
            out += [x * math.cos(a) - y * math.sin(a), x * math.sin(a) + y * math.cos(a)]
        s = 1.0 / math.sqrt(sum(z * z for z in out) / 6 + 1e-6)
        return [z * s for z in out]
    for t in range(4):
        for h in range(2):
            qh = rn(list(q[0, t, h]), P + t)
            ss, vs = [], []
            for j in range(P + t + 1):
                if not 0 <= P + t - j < W:
                    continue
                kj = rn(list(k[0, j - P, 0]), j) if j >= P else list(kc0[0, j, 0])
                vj = list(v[0, j - P, 0]) if j >= P else list(vc0[0, j, 0])
                ss.append(sum(a * c for a, c in zip(qh, kj)) / math.sqrt(6))
                vs.append(vj)
            mx = max(ss)
            ws = [math.exp(s - mx) for s in ss]
            want = [sum(w * vv[d] for w, vv in zip(ws, vs)) / sum(ws) for d in range(6)]
            _close(o[0, t, h], want, tol=1e-12, what=f"prefill brute t={t} h={h}")


# ---------------------------------------------------- shared-prompt decode pins

def pin_decode_shared_equals_copied_caches(O):
    """One prompt prefilled once, its cache copied to every sample, each sample
    with its own generated rows: decoding over the copies equals decoding over
    the one shared prompt cache plus the samples' own rows."""
    r = _rng(41)
    B, Lp, Tgen, H, Hkv, D = 3, 7, 6, 4, 2, 8
    kp = r.standard_normal((Lp, Hkv, D))
    vp = r.standard_normal((Lp, Hkv, D))
    kg = r.standard_normal((B, Tgen, Hkv, D))
    vg = r.standard_normal((B, Tgen, Hkv, D))
    q = r.standard_normal((B, H, D))
    kn = r.standard_normal((B, Hkv, D))
    vn = r.standard_normal((B, Hkv, D))
    kfull = np.concatenate([np.broadcast_to(kp, (B, Lp, Hkv, D)), kg], axis=1)
    vfull = np.concatenate([np.broadcast_to(vp, (B, Lp, Hkv, D)), vg], axis=1)
    for W in (1, 3, 8, 13):
        L = np.array([Lp + 1, Lp + 4, Lp + Tgen])
        o1, kc1, vc1 = O.attn_decode(q, kn, vn, kfull, vfull, L, W)
        o2, kc2, vc2 = O.attn_decode_shared(q, kn, vn, kp, vp, kg, vg, L, W)
        _close(o2, o1, tol=1e-12, what=f"shared vs copied W={W}")
        _close(kc2, kc1[:, Lp:], tol=0, what="sample k rows")
        _close(vc2, vc1[:, Lp:], tol=0, what="sample v rows")


def pin_decode_shared_first_generated_token(O):
    """The first generated token with W = 1 sees only itself: o = v_new."""
    r = _rng(42)
    kp, vp = r.standard_normal((5, 2, 8)), r.standard_normal((5, 2, 8))
    kg, vg = r.standard_normal((2, 4, 2, 8)), r.standard_normal((2, 4, 2, 8))
    q, kn, vn = r.standard_normal((2, 4, 8)), r.standard_normal((2, 2, 8)), r.standard_normal((2, 2, 8))
    o, kc, vc = O.attn_decode_shared(q, kn, vn, kp, vp, kg, vg, np.array([6, 6]), 1)
    _close(o, np.repeat(vn, 2, axis=1), what="W=1")
    keep = np.arange(4) != 0
    _close(kc[:, keep], kg[:, keep], tol=0, what="other k rows kept")
    _close(vc[:, 0], vn, tol=0, what="appended v")


# ------------------------------------------------------- value-embedding gate

def pin_ve_gate_zero_is_identity(O):
    """A zero gate leaves v, the caches and the output unchanged."""
    q, k, v = _prefill_case(51, T=9)
    ve = _rng(52).standard_normal(v.shape)
    kc, vc = np.zeros((2, 12, 2, 8)), np.zeros((2, 12, 2, 8))
    o0, kc0, vc0 = O.attn_prefill(q, k, v, kc, vc, 4, pos_offset=2)
    o1, kc1, vc1 = O.attn_prefill(q, k, v, kc, vc, 4, pos_offset=2, ve=ve, ve_gate=np.zeros(v.shape[:3]))
    _close(o1, o0, tol=0, what="o")
    _close(vc1, vc0, tol=0, what="v cache")


def pin_ve_gate_linearity(O):
    """Attention is linear in V: with one gate g for every token and head,
    o(v + g ve) = o(v) + g o(ve), and the cache holds v + g ve."""
    q, k, v = _prefill_case(53, T=11)
    ve = _rng(54).standard_normal(v.shape)
    kc, vc = np.zeros((2, 14, 2, 8)), np.zeros((2, 14, 2, 8))
    for g in (0.5, -1.25):
        gate = np.full(v.shape[:3], g)
        og, _, vcg = O.attn_prefill(q, k, v, kc, vc, 5, pos_offset=3, ve=ve, ve_gate=gate)
        ov, _, _ = O.attn_prefill(q, k, v, kc, vc, 5, pos_offset=3)
        oe, _, _ = O.attn_prefill(q, k, ve, kc, vc, 5, pos_offset=3)
        _close(og, ov + g * oe, tol=1e-12, what=f"linearity g={g}")
        _close(vcg[:, 3:14], v + g * ve, tol=1e-15, what="cached v'")


def pin_ve_gate_per_token_brute(O):
    """Per-token, per-head gates against the plain sum on a decode step."""
    q, kn, vn, kc, vc = _decode_case(55, B=2, Tmax=6, H=2, Hkv=2, D=4)
    r = _rng(56)
    ve, gate = r.standard_normal(vn.shape), r.standard_normal(vn.shape[:2])
    L = np.array([6, 3])
    o, _, vco = O.attn_decode(q, kn, vn, kc, vc, L, 3, ve_new=ve, ve_gate_new=gate)
    o_ref, _, _ = O.attn_decode(q, kn, vn + gate[..., None] * ve, kc, vc, L, 3)
    _close(o, o_ref, tol=1e-12, what="decode with gate")
    for b in range(2):
        for g in range(2):
            want = [vn[b, g, d] + gate[b, g] * ve[b, g, d] for d in range(4)]
            _close(vco[b, L[b] - 1, g], want, tol=1e-15, what=f"appended v' b={b} g={g}")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
