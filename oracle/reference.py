"""Plain fp64 definition of the attention-block forward (NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Every input is upcast exactly to float64 and nothing is rounded in between.
Sources (page title, section):
  [S5.4] "从文本到聊天模型" (onehacker.top), §5.4 Attention: q, k, v
         projections with shapes Q (B,T,H,D), K and V (B,T,Hkv,D); the core is
         score = Q K^T, weight = softmax(score), output = weight V.
  [S5.5] same page, §5.5 Causal Attention: a causal mask keeps each position
         from seeing later positions.
  [S5.6] same page, §5.6 RoPE: q and k are rotated according to position so
         that the scores see relative position.
  [TBL]  "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io), §1 model
         architecture table and the notes below it: RoPE as a rotation in
         complex space; RMSNorm without learnable parameters; QK-norm applied
         to q and k after RoPE; GQA (n_kv_head may be below n_head; groups of
         query heads share K/V); sliding-window attention in an SSSL pattern
         (short window = a quarter of the context).
  [S10]  "从文本到聊天模型", §10.2-10.4: the new token's K and V are appended
         to a per-layer cache, then its Q attends to every cached K/V.

Readings where the pages are silent (each is listed with its pin in the design doc):
  * RoPE pairs adjacent dims (2i, 2i+1), theta_i = base^(-2i/D), rotation by
    +p*theta_i, positions 0-based (p = pos_offset + t).  Parity unpinned for
    the pairing and the sign; the rest is pinned by closed forms/invariants.
  * RMSNorm: y = x / sqrt(mean(x^2) + eps), eps = 1e-6.  Parity unpinned for eps.
  * Scale 1/sqrt(D); no logit softcap inside attention (the +-15 softcap of the
    table belongs to the LM head); no dropout.
  * Window: key j is visible to query i iff 0 <= i - j < W (W keys including
    the query itself); W >= T is full causal attention.
  * GQA: query head h reads K/V head h // (H / Hkv).
  * Decode: seqlens[b] = L counts the new token, which sits at index and
    position L - 1; its normalised, rotated key and its raw value are written
    to the cache first, then the query attends to keys
    max(0, L - W) .. L - 1.  Older cache rows are used as stored.
  * Prefill into the cache (chunked prefill): one pos_offset P for the whole
    batch; the chunk's T tokens sit at cache rows and positions P .. P+T-1;
    their normalised, rotated keys and raw values are written there first,
    then query t (position P + t) attends to cache rows j with
    0 <= P + t - j < W.  Rows before P are used as stored.
  * Multi-sample decode over one shared prompt cache: the Lp prompt rows are
    held once (batch 1) and every sample's own rows (positions Lp..) in its
    own cache, row r holding position Lp + r; the result is that of a decode
    step over per-sample copies of the prompt cache followed by the sample's
    rows.  seqlens[b] = L in [Lp + 1, Lp + Tgen].
  * Value-embedding gate ([TBL] notes, value residual): v' = v + gate * ve,
    with ve shaped like v and one gate per (token, K/V head), both inputs;
    v' replaces v everywhere (the cache stores v').  The pages give only the
    formula; the shape of the gate is a reading.
"""
from __future__ import annotations

import math

import numpy as np

EPS = 1e-6


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or torch tensor (bf16/fp32) to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16 and fp32 both upcast exactly
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def rope_inv_freq(D: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D), i = 0 .. D/2-1, in float64 ([S5.6], [TBL])."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rope(x, positions, base: float) -> np.ndarray:
    """Rotate each adjacent pair (x_2i, x_2i+1) by the angle p*theta_i.

    x: (..., D); positions: integer array broadcastable to x.shape[:-1].
    Returns float64 of x's shape.  ([S5.6], [TBL] RoPE row and note.)
    """
    x = _f64(x)
    D = x.shape[-1]
    p = np.asarray(positions, dtype=np.float64)
    ang = p[..., None] * rope_inv_freq(D, base)          # (..., D/2)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def qk_norm(x, eps: float = EPS) -> np.ndarray:
    """Parameter-free RMSNorm over the last (head) dimension ([TBL])."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_qknorm(q, k, base: float = 10000.0, pos_offset: int = 0):
    """q (B,T,H,D), k (B,T,Hkv,D) -> (norm(rope(q)), norm(rope(k))).

    The table places QK-norm after RoPE; positions are pos_offset + t.
    """
    q, k = _f64(q), _f64(k)
    T = q.shape[1]
    pos = (pos_offset + np.arange(T))[None, :, None]      # (1,T,1)
    return qk_norm(rope(q, pos, base)), qk_norm(rope(k, pos, base))


def band_mask(T: int, W: int) -> np.ndarray:
    """visible[i, j] = 0 <= i - j < W ([S5.5] causal mask, [TBL] window)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    d = i - j
    return (d >= 0) & (d < W)


def attention_core(qn, kn, v, W: int, return_probs: bool = False):
    """softmax(q k^T / sqrt(D) restricted to the band) v, per (b, h).

    qn (B,T,H,D) and kn (B,T,Hkv,D) are the already rotated and normalised
    rows; v (B,T,Hkv,D) is raw.  Query head h reads K/V head h // (H/Hkv).
    ([S5.4] score/softmax/output, [S5.5] causal, [TBL] GQA and window.)
    """
    qn, kn, v = _f64(qn), _f64(kn), _f64(v)
    B, T, H, D = qn.shape
    Hkv = kn.shape[2]
    G = H // Hkv
    vis = band_mask(T, W)
    out = np.empty((B, T, H, D), dtype=np.float64)
    probs = np.empty((B, H, T, T), dtype=np.float64) if return_probs else None
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            g = h // G
            S = (qn[b, :, h, :] @ kn[b, :, g, :].T) * scale
            S = np.where(vis, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            P = E / E.sum(axis=1, keepdims=True)
            out[b, :, h, :] = P @ v[b, :, g, :]
            if return_probs:
                probs[b, h] = P
    return (out, probs) if return_probs else out


def attn_fwd(q, k, v, window: int, base: float = 10000.0, pos_offset: int = 0,
             return_probs: bool = False):
    """The whole prefill forward from raw q, k, v: RoPE, QK-norm, attention."""
    qn, kn = rope_qknorm(q, k, base, pos_offset)
    return attention_core(qn, kn, v, window, return_probs)


def attn_fwd_rows(q, k, v, rows, window: int, base: float = 10000.0,
                  pos_offset: int = 0) -> np.ndarray:
    """Output rows o[b, t, h, :] for a list of (b, t, h), one by one.

    Same definition as attn_fwd, evaluated only for the requested query rows
    (used to check full-size outputs on a sample).  Returns (len(rows), D).
    """
    D = q.shape[-1]
    H, Hkv = q.shape[2], k.shape[2]
    G = H // Hkv
    res = np.empty((len(rows), D), dtype=np.float64)
    for n, (b, t, h) in enumerate(rows):
        g = h // G
        lo = max(0, t - window + 1)
        keys = np.arange(lo, t + 1)
        qrow = _f64(q[b, t, h])
        krows = _f64(k[b, lo:t + 1, g])                   # (nk, D)
        vrows = _f64(v[b, lo:t + 1, g])
        qn = qk_norm(rope(qrow, pos_offset + t, base))
        kn = qk_norm(rope(krows, pos_offset + keys, base))
        s = (kn @ qn) / math.sqrt(D)
        e = np.exp(s - s.max())
        res[n] = (e / e.sum()) @ vrows
    return res


def attn_decode(q, k_new, v_new, k_cache, v_cache, seqlens, window: int,
                base: float = 10000.0, ve_new=None, ve_gate_new=None):
    """One decode step over a contiguous per-layer cache ([S10]).

    q (B,H,D); k_new, v_new (B,Hkv,D) raw; caches (B,Tmax,Hkv,D) whose rows
    before L-1 are used as stored; seqlens (B,) with L in [1, Tmax] counting
    the new token.  Returns (o (B,H,D), k_cache_out, v_cache_out) where the
    cache copies hold the appended row at index L-1.  With ve_new (B,Hkv,D)
    and ve_gate_new (B,Hkv), v_new is replaced by value_gate(v_new, ...).
    """
    q, k_new, v_new = _f64(q), _f64(k_new), value_gate(v_new, ve_new, ve_gate_new)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    L_all = np.asarray(_f64(seqlens), dtype=np.int64)
    B, H, D = q.shape
    Hkv = k_new.shape[1]
    G = H // Hkv
    o = np.empty((B, H, D), dtype=np.float64)
    for b in range(B):
        L = int(L_all[b])
        p = L - 1
        qn = qk_norm(rope(q[b], p, base))                  # (H, D)
        kn = qk_norm(rope(k_new[b], p, base))              # (Hkv, D)
        kc[b, p] = kn
        vc[b, p] = v_new[b]
        lo = max(0, L - window)
        for h in range(H):
            g = h // G
            s = (kc[b, lo:L, g] @ qn[h]) / math.sqrt(D)
            e = np.exp(s - s.max())
            o[b, h] = (e / e.sum()) @ vc[b, lo:L, g]
    return o, kc, vc


def value_gate(v, ve, gate):
    """v + gate * ve ([TBL] value residual); gate has v's shape minus the head dim."""
    v = _f64(v)
    if ve is None:
        return v
    return v + _f64(gate)[..., None] * _f64(ve)


def attn_prefill(q, k, v, k_cache, v_cache, window: int, base: float = 10000.0,
                 pos_offset: int = 0, ve=None, ve_gate=None):
    """Prefill of a chunk of T tokens into a contiguous per-layer cache
    ([S10] append K/V, then attend; [S5.5] causal mask; [TBL] window).

    q (B,T,H,D), k and v (B,T,Hkv,D) raw rows of the tokens at positions
    P .. P+T-1 (P = pos_offset); caches (B,Tmax,Hkv,D) with P + T <= Tmax,
    rows before P used as stored.  With ve (B,T,Hkv,D) and ve_gate (B,T,Hkv),
    v is replaced by value_gate(v, ve, ve_gate).  Returns (o (B,T,H,D),
    k_cache_out, v_cache_out), the cache copies holding the chunk's rows.
    """
    q, k, v = _f64(q), _f64(k), value_gate(v, ve, ve_gate)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    P = int(pos_offset)
    qn, kn = rope_qknorm(q, k, base, P)
    kc[:, P:P + T] = kn
    vc[:, P:P + T] = v
    i = P + np.arange(T)[:, None]          # query positions
    j = np.arange(P + T)[None, :]          # cache rows, one per key position
    vis = (i - j >= 0) & (i - j < window)
    o = np.empty((B, T, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = h // G
            S = (qn[b, :, h] @ kc[b, :P + T, g].T) / math.sqrt(D)
            S = np.where(vis, S, -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            o[b, :, h] = (E / E.sum(axis=1, keepdims=True)) @ vc[b, :P + T, g]
    return o, kc, vc


def attn_decode_shared(q, k_new, v_new, k_prompt, v_prompt, k_cache, v_cache, seqlens,
                       window: int, base: float = 10000.0, ve_new=None, ve_gate_new=None):
    """One decode step of B samples that share one prompt cache ([S10] §10.6:
    the prompt is prefilled once and every sample continues from its cache).

    q (B,H,D); k_new, v_new (B,Hkv,D) raw; k_prompt, v_prompt (Lp,Hkv,D) the
    prompt's rows, used as stored; k_cache, v_cache (B,Tgen,Hkv,D), row r of
    sample b holding position Lp + r; seqlens (B,) with L in [Lp+1, Lp+Tgen]
    counting the new token, at position L - 1.  The new token's normalised,
    rotated key and raw value go to row L-1-Lp of its sample's caches, then its
    query attends to positions max(0, L - W) .. L - 1.  Returns (o (B,H,D),
    k_cache_out, v_cache_out).  ve_new, ve_gate_new as in attn_decode.
    """
    q, k_new, v_new = _f64(q), _f64(k_new), value_gate(v_new, ve_new, ve_gate_new)
    kp, vp = _f64(k_prompt), _f64(v_prompt)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    L_all = np.asarray(_f64(seqlens), dtype=np.int64)
    B, H, D = q.shape
    Hkv = k_new.shape[1]
    Lp = kp.shape[0]
    G = H // Hkv
    o = np.empty((B, H, D), dtype=np.float64)
    for b in range(B):
        L = int(L_all[b])
        p = L - 1
        qn = qk_norm(rope(q[b], p, base))                  # (H, D)
        kc[b, p - Lp] = qk_norm(rope(k_new[b], p, base))
        vc[b, p - Lp] = v_new[b]
        lo = max(0, L - window)
        # the rows of positions lo .. L-1: the prompt's, then the sample's own
        keys = np.concatenate([kp[lo:Lp], kc[b, max(lo, Lp) - Lp:L - Lp]], axis=0)
        vals = np.concatenate([vp[lo:Lp], vc[b, max(lo, Lp) - Lp:L - Lp]], axis=0)
        for h in range(H):
            g = h // G
            s = (keys[:, g] @ qn[h]) / math.sqrt(D)
            e = np.exp(s - s.max())
            o[b, h] = (e / e.sum()) @ vals[:, g]
    return o, kc, vc
