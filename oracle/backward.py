"""Plain fp64 definition of the attention-block BACKWARD (NumPy), and the
forward's per-row log-sum-exp that a backward pass starts from.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Training runs the block forward, then backpropagates the loss through it and
steps the optimizer ("从文本到聊天模型" (onehacker.top), §6.5, one training
step: forward, loss.backward(), optimizer step); the attention kernel that
serves training does both passes ("Nanochat与nanoGPT对比：关键升级"
(lzwjava.github.io), §1 table, Flash Attention row). The pages print no
backward formulas: what follows is the chain rule applied to the forward that
``oracle.reference`` defines (RoPE, then parameter-free RMSNorm, then banded
GQA softmax attention), step by step in the order the forward runs backwards:

  forward (per batch b, query head h, K/V head g = h // G):
    q' = N(R(q)),  k' = N(R(k))                  R: RoPE, N: RMSNorm
    S  = q' k'^T / sqrt(D)  on the band 0 <= i - j < W, -inf elsewhere
    P  = softmax_rows(S),   o = P v
    lse_i = ln sum_j exp(S_ij)                   (the row statistic saved by
                                                  the forward: P = exp(S - lse))
  backward, given dO = dL/do:
    1. dV_g  = sum over the heads h of group g of P^T dO
    2. dP    = dO v^T
    3. dS    = P * (dP - rowsum(P * dP))          (softmax Jacobian)
    4. dq'   = dS k' / sqrt(D),   dk'_g = sum_h dS^T q' / sqrt(D)
    5. RMSNorm: y = x r, r = (mean(x^2) + eps)^-1/2
                dx = r (dy - y mean(dy * y))
    6. RoPE: a rotation of each pair (x_2i, x_2i+1) by the angle p theta_i;
       its gradient is the transposed rotation, by -p theta_i.
    7. GQA: the gradients of a K/V head sum over its G query heads (step 1
       and 4 above).

Parity of the conventions follows the forward (see ``oracle.reference``):
the RoPE pairing and sign and the epsilon are readings (parity unpinned);
everything here is pinned by central finite differences of the forward, by
the GQA = repeated-MHA identity, by float64 autograd of the attention core,
and by closed forms (tests/oracle_pins.py).
"""
from __future__ import annotations

import math

import numpy as np

from .reference import EPS, _f64, band_mask, qk_norm, rope, rope_qknorm, rope_inv_freq


def attn_fwd_lse(q, k, v, window: int, base: float = 10000.0, pos_offset: int = 0):
    """Forward output o (B,T,H,D) and the row log-sum-exp lse (B,T,H),
    lse[b,t,h] = ln sum_j exp(q'_t . k'_j / sqrt(D)) over the visible keys j,
    the natural-log statistic from which P = exp(S - lse)."""
    qn, kn = rope_qknorm(q, k, base, pos_offset)
    v = _f64(v)
    B, T, H, D = qn.shape
    G = H // kn.shape[2]
    vis = band_mask(T, window)
    o = np.empty((B, T, H, D))
    lse = np.empty((B, T, H))
    for b in range(B):
        for h in range(H):
            g = h // G
            S = np.where(vis, (qn[b, :, h] @ kn[b, :, g].T) / math.sqrt(D), -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            o[b, :, h] = (E / l) @ v[b, :, g]
            lse[b, :, h] = (m + np.log(l))[:, 0]
    return o, lse


def rope_bwd(dy, positions, base: float) -> np.ndarray:
    """Gradient through RoPE: rotate each adjacent pair of dy by -p*theta_i
    (the transpose of the forward's rotation)."""
    dy = _f64(dy)
    D = dy.shape[-1]
    p = np.asarray(positions, dtype=np.float64)
    ang = p[..., None] * rope_inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    ge, go = dy[..., 0::2], dy[..., 1::2]
    out = np.empty_like(dy)
    out[..., 0::2] = ge * c + go * s
    out[..., 1::2] = -ge * s + go * c
    return out


def qk_norm_bwd(x, dy, eps: float = EPS) -> np.ndarray:
    """Gradient through parameter-free RMSNorm y = x r, r = (mean(x^2)+eps)^-1/2,
    over the last dimension: dx = r (dy - y mean(dy * y))."""
    x, dy = _f64(x), _f64(dy)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def attention_core_bwd(qn, kn, v, do, W: int):
    """Steps 1-4 and 7: gradients of o = softmax(q'k'^T/sqrt(D) on the band) v
    with respect to q' (B,T,H,D), k' (B,T,Hkv,D) and v (B,T,Hkv,D)."""
    qn, kn, v, do = _f64(qn), _f64(kn), _f64(v), _f64(do)
    B, T, H, D = qn.shape
    Hkv = kn.shape[2]
    G = H // Hkv
    vis = band_mask(T, W)
    scale = 1.0 / math.sqrt(D)
    dq = np.zeros_like(qn)
    dk = np.zeros_like(kn)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = h // G
            S = np.where(vis, (qn[b, :, h] @ kn[b, :, g].T) * scale, -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            dv[b, :, g] += P.T @ do[b, :, h]                      # 1
            dP = do[b, :, h] @ v[b, :, g].T                       # 2
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))  # 3
            dq[b, :, h] = (dS @ kn[b, :, g]) * scale              # 4
            dk[b, :, g] += (dS.T @ qn[b, :, h]) * scale
    return dq, dk, dv


def attn_bwd(q, k, v, do, window: int, base: float = 10000.0, pos_offset: int = 0):
    """Gradients (dq, dk, dv) of the whole forward from RAW q, k, v with
    respect to those raw inputs, given dO (B,T,H,D) = dL/do."""
    q, k = _f64(q), _f64(k)
    T = q.shape[1]
    pos = (pos_offset + np.arange(T))[None, :, None]
    qr, kr = rope(q, pos, base), rope(k, pos, base)          # pre-norm rows
    qn, kn = qk_norm(qr), qk_norm(kr)
    dqn, dkn, dv = attention_core_bwd(qn, kn, v, do, window)
    dq = rope_bwd(qk_norm_bwd(qr, dqn), pos, base)            # 5, 6
    dk = rope_bwd(qk_norm_bwd(kr, dkn), pos, base)
    return dq, dk, dv
