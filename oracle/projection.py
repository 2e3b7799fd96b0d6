"""Plain fp64 definition of the bias-free q, k, v projection followed by RoPE
and QK-norm (NumPy), the step directly before the attention forward.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Sources (page title, section):
  [S5.4] "从文本到聊天模型" (onehacker.top), §5.4 Attention: the block computes
         q = c_q(x), k = c_k(x), v = c_v(x) and views them as (B, T, H, D) and
         (B, T, Hkv, D).
  [TBL]  "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io), §1 table: the
         linear layers carry no bias; separate c_q, c_k, c_v; QK-norm after
         RoPE.
  [P1]   "约100美元训出对话模型，nanochat源码全链路拆解" (ikfou.com), precision
         policy: weights are kept in fp32 and cast to the compute type in the
         linear layer.

Readings (listed in the design doc): the weights follow the linear-layer layout
(out_features, in_features): w_q (H*D, C), w_k and w_v (Hkv*D, C), already in
the compute type (the fp32 master weights are cast by the caller); output
column h*D + d of x w^T is element d of head h; q and k then get RoPE at
positions pos_offset + t and the parameter-free RMSNorm, exactly as
oracle.reference.rope_qknorm; v is the plain projection.
"""
from __future__ import annotations

import numpy as np

from .reference import _f64, rope_qknorm


def qkv_rope_qknorm(x, w_q, w_k, w_v, H: int, Hkv: int, base: float = 10000.0,
                    pos_offset: int = 0):
    """x (B, T, C); returns (q', k', v) with q' (B,T,H,D) = norm(rope(x w_q^T)),
    k' (B,T,Hkv,D) = norm(rope(x w_k^T)), v (B,T,Hkv,D) = x w_v^T, in float64."""
    x = _f64(x)
    B, T, C = x.shape
    wq, wk, wv = _f64(w_q), _f64(w_k), _f64(w_v)
    D = wq.shape[0] // H
    q = (x @ wq.T).reshape(B, T, H, D)
    k = (x @ wk.T).reshape(B, T, Hkv, D)
    v = (x @ wv.T).reshape(B, T, Hkv, D)
    qn, kn = rope_qknorm(q, k, base, pos_offset)
    return qn, kn, v
