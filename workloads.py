"""Seeded synthetic workloads for the attention-block forward.

This module holds only shapes and seeded random draws. It contains none of the
method's arithmetic (no RoPE, no normalisation, no softmax), so both the fp64
oracle under ``oracle/`` and the HIP path may take their inputs from here
without sharing any of the computation.

Shapes follow the nanochat pages:
  * d12 layer: hidden 768, 6 heads -> head dim 128, context 2048
    ("约100美元训出对话模型，nanochat源码全链路拆解" (ikfou.com), sections on
    the GPT forward and on tensor shapes B/T/H/D).
  * sliding-window pattern SSSL: three short layers with a quarter of the
    context, one full layer ("Nanochat与nanoGPT对比：关键升级"
    (lzwjava.github.io), model-architecture table, sliding-window row and the
    note below it).
  * hidden 1024 with 16 query heads -> head dim 64 (the sns.style "Nano Chat"
    article, model-configuration section); here with 4 K/V heads for GQA.
  * decode over a per-layer KV cache of capacity T ("从文本到聊天模型"
    (onehacker.top), sections 10.2-10.4).

The pages' own workloads are end-to-end training and evaluation runs on public
datasets with trained weights; seeded N(0,1) tensors of the same shapes stand
in for those activations. After QK-norm every q/k row has unit RMS whatever
the input scale, so N(0,1) inputs exercise the same operand ranges.

Seed scheme: seed = 20260000 + 100*config + 10*layer + tensor, where tensor is
0 q, 1 k, 2 v, 3 k_cache, 4 v_cache, 5 seqlens, 6 dO (the upstream gradient
of the backward pass). Draws use
``torch.Generator('cpu')`` and ``torch.randn`` in float32, then an RNE cast to
bfloat16 where the config is bf16. The same host bits feed both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_BASE = 20260000
T_Q, T_K, T_V, T_KCACHE, T_VCACHE, T_SEQLENS, T_DOUT = range(7)


def seed_for(config: int, layer: int, tensor: int) -> int:
    return SEED_BASE + 100 * config + 10 * layer + tensor


def randn(shape, seed: int, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x.to(dtype)


def randint(low: int, high_inclusive: int, shape, seed: int) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(low, high_inclusive + 1, tuple(shape), generator=g,
                         dtype=torch.int64).to(torch.int32)


@dataclass(frozen=True)
class PrefillConfig:
    idx: int
    name: str
    B: int
    T: int
    H: int
    Hkv: int
    D: int
    windows: tuple  # one entry per layer call
    dtype: torch.dtype
    rope_base: float = 10000.0
    pos_offset: int = 0


@dataclass(frozen=True)
class DecodeConfig:
    idx: int
    name: str
    B: int
    Tmax: int
    H: int
    Hkv: int
    D: int
    windows: tuple  # each window is run separately on the same inputs
    dtype: torch.dtype
    rope_base: float = 10000.0


CONFIGS = {
    0: PrefillConfig(0, "tiny-fp32", B=1, T=64, H=2, Hkv=2, D=32, windows=(64,),
                     dtype=torch.float32),
    1: PrefillConfig(1, "d12-L-prefill", B=8, T=2048, H=6, Hkv=6, D=128,
                     windows=(2048,), dtype=torch.bfloat16),
    2: PrefillConfig(2, "d12-SSSL", B=8, T=2048, H=6, Hkv=6, D=128,
                     windows=(512, 512, 512, 2048), dtype=torch.bfloat16),
    3: PrefillConfig(3, "gqa-SSSL", B=16, T=2048, H=16, Hkv=4, D=64,
                     windows=(512, 512, 512, 2048), dtype=torch.bfloat16),
    4: DecodeConfig(4, "decode", B=64, Tmax=2048, H=6, Hkv=6, D=128,
                    windows=(512, 2048), dtype=torch.bfloat16),
}


def prefill_inputs(cfg: PrefillConfig, layer: int = 0, B=None, T=None):
    """q (B,T,H,D), k and v (B,T,Hkv,D); optional B/T override for samples."""
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    q = randn((B, T, cfg.H, cfg.D), seed_for(cfg.idx, layer, T_Q), cfg.dtype)
    k = randn((B, T, cfg.Hkv, cfg.D), seed_for(cfg.idx, layer, T_K), cfg.dtype)
    v = randn((B, T, cfg.Hkv, cfg.D), seed_for(cfg.idx, layer, T_V), cfg.dtype)
    return q, k, v


def prefill_dout(cfg: PrefillConfig, layer: int = 0):
    """dL/do (B,T,H,D) for the backward of layer `layer`: N(0,1), seeded."""
    return randn((cfg.B, cfg.T, cfg.H, cfg.D), seed_for(cfg.idx, layer, T_DOUT), cfg.dtype)


def decode_inputs(cfg: DecodeConfig, set_idx: int = 0):
    """q (B,H,D), k_new/v_new (B,Hkv,D), caches (B,Tmax,Hkv,D), seqlens (B,).

    set_idx selects an independent input set (used to rotate sets so that a
    repeated timing loop does not run out of the last-level cache).
    Sequence lengths L_b are uniform in [1, Tmax]; L_b counts the new token.
    """
    c = cfg.idx + 10 * set_idx
    q = randn((cfg.B, cfg.H, cfg.D), seed_for(c, 0, T_Q), cfg.dtype)
    k_new = randn((cfg.B, cfg.Hkv, cfg.D), seed_for(c, 0, T_K), cfg.dtype)
    v_new = randn((cfg.B, cfg.Hkv, cfg.D), seed_for(c, 0, T_V), cfg.dtype)
    k_cache = randn((cfg.B, cfg.Tmax, cfg.Hkv, cfg.D), seed_for(c, 0, T_KCACHE), cfg.dtype)
    v_cache = randn((cfg.B, cfg.Tmax, cfg.Hkv, cfg.D), seed_for(c, 0, T_VCACHE), cfg.dtype)
    seqlens = randint(1, cfg.Tmax, (cfg.B,), seed_for(c, 0, T_SEQLENS))
    return q, k_new, v_new, k_cache, v_cache, seqlens


# Chunked prefill of the d12 layer: the last 512-token chunk of a 2048-token
# context, whose first 1536 positions are already in the per-layer caches.
CHUNK = dict(B=8, T=512, P=1536, Tmax=2048, H=6, Hkv=6, D=128)


def prefill_chunk_inputs(seed: int = 0, dtype=torch.bfloat16, **kw):
    """q (B,T,H,D), k and v (B,T,Hkv,D) of the chunk and the two caches
    (B,Tmax,Hkv,D) of CHUNK's sizes (overridable); every cache row is N(0,1),
    those of the chunk are overwritten by the prefill."""
    c = dict(CHUNK, **kw)
    B, T, Tmax, H, Hkv, D = c["B"], c["T"], c["Tmax"], c["H"], c["Hkv"], c["D"]
    base = SEED_BASE + 900 + 10 * seed
    q = randn((B, T, H, D), base + T_Q, dtype)
    k = randn((B, T, Hkv, D), base + T_K, dtype)
    v = randn((B, T, Hkv, D), base + T_V, dtype)
    kc = randn((B, Tmax, Hkv, D), base + T_KCACHE, dtype)
    vc = randn((B, Tmax, Hkv, D), base + T_VCACHE, dtype)
    return q, k, v, kc, vc


# Several samples continuing one d12 prompt: 64 samples of a 1536-token prompt,
# each with 1..512 tokens of its own (the new one included).
SHARED = dict(B=64, Lp=1536, Tgen=512, H=6, Hkv=6, D=128)


def decode_shared_inputs(seed: int = 0, dtype=torch.bfloat16, **kw):
    """q (B,H,D), k_new and v_new (B,Hkv,D), the prompt caches (Lp,Hkv,D), the
    samples' caches (B,Tgen,Hkv,D) and seqlens (B,) = Lp + uniform [1, Tgen]."""
    c = dict(SHARED, **kw)
    B, Lp, Tgen, H, Hkv, D = c["B"], c["Lp"], c["Tgen"], c["H"], c["Hkv"], c["D"]
    base = SEED_BASE + 800 + 10 * seed
    q = randn((B, H, D), base + T_Q, dtype)
    k_new = randn((B, Hkv, D), base + T_K, dtype)
    v_new = randn((B, Hkv, D), base + T_V, dtype)
    k_prompt = randn((Lp, Hkv, D), base + T_KCACHE + 4, dtype)
    v_prompt = randn((Lp, Hkv, D), base + T_VCACHE + 4, dtype)
    k_cache = randn((B, Tgen, Hkv, D), base + T_KCACHE, dtype)
    v_cache = randn((B, Tgen, Hkv, D), base + T_VCACHE, dtype)
    seqlens = randint(1, Tgen, (B,), base + T_SEQLENS) + Lp
    return q, k_new, v_new, k_prompt, v_prompt, k_cache, v_cache, seqlens


def small_prefill(B, T, H, Hkv, D, seed, dtype=torch.bfloat16, scale=1.0):
    """Seeded small case for parity sweeps (ragged T, odd windows, ...)."""
    q = randn((B, T, H, D), seed, torch.float32) * scale
    k = randn((B, T, Hkv, D), seed + 1, torch.float32) * scale
    v = randn((B, T, Hkv, D), seed + 2, torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


# ---- counting helpers (pure combinatorics of the band mask, no arithmetic of
# ---- the method itself): unmasked (query, key) pairs per (b, h).

def unmasked_pairs(T: int, W: int) -> int:
    """Number of (i, j) with 0 <= i - j < W and 0 <= j <= i < T."""
    if W >= T:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


def chunk_pairs(T: int, P: int, W: int) -> int:
    """Number of (t, j) with 0 <= P + t - j < W, j >= 0, t < T: query t of a
    chunk at offset P sees min(W, P + t + 1) cache rows."""
    return sum(min(W, P + t + 1) for t in range(T))


def prefill_chunk_flops(B, T, P, H, D, W) -> int:
    return 4 * D * chunk_pairs(T, P, W) * B * H


def decode_shared_bytes(seqlens, Lp, Hkv, D, W, H, elem_bytes=2):
    """Algorithmic HBM bytes of one shared-prompt decode call: every prompt row
    visible to some sample, once; each sample's own visible rows; q, o, k_new,
    v_new. (decode_bytes of the same lengths counts the prompt rows once per
    sample, as over copies.)"""
    row = Hkv * D * 2 * elem_bytes
    lo_min = min(max(0, int(L) - W) for L in seqlens)
    prompt_rows = max(0, Lp - lo_min)
    own = sum(int(L) - max(Lp, int(L) - W) for L in seqlens)
    B = len(seqlens)
    return prompt_rows * row + own * row + (2 * B * H * D + 2 * B * Hkv * D) * elem_bytes


def prefill_flops(B, T, H, D, W) -> int:
    """4*D flops per unmasked pair (2D for q.k, 2D for p*v)."""
    return 4 * D * unmasked_pairs(T, W) * B * H


def backward_flops(B, T, H, D, W) -> int:
    """10*D flops per unmasked pair: the five products of the attention
    backward (q.k again, dO.v, P^T dO, dS k, dS^T q), 2D each."""
    return 10 * D * unmasked_pairs(T, W) * B * H


def decode_bytes(seqlens, Hkv, D, W, H, elem_bytes=2) -> int:
    """Algorithmic HBM bytes of one decode call.

    K and V rows visible under the window (the appended row included, read
    from registers but counted once as its cache write), plus q, o, k_new,
    v_new.
    """
    vis = sum(min(int(L), W) for L in seqlens)
    kv = vis * Hkv * D * 2 * elem_bytes
    B = len(seqlens)
    small = (2 * B * H * D + 2 * B * Hkv * D) * elem_bytes
    return kv + small


# Fused q, k, v projection before the attention: the d12 block (hidden 768,
# 6 heads of 128) and the hidden-1024 GQA block (16 query and 4 K/V heads of
# 64), over the same B x T tokens as the prefill workloads.
QKV = {
    "d12": dict(B=8, T=2048, C=768, H=6, Hkv=6, D=128),
    "gqa": dict(B=16, T=2048, C=1024, H=16, Hkv=4, D=64),
}


def qkv_inputs(B, T, C, H, Hkv, D, seed=0, dtype=torch.bfloat16):
    """x (B,T,C) ~ N(0,1), and bias-free weights w_q (H*D,C), w_k, w_v
    (Hkv*D,C): N(0,1)/sqrt(C) drawn in fp32 (the master weights) and cast to
    the compute type, as a linear layer does."""
    base = SEED_BASE + 700 + 10 * seed
    x = randn((B, T, C), base, dtype)
    s = C ** -0.5
    wq = (randn((H * D, C), base + 1, torch.float32) * s).to(dtype)
    wk = (randn((Hkv * D, C), base + 2, torch.float32) * s).to(dtype)
    wv = (randn((Hkv * D, C), base + 3, torch.float32) * s).to(dtype)
    return x, wq, wk, wv


def qkv_flops(B, T, C, H, Hkv, D) -> int:
    """2 flops per multiply-add of the three projections."""
    return 2 * B * T * C * (H + 2 * Hkv) * D
