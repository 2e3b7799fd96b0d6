"""Prefill into the KV cache (nc_attn_prefill) vs the fp64 oracle, through the C ABI.

Each chunk's queries sit at positions pos_offset.. and attend to cache rows;
its keys and values are written to the cache first. Checked: the output, the
chunk's cache rows (k' within the tolerance, v bit for bit), every other cache
row untouched, bitwise equality with nc_attn_fwd at offset 0, a chain of
chunks followed by a decode step, and the full-size chunk the benchmark times.
Tolerances as in test_gpu_parity: bf16 max-abs <= 2e-2, mean-abs <= 2e-3;
fp32 max-abs <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_rope_amd as nc
import workloads as wl

pytestmark = pytest.mark.gpu

BF_MAX, BF_MEAN, F32_MAX = 2e-2, 2e-3, 1e-5
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _check_rounded(got, ref, dtype, what):
    """A stored value against its fp64 definition: one rounding to the element
    type, |got - ref| <= 2^-8 |ref| for bf16 (1 ulp), 1e-5 for fp32."""
    g = got.detach().double().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    d = np.abs(g - r)
    bound = 1e-5 if dtype == torch.float32 else 2.0 ** -8 * np.abs(r) + 1e-6
    print(f"[err] {what}: max {d.max():.3e}, max relative {np.max(d / np.maximum(np.abs(r), 1e-6)):.3e}", flush=True)
    assert np.all(d <= bound), f"{what}: beyond one rounding of the element type"


def _check(got, ref, dtype, what):
    d = np.abs(got.detach().double().cpu().numpy() - np.asarray(ref, dtype=np.float64))
    mx, mn = float(d.max()), float(d.mean())
    print(f"[err] {what}: max {mx:.3e} mean {mn:.3e}", flush=True)
    if dtype == torch.float32:
        assert mx <= F32_MAX, f"{what}: max abs {mx:.3e} > {F32_MAX}"
    else:
        assert mx <= BF_MAX and mn <= BF_MEAN, f"{what}: max {mx:.3e} mean {mn:.3e}"


def _run_and_check(q, k, v, kc, vc, W, P, dtype, what):
    """One prefill call on copies of the caches, checked against the oracle."""
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    o = nc.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kcd, vcd, window=W, pos_offset=P)
    torch.cuda.synchronize()
    ro, rkc, _ = oracle.attn_prefill(q, k, v, kc, vc, W, 10000.0, P)
    _check(o, ro, dtype, f"{what} o")
    T = q.shape[1]
    _check(kcd[:, P:P + T], rkc[:, P:P + T], dtype, f"{what} cached k'")
    kc_h, vc_h = kcd.cpu(), vcd.cpu()
    assert torch.equal(vc_h[:, P:P + T], v), f"{what}: cached v differs"
    keep = torch.ones(kc.shape[1], dtype=torch.bool)
    keep[P:P + T] = False
    assert torch.equal(kc_h[:, keep], kc[:, keep]), f"{what}: k rows outside the chunk changed"
    assert torch.equal(vc_h[:, keep], vc[:, keep]), f"{what}: v rows outside the chunk changed"
    return o


PREFILL_SMALL = [
    # B, T, Tmax, pos_offset, H, Hkv, D, W, dtype
    (2, 100, 300, 64, 4, 2, 64, 80, torch.bfloat16),      # query head groups, generic path
    (1, 257, 600, 128, 2, 2, 128, 128, torch.bfloat16),   # offset on a 64-key tile: scheduled tiles
    (1, 200, 700, 300, 2, 2, 128, 2048, torch.bfloat16),  # offset inside a tile, full window
    (2, 130, 400, 37, 6, 6, 128, 100, torch.bfloat16),    # odd offset and window
    (1, 64, 64, 0, 2, 2, 32, 64, torch.bfloat16),         # the whole cache in one chunk
    (1, 1, 50, 49, 4, 1, 64, 10, torch.bfloat16),         # one token at the end of the cache
    (1, 600, 1200, 512, 2, 2, 128, 256, torch.bfloat16),  # window <= T/2: two-wave D=128 kernel
    (1, 300, 1024, 96, 1, 1, 32, 192, torch.bfloat16),    # 32-column waves, offset on a half tile
    (1, 300, 1024, 160, 2, 2, 64, 128, torch.bfloat16),   # the same at D=64
    (1, 70, 200, 130, 64, 1, 32, 70, torch.bfloat16),     # 64 query heads per K/V head
    # long key ranges for few query tiles: key tiles cut into slices
    (1, 300, 2000, 1600, 2, 2, 128, 2048, torch.bfloat16),  # offset inside a tile
    (1, 256, 2048, 1536, 4, 4, 64, 1536, torch.bfloat16),   # window edge inside the slices
    (2, 200, 1800, 1536, 3, 1, 128, 2048, torch.bfloat16),  # three query heads per K/V head
    (2, 100, 300, 64, 4, 2, 64, 80, torch.float32),
    (1, 150, 400, 77, 2, 1, 128, 2048, torch.float32),
    (1, 33, 33, 0, 2, 2, 32, 5, torch.float32),
]


@pytest.mark.parametrize("case", PREFILL_SMALL, ids=lambda c: "B{}T{}Tmax{}P{}H{}Hkv{}D{}W{}-{}".format(
    *c[:8], str(c[8]).split(".")[-1]))
def test_prefill_small(case):
    B, T, Tmax, P, H, Hkv, D, W, dtype = case
    _say(f"prefill {case}")
    g = torch.Generator().manual_seed(T * 31 + P + H)
    q = torch.randn(B, T, H, D, generator=g).to(dtype)
    k = torch.randn(B, T, Hkv, D, generator=g).to(dtype)
    v = torch.randn(B, T, Hkv, D, generator=g).to(dtype)
    kc = torch.randn(B, Tmax, Hkv, D, generator=g).to(dtype)
    vc = torch.randn(B, Tmax, Hkv, D, generator=g).to(dtype)
    _run_and_check(q, k, v, kc, vc, W, P, dtype, f"prefill {case}")


@pytest.mark.parametrize("H,Hkv,D,W", [(6, 6, 128, 2048), (6, 6, 128, 256), (8, 2, 64, 300)])
def test_prefill_offset_zero_equals_fwd_bitwise(H, Hkv, D, W):
    """At offset 0 the cache path runs the same arithmetic as nc_attn_fwd."""
    _say(f"prefill at offset 0 == attn_fwd H{H} Hkv{Hkv} D{D} W{W}")
    B, T, Tmax = 2, 700, 1000
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=77 + D, dtype=torch.bfloat16)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    kc = torch.zeros(B, Tmax, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    o1 = nc.attn_fwd(q, k, v, window=W)
    o2 = nc.attn_prefill(q, k, v, kc, vc, window=W)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_chunked_prefill_then_decode():
    """Three chunks and a decode step reproduce the whole-sequence forward."""
    _say("chunks 0:256, 256:500, 500:699, then decode of token 699")
    B, T, Tmax, H, Hkv, D = 2, 700, 800, 8, 2, 128
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=5150, dtype=torch.bfloat16)
    for W in (2048, 192):
        ref = oracle.attn_fwd(q, k, v, W)
        kc = torch.zeros(B, Tmax, Hkv, D, dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        for a, b in ((0, 256), (256, 500), (500, 699)):
            o = nc.attn_prefill(q[:, a:b].contiguous().to(DEV), k[:, a:b].contiguous().to(DEV),
                                v[:, a:b].contiguous().to(DEV), kc, vc, window=W, pos_offset=a)
            torch.cuda.synchronize()
            _check(o, ref[:, a:b], torch.bfloat16, f"W={W} chunk {a}:{b}")
        L = torch.full((B,), T, dtype=torch.int32, device=DEV)
        o = nc.attn_decode(q[:, T - 1].contiguous().to(DEV), k[:, T - 1].contiguous().to(DEV),
                           v[:, T - 1].contiguous().to(DEV), kc, vc, L, window=W)
        torch.cuda.synchronize()
        _check(o, ref[:, T - 1], torch.bfloat16, f"W={W} decode after chunks")


@pytest.mark.parametrize("W", [2048, 512])
def test_prefill_chunk_full_size(W):
    """The last 512-token chunk of a 2048-token d12 context (B=8, H=Hkv=6,
    D=128) at offset 1536, as the benchmark launches it, every output element
    against the oracle."""
    _say(f"full-size chunk B8 T512 P1536 Tmax2048 W{W}")
    q, k, v, kc, vc = wl.prefill_chunk_inputs(seed=W)
    _run_and_check(q, k, v, kc, vc, W, 1536, torch.bfloat16, f"d12 chunk W={W}")


# ------------------------------------------------ value-embedding gate (v' = v + gate * ve)

@pytest.mark.parametrize("case", [
    (2, 130, 400, 37, 6, 6, 128, 100, torch.bfloat16),
    (1, 300, 2000, 1600, 2, 2, 128, 2048, torch.bfloat16),  # sliced key tiles
    (2, 100, 300, 64, 4, 2, 64, 80, torch.float32),
], ids=lambda c: "B{}T{}Tmax{}P{}H{}Hkv{}D{}W{}-{}".format(*c[:8], str(c[8]).split(".")[-1]))
def test_prefill_value_gate(case):
    B, T, Tmax, P, H, Hkv, D, W, dtype = case
    _say(f"prefill with value gate {case}")
    g = torch.Generator().manual_seed(T + P)
    q = torch.randn(B, T, H, D, generator=g).to(dtype)
    k = torch.randn(B, T, Hkv, D, generator=g).to(dtype)
    v = torch.randn(B, T, Hkv, D, generator=g).to(dtype)
    ve = torch.randn(B, T, Hkv, D, generator=g).to(dtype)
    gate = (2 * torch.rand(B, T, Hkv, generator=g)).to(dtype)
    kc = torch.randn(B, Tmax, Hkv, D, generator=g).to(dtype)
    vc = torch.randn(B, Tmax, Hkv, D, generator=g).to(dtype)
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    o = nc.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kcd, vcd, window=W, pos_offset=P,
                        ve=ve.to(DEV), ve_gate=gate.to(DEV))
    torch.cuda.synchronize()
    ro, _, rvc = oracle.attn_prefill(q, k, v, kc, vc, W, 10000.0, P, ve=ve, ve_gate=gate)
    _check(o, ro, dtype, "o")
    _check_rounded(vcd[:, P:P + T], rvc[:, P:P + T], dtype, "cached v'")
    keep = torch.ones(Tmax, dtype=torch.bool)
    keep[P:P + T] = False
    assert torch.equal(vcd.cpu()[:, keep], vc[:, keep])


def test_prefill_zero_gate_bitwise():
    """A zero gate reproduces the ungated call bit for bit (v + 0 * ve = v)."""
    _say("prefill zero gate")
    q, k, v = wl.small_prefill(2, 300, 8, 2, 128, seed=12, dtype=torch.bfloat16)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    ve = torch.randn_like(v)
    kc1 = torch.zeros(2, 400, 2, 128, dtype=torch.bfloat16, device=DEV)
    vc1, kc2, vc2 = torch.zeros_like(kc1), torch.zeros_like(kc1), torch.zeros_like(kc1)
    o1 = nc.attn_prefill(q, k, v, kc1, vc1, window=200, pos_offset=64)
    o2 = nc.attn_prefill(q, k, v, kc2, vc2, window=200, pos_offset=64, ve=ve,
                         ve_gate=torch.zeros(2, 300, 2, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(vc1, vc2) and torch.equal(kc1, kc2)


@pytest.mark.parametrize("D,sliced", [(128, False), (64, True)])
def test_prefill_cache_rows_at_rms_bound(D, sliced):
    """Cache rows before the chunk are used as stored; the attention kernels
    exponentiate with a fixed scale, which is exact for stored rows of RMS up
    to 4 (the bound nc_attn_prefill states). Rows at RMS 4 (peaky softmax,
    scores up to 4*sqrt(D)) against the oracle, unsliced and sliced."""
    B, T, Tmax, P, H, Hkv = (2, 128, 640, 512, 4, 2) if not sliced else (1, 256, 2048, 1792, 2, 1)
    _say(f"prefill cache rows at the RMS bound D={D} sliced={sliced}")
    g = torch.Generator().manual_seed(515 + D)
    q = torch.randn(B, T, H, D, generator=g).bfloat16()
    k = torch.randn(B, T, Hkv, D, generator=g).bfloat16()
    v = torch.randn(B, T, Hkv, D, generator=g).bfloat16()
    kc = torch.randn(B, Tmax, Hkv, D, generator=g)
    kc = (kc * (4.0 / kc.pow(2).mean(-1, keepdim=True).sqrt())).bfloat16()  # every row at RMS 4
    vc = torch.randn(B, Tmax, Hkv, D, generator=g).bfloat16()
    rms = kc[:, :P].float().pow(2).mean(-1).sqrt().max().item()
    assert rms <= 4.0 * (1 + 2 ** -7), rms
    _run_and_check(q, k, v, kc, vc, 2048, P, torch.bfloat16, f"rms-bound D={D}")
