"""Multi-sample decode over one shared prompt cache (nc_attn_decode_shared) vs
the fp64 oracle, through the C ABI.

Checked: the output, the appended rows (k' within the tolerance, v bit for
bit), every other row of the samples' caches and the prompt cache unchanged
bit for bit, agreement with nc_attn_decode over per-sample copies of the
prompt cache, the prefill-once-then-sample chain, and the full-size case the
benchmark times. Tolerances as in test_gpu_parity: bf16 max-abs <= 2e-2,
mean-abs <= 2e-3; fp32 max-abs <= 1e-5.
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


def _inputs(B, Lp, Tgen, H, Hkv, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    t = lambda *s: torch.randn(*s, generator=g).to(dtype)
    q, kn, vn = t(B, H, D), t(B, Hkv, D), t(B, Hkv, D)
    kp, vp = t(Lp, Hkv, D), t(Lp, Hkv, D)
    kc, vc = t(B, Tgen, Hkv, D), t(B, Tgen, Hkv, D)
    L = torch.randint(Lp + 1, Lp + Tgen + 1, (B,), generator=g, dtype=torch.int32)
    L[0] = Lp + 1
    L[-1] = Lp + Tgen
    return q, kn, vn, kp, vp, kc, vc, L


def _run_and_check(q, kn, vn, kp, vp, kc, vc, L, W, dtype, what):
    kpd, vpd, kcd, vcd = kp.to(DEV), vp.to(DEV), kc.to(DEV), vc.to(DEV)
    o = nc.attn_decode_shared(q.to(DEV), kn.to(DEV), vn.to(DEV), kpd, vpd, kcd, vcd, L.to(DEV), window=W)
    torch.cuda.synchronize()
    ro, rkc, _ = oracle.attn_decode_shared(q, kn, vn, kp, vp, kc, vc, L, W)
    _check(o, ro, dtype, f"{what} o")
    B, Lp = q.shape[0], kp.shape[0]
    rows = (L.long() - 1 - Lp)
    _check(kcd[torch.arange(B), rows.to(DEV)], rkc[np.arange(B), rows.numpy()], dtype, f"{what} appended k")
    assert torch.equal(vcd[torch.arange(B), rows.to(DEV)].cpu(), vn), f"{what}: appended v differs"
    keep = torch.ones(kc.shape[:2], dtype=torch.bool)
    keep[torch.arange(B), rows] = False
    assert torch.equal(kcd.cpu()[keep], kc[keep]) and torch.equal(vcd.cpu()[keep], vc[keep]), \
        f"{what}: other sample rows changed"
    assert torch.equal(kpd.cpu(), kp) and torch.equal(vpd.cpu(), vp), f"{what}: prompt cache changed"
    return o


SHARED_SMALL = [
    # B, Lp, Tgen, H, Hkv, D, W, dtype
    (4, 100, 50, 4, 2, 128, 2048, torch.bfloat16),
    (3, 300, 200, 6, 6, 128, 128, torch.bfloat16),   # the window leaves the prompt for long samples
    (5, 64, 64, 8, 2, 64, 100, torch.bfloat16),
    (2, 1, 30, 2, 1, 32, 5, torch.bfloat16),         # a one-token prompt
    (4, 257, 129, 16, 1, 64, 300, torch.bfloat16),   # 16 query heads per K/V head
    (70, 600, 90, 6, 6, 128, 2048, torch.bfloat16),  # enough samples that ranges are not split by size
    (3, 90, 40, 4, 2, 64, 60, torch.float32),
    (2, 33, 17, 2, 2, 32, 2048, torch.float32),
    # prompts of which a sequence sees 1024 rows or more: each range is cut at
    # the prompt's end (G = 1, 4, 8; a window shorter than the longest
    # sequence; fp32)
    (10, 1100, 60, 4, 4, 64, 4096, torch.bfloat16),
    (5, 1030, 30, 8, 2, 128, 2048, torch.bfloat16),
    (3, 1024, 20, 16, 2, 32, 1100, torch.bfloat16),
    (4, 1200, 100, 4, 2, 64, 1100, torch.bfloat16),
    (3, 1050, 20, 2, 2, 32, 4096, torch.float32),
]


@pytest.mark.parametrize("case", SHARED_SMALL, ids=lambda c: "B{}Lp{}Tgen{}H{}Hkv{}D{}W{}-{}".format(
    *c[:7], str(c[7]).split(".")[-1]))
def test_decode_shared_small(case):
    B, Lp, Tgen, H, Hkv, D, W, dtype = case
    _say(f"decode_shared {case}")
    args = _inputs(B, Lp, Tgen, H, Hkv, D, dtype, seed=Lp * 13 + Tgen + B)
    _run_and_check(*args, W, dtype, f"decode_shared {case}")


def test_decode_shared_matches_copied_caches():
    """The same step through nc_attn_decode over per-sample copies of the prompt
    cache (the copy the shared form avoids) agrees with it, both against the oracle."""
    _say("decode_shared vs nc_attn_decode over copies")
    B, Lp, Tgen, H, Hkv, D, W = 6, 400, 100, 8, 2, 128, 256
    q, kn, vn, kp, vp, kc, vc, L = _inputs(B, Lp, Tgen, H, Hkv, D, torch.bfloat16, seed=7)
    o1 = _run_and_check(q, kn, vn, kp, vp, kc, vc, L, W, torch.bfloat16, "shared")
    kfull = torch.cat([kp.unsqueeze(0).expand(B, -1, -1, -1), kc], dim=1).contiguous().to(DEV)
    vfull = torch.cat([vp.unsqueeze(0).expand(B, -1, -1, -1), vc], dim=1).contiguous().to(DEV)
    o2 = nc.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), kfull, vfull, L.to(DEV), window=W)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs()
    print(f"[err] shared vs copied: max {d.max().item():.3e}", flush=True)
    assert d.max().item() <= BF_MAX


def test_prefill_once_then_samples():
    """A prompt prefilled once at batch 1 into the prompt cache, then N samples
    each decode their first token from it: every sample's output is the last row
    of the whole-sequence forward over the prompt plus that sample's token."""
    _say("prefill at batch 1, then 5 samples decode their first token")
    Lp, N, H, Hkv, D, W = 300, 5, 8, 2, 128, 2048
    qp, kpr, vpr = wl.small_prefill(1, Lp, H, Hkv, D, seed=99, dtype=torch.bfloat16)
    kcache = torch.zeros(1, Lp, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vcache = torch.zeros_like(kcache)
    nc.attn_prefill(qp.to(DEV), kpr.to(DEV), vpr.to(DEV), kcache, vcache, window=W)
    g = torch.Generator().manual_seed(5)
    qs = torch.randn(N, H, D, generator=g).bfloat16()
    ks = torch.randn(N, Hkv, D, generator=g).bfloat16()
    vs = torch.randn(N, Hkv, D, generator=g).bfloat16()
    kc = torch.zeros(N, 8, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    L = torch.full((N,), Lp + 1, dtype=torch.int32, device=DEV)
    o = nc.attn_decode_shared(qs.to(DEV), ks.to(DEV), vs.to(DEV), kcache[0], vcache[0], kc, vc, L, window=W)
    torch.cuda.synchronize()
    for n in range(N):
        qf = torch.cat([qp, qs[n][None, None]], dim=1)
        kf = torch.cat([kpr, ks[n][None, None]], dim=1)
        vf = torch.cat([vpr, vs[n][None, None]], dim=1)
        ref = oracle.attn_fwd_rows(qf, kf, vf, [(0, Lp, h) for h in range(H)], W)
        _check(o[n], ref, torch.bfloat16, f"sample {n}")


@pytest.mark.parametrize("W", [2048, 512])
def test_decode_shared_full_size(W):
    """64 samples of a 1536-token d12 prompt (H = Hkv = 6, D = 128), each with
    1..512 tokens of its own, as the benchmark launches it."""
    _say(f"decode_shared full size B64 Lp1536 Tgen512 W{W}")
    q, kn, vn, kp, vp, kc, vc, L = wl.decode_shared_inputs(seed=W)
    _run_and_check(q, kn, vn, kp, vp, kc, vc, L, W, torch.bfloat16, f"d12 shared W={W}")


@pytest.mark.parametrize("shared", [False, True])
def test_decode_value_gate(shared):
    """The new token's value embedding (v_new + gate * ve_new) in nc_attn_decode and
    nc_attn_decode_shared against the oracle."""
    _say(f"decode with value gate, shared={shared}")
    B, Lp, Tgen, H, Hkv, D, W = 5, 200, 100, 8, 2, 128, 256
    q, kn, vn, kp, vp, kc, vc, L = _inputs(B, Lp, Tgen, H, Hkv, D, torch.bfloat16, seed=31)
    g = torch.Generator().manual_seed(32)
    ve = torch.randn(B, Hkv, D, generator=g).bfloat16()
    gate = (2 * torch.rand(B, Hkv, generator=g)).bfloat16()
    if shared:
        kcd, vcd = kc.to(DEV), vc.to(DEV)
        o = nc.attn_decode_shared(q.to(DEV), kn.to(DEV), vn.to(DEV), kp.to(DEV), vp.to(DEV), kcd, vcd,
                                  L.to(DEV), window=W, ve=ve.to(DEV), ve_gate=gate.to(DEV))
        ro, _, rvc = oracle.attn_decode_shared(q, kn, vn, kp, vp, kc, vc, L, W, ve_new=ve, ve_gate_new=gate)
        rows = L.long() - 1 - Lp
    else:
        kfull = torch.cat([kp.unsqueeze(0).expand(B, -1, -1, -1), kc], dim=1).contiguous()
        vfull = torch.cat([vp.unsqueeze(0).expand(B, -1, -1, -1), vc], dim=1).contiguous()
        kcd, vcd = kfull.to(DEV), vfull.to(DEV)
        o = nc.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), kcd, vcd, L.to(DEV), window=W,
                           ve=ve.to(DEV), ve_gate=gate.to(DEV))
        ro, _, rvc = oracle.attn_decode(q, kn, vn, kfull, vfull, L, W, ve_new=ve, ve_gate_new=gate)
        rows = L.long() - 1
    torch.cuda.synchronize()
    _check(o, ro, torch.bfloat16, "o")
    _check_rounded(vcd[torch.arange(B), rows.to(DEV)], rvc[np.arange(B), rows.numpy()], torch.bfloat16,
                   "appended v'")
