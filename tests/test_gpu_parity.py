"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerances (the stated bar for this path): bf16 I/O with fp32 accumulation:
max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 I/O: max-abs <= 1e-5.
Small shapes and the full-size workloads (every layer of the prefill
configurations, in the launches the benchmark times) compare every output
element.
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


def _err(got, ref):
    d = np.abs(got.detach().double().cpu().numpy() - np.asarray(ref, dtype=np.float64))
    return float(d.max()), float(d.mean())


def _check(got, ref, dtype, what):
    mx, mn = _err(got, ref)
    print(f"[err] {what}: max {mx:.3e} mean {mn:.3e}", flush=True)
    if dtype == torch.float32:
        assert mx <= F32_MAX, f"{what}: max abs {mx:.3e} > {F32_MAX}"
    else:
        assert mx <= BF_MAX and mn <= BF_MEAN, f"{what}: max {mx:.3e} mean {mn:.3e}"
    return mx, mn


# ---------------------------------------------------------------- prefill

SMALL_BF16 = [
    # B, T, H, Hkv, D, W, pos_offset
    (1, 1, 1, 1, 128, 1, 0),
    (2, 37, 4, 4, 64, 37, 0),
    (1, 64, 2, 2, 32, 64, 0),
    (2, 129, 6, 6, 128, 129, 5),
    (1, 200, 8, 2, 64, 50, 3),
    (1, 300, 6, 2, 128, 100, 0),
    (2, 130, 12, 2, 64, 64, 0),
    (1, 100, 16, 1, 32, 7, 0),
    (1, 70, 64, 1, 32, 70, 0),
    (1, 256, 2, 2, 128, 1, 0),
    (1, 257, 2, 1, 128, 65, 1000),
    (3, 160, 4, 2, 64, 128, 0),
    (1, 512, 1, 1, 128, 512, 0),
    (1, 333, 4, 4, 128, 2048, 0),
    (1, 190, 3, 1, 64, 33, 77),
    # one query head per K/V head and windows that are multiples of 64:
    # window-edge and diagonal tiles take the scheduled path
    (1, 700, 2, 2, 128, 128, 0),
    (2, 513, 4, 4, 64, 256, 3),
    (1, 300, 1, 1, 32, 192, 0),
    (1, 1100, 1, 1, 128, 64, 0),
    # eight query heads per K/V head at D = 128 (32 positions x 8 heads per
    # workgroup, generic masked path), and a long sequence whose window is a
    # multiple of 64 but shorter than T (window-edge tiles on every wave)
    (2, 400, 8, 1, 128, 200, 0),
    (1, 2048, 2, 2, 128, 1024, 0),
    (1, 1000, 4, 4, 64, 320, 0),
    # Most cases above launch fewer workgroups than half the device and so
    # cut their key tiles into slices; these launch enough not to
    # (432, 192, 160 and 288 workgroups), at ragged sizes
    (24, 300, 6, 6, 128, 100, 0),
    (16, 129, 16, 4, 64, 64, 0),
    (20, 130, 8, 8, 32, 37, 5),
    (6, 600, 6, 6, 128, 2048, 0),
    # few (sequence, head) pairs with bands of 24 or more key tiles: key
    # tiles cut into slices (4 slices, some of them empty for the first query
    # tiles; 3 slices with 4 query heads per workgroup; D = 32; a window of 1536)
    (1, 2048, 2, 2, 128, 2048, 0),
    (1, 1500, 4, 1, 64, 1500, 9),
    (2, 1700, 2, 2, 32, 1700, 0),
    (1, 2048, 1, 1, 128, 1536, 0),
]


@pytest.mark.parametrize("case", SMALL_BF16, ids=lambda c: "B{}T{}H{}Hkv{}D{}W{}off{}".format(*c))
def test_attn_fwd_bf16_small(case):
    B, T, H, Hkv, D, W, off = case
    _say(f"attn_fwd bf16 {case}")
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=1000 + T + H, dtype=torch.bfloat16)
    o = nc.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=W, pos_offset=off)
    torch.cuda.synchronize()
    ref = oracle.attn_fwd(q, k, v, W, 10000.0, off)
    _check(o, ref, torch.bfloat16, f"attn_fwd {case}")


SMALL_F32 = [
    (1, 64, 2, 2, 32, 64, 0),
    (2, 100, 4, 2, 64, 30, 0),
    (1, 150, 2, 1, 128, 150, 7),
    (1, 1, 1, 1, 32, 1, 0),
    (1, 131, 6, 3, 64, 1, 0),
]


@pytest.mark.parametrize("case", SMALL_F32, ids=lambda c: "B{}T{}H{}Hkv{}D{}W{}off{}".format(*c))
def test_attn_fwd_f32_small(case):
    B, T, H, Hkv, D, W, off = case
    _say(f"attn_fwd f32 {case}")
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=2000 + T, dtype=torch.float32)
    o = nc.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=W, pos_offset=off)
    torch.cuda.synchronize()
    _check(o, oracle.attn_fwd(q, k, v, W, 10000.0, off), torch.float32, f"f32 {case}")


def test_config0_tiny_fp32():
    cfg = wl.CONFIGS[0]
    _say("config 0 tiny fp32")
    q, k, v = wl.prefill_inputs(cfg)
    o = nc.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=cfg.windows[0])
    qo, ko = nc.rope_qknorm(q.to(DEV), k.to(DEV))
    torch.cuda.synchronize()
    _check(o, oracle.attn_fwd(q, k, v, cfg.windows[0]), torch.float32, "config 0 o")
    rq, rk = oracle.rope_qknorm(q, k)
    _check(qo, rq, torch.float32, "config 0 q'")
    _check(ko, rk, torch.float32, "config 0 k'")


def _full_size_properties(o, v, H, Hkv, W):
    """Every row: finite; row 0 equals v row 0 (its only visible key)."""
    G = H // Hkv
    of = o.float()
    assert torch.isfinite(of).all()
    d0 = (of[:, 0] - v[:, 0].float().repeat_interleave(G, dim=1)).abs().max().item()
    assert d0 <= BF_MAX, f"row 0 vs v0: {d0}"


# Every layer of configs 1-3 at full size, in the launch configuration the
# benchmark times, against the oracle on the WHOLE output tensor: the oracle
# runs one sequence at a time (bounded memory) and max-abs / mean-abs are
# taken over every element of o.
FULL_LAYERS = [(1, 0), (2, 0), (2, 1), (2, 2), (2, 3), (3, 0), (3, 1), (3, 2), (3, 3)]


@pytest.mark.parametrize("cidx,layer", FULL_LAYERS, ids=lambda x: str(x))
def test_full_size_prefill_whole(cidx, layer):
    cfg = wl.CONFIGS[cidx]
    W = cfg.windows[layer]
    _say(f"config {cidx} layer {layer} W={W} full size, whole tensor")
    q, k, v = wl.prefill_inputs(cfg, layer)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = nc.attn_fwd(qd, kd, vd, window=W)
    torch.cuda.synchronize()
    _full_size_properties(o, vd, cfg.H, cfg.Hkv, W)
    oc = o.cpu()
    mx, tot = 0.0, 0.0
    for b in range(cfg.B):
        ref = oracle.attn_fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], W)
        d = np.abs(oc[b:b + 1].double().numpy() - ref)
        mx = max(mx, float(d.max()))
        tot += float(d.sum())
    mn = tot / oc.numel()
    print(f"[err] config {cidx} layer {layer} whole tensor: max {mx:.3e} mean {mn:.3e}", flush=True)
    assert mx <= BF_MAX and mn <= BF_MEAN, f"config {cidx} layer {layer}: max {mx:.3e} mean {mn:.3e}"


def test_full_window_equals_causal_bitwise():
    _say("W>=T identical to W=T")
    q, k, v = wl.small_prefill(2, 700, 4, 2, 128, seed=5, dtype=torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = nc.attn_fwd(qd, kd, vd, window=700)
    b = nc.attn_fwd(qd, kd, vd, window=100000)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_pos_offset_invariance_gpu():
    _say("pos_offset invariance")
    q, k, v = wl.small_prefill(1, 400, 4, 4, 64, seed=6, dtype=torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = nc.attn_fwd(qd, kd, vd, window=128)
    b = nc.attn_fwd(qd, kd, vd, window=128, pos_offset=4096)
    torch.cuda.synchronize()
    mx, mn = _err(a, b.double().cpu().numpy())
    assert mx <= BF_MAX and mn <= BF_MEAN


def test_large_and_zero_rows():
    """QK-norm makes huge inputs safe; zero q rows give uniform weights."""
    _say("large and zero rows")
    q, k, v = wl.small_prefill(1, 150, 2, 2, 64, seed=8, dtype=torch.float32)
    q = q * 300.0
    k = k * 1e-3
    q[0, 10:20] = 0.0
    qb, kb, vb = q.bfloat16(), k.bfloat16(), v.bfloat16()
    o = nc.attn_fwd(qb.to(DEV), kb.to(DEV), vb.to(DEV), window=60)
    torch.cuda.synchronize()
    _check(o, oracle.attn_fwd(qb, kb, vb, 60), torch.bfloat16, "large/zero rows")


# ------------------------------------------------------------ rope_qknorm

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_rope_qknorm(dtype, D):
    _say(f"rope_qknorm {dtype} D={D}")
    q, k, _ = wl.small_prefill(3, 77, 6, 2, D, seed=D, dtype=dtype)
    qo, ko = nc.rope_qknorm(q.to(DEV), k.to(DEV), pos_offset=123, rope_base=500.0)
    torch.cuda.synchronize()
    rq, rk = oracle.rope_qknorm(q, k, 500.0, 123)
    _check(qo, rq, dtype, "q'")
    _check(ko, rk, dtype, "k'")


def test_rope_qknorm_in_place_full_size():
    cfg = wl.CONFIGS[1]
    _say("rope_qknorm in place, d12 shape")
    q, k, _ = wl.prefill_inputs(cfg)
    qd, kd = q.to(DEV), k.to(DEV)
    a, b = nc.rope_qknorm(qd, kd)
    qo, ko = nc.rope_qknorm(qd, kd, q_out=qd, k_out=kd)
    torch.cuda.synchronize()
    assert qo.data_ptr() == qd.data_ptr()
    assert torch.equal(qd, a) and torch.equal(kd, b)
    # sampled rows against the oracle (position-dependent rotation at large t)
    for (bb, t, h) in [(0, 0, 0), (7, 2047, 5), (3, 1000, 2)]:
        rq = oracle.qk_norm(oracle.rope(q[bb, t, h], t, 1e4))
        _check(qd[bb, t, h], rq, torch.bfloat16, f"q' row {(bb, t, h)}")


# ------------------------------------------------------------------ decode

def _decode_check(q, kn, vn, kc, vc, L, W, dtype, what):
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    o = nc.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), kcd, vcd, L.to(DEV), window=W)
    torch.cuda.synchronize()
    ro, rkc, rvc = oracle.attn_decode(q, kn, vn, kc, vc, L, W)
    _check(o, ro, dtype, f"{what} o")
    B = q.shape[0]
    idx = (L.long() - 1)
    got_k = kcd[torch.arange(B), idx.to(DEV)]
    _check(got_k, rkc[np.arange(B), idx.numpy()], dtype, f"{what} appended k")
    got_v = vcd[torch.arange(B), idx.to(DEV)].cpu()
    assert torch.equal(got_v, vn), f"{what}: appended v differs"
    # every other cache row is untouched
    mask = torch.ones(kc.shape[:2], dtype=torch.bool)
    mask[torch.arange(B), idx] = False
    assert torch.equal(kcd.cpu()[mask], kc[mask]) and torch.equal(vcd.cpu()[mask], vc[mask])



def test_prep_core_equals_fwd():
    """attn_prep followed by attn_core is exactly attn_fwd (same kernels, same workspace)."""
    _say("prep + core == fwd")
    q, k, v = wl.small_prefill(2, 300, 8, 2, 128, seed=4242)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o1 = nc.attn_fwd(q, k, v, window=200, pos_offset=7)
    ws = nc.attn_prep(k, pos_offset=7, H=8)
    o2 = nc.attn_core(q, v, ws, window=200)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)

DEC_SMALL = [
    # B, Tmax, H, Hkv, D, W, dtype
    (4, 300, 4, 2, 128, 100, torch.bfloat16),
    (3, 64, 2, 2, 32, 64, torch.float32),
    (5, 1000, 8, 2, 64, 2000, torch.bfloat16),
    (2, 129, 3, 1, 128, 1, torch.bfloat16),
    (4, 700, 16, 1, 64, 300, torch.bfloat16),
    (3, 257, 6, 2, 128, 64, torch.float32),
    (2, 90, 12, 4, 32, 40, torch.bfloat16),
]


@pytest.mark.parametrize("case", DEC_SMALL, ids=lambda c: "B{}T{}H{}Hkv{}D{}W{}-{}".format(
    *c[:6], str(c[6]).split(".")[-1]))
def test_decode_small(case):
    B, Tmax, H, Hkv, D, W, dtype = case
    _say(f"decode {case}")
    g = torch.Generator().manual_seed(Tmax * 7 + H)
    q = torch.randn(B, H, D, generator=g).to(dtype)
    kn = torch.randn(B, Hkv, D, generator=g).to(dtype)
    vn = torch.randn(B, Hkv, D, generator=g).to(dtype)
    kc = torch.randn(B, Tmax, Hkv, D, generator=g).to(dtype)
    vc = torch.randn(B, Tmax, Hkv, D, generator=g).to(dtype)
    L = torch.randint(1, Tmax + 1, (B,), generator=g, dtype=torch.int32)
    L[0] = 1
    L[-1] = Tmax
    _decode_check(q, kn, vn, kc, vc, L, W, dtype, f"decode {case}")


@pytest.mark.parametrize("W", [512, 2048])
def test_config4_decode_full_size(W):
    cfg = wl.CONFIGS[4]
    _say(f"config 4 decode W={W}")
    q, kn, vn, kc, vc, L = wl.decode_inputs(cfg)
    _decode_check(q, kn, vn, kc, vc, L, W, torch.bfloat16, f"config 4 W={W}")


def test_decode_ranked_placement_with_ties():
    """Unsplit decode over a long span (workgroups pick their (sequence, head,
    head group) by visible length): many equal lengths, lengths beyond the
    window, L = 1, and two query heads per K/V head; every output and the
    appended rows against the oracle."""
    _say("decode ranked placement")
    B, Tmax, H, Hkv, D, W = 64, 1100, 8, 4, 64, 1024  # 256 (b, g) workgroups: no split
    g = torch.Generator().manual_seed(2024)
    q = torch.randn(B, H, D, generator=g).bfloat16()
    kn = torch.randn(B, Hkv, D, generator=g).bfloat16()
    vn = torch.randn(B, Hkv, D, generator=g).bfloat16()
    kc = torch.randn(B, Tmax, Hkv, D, generator=g).bfloat16()
    vc = torch.randn(B, Tmax, Hkv, D, generator=g).bfloat16()
    pattern = [1, 1100, 700, 700, 64, 1024, 1025, 700, 3, 1100]
    L = torch.tensor([pattern[i % len(pattern)] for i in range(B)], dtype=torch.int32)
    assert nc.attn_decode_workspace_bytes(B, Tmax, H, Hkv, D, W) == 0
    _decode_check(q, kn, vn, kc, vc, L, W, torch.bfloat16, "ranked placement")


def test_decode_matches_prefill_gpu():
    """Decode of token L-1 over the prefill's k' and v equals prefill row L-1."""
    _say("decode vs prefill")
    B, T, H, Hkv, D = 2, 300, 8, 2, 128
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=44, dtype=torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for W in (64, 300):
        o_pre = nc.attn_fwd(qd, kd, vd, window=W)
        _, kprime = nc.rope_qknorm(qd, kd)
        for Lv in (1, 65, 300):
            kc = kprime.clone()
            vc = vd.clone()
            L = torch.full((B,), Lv, dtype=torch.int32, device=DEV)
            o = nc.attn_decode(qd[:, Lv - 1].contiguous(), kd[:, Lv - 1].contiguous(),
                               vd[:, Lv - 1].contiguous(), kc, vc, L, window=W)
            torch.cuda.synchronize()
            mx, mn = _err(o, o_pre[:, Lv - 1].double().cpu().numpy())
            assert mx <= BF_MAX and mn <= BF_MEAN, f"W={W} L={Lv}: {mx} {mn}"


def test_decode_workspace_reused_across_calls():
    """One workspace serves consecutive calls with different lengths and shapes."""
    _say("decode workspace reuse")
    ws = nc.decode_workspace(8, 2048, 8, 2, 128, 2048, device=DEV)
    g = torch.Generator().manual_seed(99)
    for it, (B, Tmax, H, Hkv, W) in enumerate([(8, 2048, 8, 2, 2048), (8, 2048, 8, 2, 2048),
                                               (4, 1500, 4, 2, 700), (8, 2048, 8, 2, 300)]):
        q = torch.randn(B, H, 128, generator=g).bfloat16()
        kn = torch.randn(B, Hkv, 128, generator=g).bfloat16()
        vn = torch.randn(B, Hkv, 128, generator=g).bfloat16()
        kc = torch.randn(B, Tmax, Hkv, 128, generator=g).bfloat16()
        vc = torch.randn(B, Tmax, Hkv, 128, generator=g).bfloat16()
        L = torch.randint(1, Tmax + 1, (B,), generator=g, dtype=torch.int32)
        o = nc.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), kc.to(DEV), vc.to(DEV), L.to(DEV),
                           window=W, workspace=ws)
        torch.cuda.synchronize()
        ro, _, _ = oracle.attn_decode(q, kn, vn, kc, vc, L, W)
        _check(o, ro, torch.bfloat16, f"decode reuse call {it}")
    assert nc.attn_decode_workspace_bytes(8, 2048, 8, 2, 128, 2048) > 0
