"""Fused bias-free q, k, v projection with the RoPE and QK-norm epilogue
(nc_qkv_rope_qknorm) vs the fp64 oracle (oracle.qkv_rope_qknorm), through the
C ABI, every output element.

Tolerances: q' and k' (unit-RMS rows) as for nc_rope_qknorm: bf16 max-abs <=
2e-2 and mean-abs <= 2e-3; fp32 max-abs <= 1e-5. v = x w_v^T is a plain
projection: one bf16 rounding of the fp32 accumulator, |err| <= 2^-8 |ref| +
1e-3 per element (bf16), max-abs <= 1e-5 max(1, max|ref|) (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_rope_amd as nc
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.detach().double().cpu().numpy()


def _check_unit(got, ref, dtype, what):
    d = np.abs(_np(got) - ref)
    print(f"[err] {what}: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    if dtype == torch.float32:
        assert d.max() <= 1e-5, what
    else:
        assert d.max() <= 2e-2 and d.mean() <= 2e-3, what


def _check_v(got, ref, dtype):
    g = _np(got)
    d = np.abs(g - ref)
    print(f"[err] v: max {d.max():.3e} (ref max {np.abs(ref).max():.3e}) mean {d.mean():.3e}", flush=True)
    if dtype == torch.float32:
        assert d.max() <= 1e-5 * max(1.0, float(np.abs(ref).max())), "v"
    else:
        assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 1e-3), "v beyond one rounding"


def _run(B, T, C, H, Hkv, D, off, dtype, seed):
    x, wq, wk, wv = wl.qkv_inputs(B, T, C, H, Hkv, D, seed=seed, dtype=dtype)
    q, k, v = nc.qkv_rope_qknorm(x.to(DEV), wq.to(DEV), wk.to(DEV), wv.to(DEV), H=H, Hkv=Hkv,
                                 pos_offset=off)
    torch.cuda.synchronize()
    return (x, wq, wk, wv), (q, k, v)


CASES = [
    # B, T, C, H, Hkv, D, pos_offset, dtype
    (1, 1, 64, 1, 1, 32, 0, torch.bfloat16),
    (2, 37, 128, 4, 2, 64, 5, torch.bfloat16),
    (1, 300, 64, 6, 2, 128, 0, torch.bfloat16),
    (3, 100, 192, 2, 1, 32, 1000, torch.bfloat16),
    (1, 257, 256, 16, 4, 64, 0, torch.bfloat16),
    (2, 129, 768, 6, 6, 128, 3, torch.bfloat16),
    (1, 513, 1024, 3, 1, 128, 0, torch.bfloat16),
    # head counts that leave the last 128-row group part empty
    (1, 90, 128, 3, 3, 64, 2, torch.bfloat16),
    (2, 70, 192, 6, 3, 32, 0, torch.bfloat16),
    (1, 40, 64, 5, 1, 64, 0, torch.bfloat16),
    (1, 64, 64, 2, 2, 32, 0, torch.float32),
    (2, 33, 128, 4, 2, 64, 7, torch.float32),
    (1, 20, 64, 2, 1, 128, 0, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}C{}H{}Hkv{}D{}off{}-{}".format(
    *c[:7], str(c[7]).split(".")[-1]))
def test_qkv_small(case):
    B, T, C, H, Hkv, D, off, dtype = case
    _say(f"qkv {case}")
    (x, wq, wk, wv), (q, k, v) = _run(B, T, C, H, Hkv, D, off, dtype, seed=T + C)
    rq, rk, rv = oracle.qkv_rope_qknorm(x, wq, wk, wv, H, Hkv, 10000.0, off)
    _check_unit(q, rq, dtype, "q'")
    _check_unit(k, rk, dtype, "k'")
    _check_v(v, rv, dtype)


@pytest.mark.parametrize("name", ["d12", "gqa"])
def test_qkv_full_size(name):
    s = wl.QKV[name]
    _say(f"qkv full size {name} {s}")
    (x, wq, wk, wv), (q, k, v) = _run(s["B"], s["T"], s["C"], s["H"], s["Hkv"], s["D"], 0,
                                      torch.bfloat16, seed=0)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    del q, k, v
    for b in range(s["B"]):
        rq, rk, rv = oracle.qkv_rope_qknorm(x[b:b + 1], wq, wk, wv, s["H"], s["Hkv"])
        _check_unit(qc[b:b + 1], rq, torch.bfloat16, f"q' b={b}")
        _check_unit(kc[b:b + 1], rk, torch.bfloat16, f"k' b={b}")
        _check_v(vc[b:b + 1], rv, torch.bfloat16)


def _chain_max_bar(rv):
    """Max-abs bar of the chained block. The forward's own bar (2e-2: q', k'
    rounded to bf16 before the score products, P rounded for the value product,
    o rounded once) plus the rounding of v, which the projection stores in bf16
    while the oracle keeps it in fp64: |v~_j - v_j| <= 2^-9 |v_j| moves
    o = sum_j p_j v_j by at most 2^-9 sum_j p_j |v_j| <= 2^-9 max |v|."""
    return 2e-2 + 2.0 ** -9 * float(np.abs(rv).max())


CHAIN = [
    # B, T, C, H, Hkv, D, W, pos_offset
    (2, 300, 128, 4, 2, 64, 100, 5),
    (1, 257, 256, 6, 6, 128, 257, 0),
    (1, 130, 64, 16, 1, 32, 40, 0),
    (1, 2048, 256, 2, 2, 128, 2048, 0),  # few heads, long band: key-tile slices
]


@pytest.mark.parametrize("case", CHAIN, ids=lambda c: "B{}T{}C{}H{}Hkv{}D{}W{}off{}".format(*c))
def test_projection_then_attention(case):
    """x -> nc_qkv_rope_qknorm -> nc_attn_fwd_normed, the block's attention from
    its input with q', k' written once and read once, against the oracle's
    projection followed by its attention core on the same x and weights."""
    B, T, C, H, Hkv, D, W, off = case
    _say(f"projection then attention {case}")
    (x, wq, wk, wv), (q, k, v) = _run(B, T, C, H, Hkv, D, off, torch.bfloat16, seed=T + 5)
    o = nc.attn_fwd_normed(q, k, v, window=W)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope_qknorm(x, wq, wk, wv, H, Hkv, 10000.0, off)
    ro = oracle.attention_core(rq, rk, rv, W)
    d = np.abs(_np(o) - ro)
    print(f"[err] o: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= _chain_max_bar(rv) and d.mean() <= 2e-3


def test_projection_then_attention_full_size_d12():
    s = wl.QKV["d12"]
    _say("projection then attention, d12 block, full size")
    (x, wq, wk, wv), (q, k, v) = _run(s["B"], s["T"], s["C"], s["H"], s["Hkv"], s["D"], 0, torch.bfloat16,
                                      seed=1)
    o = nc.attn_fwd_normed(q, k, v, window=s["T"]).cpu()
    mx, tot, bar = 0.0, 0.0, float("inf")
    for b in range(s["B"]):
        rq, rk, rv = oracle.qkv_rope_qknorm(x[b:b + 1], wq, wk, wv, s["H"], s["Hkv"])
        d = np.abs(o[b:b + 1].double().numpy() - oracle.attention_core(rq, rk, rv, s["T"]))
        mx, tot, bar = max(mx, float(d.max())), tot + float(d.sum()), min(bar, _chain_max_bar(rv))
    print(f"[err] o whole tensor: max {mx:.3e} (bar {bar:.3e}) mean {tot / o.numel():.3e}", flush=True)
    assert mx <= bar and tot / o.numel() <= 2e-3


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_normed_equals_fwd_after_rope_qknorm(dtype):
    """nc_rope_qknorm then nc_attn_fwd_normed against the oracle forward from raw q, k, v."""
    _say(f"rope_qknorm then attn_fwd_normed {dtype}")
    q, k, v = wl.small_prefill(2, 200, 8, 2, 64, seed=88, dtype=dtype)
    qn, kn = nc.rope_qknorm(q.to(DEV), k.to(DEV), pos_offset=3)
    o = nc.attn_fwd_normed(qn, kn, v.to(DEV), window=90)
    torch.cuda.synchronize()
    d = np.abs(_np(o) - oracle.attn_fwd(q, k, v, 90, 10000.0, 3))
    print(f"[err] o: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    if dtype == torch.float32:
        assert d.max() <= 1e-5
    else:
        assert d.max() <= 2e-2 and d.mean() <= 2e-3


NORMED = [
    # B, T, H, Hkv, D, W, dtype
    (1, 1, 2, 1, 32, 1, torch.bfloat16),
    (2, 257, 8, 1, 64, 100, torch.bfloat16),
    (1, 130, 16, 1, 32, 7, torch.bfloat16),
    (1, 300, 4, 2, 128, 300, torch.bfloat16),
    (3, 77, 6, 6, 128, 64, torch.bfloat16),
    (1, 65, 4, 2, 64, 30, torch.float32),
    (2, 40, 2, 2, 128, 40, torch.float32),
]


@pytest.mark.parametrize("case", NORMED, ids=lambda c: "B{}T{}H{}Hkv{}D{}W{}-{}".format(
    *c[:6], str(c[6]).split(".")[-1]))
def test_attn_fwd_normed_small(case):
    """nc_attn_fwd_normed on rows that are already rotated and normalised (the
    oracle's q', k' rounded to the element type) against oracle.attention_core of
    the same rounded rows: one query, one-key windows, 16 query heads per K/V
    head, every D, fp32."""
    B, T, H, Hkv, D, W, dtype = case
    _say(f"attn_fwd_normed {case}")
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=T + 3 * H + D, dtype=torch.float32)
    qn, kn = oracle.rope_qknorm(q, k, 10000.0, 0)
    qn = torch.from_numpy(qn).to(dtype)
    kn = torch.from_numpy(kn).to(dtype)
    v = v.to(dtype)
    o = nc.attn_fwd_normed(qn.to(DEV), kn.to(DEV), v.to(DEV), window=W)
    torch.cuda.synchronize()
    ref = oracle.attention_core(qn.double().numpy(), kn.double().numpy(), v.double().numpy(), W)
    d = np.abs(_np(o) - ref)
    print(f"[err] o: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    if dtype == torch.float32:
        assert d.max() <= 1e-5
    else:
        assert d.max() <= 2e-2 and d.mean() <= 2e-3
