"""Attention backward (nc_attn_bwd) and the forward's row log-sum-exp
(nc_attn_fwd_lse) vs the fp64 oracle, through the C ABI.

The gradients come from the HIP chain itself: nc_attn_fwd_lse gives o and lse,
nc_attn_bwd takes them with dO; the oracle computes dq, dk, dv from q, k, v
and dO alone (oracle.attn_bwd), element by element over whole tensors.

Tolerances. lse (fp32 output of bf16 arithmetic): max-abs <= 2^-8 sqrt(D) +
2^-9 and mean-abs <= 4e-3 (2^-8). The bf16 rounding of q' and k' (2^-9
relative per element, both unit-RMS rows) moves a score q'.k'/sqrt(D) by at
most 2^-8 sqrt(D), and the row sum is formed from the bf16-rounded
exponentials the MFMA consumes (2^-9 relative each, which a row of one key
keeps whole). Measured: up to 1.0e-2 over the 524,288 rows of a GQA layer, a
mean of 3e-4 to 9e-4 on long rows, 2.8e-3 on one-key rows.
Gradients in bf16: max-abs <= 2e-2 * max|ref| and mean-abs <= 1e-2 * mean|ref|
over each tensor: the gradients are sums of many terms with cancellation
(their largest elements are 20-40 times their RMS at T = 2048), so a bar
relative to the tensor's own scale is the meaningful one. The bf16 rounding of
the output alone is 2^-9 relative; with the bf16 MFMA operands (q', k', P, dS,
dO) an emulation of the kernels' roundings gives 0.26-1.1% of max|ref| and
0.33-0.38% of mean|ref|. Both bars add an absolute 1e-5 for tensors whose
exact value is zero (a single visible key gives dq = dk = 0 exactly, and the
kernel leaves the fp32 rounding of dO.v - dO.o, two D-term sums, about
D * 2^-24 of their terms: up to 1.1e-6 measured). fp32: max-abs <=
1e-5 * max(1, max|ref|) for the gradients, 1e-5 for o and lse.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_rope_amd as nc
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def LSE_MAX(D):
    return 2.0 ** -8 * D ** 0.5 + 2.0 ** -9


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.detach().double().cpu().numpy()


def _check_abs(got, ref, mx_tol, mn_tol, what):
    d = np.abs(_np(got) - ref)
    print(f"[err] {what}: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= mx_tol and d.mean() <= mn_tol, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _check_grad(got, ref, dtype, what):
    g = _np(got)
    d = np.abs(g - ref)
    amax, amean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    print(f"[err] {what}: max {d.max():.3e} (ref max {amax:.3e}) mean {d.mean():.3e} "
          f"(ref mean {amean:.3e})", flush=True)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    if dtype == torch.float32:
        assert d.max() <= 1e-5 * max(1.0, amax), f"{what}: max {d.max():.3e}"
    else:
        assert d.max() <= 2e-2 * amax + 1e-5 and d.mean() <= 1e-2 * amean + 1e-5, \
            f"{what}: max {d.max():.3e} vs {2e-2 * amax:.3e}, mean {d.mean():.3e} vs {1e-2 * amean:.3e}"


def _run(q, k, v, do, W, off):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = nc.attn_fwd_lse(qd, kd, vd, window=W, pos_offset=off)
    dq, dk, dv = nc.attn_bwd(qd, kd, vd, o, dod, lse, window=W, pos_offset=off)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


SMALL = [
    # B, T, H, Hkv, D, W, pos_offset, dtype
    (1, 1, 1, 1, 128, 1, 0, torch.bfloat16),
    (2, 37, 4, 4, 64, 37, 0, torch.bfloat16),
    (1, 64, 2, 2, 32, 64, 0, torch.bfloat16),
    (2, 129, 6, 6, 128, 129, 5, torch.bfloat16),
    (1, 200, 8, 2, 64, 50, 3, torch.bfloat16),
    (1, 300, 6, 2, 128, 100, 0, torch.bfloat16),
    (1, 100, 16, 1, 32, 7, 0, torch.bfloat16),
    (1, 256, 2, 2, 128, 1, 0, torch.bfloat16),
    (3, 160, 4, 2, 64, 128, 0, torch.bfloat16),
    (1, 333, 4, 4, 128, 2048, 0, torch.bfloat16),
    (1, 513, 2, 1, 128, 256, 11, torch.bfloat16),
    (2, 1000, 2, 2, 64, 300, 0, torch.bfloat16),
    (1, 64, 2, 2, 32, 64, 0, torch.float32),
    (2, 100, 4, 2, 64, 30, 0, torch.float32),
    (1, 150, 2, 1, 128, 150, 7, torch.float32),
    (1, 1, 1, 1, 32, 1, 0, torch.float32),
    (1, 131, 6, 3, 64, 1, 0, torch.float32),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}T{}H{}Hkv{}D{}W{}off{}-{}".format(
    *c[:7], str(c[7]).split(".")[-1]))
def test_backward_small(case):
    B, T, H, Hkv, D, W, off, dtype = case
    _say(f"backward {case}")
    q, k, v = wl.small_prefill(B, T, H, Hkv, D, seed=3000 + T + D, dtype=dtype)
    do = wl.randn((B, T, H, D), 3500 + T, dtype)
    o, lse, dq, dk, dv = _run(q, k, v, do, W, off)
    ro, rlse = oracle.attn_fwd_lse(q, k, v, W, 10000.0, off)
    if dtype == torch.float32:
        _check_abs(o, ro, 1e-5, 1e-5, "o")
        _check_abs(lse, rlse, 1e-5, 1e-5, "lse")
    else:
        _check_abs(o, ro, 2e-2, 2e-3, "o")
        _check_abs(lse, rlse, LSE_MAX(D), 4e-3, "lse")
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, W, 10000.0, off)
    _check_grad(dq, rq, dtype, "dq")
    _check_grad(dk, rk, dtype, "dk")
    _check_grad(dv, rv, dtype, "dv")


def test_fwd_lse_output_equals_fwd():
    """nc_attn_fwd_lse's o equals nc_attn_fwd's (bit for bit where both run
    the same kernel; at D = 128 the lse form runs the two-wave kernel, whose
    rounding order may differ in the last bit)."""
    _say("fwd_lse o vs fwd")
    for (D, W) in ((64, 300), (128, 200), (32, 1000)):
        q, k, v = wl.small_prefill(2, 700, 4, 2, D, seed=77 + D, dtype=torch.bfloat16)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        o1 = nc.attn_fwd(qd, kd, vd, window=W)
        o2, _ = nc.attn_fwd_lse(qd, kd, vd, window=W)
        torch.cuda.synchronize()
        if D != 128:
            assert torch.equal(o1, o2), f"D={D}"
        else:
            assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -7


FULL_LAYERS = [(1, 0), (2, 0), (2, 1), (2, 2), (2, 3), (3, 0), (3, 1), (3, 2), (3, 3)]


@pytest.mark.parametrize("cidx,layer", FULL_LAYERS, ids=lambda x: str(x))
def test_backward_full_size_whole(cidx, layer):
    """Every layer of configs 1-3 at full size: lse and the three gradients
    against the oracle on whole tensors (the oracle runs one sequence at a time)."""
    cfg = wl.CONFIGS[cidx]
    W = cfg.windows[layer]
    _say(f"backward config {cidx} layer {layer} W={W} full size")
    q, k, v = wl.prefill_inputs(cfg, layer)
    do = wl.prefill_dout(cfg, layer)
    o, lse, dq, dk, dv = _run(q, k, v, do, W, 0)
    got = [_np(x) for x in (lse, dq, dk, dv)]
    del o, lse, dq, dk, dv
    refs = [[], [], [], []]
    for b in range(cfg.B):
        _, rl = oracle.attn_fwd_lse(q[b:b + 1], k[b:b + 1], v[b:b + 1], W)
        rq, rk, rv = oracle.attn_bwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], do[b:b + 1], W)
        for lst, x in zip(refs, (rl, rq, rk, rv)):
            lst.append(x)
    refs = [np.concatenate(r, axis=0) for r in refs]
    d = np.abs(got[0] - refs[0])
    print(f"[err] lse: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= LSE_MAX(cfg.D) and d.mean() <= 4e-3
    for name, g, r in zip(("dq", "dk", "dv"), got[1:], refs[1:]):
        dd = np.abs(g - r)
        amax, amean = float(np.abs(r).max()), float(np.abs(r).mean())
        print(f"[err] {name}: max {dd.max():.3e} (ref max {amax:.3e}) mean {dd.mean():.3e} "
              f"(ref mean {amean:.3e})", flush=True)
        assert np.all(np.isfinite(g))
        assert dd.max() <= 2e-2 * amax + 1e-5 and dd.mean() <= 1e-2 * amean + 1e-5, name
