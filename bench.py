#!/usr/bin/env python3
"""Benchmark of the attention-block forward on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--settle-ms 100]

A step is one ``nc_attn_fwd`` call (RoPE + QK-norm + banded attention, the
prefill path end to end: the k'/table input stage and the attention kernel)
over the d12 L-layer batch: B=8, T=2048, H=Hkv=6, D=128, full causal window,
bf16, inputs resident in HBM. Four independent input sets are rotated so
repeated steps do not run out of the 256 MB last-level cache. ``value`` is
attention-forward TFLOP/s counting 4*D flops per unmasked (query, key) pair.

The same run also times, with HIP events on the launch stream:
  * the attention kernel alone (``nc_attn_core`` on workspaces filled by
    ``nc_attn_prep``), the basis of ``roofline`` (against the 2516.6 TFLOP/s
    bf16 dense peak);
  * the split-KV decode over a 2048-slot cache (B=64, H=Hkv=6, D=128) at
    window 512 and 2048, as HBM GB/s of algorithmic bytes;
  * ``nc_rope_qknorm`` on the d12 q and k, as HBM GB/s;
  * a 1 GiB device-to-device copy (torch), the practical HBM reference that the
    decode and rope figures are also given against (``frac_copy``);
  * the d12 SSSL and GQA SSSL stacks (4 ``nc_attn_fwd`` layer calls);
and, on the host, the fp64 oracle on a bounded sample (``cpu_baseline``).

Every timed part first runs untimed for about ``--settle-ms`` of back-to-back
GPU work, then ``--warmup`` untimed calls, then exactly ``--steps`` timed calls.
The settling run is there because the engine clock ramps up over the first
~30 ms of load after the GPU has been idle (the step runs about 20% slower at
first); without it the numbers depend on how long the host paused before the
part started.

Only rank 0 of a 1-GPU job exists here: ``--gpus`` above 1 exits.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention fwd TFLOP/s (unmasked pairs) + % bf16 MFMA peak; decode HBM GB/s"
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_d12_pmc.txt")
KERNEL_SOURCES = ["transformer_attention_rope_amd/csrc/attn_fwd.hip",
                  "transformer_attention_rope_amd/csrc/device_common.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the attention kernel from the committed PMC
    summary, or None when missing or taken on a different kernel source."""
    if not os.path.exists(PMC_FILE):
        return None
    kv = {}
    for line in open(PMC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def event_time_ms(fn, n, torch):
    """Average ms per call of fn() over n back-to-back calls on the current
    stream, bracketed by synchronisations."""
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(n):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def trial_times_ms(fn, trials, n, torch):
    """Per-call ms of `trials` separate runs of n back-to-back calls each."""
    return [event_time_ms(fn, n, torch) for _ in range(trials)]


def median(xs):
    xs = sorted(xs)
    m = len(xs) // 2
    return xs[m] if len(xs) % 2 else 0.5 * (xs[m - 1] + xs[m])


def settle(fn, ms, torch):
    """Run fn(i) untimed, keeping the GPU busy, until at least ms of GPU time
    has passed since the first call; returns the number of calls made."""
    if ms <= 0:
        return 0
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    start.record()
    n, chunk, prev = 0, 8, None
    while True:
        for _ in range(chunk):
            fn(n)
            n += 1
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        if prev is not None:           # one chunk stays queued while we look
            prev.synchronize()
            if start.elapsed_time(prev) >= ms:
                break
        prev = ev
    torch.cuda.synchronize()
    return n


def cpu_baseline(budget_s: float):
    """fp64 oracle on the d12 L-layer workload, one (b, h) head (full T=2048)
    at a time, until every head is done or about budget_s seconds passed."""
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cfg = wl.CONFIGS[1]
    W = cfg.windows[0]
    q, k, v = wl.prefill_inputs(cfg, 0)
    t0 = time.perf_counter()
    n = 0
    for b in range(cfg.B):
        for h in range(cfg.H):
            g = h // (cfg.H // cfg.Hkv)
            oracle.attn_fwd(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1], W)
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = wl.prefill_flops(1, cfg.T, n, cfg.D, W)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"d12 L-layer prefill, {n} of {cfg.B * cfg.H} (b,h) heads "
                      f"(T=2048, D=128, full causal), fp64 NumPy, {dt:.1f} s wall",
            "host_cpu_count": os.cpu_count(),
            "per_config_wall_s": oracle_wall_per_config()}


def oracle_wall_per_config():
    """Oracle wall time of each whole configuration, from a timed sample:
    config 0 whole; configs 1-3 one (b, h) head per layer, scaled by the
    heads; config 4 eight sequences per window, scaled by the batch."""
    import oracle
    import workloads as wl
    res = {}
    c0 = wl.CONFIGS[0]
    q, k, v = wl.prefill_inputs(c0)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, c0.windows[0])
    res["0"] = round(time.perf_counter() - t0, 4)
    for cidx in (1, 2, 3):
        c = wl.CONFIGS[cidx]
        tot = 0.0
        for l, w in enumerate(c.windows):
            q, k, v = wl.prefill_inputs(c, l, B=1)
            t0 = time.perf_counter()
            oracle.attn_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], w)
            tot += (time.perf_counter() - t0) * c.B * c.H
        res[str(cidx)] = round(tot, 2)
    c4 = wl.CONFIGS[4]
    q, kn, vn, kc, vc, L = wl.decode_inputs(c4)
    for w in c4.windows:
        t0 = time.perf_counter()
        oracle.attn_decode(q[:8], kn[:8], vn[:8], kc[:8], vc[:8], L[:8], w)
        res[f"4_W{w}"] = round((time.perf_counter() - t0) * c4.B / 8, 3)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed back-to-back GPU work before each timed part (clock ramp)")
    ap.add_argument("--sets", type=int, default=4, help="rotated input sets (defeats the MALL)")
    ap.add_argument("--only", default="all",
                    choices=["all", "fwd", "core", "decode", "rope", "stacks", "prefill", "shared", "gate",
                             "bwd", "qkv", "copy"],
                    help="run one part (used for profiler runs); 'copy' runs a plain "
                         "1 GiB device copy for counter calibration")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the attention forward shards over batch or K/V heads with no exchange). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attention_rope_amd as nc
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    K, Wm = args.steps, args.warmup
    out = {}
    settled = {}   # calls made by the settling run of each part

    def prime(name, fn):
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        settled[name] = settle(fn, args.settle_ms, torch)
        for i in range(Wm):
            fn(i)

    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    # ------------------------------------------------ step: d12 L-layer prefill
    cfg = wl.CONFIGS[1]
    W = cfg.windows[0]
    flops = wl.prefill_flops(cfg.B, cfg.T, cfg.H, cfg.D, W)
    if args.only in ("all", "fwd", "core"):
        sets = []
        for s in range(args.sets):
            q, k, v = wl.prefill_inputs(cfg, layer=s)  # set s uses layer index s in the seed
            sets.append((q.to(dev), k.to(dev), v.to(dev), torch.empty_like(q, device=dev)))
        nws = nc.attn_fwd_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.Hkv, cfg.D, 0, cfg.dtype)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)

        def step(i):
            q, k, v, o = sets[i % len(sets)]
            nc.attn_fwd(q, k, v, window=W, out=o, workspace=ws)

        if args.only in ("all", "fwd"):
            prime("step", step)
            ms = event_time_ms(step, K, torch)
            out["step_ms"] = ms
            # the timing protocol's median of 5 trials of 50 launches, and the
            # same with one input set (no rotation: the 256 MB last-level cache
            # then holds part of the inputs between steps)
            out["trials_ms"] = trial_times_ms(step, 5, min(50, K), torch)

            def step1(i):
                q, k, v, o = sets[0]
                nc.attn_fwd(q, k, v, window=W, out=o, workspace=ws)

            prime("step_one_set", step1)
            out["one_set_trials_ms"] = trial_times_ms(step1, 5, min(50, K), torch)
        if args.only in ("all", "core"):
            # one prepared workspace (k' and table) per input set
            wss = [nc.attn_prep(k, workspace=torch.empty_like(ws)) for (q, k, v, o) in sets]

            def kern(i):
                q, k, v, o = sets[i % len(sets)]
                nc.attn_core(q, v, wss[i % len(sets)], window=W, out=o)

            prime("core", kern)
            out["kern_ms"] = event_time_ms(kern, K, torch)
            del wss
        del sets, ws

    if args.only in ("fwd", "core"):
        out["settle_calls"] = settled
        print(json.dumps(out))
        return

    # --------------------------------------- device copy (HBM reference)
    copy_gbs = None
    if args.only in ("all", "decode", "rope"):
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)

        def cstep(i):
            dst.copy_(src)

        settle(cstep, args.settle_ms, torch)
        cms = event_time_ms(cstep, 20, torch)
        copy_gbs = 2 * n / (cms * 1e-3) / 1e9  # bytes read + written
        del src, dst

    # ------------------------------------------------------------ decode
    dec = {}
    if args.only in ("all", "decode"):
        dcfg = wl.CONFIGS[4]
        dsets = []
        for s in range(args.sets):
            q, kn, vn, kc, vc, L = wl.decode_inputs(dcfg, set_idx=s)
            dsets.append([t.to(dev) for t in (q, kn, vn, kc, vc, L)] + [torch.empty_like(q, device=dev)])
        for Wd in dcfg.windows:
            wsd = nc.decode_workspace(dcfg.B, dcfg.Tmax, dcfg.H, dcfg.Hkv, dcfg.D, Wd, device=dev)

            def dstep(i, Wd=Wd, wsd=wsd):
                q, kn, vn, kc, vc, L, o = dsets[i % len(dsets)]
                nc.attn_decode(q, kn, vn, kc, vc, L, window=Wd, out=o, workspace=wsd)

            prime(f"decode_W{Wd}", dstep)
            ms = event_time_ms(dstep, K, torch)
            nbytes = sum(wl.decode_bytes(ds[5].cpu().tolist(), dcfg.Hkv, dcfg.D, Wd, dcfg.H)
                         for ds in dsets) / len(dsets)
            gbs = nbytes / (ms * 1e-3) / 1e9
            dec[f"W{Wd}"] = {"us_per_call": round(ms * 1e3, 2), "GB_per_s": round(gbs, 1),
                             "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                             "frac_copy": round(gbs / copy_gbs, 4),
                             "algorithmic_bytes": int(nbytes)}
        del dsets
        if args.only == "decode":
            print(json.dumps(dec))
            return

    # ------------------------------------------------------- rope_qknorm
    rope = {}
    if args.only in ("all", "rope"):
        rsets = []
        for s in range(args.sets):
            q, k, _ = wl.prefill_inputs(cfg, layer=s)
            rsets.append((q.to(dev), k.to(dev), torch.empty_like(q, device=dev),
                          torch.empty_like(k, device=dev)))

        def rstep(i):
            q, k, qo, ko = rsets[i % len(rsets)]
            nc.rope_qknorm(q, k, q_out=qo, k_out=ko)

        prime("rope", rstep)
        ms = event_time_ms(rstep, K, torch)
        nbytes = 2 * (rsets[0][0].numel() + rsets[0][1].numel()) * 2
        gbs = nbytes / (ms * 1e-3) / 1e9
        rope = {"workload": "q,k of the d12 layer (8x2048x6x128 each), bf16, read + write",
                "us_per_call": round(ms * 1e3, 2), "GB_per_s": round(gbs, 1),
                "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                "frac_copy": round(gbs / copy_gbs, 4)}
        del rsets
        if args.only == "rope":
            print(json.dumps(rope))
            return

    # -------------------------------------------------- SSSL / GQA stacks
    stacks = {}
    if args.only in ("all", "stacks"):
        for cidx in (2, 3):
            c = wl.CONFIGS[cidx]
            layers = [tuple(t.to(dev) for t in wl.prefill_inputs(c, layer=l)) for l in range(4)]
            outs = [torch.empty_like(l[0]) for l in layers]
            wsc = torch.empty(nc.attn_fwd_workspace_bytes(c.B, c.T, c.H, c.Hkv, c.D, 0, c.dtype),
                              dtype=torch.uint8, device=dev)

            def sstep(i, layers=layers, outs=outs, wsc=wsc, c=c):
                for l, (q, k, v) in enumerate(layers):
                    nc.attn_fwd(q, k, v, window=c.windows[l], out=outs[l], workspace=wsc)

            prime(c.name, sstep)
            ms = event_time_ms(sstep, K, torch)
            fl = sum(wl.prefill_flops(c.B, c.T, c.H, c.D, w) for w in c.windows)
            tf = fl / (ms * 1e-3) / 1e12
            stacks[c.name] = {"shape": f"B={c.B} T={c.T} H={c.H} Hkv={c.Hkv} D={c.D} "
                                       f"windows={list(c.windows)}",
                              "us_per_stack": round(ms * 1e3, 2), "TFLOP_per_s": round(tf, 1),
                              "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                              "stack_trials_median_us": round(
                                  median(trial_times_ms(sstep, 5, min(13, K), torch)) * 1e3, 2)}
            # each layer alone (prep + attention), and its attention kernel alone
            per = []
            for l, (q, k, v) in enumerate(layers):
                w_l = c.windows[l]

                def lstep(i, q=q, k=k, v=v, l=l, w_l=w_l):
                    nc.attn_fwd(q, k, v, window=w_l, out=outs[l], workspace=wsc)

                wsl = nc.attn_prep(k, H=c.H, workspace=torch.empty_like(wsc))

                def kstep(i, q=q, v=v, l=l, w_l=w_l, wsl=wsl):
                    nc.attn_core(q, v, wsl, window=w_l, out=outs[l])

                prime(f"{c.name}_layer{l}", lstep)
                ms_l = event_time_ms(lstep, K, torch)
                prime(f"{c.name}_core{l}", kstep)
                ms_k = event_time_ms(kstep, K, torch)
                fl_l = wl.prefill_flops(c.B, c.T, c.H, c.D, w_l)
                per.append({"window": w_l, "us": round(ms_l * 1e3, 2),
                            "frac_bf16_peak": round(fl_l / (ms_l * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                            "kernel_us": round(ms_k * 1e3, 2),
                            "kernel_frac_bf16_peak": round(fl_l / (ms_k * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
                del wsl
            stacks[c.name]["layers"] = per
            del layers, outs, wsc
        if args.only == "stacks":
            print(json.dumps(stacks))
            return

    # ------------------------------------------- training: forward + backward
    bwd = {}
    if args.only in ("all", "bwd"):
        for cidx in (1, 2, 3):
            c = wl.CONFIGS[cidx]
            per = []
            for l in range(len(c.windows)):
                if cidx == 2 and l > 0 and c.windows[l] == c.windows[0]:
                    continue  # layers 1, 2 of a stack repeat layer 0's shape and window
                if cidx == 3 and l > 0 and c.windows[l] == c.windows[0]:
                    continue
                w_l = c.windows[l]
                q, k, v = (t.to(dev) for t in wl.prefill_inputs(c, layer=l))
                do = wl.prefill_dout(c, layer=l).to(dev)
                o = torch.empty_like(q)
                lse = torch.empty(c.B, c.T, c.H, dtype=torch.float32, device=dev)
                wsf = torch.empty(nc.attn_fwd_workspace_bytes(c.B, c.T, c.H, c.Hkv, c.D, 0, c.dtype),
                                  dtype=torch.uint8, device=dev)
                wsb = torch.empty(nc.attn_bwd_workspace_bytes(c.B, c.T, c.H, c.Hkv, c.D, c.dtype),
                                  dtype=torch.uint8, device=dev)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

                def fstep(i, q=q, k=k, v=v, o=o, lse=lse, wsf=wsf, w_l=w_l):
                    nc.attn_fwd_lse(q, k, v, window=w_l, out=o, lse=lse, workspace=wsf)

                def bstep(i, q=q, k=k, v=v, o=o, lse=lse, do=do, wsb=wsb, w_l=w_l, dq=dq, dk=dk, dv=dv):
                    nc.attn_bwd(q, k, v, o, do, lse, window=w_l, dq=dq, dk=dk, dv=dv, workspace=wsb)

                prime(f"fwd_lse_c{cidx}_l{l}", fstep)
                ms_f = event_time_ms(fstep, K, torch)
                prime(f"bwd_c{cidx}_l{l}", bstep)
                ms_b = event_time_ms(bstep, K, torch)
                pairs = wl.unmasked_pairs(c.T, w_l) * c.B * c.H
                tf_b = wl.backward_flops(c.B, c.T, c.H, c.D, w_l) / (ms_b * 1e-3) / 1e12
                tf_f = wl.prefill_flops(c.B, c.T, c.H, c.D, w_l) / (ms_f * 1e-3) / 1e12
                per.append({"layer": l, "window": w_l, "fwd_lse_us": round(ms_f * 1e3, 2),
                            "fwd_lse_frac_bf16_peak": round(tf_f / PEAK_BF16_TFLOPS, 4),
                            "bwd_us": round(ms_b * 1e3, 2), "bwd_TFLOP_per_s": round(tf_b, 1),
                            "bwd_frac_bf16_peak": round(tf_b / PEAK_BF16_TFLOPS, 4),
                            "unmasked_pairs": pairs})
                del q, k, v, do, o, lse, wsf, wsb, dq, dk, dv
            bwd[c.name] = {"shape": f"B={c.B} T={c.T} H={c.H} Hkv={c.Hkv} D={c.D}", "layers": per}
        bwd["flops"] = ("backward: 10*D per unmasked pair (q.k recomputed, dO.v, P^T dO, dS k, dS^T q); "
                        "forward: 4*D")
        if args.only == "bwd":
            print(json.dumps(bwd))
            return

    # ---------------------- fused q, k, v projection with RoPE + QK-norm epilogue
    qkv = {}
    if args.only in ("all", "qkv"):
        for name, sh in wl.QKV.items():
            qsets = []
            for s_ in range(args.sets):
                x, wq, wk, wv = (t.to(dev) for t in wl.qkv_inputs(**sh, seed=s_))
                qsets.append((x, wq, wk, wv))
            B, T, C, H, Hkv, D = sh["B"], sh["T"], sh["C"], sh["H"], sh["Hkv"], sh["D"]
            qo = torch.empty(B, T, H, D, dtype=torch.bfloat16, device=dev)
            ko = torch.empty(B, T, Hkv, D, dtype=torch.bfloat16, device=dev)
            vo = torch.empty_like(ko)
            wsq = torch.empty(nc.qkv_rope_qknorm_workspace_bytes(T, D), dtype=torch.uint8, device=dev)

            def qstep(i, qsets=qsets, H=H, Hkv=Hkv, qo=qo, ko=ko, vo=vo, wsq=wsq):
                x, wq, wk, wv = qsets[i % len(qsets)]
                nc.qkv_rope_qknorm(x, wq, wk, wv, H=H, Hkv=Hkv, q_out=qo, k_out=ko, v_out=vo, workspace=wsq)

            prime(f"qkv_{name}", qstep)
            ms = event_time_ms(qstep, K, torch)
            fl = wl.qkv_flops(B, T, C, H, Hkv, D)
            tf = fl / (ms * 1e-3) / 1e12
            nbytes = (B * T * C + (H + 2 * Hkv) * D * C + B * T * (H + 2 * Hkv) * D) * 2
            # the attention block's input side end to end: x -> q', k', v -> o
            # (causal, full window), attention read straight from q', k'
            oo = torch.empty_like(qo)
            wsn = nc.attn_fwd_normed_workspace_bytes(B, T, H, Hkv, D)
            wsn = torch.empty(max(wsn, 1), dtype=torch.uint8, device=dev)

            def nstep(i, qo=qo, ko=ko, vo=vo, oo=oo, wsn=wsn, T=T):
                nc.attn_fwd_normed(qo, ko, vo, window=T, out=oo, workspace=wsn)

            def bstep(i, qstep=qstep, nstep=nstep):
                qstep(i)
                nstep(i)

            prime(f"normed_{name}", nstep)
            ms_n = event_time_ms(nstep, K, torch)
            prime(f"block_{name}", bstep)
            ms_b = event_time_ms(bstep, K, torch)
            fl_a = wl.prefill_flops(B, T, H, D, T)
            qkv[name] = {"shape": f"x (B={B}, T={T}, C={C}) -> q' (H={H}), k', v (Hkv={Hkv}), D={D}, bf16",
                         "us_per_call": round(ms * 1e3, 2), "TFLOP_per_s": round(tf, 1),
                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "GFLOP": round(fl / 1e9, 2),
                         "algorithmic_bytes": nbytes,
                         "attn_from_normed_us": round(ms_n * 1e3, 2),
                         "attn_from_normed_frac_bf16_peak": round(
                             fl_a / (ms_n * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "x_to_o_us": round(ms_b * 1e3, 2),
                         "x_to_o_TFLOP_per_s": round((fl + fl_a) / (ms_b * 1e-3) / 1e12, 1)}
            del qsets, qo, ko, vo, wsq, oo, wsn
        qkv["flops"] = ("2 per multiply-add of the three projections (table and epilogue not counted); "
                        "attention 4*D per unmasked pair, causal")
        if args.only == "qkv":
            print(json.dumps(qkv))
            return

    # ------------------------------------- prefill into the KV cache (chunked)
    pre = {}
    if args.only in ("all", "prefill"):
        ch = wl.CHUNK
        B, Tc, P, Tmax, H, Hkv, D = ch["B"], ch["T"], ch["P"], ch["Tmax"], ch["H"], ch["Hkv"], ch["D"]
        psets = []
        for s_ in range(args.sets):
            q, k, v, kc, vc = wl.prefill_chunk_inputs(seed=s_)
            psets.append([t.to(dev) for t in (q, k, v, kc, vc)] + [torch.empty_like(q, device=dev)])
        wsp = torch.empty(max(nc.attn_prefill_workspace_bytes(B, Tc, Tmax, H, Hkv, D), 1),
                          dtype=torch.uint8, device=dev)
        wsp_full = torch.empty(max(nc.attn_prefill_workspace_bytes(B, Tmax, Tmax, H, Hkv, D), 1),
                               dtype=torch.uint8, device=dev)

        def tf_entry(ms, fl, **extra):
            tf = fl / (ms * 1e-3) / 1e12
            return dict(extra, us_per_call=round(ms * 1e3, 2), TFLOP_per_s=round(tf, 1),
                        frac_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))

        for Wp in (2048, 512):
            def pstep(i, Wp=Wp):
                q, k, v, kc, vc, o = psets[i % len(psets)]
                nc.attn_prefill(q, k, v, kc, vc, window=Wp, pos_offset=P, out=o, workspace=wsp)

            prime(f"prefill_chunk_W{Wp}", pstep)
            ms = event_time_ms(pstep, K, torch)
            pre[f"chunk_W{Wp}"] = tf_entry(
                ms, wl.prefill_chunk_flops(B, Tc, P, H, D, Wp),
                workload=f"last {Tc}-token chunk at offset {P} of a {Tmax}-token context, "
                         f"B={B} H=Hkv={H} D={D} window={Wp}: k', v into the caches, then attention")
        del psets
        # the whole context: four chunks of 512, and one call of 2048, into the caches
        full = []
        for s_ in range(args.sets):
            q, k, v = wl.prefill_inputs(cfg, layer=s_)
            kc = torch.empty(B, Tmax, Hkv, D, dtype=torch.bfloat16, device=dev)
            full.append((q.to(dev), k.to(dev), v.to(dev), kc, torch.empty_like(kc),
                         torch.empty_like(q, device=dev)))
        cuts = [(a, a + Tc) for a in range(0, Tmax, Tc)]
        views = [[tuple(t[:, a:b] for t in (q, k, v, o)) for a, b in cuts] for (q, k, v, _, _, o) in full]
        chunks = [[tuple(t.contiguous() for t in vw[:3]) + (vw[3].contiguous(),) for vw in sv]
                  for sv in views]

        def cstep4(i):
            j = i % len(full)
            kc, vc = full[j][3], full[j][4]
            for (a, _), (q, k, v, o) in zip(cuts, chunks[j]):
                nc.attn_prefill(q, k, v, kc, vc, window=W, pos_offset=a, out=o, workspace=wsp)

        prime("prefill_4x512", cstep4)
        ms = event_time_ms(cstep4, K, torch)
        pre["context_4x512_W2048"] = tf_entry(
            ms, flops, workload=f"B={B} T={Tmax} H=Hkv={H} D={D} full causal, prefilled into the "
                                f"caches in {len(cuts)} chunks of {Tc} (one call each)")

        def cstep1(i):
            q, k, v, kc, vc, o = full[i % len(full)]
            nc.attn_prefill(q, k, v, kc, vc, window=W, out=o, workspace=wsp_full)

        prime("prefill_1x2048", cstep1)
        ms = event_time_ms(cstep1, K, torch)
        pre["context_1x2048_W2048"] = tf_entry(
            ms, flops, workload=f"the same context in one call (k', v written to the caches; "
                                f"compare the headline step, which keeps k' in its workspace)")
        del full, views, chunks, wsp, wsp_full
        if args.only == "prefill":
            print(json.dumps(pre))
            return

    # ----------------------------- several samples over one shared prompt cache
    shd = {}
    if args.only in ("all", "shared"):
        sc = wl.SHARED
        B, Lp, Tgen, H, Hkv, D = sc["B"], sc["Lp"], sc["Tgen"], sc["H"], sc["Hkv"], sc["D"]
        ssets, csets = [], []
        for s_ in range(args.sets):
            q, kn, vn, kp, vp, kc, vc, L = wl.decode_shared_inputs(seed=s_)
            ssets.append([t.to(dev) for t in (q, kn, vn, kp, vp, kc, vc, L)] + [torch.empty_like(q, device=dev)])
            # the per-sample copies of the prompt cache that the shared form avoids
            kf = torch.cat([kp.unsqueeze(0).expand(B, -1, -1, -1), kc], dim=1).contiguous()
            vf = torch.cat([vp.unsqueeze(0).expand(B, -1, -1, -1), vc], dim=1).contiguous()
            csets.append((kf.to(dev), vf.to(dev)))
        for Wd in (2048, 512):
            wss = torch.empty(max(nc.attn_decode_shared_workspace_bytes(B, Lp, Tgen, H, Hkv, D, Wd), 1),
                              dtype=torch.uint8, device=dev)
            wsc = nc.decode_workspace(B, Lp + Tgen, H, Hkv, D, Wd, device=dev)

            def sstep_(i, Wd=Wd, wss=wss):
                q, kn, vn, kp, vp, kc, vc, L, o = ssets[i % len(ssets)]
                nc.attn_decode_shared(q, kn, vn, kp, vp, kc, vc, L, window=Wd, out=o, workspace=wss)

            def cstep_(i, Wd=Wd, wsc=wsc):
                q, kn, vn, kp, vp, kc, vc, L, o = ssets[i % len(ssets)]
                kf, vf = csets[i % len(csets)]
                nc.attn_decode(q, kn, vn, kf, vf, L, window=Wd, out=o, workspace=wsc)

            prime(f"shared_W{Wd}", sstep_)
            ms_s = event_time_ms(sstep_, K, torch)
            prime(f"copied_W{Wd}", cstep_)
            ms_c = event_time_ms(cstep_, K, torch)
            lens = [ss[7].cpu().tolist() for ss in ssets]
            ub = sum(wl.decode_shared_bytes(l, Lp, Hkv, D, Wd, H) for l in lens) / len(lens)
            cb = sum(wl.decode_bytes(l, Hkv, D, Wd, H) for l in lens) / len(lens)
            shd[f"W{Wd}"] = {"us_per_call": round(ms_s * 1e3, 2),
                             "unique_bytes": int(ub),
                             "GB_per_s_unique": round(ub / (ms_s * 1e-3) / 1e9, 1),
                             "copied_caches_us_per_call": round(ms_c * 1e3, 2),
                             "copied_caches_bytes": int(cb),
                             "speedup_vs_copied": round(ms_c / ms_s, 3)}
        shd["workload"] = (f"{B} samples of a {Lp}-token prompt (one shared prompt cache), each with "
                           f"1..{Tgen} tokens of its own, H=Hkv={H} D={D}, bf16; against nc_attn_decode "
                           f"over per-sample copies of the prompt cache")
        del ssets, csets
        if args.only == "shared":
            print(json.dumps(shd))
            return

    # ------------------------------- value-embedding gate (v' = v + gate * ve)
    gate = {}
    if args.only in ("all", "gate"):
        ch = wl.CHUNK
        B, Tc, P, Tmax, H, Hkv, D = ch["B"], ch["T"], ch["P"], ch["Tmax"], ch["H"], ch["Hkv"], ch["D"]
        gsets = []
        for s_ in range(args.sets):
            q, k, v, kc, vc = [t.to(dev) for t in wl.prefill_chunk_inputs(seed=s_)]
            gsets.append((q, k, v, kc, vc, torch.randn_like(v), torch.rand(B, Tc, Hkv, device=dev).to(v.dtype),
                          torch.empty_like(q)))
        wsg = torch.empty(max(nc.attn_prefill_workspace_bytes(B, Tc, Tmax, H, Hkv, D), 1), dtype=torch.uint8,
                          device=dev)
        for with_gate in (False, True):
            def gstep(i, with_gate=with_gate):
                q, k, v, kc, vc, ve, g, o = gsets[i % len(gsets)]
                nc.attn_prefill(q, k, v, kc, vc, window=2048, pos_offset=P, out=o, workspace=wsg,
                                ve=ve if with_gate else None, ve_gate=g if with_gate else None)

            prime(f"gate_prefill_{with_gate}", gstep)
            gate[f"prefill_chunk_W2048_{'gated' if with_gate else 'plain'}_us"] = round(event_time_ms(gstep, K, torch) * 1e3, 2)
        del gsets, wsg
        dcfg = wl.CONFIGS[4]
        dsets = []
        for s_ in range(args.sets):
            q, kn, vn, kc, vc, L = [t.to(dev) for t in wl.decode_inputs(dcfg, set_idx=s_)]
            dsets.append((q, kn, vn, kc, vc, L, torch.randn_like(vn), torch.rand(dcfg.B, dcfg.Hkv, device=dev).to(vn.dtype),
                          torch.empty_like(q)))
        wsd = nc.decode_workspace(dcfg.B, dcfg.Tmax, dcfg.H, dcfg.Hkv, dcfg.D, 512, device=dev)
        for with_gate in (False, True):
            def dstep_(i, with_gate=with_gate):
                q, kn, vn, kc, vc, L, ve, g, o = dsets[i % len(dsets)]
                nc.attn_decode(q, kn, vn, kc, vc, L, window=512, out=o, workspace=wsd,
                               ve=ve if with_gate else None, ve_gate=g if with_gate else None)

            prime(f"gate_decode_{with_gate}", dstep_)
            gate[f"decode_W512_{'gated' if with_gate else 'plain'}_us"] = round(event_time_ms(dstep_, K, torch) * 1e3, 2)
        gate["workload"] = ("nc_attn_prefill on the d12 chunk (512 tokens at offset 1536, W=2048) and nc_attn_decode "
                            "on the B=64 d12 decode (W=512), each with and without the value-embedding pair")
        del dsets, wsd
        if args.only == "gate":
            print(json.dumps(gate))
            return

    # ---------------------------------------------------------------- line
    step_ms = out["step_ms"]
    value = flops / (step_ms * 1e-3) / 1e12
    kern_tf = flops / (out["kern_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "settle_ms": args.settle_ms,
        "settle_calls": settled,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "d12 L-layer prefill attention forward, B=8 T=2048 H=Hkv=6 D=128 "
                               "window=2048 (full causal), bf16: q rotated and normalised in the "
                               "attention kernel's load, k through the input-stage kernel "
                               "(attn_prep_kernel writes k' and the q table), then the attention kernel",
                   "B": cfg.B, "T": cfg.T, "H": cfg.H, "Hkv": cfg.Hkv, "D": cfg.D, "window": W,
                   "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "step_trials": {"trials": 5, "launches": min(50, K), "median_ms": round(median(out["trials_ms"]), 5),
                        "ms": [round(x, 5) for x in out["trials_ms"]],
                        "one_input_set_median_ms": round(median(out["one_set_trials_ms"]), 5),
                        "note": "rotated: 4 input sets (~300 MB, beyond the 256 MB last-level cache); "
                                "one set: the same inputs every step"},
        "roofline": {"bound": "mfma", "achieved": round(kern_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(),
                     "kernel": "attn_fwd_bf16_kernel<128, 8>",
                     "kernel_us": round(out["kern_ms"] * 1e3, 2),
                     "flops_per_launch": flops},
        "device_copy_GB_per_s": round(copy_gbs, 1) if copy_gbs else None,
        "decode": dec,
        "rope_qknorm": rope,
        "stacks": stacks,
        "backward": bwd,
        "qkv_projection": qkv,
        "prefill_cache": pre,
        "decode_shared_prompt": shd,
        "value_gate": gate,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
