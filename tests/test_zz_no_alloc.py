"""nc_attn_fwd_noalloc, the forward that allocates nothing (its workspace is
the library's static per-device scratch), against nc_attn_fwd through the C
ABI: two calls in a row, the second with a smaller input, each bit for bit
equal to nc_attn_fwd on the same inputs (same kernels, same workspace
contents), the smaller one also against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_rope_amd as nc
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_fwd_noalloc_two_calls_match_fwd():
    cfg = wl.CONFIGS[1]
    q1, k1, v1 = wl.prefill_inputs(cfg)                                  # d12 layer: 25.7 MB of scratch
    q2, k2, v2 = wl.small_prefill(1, 2048, 2, 2, 128, seed=4321)          # smaller, cut into slices
    calls = [(q1, k1, v1, 2048, 0), (q2, k2, v2, 2048, 5)]
    for i, (q, k, v, W, off) in enumerate(calls):
        print(f"[case] noalloc call {i} shape {tuple(q.shape)} W={W}", flush=True)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        ref = nc.attn_fwd(qd, kd, vd, window=W, pos_offset=off)
        out = torch.empty_like(qd)
        got = nc.attn_fwd_noalloc(qd, kd, vd, window=W, out=out, pos_offset=off)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), f"call {i}: differs from nc_attn_fwd"
    d = np.abs(out.double().cpu().numpy() - oracle.attn_fwd(q2, k2, v2, 2048, 10000.0, 5))
    print(f"[err] second call vs oracle: max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
