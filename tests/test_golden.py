"""The oracle reproduces its stored outputs (written by tests/golden/make_golden.py,
which calls only the oracle).  Guards against unnoticed changes of the oracle."""
import os

import numpy as np

import oracle
import workloads as wl

G = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_fp32_golden():
    cfg = wl.CONFIGS[0]
    q, k, v = wl.prefill_inputs(cfg)
    o = oracle.attn_fwd(q, k, v, cfg.windows[0], cfg.rope_base, cfg.pos_offset)
    qn, kn = oracle.rope_qknorm(q, k, cfg.rope_base, cfg.pos_offset)
    np.testing.assert_allclose(o.reshape(-1, cfg.D),
                               np.loadtxt(os.path.join(G, "tiny_fp32_attn_out.txt")),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(qn.reshape(-1, cfg.D),
                               np.loadtxt(os.path.join(G, "tiny_fp32_q_rope_qknorm.txt")),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(kn.reshape(-1, cfg.D),
                               np.loadtxt(os.path.join(G, "tiny_fp32_k_rope_qknorm.txt")),
                               rtol=0, atol=1e-13)
