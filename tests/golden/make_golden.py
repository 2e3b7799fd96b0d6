"""Writes the stored oracle outputs under tests/golden/.

Calls only the fp64 oracle (``oracle/``) on seeded inputs from ``workloads``;
no value here comes from the HIP path.  Re-run after a deliberate change of
the oracle's arithmetic, and name the passage of the pages that justifies the
change in the commit message:

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def main():
    cfg = wl.CONFIGS[0]
    q, k, v = wl.prefill_inputs(cfg)
    o = oracle.attn_fwd(q, k, v, cfg.windows[0], cfg.rope_base, cfg.pos_offset)
    qn, kn = oracle.rope_qknorm(q, k, cfg.rope_base, cfg.pos_offset)
    hdr = ("oracle output, tiny fp32 config: B=1 T=64 H=Hkv=2 D=32, full causal, "
           "RoPE base 1e4, eps 1e-6; rows in (b,t,h) order, D values per row")
    np.savetxt(os.path.join(HERE, "tiny_fp32_attn_out.txt"), o.reshape(-1, cfg.D),
               fmt="%.17g", header=hdr)
    np.savetxt(os.path.join(HERE, "tiny_fp32_q_rope_qknorm.txt"), qn.reshape(-1, cfg.D),
               fmt="%.17g", header="oracle rope_qknorm(q) for the same config")
    np.savetxt(os.path.join(HERE, "tiny_fp32_k_rope_qknorm.txt"), kn.reshape(-1, cfg.D),
               fmt="%.17g", header="oracle rope_qknorm(k) for the same config")


if __name__ == "__main__":
    main()
