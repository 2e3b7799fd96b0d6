"""Entry points on several streams and inside a captured HIP graph.

The library enqueues kernels on the caller's stream and allocates, frees and
synchronises nothing, so its calls can be split over streams (ordered by
events) and captured into a graph. Results must equal those of the same calls
run eagerly on one stream, bit for bit. Graph replays are interleaved with
eager work and synchronisation, and every replay is checked.
"""
import pytest
import torch

import transformer_attention_rope_amd as nc
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def test_prep_and_core_on_two_streams():
    """nc_attn_prep on one stream, nc_attn_core on another after an event, and two
    independent forwards on two streams with their own workspaces."""
    _say("prep / core split over two streams")
    B, T, H, Hkv, D = 2, 700, 8, 2, 128
    q, k, v = [t.to(DEV) for t in wl.small_prefill(B, T, H, Hkv, D, seed=606)]
    q2, k2, v2 = [t.to(DEV) for t in wl.small_prefill(B, T, H, Hkv, D, seed=707)]
    ref = nc.attn_fwd(q, k, v, window=256)
    ref2 = nc.attn_fwd(q2, k2, v2, window=2048)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    nbytes = nc.attn_fwd_workspace_bytes(B, T, H, Hkv, D)
    ws1 = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    o2 = torch.empty_like(q2)
    ev = torch.cuda.Event()
    with torch.cuda.stream(s1):
        nc.attn_prep(k, H=H, workspace=ws1)
        ev.record(s1)
        nc.attn_fwd(q2, k2, v2, window=2048, out=o2, workspace=ws2)  # independent work on s1
    with torch.cuda.stream(s2):
        s2.wait_event(ev)
        nc.attn_core(q, v, ws1, window=256, out=o)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    assert torch.equal(o2, ref2)


def test_graph_capture_and_replay():
    """A forward, a chunked prefill and a decode step captured into one graph and
    replayed three times, with eager work and synchronisation in between."""
    _say("graph capture of attn_fwd, attn_prefill, attn_decode")
    B, T, H, Hkv, D = 2, 300, 8, 2, 128
    q, k, v = [t.to(DEV) for t in wl.small_prefill(B, T, H, Hkv, D, seed=808)]
    g = torch.Generator().manual_seed(9)
    Tmax = 512
    kc0 = torch.randn(B, Tmax, Hkv, D, generator=g).bfloat16().to(DEV)
    vc0 = torch.randn(B, Tmax, Hkv, D, generator=g).bfloat16().to(DEV)
    qd = torch.randn(B, H, D, generator=g).bfloat16().to(DEV)
    kn = torch.randn(B, Hkv, D, generator=g).bfloat16().to(DEV)
    vn = torch.randn(B, Hkv, D, generator=g).bfloat16().to(DEV)
    L = torch.tensor([T + 101, T + 7], dtype=torch.int32, device=DEV)

    # static buffers the graph reads and writes
    o_f = torch.empty_like(q)
    o_p = torch.empty_like(q)
    o_d = torch.empty_like(qd)
    kc, vc = kc0.clone(), vc0.clone()
    ws_f = torch.empty(nc.attn_fwd_workspace_bytes(B, T, H, Hkv, D), dtype=torch.uint8, device=DEV)
    ws_p = torch.empty(max(nc.attn_prefill_workspace_bytes(B, T, Tmax, H, Hkv, D), 1), dtype=torch.uint8,
                       device=DEV)
    ws_d = nc.decode_workspace(B, Tmax, H, Hkv, D, 128, device=DEV)

    def calls():
        nc.attn_fwd(q, k, v, window=128, out=o_f, workspace=ws_f)
        nc.attn_prefill(q, k, v, kc, vc, window=2048, pos_offset=100, out=o_p, workspace=ws_p)
        nc.attn_decode(qd, kn, vn, kc, vc, L, window=128, out=o_d, workspace=ws_d)

    calls()  # eager reference (and warm-up of the library on this stream)
    torch.cuda.synchronize()
    ref_f, ref_p, ref_d = o_f.clone(), o_p.clone(), o_d.clone()
    ref_kc, ref_vc = kc.clone(), vc.clone()

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t_ in (o_f, o_p, o_d):
            t_.zero_()
        kc.copy_(kc0)
        vc.copy_(vc0)
        _ = (q.float() @ q.float().transpose(-1, -2).contiguous()).sum()  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_f, ref_f), f"replay {rep}: attn_fwd"
        assert torch.equal(o_p, ref_p), f"replay {rep}: attn_prefill"
        assert torch.equal(o_d, ref_d), f"replay {rep}: attn_decode"
        assert torch.equal(kc, ref_kc) and torch.equal(vc, ref_vc), f"replay {rep}: caches"
