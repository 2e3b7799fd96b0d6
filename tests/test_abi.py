"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import transformer_attention_rope_amd as nc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nc_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(nc_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_is_built():
    assert os.path.exists(nc.library_path()), "run __graft_entry__.build() first"


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 9, names
    L = ctypes.CDLL(nc.library_path())
    for n in names:
        assert hasattr(L, n), f"{n} declared in nc_attn.h but not exported"
    # and the binding knows every one of them
    assert set(names) == set(nc._SIGS), (set(names) ^ set(nc._SIGS))


def test_version_and_strings():
    L = nc.lib()
    assert L.nc_abi_version() == 10
    for s in range(4):
        assert L.nc_status_string(s)
    assert b"unknown" in L.nc_status_string(99)


P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced on these paths


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, B=1, T=8, H=2, Hkv=2, D=64, window=8, base=1e4, off=0, dt=0,
             ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    L = nc.lib()
    return L.nc_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["T"], a["H"], a["Hkv"], a["D"],
                         a["window"], a["base"], a["off"], a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(q=None), 1, "q is NULL"),
    (dict(v=P + 4), 1, "not 16-byte aligned"),
    (dict(B=0), 1, "sizes"),
    (dict(T=-1), 1, "sizes"),
    (dict(H=3, Hkv=2), 1, "multiple"),
    (dict(D=48), 2, "head dim"),
    (dict(D=256), 2, "head dim"),
    (dict(window=0), 1, "window"),
    (dict(off=-5), 1, "pos_offset"),
    (dict(base=0.0), 1, "rope_base"),
    (dict(base=float("inf")), 1, "rope_base"),
    (dict(base=float("nan")), 1, "rope_base"),
    (dict(dt=7), 1, "dtype"),
    (dict(wsb=16), 1, "workspace"),
    (dict(ws=None), 1, "ws is NULL"),
    (dict(B=1 << 20, T=1 << 12, H=1 << 4), 1, "exceed"),
    (dict(T=1 << 22, H=8, Hkv=8, D=128), 2, "2^32"),
])
def test_attn_fwd_validation(kw, status, frag):
    assert _fwd(**kw) == status
    assert frag in nc.lib().nc_last_error().decode()


def test_prep_core_validation():
    L = nc.lib()
    need = L.nc_attn_fwd_workspace_bytes(1, 8, 2, 2, 64, 0, 0)
    assert L.nc_attn_prep(None, 1, 8, 2, 64, 1e4, 0, 0, P, need, None) == 1
    assert b"k is NULL" in L.nc_last_error()
    assert L.nc_attn_prep(P, 1, 8, 2, 64, 1e4, 0, 0, P, need - 1, None) == 1
    assert b"workspace" in L.nc_last_error()
    assert L.nc_attn_prep(P, 1, 8, 2, 64, -1.0, 0, 0, P, need, None) == 1
    assert L.nc_attn_core(P, P, P, 1, 8, 2, 2, 64, 0, 0, P, need, None) == 1
    assert b"window" in L.nc_last_error()
    assert L.nc_attn_core(P, P, None, 1, 8, 2, 2, 64, 8, 0, P, need, None) == 1
    assert b"o is NULL" in L.nc_last_error()
    assert L.nc_attn_core(P, P, P, 1, 8, 2, 2, 64, 8, 0, None, need, None) == 1
    assert b"ws is NULL" in L.nc_last_error()
    assert L.nc_attn_core(P, P, P, 1, 8, 3, 2, 64, 8, 0, P, need, None) == 1


def test_rope_qknorm_validation():
    L = nc.lib()
    assert L.nc_rope_qknorm(P, P, None, P, 1, 4, 2, 2, 32, 1e4, 0, 0, None, 0, None) == 1
    assert b"q_out is NULL" in L.nc_last_error()
    assert L.nc_rope_qknorm(P, P, P, P, 1, 4, 2, 2, 96, 1e4, 0, 0, None, 0, None) == 2
    assert L.nc_rope_qknorm(P, P, P, P, 1, 4, 2, 2, 32, -1.0, 0, 0, None, 0, None) == 1
    assert L.nc_rope_qknorm(P, P, P, P, 1, 4, 2, 2, 32, 1e4, (1 << 30), 0, None, 0, None) == 1
    assert b"exceeds" in L.nc_last_error()


def _dec(**kw):
    a = dict(q=P, kn=P, vn=P, ve=None, vg=None, kc=P, vc=P, sl=P, o=P, B=4, Tmax=2048, H=8, Hkv=2, D=128,
             window=512, base=1e4, dt=0, ws=P, wsb=1 << 24, stream=None)
    a.update(kw)
    L = nc.lib()
    return L.nc_attn_decode(a["q"], a["kn"], a["vn"], a["ve"], a["vg"], a["kc"], a["vc"], a["sl"], a["o"], a["B"],
                            a["Tmax"], a["H"], a["Hkv"], a["D"], a["window"], a["base"], a["dt"],
                            a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(sl=None), 1, "seqlens is NULL"),
    (dict(sl=P + 2), 1, "4-byte"),
    (dict(kc=None), 1, "k_cache is NULL"),
    (dict(Tmax=0), 1, "sizes"),
    (dict(H=256, Hkv=2), 2, "exceed 64"),
    (dict(window=-1), 1, "window"),
    (dict(D=16), 2, "head dim"),
    (dict(ws=None), 1, "ws is NULL"),
    (dict(wsb=8), 1, "workspace"),
    (dict(ve=P), 1, "both be NULL"),
    (dict(ve=P, vg=P + 3, dt=1), 1, "ve_gate is not aligned"),
])
def test_decode_validation(kw, status, frag):
    assert _dec(**kw) == status
    assert frag in nc.lib().nc_last_error().decode()


def _pre(**kw):
    a = dict(q=P, k=P, v=P, ve=None, vg=None, kc=P, vc=P, o=P, B=2, T=64, Tmax=256, H=4, Hkv=2, D=64,
             window=128, base=1e4, off=128, dt=0, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    L = nc.lib()
    return L.nc_attn_prefill(a["q"], a["k"], a["v"], a["ve"], a["vg"], a["kc"], a["vc"], a["o"], a["B"], a["T"],
                             a["Tmax"], a["H"], a["Hkv"], a["D"], a["window"], a["base"], a["off"],
                             a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(vc=None), 1, "v_cache is NULL"),
    (dict(kc=P + 8), 1, "not 16-byte aligned"),
    (dict(off=193), 1, "exceeds Tmax"),
    (dict(off=-1), 1, "pos_offset"),
    (dict(Tmax=0, off=0), 1, "Tmax"),
    (dict(window=0), 1, "window"),
    (dict(D=80), 2, "head dim"),
    (dict(H=5), 1, "multiple"),
    (dict(ws=None), 1, "ws is NULL"),
    (dict(wsb=255), 1, "workspace"),
    (dict(Tmax=1 << 22, H=8, Hkv=8, D=128, off=0), 2, "2^32"),
    (dict(B=1 << 12, Tmax=1 << 18, Hkv=4, H=4, off=0), 1, "cache rows"),
    (dict(ve=P), 1, "both be NULL"),
    (dict(vg=P), 1, "both be NULL"),
    (dict(ve=P + 2, vg=P), 1, "ve is not 16-byte aligned"),
    (dict(ve=P, vg=P + 1), 1, "ve_gate is not aligned"),
])
def test_prefill_validation(kw, status, frag):
    assert _pre(**kw) == status
    assert frag in nc.lib().nc_last_error().decode()


def _dsh(**kw):
    a = dict(q=P, kn=P, vn=P, ve=None, vg=None, kp=P, vp=P, Lp=1536, kc=P, vc=P, sl=P, o=P, B=64, Tgen=512,
             H=6, Hkv=6, D=128, window=2048, base=1e4, dt=0, ws=P, wsb=1 << 24, stream=None)
    a.update(kw)
    L = nc.lib()
    return L.nc_attn_decode_shared(a["q"], a["kn"], a["vn"], a["ve"], a["vg"], a["kp"], a["vp"], a["Lp"], a["kc"], a["vc"],
                                   a["sl"], a["o"], a["B"], a["Tgen"], a["H"], a["Hkv"], a["D"],
                                   a["window"], a["base"], a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(kp=None), 1, "k_prompt is NULL"),
    (dict(vp=P + 4), 1, "not 16-byte aligned"),
    (dict(Lp=0), 1, "Lp"),
    (dict(Tgen=0), 1, "sizes"),
    (dict(sl=None), 1, "seqlens is NULL"),
    (dict(window=0), 1, "window"),
    (dict(H=512, Hkv=4), 2, "exceed 64"),
    (dict(D=96), 2, "head dim"),
    (dict(ws=None), 1, "ws is NULL"),
    (dict(wsb=64), 1, "workspace"),
    (dict(Lp=1 << 30), 1, "exceeds"),
    (dict(vg=P), 1, "both be NULL"),
])
def test_decode_shared_validation(kw, status, frag):
    assert _dsh(**kw) == status
    assert frag in nc.lib().nc_last_error().decode()


def test_workspace_queries():
    L = nc.lib()
    assert L.nc_rope_qknorm_workspace_bytes(2048, 128, 0) == 0
    # (cos, sin) per position and frequency (two fp16 for bf16, two fp32 for
    # fp32), then k', each part rounded up to 256 bytes
    assert L.nc_attn_fwd_workspace_bytes(8, 2048, 6, 6, 128, 0, 0) == 2048 * 64 * 4 + 8 * 2048 * 6 * 128 * 2
    assert L.nc_attn_fwd_workspace_bytes(8, 2048, 6, 6, 128, 0, 1) == 2048 * 64 * 8 + 8 * 2048 * 6 * 128 * 4
    assert L.nc_attn_fwd_workspace_bytes(1, 3, 2, 2, 32, 0, 0) == 256 + 512  # 3*16*4, 3*2*32*2 (no slices: one key tile)
    assert L.nc_attn_fwd_workspace_bytes(1, 3, 2, 2, 32, 0, 1) == 512 + 768  # 3*16*8, 3*2*32*4
    assert L.nc_attn_fwd_workspace_bytes(1, 3, 2, 2, 32, 0, 7) == 0
    # chunked prefill: the table of the chunk's positions; fp32 never slices
    assert L.nc_attn_prefill_workspace_bytes(2, 64, 256, 4, 2, 64, 1) == 64 * 32 * 8
    assert L.nc_attn_prefill_workspace_bytes(1, 3, 3, 2, 2, 32, 0) == 256
    assert L.nc_attn_prefill_workspace_bytes(1, 0, 3, 2, 2, 32, 1) == 0
    assert L.nc_attn_prefill_workspace_bytes(1, 4, 3, 2, 2, 32, 0) == 0  # Tmax < T
    # bf16 launches far below a full device get room for key-tile slices: the
    # d12 chunk (96 workgroups of 256 columns, or 192 of 128) takes up to two
    # slices of fp32 rows of D + 1 values (output and row sum)
    rows = 8 * 512 * 6
    assert L.nc_attn_prefill_workspace_bytes(8, 512, 2048, 6, 6, 128, 0) == \
        512 * 64 * 4 + 2 * rows * 129 * 4
    # a full device of workgroups (the d12 layer) gets none
    assert L.nc_attn_fwd_workspace_bytes(8, 2048, 6, 6, 128, 0, 0) == 2048 * 64 * 4 + 8 * 2048 * 6 * 128 * 2
    # few (sequence, head) pairs: the key range is split and needs chunk states
    n = L.nc_attn_decode_workspace_bytes(2, 2048, 6, 6, 128, 2048)
    assert n > 0 and n % 256 == 0
    # one workgroup per (sequence, head) already fills the device: no split
    assert L.nc_attn_decode_workspace_bytes(64, 2048, 6, 6, 128, 2048) == 0
    assert L.nc_attn_decode_workspace_bytes(0, 2048, 6, 6, 128, 2048) == 0
    # a shared prompt may be cut at its end and its part run in two chunks:
    # two more chunk states per (b, h) than the unsplit range, so room for three
    assert L.nc_attn_decode_shared_workspace_bytes(64, 1536, 512, 6, 6, 128, 2048) == 64 * 6 * 3 * 130 * 4
    assert L.nc_attn_decode_shared_workspace_bytes(64, 1536, 512, 6, 6, 128, 1600) == 64 * 6 * 3 * 130 * 4
    assert L.nc_attn_decode_shared_workspace_bytes(64, 0, 512, 6, 6, 128, 2048) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 32)
    with pytest.raises(ValueError, match="GPU"):
        nc.attn_fwd(q, q, q, window=4)
    with pytest.raises(ValueError, match="GPU"):
        nc.rope_qknorm(q, q)
    with pytest.raises(ValueError, match="GPU"):
        nc.attn_prefill(q, q, q, torch.zeros(1, 8, 2, 32), torch.zeros(1, 8, 2, 32), window=4)


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, T=8, H=2, Hkv=2, D=64, window=8,
             base=1e4, off=0, dt=0, ws=P, wsb=1 << 24, stream=None)
    a.update(kw)
    return nc.lib().nc_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                a["dv"], a["B"], a["T"], a["H"], a["Hkv"], a["D"], a["window"],
                                a["base"], a["off"], a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(dq=None), 1, "dq is NULL"),
    (dict(do=P + 8), 1, "dout is not 16-byte aligned"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(lse=P + 2), 1, "lse is not 4-byte aligned"),
    (dict(H=3, Hkv=2), 1, "multiple"),
    (dict(D=80), 2, "head dim"),
    (dict(window=0), 1, "window"),
    (dict(off=-1), 1, "pos_offset"),
    (dict(wsb=100), 1, "workspace"),
    (dict(T=1 << 21, H=16, Hkv=1, D=128), 2, "2^32"),
])
def test_attn_bwd_validation(kw, status, frag):
    assert _bwd(**kw) == status
    assert frag in nc.lib().nc_last_error().decode()


def test_attn_fwd_lse_validation():
    L = nc.lib()
    st = L.nc_attn_fwd_lse(P, P, P, P, None, 1, 8, 2, 2, 64, 8, 1e4, 0, 0, P, 1 << 20, None)
    assert st == 1 and b"lse is NULL" in L.nc_last_error()
    st = L.nc_attn_fwd_lse(P, P, P, P, P + 1, 1, 8, 2, 2, 64, 8, 1e4, 0, 0, P, 1 << 20, None)
    assert st == 1 and b"4-byte" in L.nc_last_error()


def test_bwd_workspace_bytes():
    L = nc.lib()
    # bf16 d12 layer: the table, five bf16 tensors of the layer's size and the stats
    n = L.nc_attn_bwd_workspace_bytes(8, 2048, 6, 6, 128, 0)
    elems = 8 * 2048 * 6 * 128
    assert n >= 5 * elems * 2  # k', k'^T, q', q'^T, dO^T
    assert L.nc_attn_bwd_workspace_bytes(8, 2048, 6, 6, 96, 0) == 0
    assert L.nc_attn_bwd_workspace_bytes(8, 2048, 6, 4, 128, 0) == 0
    assert L.nc_attn_bwd_workspace_bytes(1, 64, 2, 2, 32, 1) > 0


def test_fwd_noalloc_rejects_beyond_scratch():
    """Sizes whose workspace exceeds the static 64 MiB scratch are refused on
    the host, before any HIP call."""
    L = nc.lib()
    # B=32 d12 layer: k' alone is 100 MB
    st = L.nc_attn_fwd_noalloc(P, P, P, P, 32, 2048, 6, 6, 128, 2048, 1e4, 0, 0, None)
    assert st == 1 and b"beyond the library's static" in L.nc_last_error()
    st = L.nc_attn_fwd_noalloc(P, P, P, P, 1, 8, 2, 2, 48, 8, 1e4, 0, 0, None)
    assert st == 2 and b"head dim" in L.nc_last_error()


def test_qkv_validation():
    L = nc.lib()

    def call(**kw):
        a = dict(x=P, wq=P, wk=P, wv=P, q=P, k=P, v=P, B=1, T=8, C=64, H=2, Hkv=2, D=64, base=1e4, off=0,
                 dt=0, ws=P, wsb=1 << 20)
        a.update(kw)
        return L.nc_qkv_rope_qknorm(a["x"], a["wq"], a["wk"], a["wv"], a["q"], a["k"], a["v"], a["B"],
                                    a["T"], a["C"], a["H"], a["Hkv"], a["D"], a["base"], a["off"], a["dt"],
                                    a["ws"], a["wsb"], None)
    assert call(C=100) == 2 and b"multiple of 64" in L.nc_last_error()
    assert call(C=0) == 1
    assert call(wk=None) == 1 and b"w_k is NULL" in L.nc_last_error()
    assert call(v=P + 8) == 1 and b"v_out is not 16-byte aligned" in L.nc_last_error()
    assert call(D=96) == 2
    assert call(wsb=8) == 1 and b"workspace" in L.nc_last_error()
    assert call(ws=None) == 1
    assert L.nc_qkv_rope_qknorm_workspace_bytes(2048, 128, 0) >= 2048 * 64 * 4


def test_fwd_normed_validation():
    L = nc.lib()

    def call(**kw):
        a = dict(q=P, k=P, v=P, o=P, B=1, T=8, H=2, Hkv=2, D=64, W=8, dt=0, ws=P, wsb=1 << 20)
        a.update(kw)
        return L.nc_attn_fwd_normed(a["q"], a["k"], a["v"], a["o"], a["B"], a["T"], a["H"], a["Hkv"],
                                    a["D"], a["W"], a["dt"], a["ws"], a["wsb"], None)
    assert call(W=0) == 1 and b"window" in L.nc_last_error()
    assert call(k=None) == 1 and b"k is NULL" in L.nc_last_error()
    assert call(D=48) == 2 and b"head dim" in L.nc_last_error()
    assert call(H=3) != 0
    # a short sequence on many heads runs in one slice: no workspace at all
    assert L.nc_attn_fwd_normed_workspace_bytes(1, 8, 2, 2, 64, 0) == 0
    assert L.nc_attn_fwd_normed_workspace_bytes(0, 8, 2, 2, 64, 0) == 0
