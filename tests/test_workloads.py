"""The benchmark's algorithmic counts (pairs, flops, bytes) against brute-force
enumeration on small cases (CPU only)."""
import itertools

import pytest

import workloads as wl


@pytest.mark.parametrize("T,W", [(1, 1), (7, 3), (16, 16), (20, 64), (33, 8)])
def test_unmasked_pairs_brute(T, W):
    brute = sum(1 for i, j in itertools.product(range(T), range(T)) if 0 <= i - j < W)
    assert wl.unmasked_pairs(T, W) == brute


@pytest.mark.parametrize("T,P,W", [(1, 0, 1), (5, 0, 5), (5, 7, 3), (9, 4, 100), (12, 30, 10)])
def test_chunk_pairs_brute(T, P, W):
    """Query t of a chunk at offset P sees cache rows j with 0 <= P + t - j < W."""
    brute = sum(1 for t in range(T) for j in range(P + T) if 0 <= P + t - j < W)
    assert wl.chunk_pairs(T, P, W) == brute
    if P == 0:
        assert wl.chunk_pairs(T, 0, W) == wl.unmasked_pairs(T, W)


def test_flops_are_4D_per_pair():
    assert wl.prefill_flops(2, 10, 3, 8, 4) == 4 * 8 * wl.unmasked_pairs(10, 4) * 2 * 3
    assert wl.prefill_chunk_flops(2, 10, 5, 3, 8, 4) == 4 * 8 * wl.chunk_pairs(10, 5, 4) * 2 * 3


@pytest.mark.parametrize("W", [3, 6, 50])
def test_decode_bytes_brute(W):
    """Visible K and V rows per sequence (its window), plus q, o, k_new, v_new."""
    seqlens, Hkv, D, H, e = [1, 4, 9], 2, 8, 4, 2
    rows = sum(len([j for j in range(L) if L - 1 - j < W]) for L in seqlens)
    want = rows * Hkv * D * 2 * e + (2 * 3 * H * D + 2 * 3 * Hkv * D) * e
    assert wl.decode_bytes(seqlens, Hkv, D, W, H) == want


@pytest.mark.parametrize("W", [2, 5, 9, 40])
def test_decode_shared_bytes_brute(W):
    """Every prompt row some sample sees, once; each sample's own visible rows."""
    Lp, seqlens, Hkv, D, H, e = 6, [7, 9, 12], 2, 8, 4, 2
    prompt_rows = {j for L in seqlens for j in range(L) if L - 1 - j < W and j < Lp}
    own = sum(1 for L in seqlens for j in range(L) if L - 1 - j < W and j >= Lp)
    want = (len(prompt_rows) + own) * Hkv * D * 2 * e + (2 * 3 * H * D + 2 * 3 * Hkv * D) * e
    assert wl.decode_shared_bytes(seqlens, Lp, Hkv, D, W, H) == want
