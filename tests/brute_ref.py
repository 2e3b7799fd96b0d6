"""Pure-Python brute force of the attention-block forward, for tiny shapes.

Used only to pin the NumPy oracle.  It evaluates the definition scalar by
scalar with explicit loops and the ``math`` module, enumerating every
(query, key) pair and testing visibility pair by pair, so it shares neither
vectorisation nor masking code with the oracle.  It keeps the same readings
of the pages (adjacent RoPE pairs, +p*theta, eps 1e-6, 0 <= i-j < W,
kv head = h // G).
"""
import math


def brute_attn(q, k, v, W, base=10000.0, pos_offset=0, eps=1e-6):
    """q[b][t][h][d], k/v[b][t][g][d] nested lists of floats -> o nested list."""
    B, T, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    G = H // Hkv

    def rot_norm(row, p):
        out = [0.0] * D
        for i in range(D // 2):
            theta = base ** (-(2.0 * i) / D)
            a = p * theta
            x, y = row[2 * i], row[2 * i + 1]
            out[2 * i] = x * math.cos(a) - y * math.sin(a)
            out[2 * i + 1] = x * math.sin(a) + y * math.cos(a)
        ms = sum(z * z for z in out) / D
        r = 1.0 / math.sqrt(ms + eps)
        return [z * r for z in out]

    o = [[[[0.0] * D for _ in range(H)] for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(T):
                qi = rot_norm(q[b][i][h], pos_offset + i)
                scores = []
                for j in range(T):
                    if 0 <= i - j < W:
                        kj = rot_norm(k[b][j][g], pos_offset + j)
                        s = sum(qi[d] * kj[d] for d in range(D)) / math.sqrt(D)
                        scores.append((j, s))
                mx = max(s for _, s in scores)
                den = sum(math.exp(s - mx) for _, s in scores)
                for j, s in scores:
                    w = math.exp(s - mx) / den
                    for d in range(D):
                        o[b][i][h][d] += w * v[b][j][g][d]
    return o
