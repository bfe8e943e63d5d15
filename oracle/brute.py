"""Brute-force checkers for the oracle (pure Python loops, tiny shapes only).

TEST INFRASTRUCTURE ONLY: used by the tests to pin ``oracle.py``; it imports
nothing from it and nothing from the GPU library.

``brute_rel_attn`` evaluates the four-term score of A^rel (Dai et al.,
Transformer-XL, Sec. 3.3) the naive way the paper describes: the position key
W_kR R_{i-j} is recomputed for every (i, j) pair, at quadratic cost.

``appb_terms`` follows the paper's Appendix B route instead: build the reversed
matrix Q of position keys, form B~ = q Q^T and d~ = (Q v)^T, and obtain rows of
B and D by left-shifting.  It is an independent computation of terms (b) and (d).
"""
from __future__ import annotations

import math

__all__ = ["brute_rel_attn", "appb_terms", "brute_sinusoid"]


def _matvec(W, x):
    """y = W x for a list-of-rows matrix."""
    return [sum(wr[c] * x[c] for c in range(len(x))) for wr in W]


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def brute_sinusoid(n_pos, d):
    """Vaswani sinusoid row by row (same reading as the oracle, written with
    math.sin/cos per entry)."""
    rows = []
    for p in range(n_pos):
        row = []
        for c in range(d):
            k2 = c - (c % 2)
            ang = p / math.pow(10000.0, k2 / d)
            row.append(math.sin(ang) if c % 2 == 0 else math.cos(ang))
        rows.append(row)
    return rows


def brute_rel_attn(h, mem_log, W_q, W_kE, W_kR, W_v, u, v, R, n_heads, d_head, scale):
    """Nested loops over batch, head, query and key.  Arguments are nested lists:
    h [B][L][d], mem_log [B][M][d], W_* [H*dh][d], u, v [H][dh], R [>=M+L][d].
    Returns out [B][L][H*dh] and the score matrix s [B][H][L][M+L] (None where
    masked).  Mask: key j of [memory ; segment] visible iff j <= M + i."""
    B = len(h)
    L = len(h[0])
    M = len(mem_log[0]) if B and mem_log[0] is not None else 0
    out = [[[0.0] * (n_heads * d_head) for _ in range(L)] for _ in range(B)]
    scores = [[[[None] * (M + L) for _ in range(L)] for _ in range(n_heads)] for _ in range(B)]
    for b in range(B):
        ext = [list(row) for row in mem_log[b]] + [list(row) for row in h[b]]
        q_all = [_matvec(W_q, x) for x in h[b]]
        k_all = [_matvec(W_kE, x) for x in ext]
        v_all = [_matvec(W_v, x) for x in ext]
        for hh in range(n_heads):
            lo, hi = hh * d_head, (hh + 1) * d_head
            for i in range(L):
                qi = q_all[i][lo:hi]
                s_row = []
                for j in range(M + L):
                    if j > M + i:
                        continue
                    kj = k_all[j][lo:hi]
                    # W_kR R_{i-j}, recomputed for this pair (distance M + i - j)
                    rk = _matvec(W_kR, R[M + i - j])[lo:hi]
                    a = _dot(qi, kj)
                    bb = _dot(qi, rk)
                    c = _dot(u[hh], kj)
                    dd = _dot(v[hh], rk)
                    s = scale * (a + bb + c + dd)
                    scores[b][hh][i][j] = s
                    s_row.append((j, s))
                mx = max(s for _, s in s_row)
                ex = [(j, math.exp(s - mx)) for j, s in s_row]
                z = sum(e for _, e in ex)
                for c in range(d_head):
                    out[b][i][lo + c] = sum(e * v_all[j][lo + c] for j, e in ex) / z
    return out, scores


def appb_terms(q, r, v, M):
    """Terms (b) and (d) for one head by the Appendix B procedure.

    q: [L][dh] queries, r: [M+L][dh] with r[delta] = W_kR R_delta, v: [dh].
    Q is r in reversed order (Q_k = W_kR R_{M+L-1-k}); B~ = q Q^T; row i of B is
    row i of B~ shifted left by L-1-i with zeros entering from the right; D is
    built the same way from the single row d~ = (Q v)^T.  Returns (B, D) as
    [L][M+L] lists."""
    L = len(q)
    n = M + L
    Q = [r[n - 1 - k] for k in range(n)]
    Bt = [[_dot(q[i], Q[k]) for k in range(n)] for i in range(L)]
    dt = [_dot(v, Q[k]) for k in range(n)]

    def left_shift(row, s):
        return row[s:] + [0.0] * s

    Bm = [left_shift(Bt[i], L - 1 - i) for i in range(L)]
    Dm = [left_shift(dt, L - 1 - i) for i in range(L)]
    return Bm, Dm
