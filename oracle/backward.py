"""CPU oracle (float64, numpy) for the backward pass of the relative attention.

TEST INFRASTRUCTURE ONLY.  Only the tests and the smoke check may import this
module.  It shares no code with the GPU library.

Source: Dai et al., "Transformer-XL", Sec. 3.3 (the score A^rel with its four
terms, Masked-Softmax and the value sum) and Sec. 3.2 (the memory enters with a
stop-gradient, so no gradient reaches the cached states themselves; the keys and
values computed from them are ordinary tensors of the segment's graph).

Gradients are taken with respect to the tensors the attention core consumes:
the per-head queries q, keys k and values val over [memory ; segment], the
position keys r[delta] = W_kR R_delta, and the biases u, v; and, through
r = R W_kR^T, with respect to W_kR.  The chain rule is written out term by term
(softmax Jacobian, then each of the four score terms); nothing is blocked,
fused or reordered.
"""
from __future__ import annotations

import numpy as np

from .oracle import rel_attn_terms

__all__ = ["attn_core", "attn_core_bwd", "rel_attn_bwd"]


def attn_core(q, k, val, r, u, v, M, scale):
    """Forward of the attention core for one batch row and head.

    q [L, dh], k, val [M+L, dh], r [M+L, dh] (r[delta] = W_kR R_delta), u, v [dh].
      A_ij = q_i.k_j + q_i.r[M+i-j] + u.k_j + v.r[M+i-j]   (four terms, Sec. 3.3)
      P    = softmax_j(scale * A_ij over visible j <= M + i)
      out  = P val
    The terms are the forward oracle's (per-pair lookup of r at delta).
    Returns (out [L, dh], P [L, M+L])."""
    ac, bd, cc, dd, vis = rel_attn_terms(q, k, r, u, v, M)
    s = np.where(vis, scale * (ac + bd + cc + dd), -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    P = np.exp(s)
    P = P / P.sum(axis=1, keepdims=True)
    return P @ val, P


def attn_core_bwd(q, k, val, r, u, v, M, scale, d_out):
    """Backward of ``attn_core`` for one batch row and head, given
    d_out = dLoss/d out [L, dh].  Returns a dict of dLoss/d{q, k, val, r, u, v}.

      d val_j   = sum_i P_ij d_out_i
      dP_ij     = d_out_i . val_j
      dS_ij     = P_ij (dP_ij - sum_j' P_ij' dP_ij')       (softmax Jacobian)
      dA_ij     = scale * dS_ij
      (a) q_i.k_j      -> dq_i += dA_ij k_j,        dk_j += dA_ij q_i
      (b) q_i.r[delta] -> dq_i += dA_ij r[delta],   dr[delta] += dA_ij q_i
      (c) u.k_j        -> du   += dA_ij k_j,        dk_j += dA_ij u
      (d) v.r[delta]   -> dv   += dA_ij r[delta],   dr[delta] += dA_ij v
    with delta = M + i - j over the visible pairs j <= M + i.  The sums over
    keys run per query row i; for a fixed i, j -> delta = M + i - j walks the
    visible keys and the distances 0 .. M+i in opposite orders."""
    L = q.shape[0]
    _, P = attn_core(q, k, val, r, u, v, M, scale)
    d_val = P.T @ d_out
    dP = d_out @ val.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dA = scale * dS                      # zero on masked pairs, where P is 0
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dr = np.zeros_like(r)
    du = np.zeros_like(u)
    dv = np.zeros_like(v)
    for i in range(L):
        nv = M + i + 1                   # visible keys j = 0 .. M+i
        g = dA[i, :nv]                   # g[j]
        g_by_delta = g[::-1]             # g at j = M+i-delta, delta = 0 .. M+i
        r_vis = r[:nv]                   # r[delta], delta = 0 .. M+i
        dq[i] += g @ k[:nv]                              # (a)
        dk[:nv] += np.outer(g, q[i])
        dq[i] += g_by_delta @ r_vis                      # (b)
        dr[:nv] += np.outer(g_by_delta, q[i])
        du += g @ k[:nv]                                 # (c)
        dk[:nv] += np.outer(g, u)
        dv += g_by_delta @ r_vis                         # (d)
        dr[:nv] += np.outer(g_by_delta, v)
    return dict(q=dq, k=dk, val=d_val, r=dr, u=du, v=dv)


def _heads(x, H, dh):
    return x.reshape(x.shape[:-1] + (H, dh))


def rel_attn_bwd(h, mem_log, W_q, W_kE, W_kR, W_v, u, v, R, n_heads, d_head, scale, d_out,
                 Rk=None):
    """Backward of one relative-attention layer (Sec. 3.3 summary equations)
    with respect to the attention core's inputs, for all batch rows and heads.

    h [B, L, d], mem_log [B, M, d] (oldest first), d_out [B, L, H*d_head].
    Projections as in the forward: q = h W_q^T, k = h~ W_kE^T, val = h~ W_v^T
    with h~ = [mem ; h]; r = R W_kR^T (or the given Rk [M+L, H, dh]).
    Returns dict with
      q   [B, L, H, dh]     dLoss/dq
      k   [B, M+L, H, dh]   dLoss/dk   (memory rows included: SG stops the
      val [B, M+L, H, dh]   dLoss/dval  gradient at the cached states, not here)
      u, v [H, dh]          summed over batch rows, queries and keys
      r   [M+L, H, dh]      dLoss/dr, summed over batch rows
      W_kR [H*dh, d_pos]    dLoss/dW_kR = sum_delta dr[delta] (x) R_delta
                            (only when r is computed from W_kR and R)."""
    B, L, _ = h.shape
    M = mem_log.shape[1]
    H, dh = n_heads, d_head
    ht = np.concatenate([mem_log, h], axis=1)
    q = _heads(h @ W_q.T, H, dh)
    k = _heads(ht @ W_kE.T, H, dh)
    val = _heads(ht @ W_v.T, H, dh)
    r = Rk if Rk is not None else _heads(R[:M + L] @ W_kR.T, H, dh)
    g = _heads(d_out, H, dh)
    out = dict(q=np.zeros_like(q), k=np.zeros_like(k), val=np.zeros_like(val),
               r=np.zeros_like(r), u=np.zeros((H, dh)), v=np.zeros((H, dh)))
    for b in range(B):
        for hh in range(H):
            gr = attn_core_bwd(q[b, :, hh], k[b, :, hh], val[b, :, hh], r[:, hh], u[hh], v[hh],
                               M, scale, g[b, :, hh])
            out["q"][b, :, hh] = gr["q"]
            out["k"][b, :, hh] = gr["k"]
            out["val"][b, :, hh] = gr["val"]
            out["r"][:, hh] += gr["r"]
            out["u"][hh] += gr["u"]
            out["v"][hh] += gr["v"]
    if Rk is None:
        out["W_kR"] = out["r"].reshape(M + L, H * dh).T @ R[:M + L]
    return out
