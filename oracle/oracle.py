"""CPU oracle (float64, numpy) for the Transformer-XL relative-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU
library and never reads anything the GPU path produced.

Source: Dai et al., "Transformer-XL: Attentive Language Models Beyond a
Fixed-Length Context".  Each function names the passage it follows.  Where the
paper leaves a step open, the reading taken is stated in the docstring.

Conventions
  * Batched tensors are [batch, length, features]; heads split the feature axis
    into consecutive blocks of d_head (head h owns features h*d_head ...).
  * Memory is a ring buffer: logical row p (oldest first) lives at physical
    slot (start + p) mod M.
  * Key index j runs over the extended context [memory ; segment] (0 .. M+L-1);
    query index i runs over the segment (0 .. L-1); the relative distance is
    delta = M + i - j.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "sinusoid", "logical_memory", "rel_proj", "rel_attn_fwd", "rel_attn_terms",
    "mem_update", "layer_norm", "stack_layer", "segment_step", "segment_stream",
]


# --------------------------------------------------------------------------- R
def sinusoid(n_pos: int, d: int) -> np.ndarray:
    """Relative position table R, row delta = distance delta (delta = 0..n_pos-1).

    Sec. 3.3 states R is the sinusoid encoding matrix of Vaswani et al. (2017)
    with no learnable parameters, and that row i of R encodes a relative
    distance of i.  No page prints the formula; the reading taken is Vaswani's:
    column 2k holds sin(delta / 10000^(2k/d)), column 2k+1 holds
    cos(delta / 10000^(2k/d))."""
    R = np.zeros((n_pos, d), dtype=np.float64)
    pos = np.arange(n_pos, dtype=np.float64)
    for c in range(d):
        k2 = c - (c % 2)                      # the even index 2k of this pair
        angle = pos / (10000.0 ** (k2 / d))
        R[:, c] = np.sin(angle) if c % 2 == 0 else np.cos(angle)
    return R


# ----------------------------------------------------------------- memory ring
def logical_memory(mem_phys: np.ndarray, start: int) -> np.ndarray:
    """Oldest-first view of a ring-buffered memory [B, M, d]."""
    M = mem_phys.shape[1]
    if M == 0:
        return mem_phys.copy()
    idx = (start + np.arange(M)) % M
    return mem_phys[:, idx, :]


def mem_update(mem_phys: np.ndarray, start: int, h: np.ndarray):
    """Memory update of Sec. 3.2: the memory caches the M most recent hidden
    states, possibly spanning several segments.  Reading taken (first-in
    first-out): the new logical memory is the last M rows of [memory ; h],
    written after the segment has used the old memory.

    Returns (new physical ring, new start).  When L < M the L oldest slots are
    overwritten in place and start advances by L; when L >= M the ring holds
    the last M rows of h in order and start becomes 0."""
    B, M, d = mem_phys.shape
    L = h.shape[1]
    out = mem_phys.copy()
    if M == 0:
        return out, 0
    if L >= M:
        out[:, :, :] = h[:, L - M:, :]
        return out, 0
    slots = (start + np.arange(L)) % M
    out[:, slots, :] = h
    return out, (start + L) % M


# ----------------------------------------------------------------- projections
def _heads(x: np.ndarray, n_heads: int, d_head: int) -> np.ndarray:
    """[..., n_heads*d_head] -> [..., n_heads, d_head]."""
    return x.reshape(x.shape[:-1] + (n_heads, d_head))


def rel_proj(R: np.ndarray, W_kR: np.ndarray, n_heads: int, d_head: int) -> np.ndarray:
    """Position keys r[delta] = W_kR R_delta for every distance (App. B, matrix Q
    stores the same rows in reversed order).  Returns [n_pos, n_heads, d_head]."""
    return _heads(R @ W_kR.T, n_heads, d_head)


# ------------------------------------------------------------------- attention
def rel_attn_terms(q, k, r, u, v, M):
    """The four score terms of A^rel (Sec. 3.3) for one (batch, head).

    q [L, dh], k [M+L, dh], r [M+L, dh] (r[delta] = W_kR R_delta), u, v [dh].
    Returns (ac, bd, cc, dd, visible), each [L, M+L]:
      (a) ac[i,j] = q_i . k_j                       content addressing
      (b) bd[i,j] = q_i . W_kR R_{i-j}              content-dependent position bias
      (c) cc[i,j] = u . k_j                         global content bias
      (d) dd[i,j] = v . W_kR R_{i-j}                global position bias
    The distance between query i and key j of [memory ; segment] is
    delta = M + i - j (App. B: row i of matrix B pairs column j with R_{M+i-j}).
    Terms (b) and (d) are evaluated per pair: the scalars q_i . r[delta] and
    v . r[delta] are formed for every delta and then looked up at each pair's own
    delta.  Entries with delta < 0 (future keys) are set to 0 and reported as
    not visible."""
    L = q.shape[0]
    n = k.shape[0]
    i = np.arange(L)[:, None]
    j = np.arange(n)[None, :]
    delta = M + i - j
    visible = delta >= 0
    dcl = np.clip(delta, 0, n - 1)
    ac = q @ k.T
    bd = np.take_along_axis(q @ r.T, dcl, axis=1)
    cc = np.broadcast_to((k @ u)[None, :], (L, n)).copy()
    dd = (r @ v)[dcl]
    for t in (bd, dd):
        t[~visible] = 0.0
    ac = np.where(visible, ac, 0.0)
    cc = np.where(visible, cc, 0.0)
    return ac, bd, cc, dd, visible


def rel_attn_fwd(h, mem_log, W_q, W_kE, W_kR, W_v, u, v, R=None, n_heads=1, d_head=None,
                 scale=None, Rk=None, return_terms=False):
    """One relative-attention forward over a cached memory (Sec. 3.3 summary
    equations, single head generalised to n_heads).

      h~   = [SG(m) ; h]                                  (concatenation, length)
      q, k, val = h W_q^T,  h~ W_kE^T,  h~ W_v^T
      A_ij = q_i.k_j + q_i.W_kR R_{i-j} + u.k_j + v.W_kR R_{i-j}
      a    = Masked-Softmax(A) val

    Readings taken where the paper is silent:
      * scale: the summary applies Masked-Softmax to A directly; scale multiplies
        the sum of the four terms.  Default 1/sqrt(d_head) (the scaled
        dot-product attention of Vaswani et al., which the model builds on);
        scale=1 is the literal formula.
      * mask: query i sees every memory slot and the segment keys j <= i, i.e.
        key j of [memory ; segment] is visible iff j <= M + i (Sec. 3.3 lets
        q_i attend on k_{<=i}; App. B's matrix B has zeros past R_0).
      * heads: head h uses rows h*d_head .. of W_q, W_kE, W_kR, W_v and u[h],
        v[h]; R is shared by all heads; the output concatenates the heads.

    h [B, L, d], mem_log [B, M, d] (oldest first).  If Rk is given
    ([M+L, H, dh]) it replaces W_kR R.  Returns out [B, L, H*d_head] (and the
    term matrices [B, H, L, M+L] if return_terms)."""
    B, L, d = h.shape
    M = mem_log.shape[1]
    H = n_heads
    dh = d_head if d_head is not None else W_q.shape[0] // H
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    ht = np.concatenate([mem_log, h], axis=1)
    q = _heads(h @ W_q.T, H, dh)
    k = _heads(ht @ W_kE.T, H, dh)
    val = _heads(ht @ W_v.T, H, dh)
    r = Rk if Rk is not None else rel_proj(R[:M + L], W_kR, H, dh)
    out = np.zeros((B, L, H, dh))
    terms = None
    if return_terms:
        terms = {t: np.zeros((B, H, L, M + L)) for t in ("ac", "bd", "cc", "dd", "p")}
    for b in range(B):
        for hh in range(H):
            ac, bd, cc, dd, vis = rel_attn_terms(q[b, :, hh], k[b, :, hh], r[:, hh],
                                                 u[hh], v[hh], M)
            s = scale * (ac + bd + cc + dd)
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, hh] = p @ val[b, :, hh]
            if return_terms:
                for name, t in (("ac", ac), ("bd", bd), ("cc", cc), ("dd", dd), ("p", p)):
                    terms[name][b, hh] = t
    out = out.reshape(B, L, H * dh)
    return (out, terms) if return_terms else out


# ---------------------------------------------------------------- full layer
def layer_norm(x: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the feature axis, no affine parameters (gain 1, bias 0).
    The summary equations name LayerNorm without parameters; eps 1e-5 is the
    reading taken."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def stack_layer(a, h, W_o, W_ff1, W_ff2):
    """The rest of one layer after attention (Sec. 3.3 summary equations):
      o  = LayerNorm(Linear(a) + h)
      h' = Positionwise-Feed-Forward(o)
    Reading taken for the feed-forward block (no biases anywhere, ReLU, residual
    and LayerNorm): h' = LayerNorm(o + ReLU(o W_ff1^T) W_ff2^T)."""
    o = layer_norm(a @ W_o.T + h)
    f = np.maximum(o @ W_ff1.T, 0.0) @ W_ff2.T
    return layer_norm(o + f)


def segment_step(h, layers, mems, start, u, v, R, n_heads, d_head, scale=None, Rks=None):
    """One segment through an N-layer Transformer-XL (Sec. 3.3, for n = 1..N).

    mems[n] is layer n's physical memory ring (all layers share ``start``).
    Layer n attends over [memory_n ; h^{n-1}] and its memory is then updated with
    its own input h^{n-1} (the summary equation extends h^{n-1} with m^{n-1}).
    u and v are shared by all layers (the summary gives them no layer index).
    A layer without W_o returns the attention output itself.

    Returns (h_out, new_mems, new_start, per-layer outputs)."""
    outs = []
    new_mems = []
    new_start = start
    x = h
    for n, lay in enumerate(layers):
        mem_log = logical_memory(mems[n], start)
        Rk = None if Rks is None else Rks[n]
        a = rel_attn_fwd(x, mem_log, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, u, v, R,
                         n_heads, d_head, scale, Rk=Rk)
        y = a if lay.W_o is None else stack_layer(a, x, lay.W_o, lay.W_ff1, lay.W_ff2)
        m_new, new_start = mem_update(mems[n], start, x)
        new_mems.append(m_new)
        outs.append(y)
        x = y
    return x, new_mems, new_start, outs


def segment_stream(segments, layers, mems, u, v, R, n_heads, d_head, scale=None, start=0):
    """Run consecutive segments, carrying every layer's memory (Sec. 3.2,
    segment-level recurrence with state reuse).  Returns the list of per-segment
    outputs, the final rings and the final start."""
    outs = []
    for h in segments:
        y, mems, start, _ = segment_step(h, layers, mems, start, u, v, R, n_heads, d_head, scale)
        outs.append(y)
    return outs, mems, start
