"""Pins of the CPU oracle's backward pass (CPU only).

The gradients of oracle.backward are checked against two routes that share
nothing with it: central finite differences of the forward in float64, and
torch autograd through torch's own scaled-dot-product attention with the
position terms added as a bias formed pair by pair.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob
from synth import random_case


def _core_case(seed, L, M, dh, w=0.7):
    rng = np.random.default_rng(seed)
    n = M + L
    return dict(q=rng.normal(0, w, (L, dh)), k=rng.normal(0, w, (n, dh)),
                val=rng.normal(0, 1, (n, dh)), r=rng.normal(0, w, (n, dh)),
                u=rng.normal(0, w, dh), v=rng.normal(0, w, dh)), rng.normal(0, 1, (L, dh))


@pytest.mark.parametrize("L,M,dh", [(4, 5, 3), (6, 0, 2), (3, 7, 4), (1, 4, 3)])
def test_core_gradients_match_finite_differences(L, M, dh):
    """Every gradient of the core against central differences of the loss
    sum(out * G) (float64, step 1e-6)."""
    t, G = _core_case(11 + L + M, L, M, dh)
    scale = 0.83

    def loss(tt):
        out, _ = ob.attn_core(tt["q"], tt["k"], tt["val"], tt["r"], tt["u"], tt["v"], M, scale)
        return float((out * G).sum())

    g = ob.attn_core_bwd(t["q"], t["k"], t["val"], t["r"], t["u"], t["v"], M, scale, G)
    eps = 1e-6
    for name in ("q", "k", "val", "r", "u", "v"):
        fd = np.zeros_like(t[name])
        for idx in np.ndindex(t[name].shape):
            tp = {k: x.copy() for k, x in t.items()}
            tm = {k: x.copy() for k, x in t.items()}
            tp[name][idx] += eps
            tm[name][idx] -= eps
            fd[idx] = (loss(tp) - loss(tm)) / (2 * eps)
        err = np.max(np.abs(fd - g[name])) / max(1e-12, np.max(np.abs(fd)))
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("L,M,dh", [(5, 6, 4), (8, 0, 3), (7, 9, 8)])
def test_core_gradients_match_torch_autograd(L, M, dh):
    """torch autograd through F.scaled_dot_product_attention(q + u, k, val) with
    the additive bias scale * (q_i + v) . r[M+i-j] (gathered per pair by index)
    and -inf on future keys."""
    t, G = _core_case(3 * L + M, L, M, dh)
    scale = 1.0 / math.sqrt(dh)
    g = ob.attn_core_bwd(t["q"], t["k"], t["val"], t["r"], t["u"], t["v"], M, scale, G)
    T = {k: torch.tensor(x, requires_grad=True) for k, x in t.items()}
    n = M + L
    delta = torch.tensor([[M + i - j for j in range(n)] for i in range(L)])
    vis = delta >= 0
    rg = T["r"][delta.clamp(min=0)]                       # [L, n, dh]: r[M+i-j]
    bias = scale * ((T["q"] + T["v"])[:, None, :] * rg).sum(-1)
    bias = torch.where(vis, bias, torch.tensor(-math.inf, dtype=torch.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        (T["q"] + T["u"])[None], T["k"][None], T["val"][None], attn_mask=bias[None],
        scale=scale)[0]
    (out * torch.tensor(G)).sum().backward()
    for name in ("q", "k", "val", "r", "u", "v"):
        ref = T[name].grad.numpy()
        assert np.max(np.abs(ref - g[name])) <= 1e-10 * max(1.0, np.max(np.abs(ref))), name


def test_layer_w_kr_gradient_matches_finite_differences():
    """Through the projection r = R W_kR^T: dLoss/dW_kR from rel_attn_bwd against
    central differences of the forward oracle for sampled entries."""
    B, d, H, dh, L, M = 2, 6, 2, 3, 4, 5
    wl = random_case(5, B, d, H, dh, L, M, "f32", w_std=0.5)
    lay = wl.layers[0]
    R = oracle.sinusoid(M + L, d)
    h, mem = wl.segments[0], wl.mem[0]
    rng = np.random.default_rng(9)
    G = rng.normal(0, 1, (B, L, H * dh))
    scale = 0.6
    g = ob.rel_attn_bwd(h, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H, dh,
                        scale, G)

    def loss(W):
        out = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, W, lay.W_v, wl.u, wl.v, R, H, dh,
                                  scale)
        return float((out * G).sum())

    eps = 1e-6
    for idx in [(0, 0), (1, 3), (4, 5), (5, 2), (2, 1)]:
        Wp, Wm = lay.W_kR.copy(), lay.W_kR.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        fd = (loss(Wp) - loss(Wm)) / (2 * eps)
        assert abs(fd - g["W_kR"][idx]) <= 1e-6 * max(1.0, abs(fd)), idx


def test_layer_gradients_sum_core_gradients():
    """rel_attn_bwd's batch/head bookkeeping: per-(b, h) core gradients land in
    their slots, and r, u, v gradients are summed over batch rows."""
    B, d, H, dh, L, M = 2, 6, 2, 3, 3, 4
    wl = random_case(8, B, d, H, dh, L, M, "f32", w_std=0.5)
    lay = wl.layers[0]
    R = oracle.sinusoid(M + L, d)
    h, mem = wl.segments[0], wl.mem[0]
    G = np.random.default_rng(1).normal(0, 1, (B, L, H * dh))
    scale = 0.5
    g = ob.rel_attn_bwd(h, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H, dh,
                        scale, G)
    ht = np.concatenate([mem, h], axis=1)
    q = (h @ lay.W_q.T).reshape(B, L, H, dh)
    k = (ht @ lay.W_kE.T).reshape(B, M + L, H, dh)
    val = (ht @ lay.W_v.T).reshape(B, M + L, H, dh)
    r = (R @ lay.W_kR.T).reshape(M + L, H, dh)
    dr = np.zeros_like(r)
    for b in range(B):
        for hh in range(H):
            c = ob.attn_core_bwd(q[b, :, hh], k[b, :, hh], val[b, :, hh], r[:, hh], wl.u[hh],
                                 wl.v[hh], M, scale, G.reshape(B, L, H, dh)[b, :, hh])
            assert np.allclose(g["q"][b, :, hh], c["q"], rtol=0, atol=1e-12)
            assert np.allclose(g["k"][b, :, hh], c["k"], rtol=0, atol=1e-12)
            dr[:, hh] += c["r"]
    assert np.allclose(g["r"], dr, rtol=0, atol=1e-12)
