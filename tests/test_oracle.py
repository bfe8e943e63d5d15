"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a hand-worked example, brute force
on tiny inputs, the paper's Appendix B route, a library routine the method
reduces to, or an invariant the paper states.  The last test plants plausible
mistakes in the oracle and checks that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from synth import random_case

HERE = os.path.dirname(os.path.abspath(__file__))


def _tolist(a):
    return np.asarray(a).tolist()


def _case(seed=0, B=2, d=6, H=2, dh=3, L=4, M=5, w=0.5):
    wl = random_case(seed, B, d, H, dh, L, M, "f32", w_std=w)
    lay = wl.layers[0]
    R = oracle.sinusoid(M + L, d)
    return wl, lay, R


# ------------------------------------------------------------ hand example
def test_hand_worked_example():
    """Closed-form scores of a 2-query example derived by hand from Sec. 3.3."""
    ex = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))
    h = np.array(ex["h"])
    mem = np.array(ex["mem"])
    u = np.array(ex["u"])
    v = np.array(ex["v"])
    I2 = np.eye(2)
    R = oracle.sinusoid(3, 2)
    out, terms = oracle.rel_attn_fwd(h, mem, I2, I2, I2, I2, u, v, R, 1, 2, scale=1.0,
                                     return_terms=True)
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(2), math.sin(2)
    s0 = [0.5 + 1.5 * c1, 2.5]
    s1_ = [1.5 + s2 + 1.5 * c2, 1 + s1 + 1.5 * c1, 4.0]

    def softmax(xs):
        m = max(xs)
        e = [math.exp(x - m) for x in xs]
        z = sum(e)
        return [x / z for x in e]

    p0 = softmax(s0)
    p1 = softmax(s1_)
    want = np.array([[p0[0], p0[1]], [p1[0] + p1[2], p1[1] + p1[2]]])
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-14)
    s = terms["ac"] + terms["bd"] + terms["cc"] + terms["dd"]
    np.testing.assert_allclose(s[0, 0, 0, :2], s0, atol=1e-14)
    np.testing.assert_allclose(s[0, 0, 1, :3], s1_, atol=1e-14)
    assert terms["p"][0, 0, 0, 2] == 0.0          # future key masked


# ------------------------------------------------------------------- sinusoid
def test_sinusoid_closed_form():
    R = oracle.sinusoid(7, 8)
    assert np.array_equal(R[0], np.array([0, 1] * 4, dtype=float))
    assert R[1, 0] == math.sin(1.0) and R[1, 1] == math.cos(1.0)
    assert abs(R[5, 6] - math.sin(5 / 10000 ** (6 / 8))) < 1e-15
    assert abs(R[5, 7] - math.cos(5 / 10000 ** (6 / 8))) < 1e-15
    np.testing.assert_allclose(R, np.array(brute.brute_sinusoid(7, 8)), atol=1e-15)


def test_sinusoid_relative_invariance():
    """R_a . R_b = sum_k cos((a-b) w_k) depends only on a-b: the property that
    lets the encoding carry relative distance."""
    d = 16
    R = oracle.sinusoid(40, d)
    G = R @ R.T
    for off in (0, 1, 5, 17):
        diag = np.diagonal(G, offset=off)
        np.testing.assert_allclose(diag, diag[0], atol=1e-12)
        w = 1.0 / 10000 ** (np.arange(0, d, 2) / d)
        assert abs(diag[0] - np.cos(off * w).sum()) < 1e-12


# -------------------------------------------------------------- brute force
@pytest.mark.parametrize("shape", [
    dict(B=1, d=4, H=1, dh=4, L=3, M=0),
    dict(B=2, d=6, H=2, dh=3, L=4, M=5),
    dict(B=1, d=8, H=2, dh=4, L=5, M=2),
    dict(B=2, d=5, H=1, dh=5, L=1, M=6),
    dict(B=1, d=16, H=1, dh=16, L=8, M=8),      # the tiny fp32 workload's shape
])
def test_brute_force_tiny(shape):
    """Pure-Python loops recomputing W_kR R_{i-j} per pair (the quadratic route
    of Sec. 3.3) agree with the oracle."""
    wl, lay, R = _case(seed=7 + shape["L"], **shape)
    h = wl.segments[0]
    mem = wl.mem[0]
    scale = 1.0 / math.sqrt(shape["dh"])
    got = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R,
                              shape["H"], shape["dh"], scale)
    ref, _ = brute.brute_rel_attn(_tolist(h), _tolist(mem), _tolist(lay.W_q), _tolist(lay.W_kE),
                                  _tolist(lay.W_kR), _tolist(lay.W_v), _tolist(wl.u),
                                  _tolist(wl.v), _tolist(R), shape["H"], shape["dh"], scale)
    ref = np.array(ref)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


# ------------------------------------------------- reduction to textbook attn
@pytest.mark.parametrize("M", [0, 3, 9])
def test_reduces_to_causal_attention(M):
    """u = v = 0 and W_kR = 0 leave term (a) alone: the layer is then causal
    scaled-dot-product attention with the memory as a visible prefix, as
    computed by torch's library routine in float64."""
    B, d, H, dh, L = 2, 12, 3, 4, 6
    wl, lay, R = _case(seed=11, B=B, d=d, H=H, dh=dh, L=L, M=M)
    h, mem = wl.segments[0], wl.mem[0]
    z = np.zeros_like
    scale = 0.37
    got = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, z(lay.W_kR), lay.W_v, z(wl.u),
                              z(wl.v), R, H, dh, scale)
    ht = np.concatenate([mem, h], axis=1)
    q = torch.tensor(h @ lay.W_q.T).reshape(B, L, H, dh).transpose(1, 2)
    k = torch.tensor(ht @ lay.W_kE.T).reshape(B, M + L, H, dh).transpose(1, 2)
    val = torch.tensor(ht @ lay.W_v.T).reshape(B, M + L, H, dh).transpose(1, 2)
    mask = torch.tensor(np.arange(M + L)[None, :] <= M + np.arange(L)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, val, attn_mask=mask,
                                                           scale=scale)
    ref = ref.transpose(1, 2).reshape(B, L, H * dh).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("M", [0, 4, 7])
def test_shaw_variant_two_terms(M):
    """The Shaw et al. (2018) form compared in Sec. 3.3 keeps only terms (a) and
    (b), with a learned table R_hat in place of W_kR R.  Taking u = v = 0 and the
    caller's Rk = R_hat must give: torch's scaled-dot-product attention in
    float64 with an additive bias scale * q_i . R_hat[M+i-j], the bias formed
    pair by pair in Python loops."""
    B, d, H, dh, L = 2, 10, 2, 5, 6
    wl, lay, R = _case(seed=19, B=B, d=d, H=H, dh=dh, L=L, M=M)
    h, mem = wl.segments[0], wl.mem[0]
    rng = np.random.default_rng(3)
    R_hat = rng.normal(0.0, 0.5, (M + L, H, dh))
    z = np.zeros_like
    scale = 0.41
    got = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, None, lay.W_v, z(wl.u), z(wl.v), None,
                              H, dh, scale, Rk=R_hat)
    ht = np.concatenate([mem, h], axis=1)
    qn = (h @ lay.W_q.T).reshape(B, L, H, dh)
    bias = np.full((B, H, L, M + L), -np.inf)
    for b in range(B):
        for hh in range(H):
            for i in range(L):
                for j in range(M + i + 1):
                    bias[b, hh, i, j] = scale * sum(qn[b, i, hh, c] * R_hat[M + i - j, hh, c]
                                                    for c in range(dh))
    q = torch.tensor(qn).transpose(1, 2)
    k = torch.tensor(ht @ lay.W_kE.T).reshape(B, M + L, H, dh).transpose(1, 2)
    val = torch.tensor(ht @ lay.W_v.T).reshape(B, M + L, H, dh).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, val,
                                                           attn_mask=torch.tensor(bias),
                                                           scale=scale)
    ref = ref.transpose(1, 2).reshape(B, L, H * dh).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


# --------------------------------------------------------- term invariants
def test_term_structure():
    """(c) does not depend on the query position and (d) depends only on i - j
    (Sec. 3.3: global content bias and global positional bias).  (b) is
    Toeplitz only when every query row is equal."""
    B, d, H, dh, L, M = 1, 8, 2, 4, 7, 5
    wl, lay, R = _case(seed=3, B=B, d=d, H=H, dh=dh, L=L, M=M)
    h, mem = wl.segments[0], wl.mem[0]
    _, t = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H,
                               dh, return_terms=True)
    vis = np.arange(M + L)[None, :] <= M + np.arange(L)[:, None]
    for hh in range(H):
        cc, dd, bd = t["cc"][0, hh], t["dd"][0, hh], t["bd"][0, hh]
        for i in range(L):
            np.testing.assert_array_equal(cc[i, vis[i]], cc[L - 1, vis[i]])
        for i in range(L - 1):
            for j in range(M + i + 1):
                assert abs(dd[i, j] - dd[i + 1, j + 1]) < 1e-13
        assert any(abs(bd[i, j] - bd[i + 1, j + 1]) > 1e-6
                   for i in range(L - 1) for j in range(M + i + 1))
    # equal query rows make (b) Toeplitz as well
    h_eq = np.repeat(h[:, :1, :], L, axis=1)
    _, t2 = oracle.rel_attn_fwd(h_eq, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R,
                                H, dh, return_terms=True)
    bd = t2["bd"][0, 0]
    for i in range(L - 1):
        for j in range(M + i + 1):
            assert abs(bd[i, j] - bd[i + 1, j + 1]) < 1e-13


# ------------------------------------------------------------- App. B route
@pytest.mark.parametrize("L,M", [(4, 5), (6, 0), (1, 7), (5, 5)])
def test_appendix_b_shift_route(L, M):
    """Terms (b) and (d) equal the left-shifted rows of B~ = q Q^T and
    d~ = (Q v)^T with Q the reversed position-key matrix (App. B)."""
    B, d, H, dh = 1, 8, 2, 4
    wl, lay, R = _case(seed=5, B=B, d=d, H=H, dh=dh, L=L, M=M)
    h, mem = wl.segments[0], wl.mem[0]
    _, t = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H,
                               dh, return_terms=True)
    r = (R[:M + L] @ lay.W_kR.T).reshape(M + L, H, dh)
    q = (h[0] @ lay.W_q.T).reshape(L, H, dh)
    for hh in range(H):
        Bm, Dm = brute.appb_terms(_tolist(q[:, hh]), _tolist(r[:, hh]), _tolist(wl.v[hh]), M)
        np.testing.assert_allclose(t["bd"][0, hh], np.array(Bm), atol=1e-13)
        np.testing.assert_allclose(t["dd"][0, hh], np.array(Dm), atol=1e-13)


# ------------------------------------------------------ concat equivalence
@pytest.mark.parametrize("L,M", [(5, 7), (8, 8), (3, 1)])
def test_memory_equals_concatenated_sequence(L, M):
    """A segment attending over memory X[:M] gives the last L rows of the same
    layer run with no memory over the whole sequence X (Sec. 3.2, 3.3)."""
    B, d, H, dh = 2, 8, 2, 4
    wl, lay, R = _case(seed=9, B=B, d=d, H=H, dh=dh, L=L, M=M)
    X = np.concatenate([wl.mem[0], wl.segments[0]], axis=1)
    args = (lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H, dh)
    seg = oracle.rel_attn_fwd(X[:, M:], X[:, :M], *args)
    full = oracle.rel_attn_fwd(X, X[:, :0], *args)
    np.testing.assert_allclose(seg, full[:, M:], atol=1e-12)


# ------------------------------------------------------------- stream / ring
def test_ring_stream_matches_explicit_memory():
    """The ring buffer reproduces 'memory = last M hidden states' over many
    segments, including L < M, L = M and L > M (Sec. 3.2)."""
    for (L, M) in [(3, 7), (4, 4), (6, 4)]:
        B, d, H, dh = 1, 8, 2, 4
        wl = random_case(21, B, d, H, dh, L, M, "f32", w_std=0.4, n_segments=5)
        lay = wl.layers[0]
        R = oracle.sinusoid(M + L, d)
        outs, mems, start = oracle.segment_stream(wl.segments, wl.layers, [wl.mem[0]], wl.u,
                                                  wl.v, R, H, dh)
        hist = wl.mem[0]
        for s, h in enumerate(wl.segments):
            want = oracle.rel_attn_fwd(h, hist, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v,
                                       R, H, dh)
            np.testing.assert_allclose(outs[s], want, atol=1e-13)
            hist = np.concatenate([hist, h], axis=1)[:, -M:]
        np.testing.assert_array_equal(oracle.logical_memory(mems[0], start), hist)


def test_ring_rotation_invariance_and_resume():
    B, d, H, dh, L, M = 2, 8, 2, 4, 3, 7
    wl = random_case(23, B, d, H, dh, L, M, "f32", w_std=0.4, n_segments=4)
    R = oracle.sinusoid(M + L, d)
    base, _, _ = oracle.segment_stream(wl.segments, wl.layers, [wl.mem[0]], wl.u, wl.v, R, H, dh)
    # the same logical memory stored with a rotated ring start gives the same outputs
    rot = 4
    phys = np.roll(wl.mem[0], rot, axis=1)      # logical p now at slot (p + rot) % M
    got, _, _ = oracle.segment_stream(wl.segments, wl.layers, [phys], wl.u, wl.v, R, H, dh,
                                      start=rot)
    for a, b in zip(base, got):
        np.testing.assert_array_equal(a, b)
    # checkpoint after 2 segments, resume: bit-identical
    o1, m1, s1 = oracle.segment_stream(wl.segments[:2], wl.layers, [wl.mem[0]], wl.u, wl.v, R,
                                       H, dh)
    o2, _, _ = oracle.segment_stream(wl.segments[2:], wl.layers, m1, wl.u, wl.v, R, H, dh,
                                     start=s1)
    for a, b in zip(base, o1 + o2):
        np.testing.assert_array_equal(a, b)


def test_mem_update_edges():
    mem = np.arange(2 * 4 * 1, dtype=float).reshape(2, 4, 1)
    h = 100 + np.arange(2 * 6 * 1, dtype=float).reshape(2, 6, 1)
    m2, s2 = oracle.mem_update(mem, 3, h)               # L > M
    assert s2 == 0
    np.testing.assert_array_equal(m2, h[:, 2:])
    m3, s3 = oracle.mem_update(mem, 3, h[:, :2])        # L < M, wraps around
    assert s3 == 1
    np.testing.assert_array_equal(m3[:, [3, 0]], h[:, :2])
    np.testing.assert_array_equal(m3[:, [1, 2]], mem[:, [1, 2]])
    m4, s4 = oracle.mem_update(mem[:, :0], 0, h)        # no memory
    assert m4.shape == (2, 0, 1) and s4 == 0


# --------------------------------------------------------------- sanity
def test_softmax_rows_and_convex_hull():
    B, d, H, dh, L, M = 2, 8, 2, 4, 6, 5
    wl, lay, R = _case(seed=13, B=B, d=d, H=H, dh=dh, L=L, M=M, w=1.0)
    h, mem = wl.segments[0], wl.mem[0]
    out, t = oracle.rel_attn_fwd(h, mem, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H,
                                 dh, return_terms=True)
    np.testing.assert_allclose(t["p"].sum(-1), 1.0, atol=1e-14)
    ht = np.concatenate([mem, h], axis=1)
    val = (ht @ lay.W_v.T).reshape(B, M + L, H, dh)
    o = out.reshape(B, L, H, dh)
    for b in range(B):
        for i in range(L):
            vis = val[b, :M + i + 1]
            assert np.all(o[b, i] <= vis.max(0) + 1e-12)
            assert np.all(o[b, i] >= vis.min(0) - 1e-12)


def test_stack_layer_pieces_match_torch():
    """The W_o / LayerNorm / ReLU feed-forward block against torch.nn.functional."""
    rng = np.random.default_rng(4)
    B, L, d, hd, di = 2, 3, 8, 6, 16
    a = rng.normal(size=(B, L, hd))
    h = rng.normal(size=(B, L, d))
    W_o = rng.normal(size=(d, hd))
    W1 = rng.normal(size=(di, d))
    W2 = rng.normal(size=(d, di))
    got = oracle.stack_layer(a, h, W_o, W1, W2)
    F = torch.nn.functional
    T = torch.tensor
    o = F.layer_norm(F.linear(T(a), T(W_o)) + T(h), (d,), eps=1e-5)
    ref = F.layer_norm(o + F.linear(F.relu(F.linear(o, T(W1))), T(W2)), (d,), eps=1e-5)
    np.testing.assert_allclose(got, ref.numpy(), atol=1e-12)


def test_batch_independence():
    """Batch rows never mix: a run on a subset of the batch equals those rows of
    the full run (lets large-shape parity sample batch rows)."""
    B, d, H, dh, L, M = 3, 8, 2, 4, 4, 6
    wl, lay, R = _case(seed=17, B=B, d=d, H=H, dh=dh, L=L, M=M)
    args = (lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H, dh)
    full = oracle.rel_attn_fwd(wl.segments[0], wl.mem[0], *args)
    part = oracle.rel_attn_fwd(wl.segments[0][1:2], wl.mem[0][1:2], *args)
    np.testing.assert_array_equal(full[1:2], part)


# --------------------------------------------------- planted mistakes (CPU)
def _pins_pass():
    """Run the pins that exercise rel_attn_terms; True if all of them pass."""
    try:
        test_hand_worked_example()
        for shp in (dict(B=2, d=6, H=2, dh=3, L=4, M=5), dict(B=1, d=4, H=1, dh=4, L=3, M=0)):
            test_brute_force_tiny(shp)
        test_appendix_b_shift_route(4, 5)
        test_memory_equals_concatenated_sequence(5, 7)
        test_term_structure()
    except AssertionError:
        return False
    return True


def _mutants(orig):
    def wrong_delta(q, k, r, u, v, M):            # forgot the memory offset
        return orig(q, k, r, u, v, 0)

    def drop_c(q, k, r, u, v, M):                 # dropped term (c)
        ac, bd, cc, dd, vis = orig(q, k, r, u, v, M)
        return ac, bd, 0 * cc, dd, vis

    def sign_d(q, k, r, u, v, M):                 # wrong sign on term (d)
        ac, bd, cc, dd, vis = orig(q, k, r, u, v, M)
        return ac, bd, cc, -dd, vis

    def reversed_r(q, k, r, u, v, M):             # R indexed by j - i order
        return orig(q, k, r[::-1].copy(), u, v, M)

    def swapped_uv(q, k, r, u, v, M):             # u and v exchanged
        return orig(q, k, r, v, u, M)

    def mask_strict(q, k, r, u, v, M):            # query cannot see itself
        ac, bd, cc, dd, vis = orig(q, k, r, u, v, M)
        vis = vis.copy()
        L = q.shape[0]
        vis[np.arange(L), M + np.arange(L)] = False
        return ac, bd, cc, dd, vis

    return [wrong_delta, drop_c, sign_d, reversed_r, swapped_uv, mask_strict]


def test_pins_catch_planted_mistakes(monkeypatch):
    from oracle import oracle as mod
    orig = mod.rel_attn_terms
    assert _pins_pass()
    for mut in _mutants(orig):
        monkeypatch.setattr(mod, "rel_attn_terms", mut)
        assert not _pins_pass(), f"pins missed planted mistake {mut.__name__}"
        monkeypatch.setattr(mod, "rel_attn_terms", orig)


# ------------------------------------------------ N-layer recurrence (CPU)
def _brute_stack_stream(wl, R, H, dh, scale, n_seg):
    """Independent route for an N-layer stream (Sec. 3.2 recurrence and the
    Sec. 3.3 summary equations, for n = 1..N): the attention of each layer is
    the pure-Python brute force, the rest of the layer is torch's functional
    linear / relu / layer_norm in float64, and layer n's memory is rebuilt from
    scratch as the last M rows of everything layer n has been given as input
    (its own input history), with no ring buffer."""
    F = torch.nn.functional
    T = torch.tensor
    M = wl.cfg.mem_len
    d = wl.cfg.d_model
    hist = [wl.mem[n].copy() for n in range(len(wl.layers))]   # logical, oldest first
    outs, per_layer = [], []
    for s in range(n_seg):
        x = wl.segments[s]
        layer_outs = []
        for n, lay in enumerate(wl.layers):
            a, _ = brute.brute_rel_attn(_tolist(x), _tolist(hist[n][:, -M:] if M else hist[n][:, :0]),
                                        _tolist(lay.W_q), _tolist(lay.W_kE), _tolist(lay.W_kR),
                                        _tolist(lay.W_v), _tolist(wl.u), _tolist(wl.v),
                                        _tolist(R), H, dh, scale)
            a = T(np.array(a))
            o = F.layer_norm(F.linear(a, T(lay.W_o)) + T(x), (d,), eps=1e-5)
            y = F.layer_norm(o + F.linear(F.relu(F.linear(o, T(lay.W_ff1))), T(lay.W_ff2)),
                             (d,), eps=1e-5).numpy()
            hist[n] = np.concatenate([hist[n], x], axis=1)   # layer n cached its own input
            layer_outs.append(y)
            x = y
        outs.append(x)
        per_layer.append(layer_outs)
    return outs, per_layer, [h[:, -M:] for h in hist]


def _stack_case():
    from synth import Config, make_workload
    cfg = Config("stack3_tiny", batch=2, d_model=8, n_heads=2, d_head=4, seg_len=3, mem_len=4,
                 n_layers=3, n_segments=3, dtype="f32", w_std=0.4, seed=31, d_inner=12)
    return cfg, make_workload(cfg)


def _stack_pin_passes():
    cfg, wl = _stack_case()
    H, dh, M = cfg.n_heads, cfg.d_head, cfg.mem_len
    R = oracle.sinusoid(M + cfg.seg_len, cfg.d_model)
    scale = 1.0 / math.sqrt(dh)
    want, want_layers, want_mem = _brute_stack_stream(wl, R, H, dh, scale, cfg.n_segments)
    mems = [m.copy() for m in wl.mem]
    start = 0
    for s in range(cfg.n_segments):
        y, mems, start, layer_outs = oracle.segment_step(wl.segments[s], wl.layers, mems, start,
                                                         wl.u, wl.v, R, H, dh, scale)
        if np.max(np.abs(y - want[s])) > 1e-11:
            return False
        for n in range(cfg.n_layers):
            if np.max(np.abs(layer_outs[n] - want_layers[s][n])) > 1e-11:
                return False
    for n in range(cfg.n_layers):
        # layer 0 caches the segment inputs themselves (exact); deeper layers
        # cache outputs of the layer below, formed by the two routes
        got = oracle.logical_memory(mems[n], start)
        if got.shape != want_mem[n].shape or np.max(np.abs(got - want_mem[n])) > 1e-11:
            return False
    return True


def test_stack_recurrence_three_layers():
    """Three full layers (W_o, LayerNorm, ReLU feed-forward), each with its own
    memory, over three segments with L < M: every layer output and final ring of
    oracle.segment_step equals the independent brute-force route."""
    assert _stack_pin_passes()


def _stack_mutants(orig):
    """Plausible mistakes in the N-layer recurrence, each a variant of
    segment_step (Sec. 3.3 summary: layer n attends over [SG(m^{n-1}) ; h^{n-1}]
    and caches h^{n-1})."""
    from oracle import oracle as mod

    def run(h, layers, mems, start, u, v, R, H, dh, scale=None, Rks=None, *, seg_input=False,
            shared_mem=False, cache_output=False):
        outs, new_mems, x, new_start = [], [], h, start
        for n, lay in enumerate(layers):
            src = mems[0] if shared_mem else mems[n]
            inp = h if seg_input else x
            a = mod.rel_attn_fwd(inp, mod.logical_memory(src, start), lay.W_q, lay.W_kE, lay.W_kR,
                                 lay.W_v, u, v, R, H, dh, scale)
            y = mod.stack_layer(a, inp, lay.W_o, lay.W_ff1, lay.W_ff2)
            m_new, new_start = mod.mem_update(src, start, y if cache_output else inp)
            new_mems.append(m_new)
            outs.append(y)
            x = y
        return x, new_mems, new_start, outs

    def segment_input_to_every_layer(*a, **k):
        return run(*a, **k, seg_input=True)

    def one_shared_memory(*a, **k):
        return run(*a, **k, shared_mem=True)

    def memory_caches_layer_output(*a, **k):
        return run(*a, **k, cache_output=True)

    return [segment_input_to_every_layer, one_shared_memory, memory_caches_layer_output]


def test_stack_pin_catches_planted_mistakes(monkeypatch):
    from oracle import oracle as mod
    orig = mod.segment_step
    assert _stack_pin_passes()
    for mut in _stack_mutants(orig):
        monkeypatch.setattr(mod, "segment_step", mut)
        monkeypatch.setattr(oracle, "segment_step", mut)
        assert not _stack_pin_passes(), f"stack pin missed planted mistake {mut.__name__}"
        monkeypatch.setattr(mod, "segment_step", orig)
        monkeypatch.setattr(oracle, "segment_step", orig)
