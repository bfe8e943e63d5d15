"""GPU parity of the backward (txl_rel_attn_bwd) against the CPU oracle's
backward (oracle.backward, pinned by finite differences and torch autograd).

Tolerance as for the bf16 path: max|gpu - oracle| <= 2e-2 * max|oracle| per
gradient tensor.  Gradients that sum over batch rows (d_Rk, d_u, d_v, d_W_kR)
are compared whole, for the full train-shaped batch (22 rows) too."""
import numpy as np
import pytest

import synth
from gpu_helpers import (DeviceLayers, assert_close, from_dev, log, nan_empty, poisoned, to_dev,
                         workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def txl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_xl_relative_attn_amd as mod
    return mod


def _run(txl, cfg, b_idx, use_rk=False, with_wkr=True, seed=7, oracle_rows=False):
    import torch
    import oracle
    log(f"[case] backward {cfg.name} B={cfg.batch} L={cfg.seg_len} M={cfg.mem_len} "
        f"H={cfg.n_heads} dh={cfg.d_head} d={cfg.d_model} rk={use_rk} wkr={with_wkr}")
    wl = synth.make_workload(cfg, n_segments=1)
    c = cfg
    H, dh, L, M, B = c.n_heads, c.d_head, c.seg_len, c.mem_len, c.batch
    P = M + L
    rng = np.random.default_rng(seed)
    G = synth.round_to(rng.normal(0.0, 1.0, (B, L, H * dh)), "bf16")
    dl = DeviceLayers(wl)
    shp = dl.shape()
    w = dl.W[0]
    Rk = None
    Rk_host = None
    if use_rk:
        Rk_host = synth.round_to(rng.normal(0.0, 0.5, (P, H, dh)), "bf16")
        Rk = to_dev(Rk_host, "bf16")
    f32 = dict(dtype=torch.float32, device="cuda")
    d_q = poisoned((B, L, H, dh), torch.float32)
    d_k = poisoned((B, P, H, dh), torch.float32)
    d_val = poisoned((B, P, H, dh), torch.float32)
    d_u = poisoned((H, dh), torch.float32)
    d_v = poisoned((H, dh), torch.float32)
    d_Rk = poisoned((P, H, dh), torch.float32)
    d_W = poisoned((H * dh, c.d_pos), torch.float32) if with_wkr else None
    ws = workspace(txl.txl_rel_attn_bwd_workspace_bytes(shp))
    h = to_dev(wl.segments[0], "bf16")
    txl.txl_rel_attn_bwd(shp, h, dl.mem[0] if M else None, 0, w["W_q"], w["W_kE"],
                         None if use_rk else w["W_kR"], w["W_v"], dl.u, dl.v,
                         None if use_rk else dl.R, Rk, to_dev(G, "bf16"), d_q, d_k, d_val, d_u,
                         d_v, d_Rk, d_W, ws)
    torch.cuda.synchronize()
    lay = wl.layers[0]
    R = oracle.sinusoid(P, c.d_pos)
    scale = 1.0 / np.sqrt(dh)
    if oracle_rows:
        from oracle_pool import oracle_bwd_rows
        assert not use_rk and np.array_equal(b_idx, np.arange(B))
        log(f"  oracle backward on {B} rows in worker processes")
        want = oracle_bwd_rows(cfg, seed)
    else:
        want = oracle.backward.rel_attn_bwd(wl.segments[0][b_idx], wl.mem[0][b_idx], lay.W_q,
                                            lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v, R, H, dh,
                                            scale, G[b_idx], Rk=Rk_host)
    assert_close(from_dev(d_q)[b_idx], want["q"], "bf16", "d_q")
    assert_close(from_dev(d_k)[b_idx], want["k"], "bf16", "d_k")
    assert_close(from_dev(d_val)[b_idx], want["val"], "bf16", "d_val")
    return dict(d_Rk=from_dev(d_Rk), d_u=from_dev(d_u), d_v=from_dev(d_v),
                d_W=None if d_W is None else from_dev(d_W)), want


def _check_summed(got, want, full_batch):
    if not full_batch:
        return
    assert_close(got["d_Rk"], want["r"], "bf16", "d_Rk")
    assert_close(got["d_u"], want["u"], "bf16", "d_u")
    assert_close(got["d_v"], want["v"], "bf16", "d_v")
    if got["d_W"] is not None:
        assert_close(got["d_W"], want["W_kR"], "bf16", "d_W_kR")


def test_bwd_small(txl):
    cfg = synth.Config("bwd_small", 2, 128, 2, 64, 64, 40, 1, 1, "bf16", 0.05, 321)
    got, want = _run(txl, cfg, np.arange(2))
    _check_summed(got, want, True)


def test_bwd_odd_head_packed(txl):
    """d_model 410 (rows repacked to 448), d_head 41, memory 150, one query group
    plus a ragged tail."""
    cfg = synth.Config("bwd_odd", 2, 410, 10, 41, 150, 150, 1, 1, "bf16", 0.02, 1002)
    got, want = _run(txl, cfg, np.arange(2))
    _check_summed(got, want, True)


def test_bwd_no_memory_and_caller_rk(txl):
    """M = 0 with the caller's position keys (no W_kR gradient)."""
    cfg = synth.Config("bwd_nomem", 2, 128, 2, 64, 96, 0, 1, 1, "bf16", 0.05, 55)
    got, want = _run(txl, cfg, np.arange(2), use_rk=True, with_wkr=False)
    _check_summed(got, want, True)


def test_bwd_split_forward(txl):
    """A single (b, h) with a long memory: the recomputed forward uses key-range
    splits, whose combine provides the log-sum-exp."""
    cfg = synth.Config("bwd_split", 1, 64, 1, 64, 32, 1500, 1, 1, "bf16", 0.05, 77)
    got, want = _run(txl, cfg, np.arange(1))
    _check_summed(got, want, True)


def test_bwd_train_shaped_two_rows(txl):
    """Train-shaped layer (segment 512, memory 512, 8 heads of 64, d_model 512)
    with 2 batch rows: every gradient, summed ones included."""
    cfg = synth.get_config("train_l512_m512", batch=2)
    got, want = _run(txl, cfg, np.arange(2))
    _check_summed(got, want, True)


def test_bwd_train_shaped_full_batch(txl):
    """The full train-shaped batch (22 rows): every row's d_q, d_k, d_val, and
    the gradients summed over all 22 rows (d_Rk, d_u, d_v, d_W_kR), which go
    through the per-row ordered sums.  The oracle runs one row per worker
    process."""
    cfg = synth.get_config("train_l512_m512")
    got, want = _run(txl, cfg, np.arange(cfg.batch), oracle_rows=True)
    _check_summed(got, want, True)


def test_bwd_odd_batch(txl):
    """Three batch rows: the dRk product takes one batch row per partial (pairs
    when the count is even), and the partials are summed in order."""
    cfg = synth.Config("bwd_odd_batch", 3, 128, 2, 64, 96, 64, 1, 1, "bf16", 0.05, 303)
    got, want = _run(txl, cfg, np.arange(3))
    _check_summed(got, want, True)


def test_bwd_long_segment(txl):
    """Segment 640 > 512: the key-side products stage their shared operand in
    two K chunks, and workgroups whose band starts in the second chunk skip the
    first."""
    cfg = synth.Config("bwd_long_seg", 1, 128, 2, 64, 640, 96, 1, 1, "bf16", 0.05, 91)
    got, want = _run(txl, cfg, np.arange(1))
    _check_summed(got, want, True)


@pytest.mark.parametrize("case", ["train_two_rows", "caller_rk_no_memory"])
def test_bwd_saved_matches_recompute(txl, case):
    """txl_rel_attn_fwd_train + txl_rel_attn_bwd_saved give txl_rel_attn_fwd's
    output and txl_rel_attn_bwd's gradients bit for bit (same kernels, no
    recompute), and the gradients match the oracle."""
    import torch
    import oracle
    if case == "train_two_rows":
        cfg = synth.get_config("train_l512_m512", batch=2)
        use_rk = False
    else:
        cfg = synth.Config("bwd_saved_nomem", 2, 128, 2, 64, 96, 0, 1, 1, "bf16", 0.05, 57)
        use_rk = True
    log(f"[case] backward from saved state {case}")
    wl = synth.make_workload(cfg, n_segments=1)
    c = cfg
    H, dh, L, M, B = c.n_heads, c.d_head, c.seg_len, c.mem_len, c.batch
    P = M + L
    rng = np.random.default_rng(11)
    G = synth.round_to(rng.normal(0.0, 1.0, (B, L, H * dh)), "bf16")
    dl = DeviceLayers(wl)
    shp = dl.shape()
    w = dl.W[0]
    Rk_host = synth.round_to(rng.normal(0.0, 0.5, (P, H, dh)), "bf16") if use_rk else None
    Rk = to_dev(Rk_host, "bf16") if use_rk else None
    h = to_dev(wl.segments[0], "bf16")
    mem = dl.mem[0] if M else None
    W_kR = None if use_rk else w["W_kR"]
    R = None if use_rk else dl.R
    f32 = dict(dtype=torch.float32, device="cuda")

    def grads():
        return [nan_empty((B, L, H, dh), **f32), nan_empty((B, P, H, dh), **f32),
                nan_empty((B, P, H, dh), **f32), nan_empty((H, dh), **f32),
                nan_empty((H, dh), **f32), nan_empty((P, H, dh), **f32),
                None if use_rk else nan_empty((H * dh, c.d_pos), **f32)]
    g_ref, g_sav = grads(), grads()
    dG = to_dev(G, "bf16")
    ws_ref = workspace(txl.txl_rel_attn_bwd_workspace_bytes(shp))
    txl.txl_rel_attn_bwd(shp, h, mem, 0, w["W_q"], w["W_kE"], W_kR, w["W_v"], dl.u, dl.v, R, Rk,
                         dG, *g_ref, ws_ref)
    out_ref = nan_empty((B, L, H, dh), dtype=torch.bfloat16, device="cuda")
    ws_f = workspace(txl.txl_rel_attn_workspace_bytes(shp))
    txl.txl_rel_attn_fwd(shp, h, mem, 0, w["W_q"], w["W_kE"], W_kR, w["W_v"], dl.u, dl.v, R, Rk,
                         out_ref, ws_f)
    out = torch.full_like(out_ref, float("nan"))
    ws = workspace(txl.txl_rel_attn_bwd_workspace_bytes(shp))
    txl.txl_rel_attn_fwd_train(shp, h, mem, 0, w["W_q"], w["W_kE"], W_kR, w["W_v"], dl.u, dl.v,
                               R, Rk, out, ws)
    txl.txl_rel_attn_bwd_saved(shp, dl.u, dl.v, R, use_rk, out, dG, *g_sav, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref), "forward output differs from txl_rel_attn_fwd"
    names = ["d_q", "d_k", "d_val", "d_u", "d_v", "d_Rk", "d_W_kR"]
    for n, a, b in zip(names, g_sav, g_ref):
        if a is not None:
            assert torch.equal(a, b), f"{n} differs from txl_rel_attn_bwd"
    lay = wl.layers[0]
    want = oracle.backward.rel_attn_bwd(wl.segments[0][:1], wl.mem[0][:1], lay.W_q, lay.W_kE,
                                        lay.W_kR, lay.W_v, wl.u, wl.v,
                                        oracle.sinusoid(P, c.d_pos), H, dh, 1.0 / np.sqrt(dh),
                                        G[:1], Rk=Rk_host)
    assert_close(from_dev(g_sav[0])[:1], want["q"], "bf16", "d_q")
    assert_close(from_dev(g_sav[1])[:1], want["k"], "bf16", "d_k")
    assert_close(from_dev(g_sav[2])[:1], want["val"], "bf16", "d_val")
