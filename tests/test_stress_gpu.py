"""GPU parity in the regimes the near-uniform workloads do not reach.

* Peaked softmax (Sec. 3.3 Masked-Softmax): the eval-shaped layer with weights
  N(0, 0.1), where the maxima of later key blocks exceed earlier ones by more
  than the kernel's lazy-rescale threshold.
* A bf16 case with the literal scale 1 whose first key block scores below
  -128 in base-2 units (the first reference maximum of a fresh split) and whose
  every later block raises the maximum by more than the threshold.
* The memory-less window of the vanilla model that Sec. 3.1 evaluates and
  Table 9 times: full layers with M = 0 at window lengths 800 and 1800.

The kernel's online softmax works in base 2 and moves its reference maximum
only when a 32-key block's maximum exceeds it by more than 8; before the first
visible key of a key range the first block's maximum becomes the reference.
`_lazy_rescales` replays that rule on the oracle's scores (CPU) to show the
rescale branch is taken by these inputs.
Tolerances: max|gpu - oracle| <= 2e-2 * max|oracle| (bf16), except in the
peaked eval-shaped case.  There the logits have a spread of about 10 (natural
units) and rounding the matrix-core operands (q+u, q+v, K, V, Rk, P) to bf16
moves the exact answer by more than 2e-2 for any bf16 kernel.  That case's
tolerance is the larger of 2e-2 and 1.25 S, with S the oracle's own
sensitivity: the largest relative change of the fp64 oracle output over three
random elementwise perturbations of W_q, W_kE, W_kR and W_v by 1 + U(-2^-8,
2^-8) (two bf16 roundings of a product's operands), per segment; the 25 %
covers the spread of a maximum over 262,144 outputs between two rounding
patterns.  A CPU model that rounds exactly the kernel's operands to bf16 gives
2.5e-2 on segment 0 of this case; S is 4.9e-2 and 5.1e-2 on its two segments.
"""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import (TOL, DeviceLayers, assert_close, from_dev, log, rel_err,
                         run_attn_stream, to_dev, workspace)

pytestmark = pytest.mark.gpu

THRESH = 8.0   # base-2 units


@pytest.fixture(scope="module")
def txl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_xl_relative_attn_amd as mod
    return mod


def _n_split(B, H, L, M):
    """The library's key-range split count for a bf16 layer (two workgroup
    slots per compute unit, every split >= 4 key blocks, at most 16)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = B * H * ((L + 127) // 128)
    nb_min = (M + min(L, 128) + 31) // 32
    return max(1, min(2 * cus // wgs, 16, max(1, nb_min // 4)))


def _lazy_rescales(terms, scale, M, L, n_split):
    """Replay the lazy reference-maximum rule on the oracle's scores for query
    group 0 (queries < 128).  Returns (rescales of a non-empty accumulator,
    fresh starts whose block maximum is below -128)."""
    s = terms["ac"] + terms["bd"] + terms["cc"] + terms["dd"]       # [B, H, L, M+L]
    Lq = min(L, 128)
    n = M + L
    vis = np.arange(n)[None, :] <= M + np.arange(L)[:, None]
    s2 = np.where(vis, s * scale * math.log2(math.e), -np.inf)[:, :, :Lq]
    nb = (M + Lq + 31) // 32
    pad = nb * 32 - n
    if pad > 0:
        s2 = np.concatenate([s2, np.full(s2.shape[:-1] + (pad,), -np.inf)], axis=-1)
    bmax = s2[..., :nb * 32].reshape(s2.shape[:-1] + (nb, 32)).max(-1)   # [B, H, Lq, nb]
    rescales = deep = 0
    for sp in range(n_split):
        lo, hi = sp * nb // n_split, (sp + 1) * nb // n_split
        ref = np.full(bmax.shape[:-1], -np.inf)
        fresh = np.ones(bmax.shape[:-1], bool)
        for t in range(lo, hi):
            mb = bmax[..., t]
            first = fresh & (mb > -np.inf)
            deep += int(np.sum(first & (mb < -128.0)))
            up = ~fresh & (mb > ref + THRESH)
            rescales += int(np.sum(up))
            ref = np.where(first | up, mb, ref)
            fresh &= ~first
    return rescales, deep


def _bf16_sensitivity(x, mem_log, wl, R, scale, seeds=(20190109, 2019, 109)):
    """Largest relative change of the oracle's output for segment input x over
    `seeds` perturbations of the four projection weights by 1 + U(-2^-8, 2^-8)
    elementwise."""
    import oracle
    c = wl.cfg
    lay = wl.layers[0]
    args = (wl.u, wl.v, R, c.n_heads, c.d_head, scale)
    base = oracle.rel_attn_fwd(x, mem_log, lay.W_q, lay.W_kE, lay.W_kR, lay.W_v, *args)
    worst = 0.0
    for seed in seeds:
        rng = np.random.default_rng(seed)

        def pert(W):
            return W * (1.0 + rng.uniform(-2.0 ** -8, 2.0 ** -8, W.shape))

        moved = oracle.rel_attn_fwd(x, mem_log, pert(lay.W_q), pert(lay.W_kE), pert(lay.W_kR),
                                    pert(lay.W_v), *args)
        worst = max(worst, rel_err(moved, base))
    return worst


def test_peaked_softmax_eval_shape(txl):
    """Eval-shaped layer (d_model 1024, 16 heads of 64, segment 128, memory
    1600, scale 1/sqrt(d_head)) at 2 batch rows with weights and u, v
    ~ N(0, 0.1), two segments."""
    import oracle
    cfg = synth.get_config("eval_l128_m1600", batch=2, w_std=0.1, seed=4101)
    log("[case] peaked softmax eval shape, w_std 0.1")
    wl = synth.make_workload(cfg, n_segments=2)
    outs, _, _ = run_attn_stream(wl, 2)
    sc = 1.0 / math.sqrt(cfg.d_head)
    R = oracle.sinusoid(cfg.n_pos, cfg.d_pos)
    mem = wl.mem[0]
    start = 0
    for s in range(2):
        mem_log = oracle.logical_memory(mem, start)
        sens = _bf16_sensitivity(wl.segments[s], mem_log, wl, R, sc)
        tol = max(TOL["bf16"], 1.25 * sens)
        log(f"  segment {s}: oracle sensitivity to bf16-sized weight perturbations {sens:.3e}")
        want, terms = oracle.rel_attn_fwd(wl.segments[s], mem_log,
                                          wl.layers[0].W_q, wl.layers[0].W_kE,
                                          wl.layers[0].W_kR, wl.layers[0].W_v, wl.u, wl.v, R,
                                          cfg.n_heads, cfg.d_head, sc, return_terms=True)
        if s == 0:
            ns = _n_split(cfg.batch, cfg.n_heads, cfg.seg_len, cfg.mem_len)
            resc, _ = _lazy_rescales(terms, sc, cfg.mem_len, cfg.seg_len, ns)
            log(f"  {ns} key splits; lazy-rule rescales of segment 0 (replayed on the CPU): {resc}")
            assert resc > 0
        del terms
        err = rel_err(outs[s], want)
        log(f"  segment {s}: max|gpu-oracle|/max|oracle| = {err:.3e} (tol {tol:.3e})")
        assert np.all(np.isfinite(outs[s])) and err <= tol
        mem, start = oracle.mem_update(mem, start, wl.segments[s])


def test_rescale_from_very_negative_first_block(txl):
    """scale = 1 on the bf16 path.  W_q = 0 and every row of [memory ; segment]
    carries a component along g = W_kE^T u sized so that u.k_j (term (c)) equals
    a per-block level beta: -200 for keys 0..31, then -100, -40, -20, -8, 0, 6
    and 12.  A fresh key range starting at block 0 meets a block maximum below
    -128 in base-2 units, and every later block raises the maximum by more than
    8 (the rescale of a non-empty accumulator)."""
    import torch
    import oracle
    B, d, H, dh, L, M = 2, 64, 1, 64, 32, 224
    cfg = synth.Config("ramp", B, d, H, dh, L, M, 1, 1, "bf16", 0.05, 9001)
    wl = synth.make_workload(cfg, n_segments=1)
    lay = wl.layers[0]
    lay.W_q = np.zeros_like(lay.W_q)
    g = lay.W_kE.T @ wl.u[0]
    levels = np.array([-200.0, -100.0, -40.0, -20.0, -8.0, 0.0, 6.0, 12.0])
    beta = levels[np.arange(M + L) // 32]
    ext = np.concatenate([wl.mem[0], wl.segments[0]], axis=1)
    ext = synth.round_to(ext + beta[None, :, None] * (g / (g @ g))[None, None, :], "bf16")
    wl.mem[0] = ext[:, :M].copy()
    wl.segments[0] = ext[:, M:].copy()
    log("[case] bf16 scale 1, very negative first block, ramped block maxima")
    outs, _, _ = run_attn_stream(wl, 1, scale=1.0)
    R = oracle.sinusoid(M + L, d)
    want, terms = oracle.rel_attn_fwd(wl.segments[0], wl.mem[0], lay.W_q, lay.W_kE, lay.W_kR,
                                      lay.W_v, wl.u, wl.v, R, H, dh, 1.0, return_terms=True)
    ns = _n_split(B, H, L, M)
    resc, deep = _lazy_rescales(terms, 1.0, M, L, ns)
    log(f"  {ns} key splits; fresh starts below -128: {deep}; rescales: {resc}")
    assert deep > 0 and resc > 0
    assert_close(outs[0], want, "bf16", "segment 0")
    _ = torch


@pytest.mark.parametrize("L,n_layers", [(800, 3), (1800, 2)], ids=["window800", "window1800"])
def test_vanilla_window_stack(txl, L, n_layers):
    """Sec. 3.1's vanilla evaluation runs a whole window from scratch: full
    layers (W_o, LayerNorm, ReLU feed-forward of width 4096) with no memory,
    d_model 1024, 16 heads of 64, one batch row; the shape Table 9 times."""
    import torch
    import oracle
    cfg = synth.Config(f"vanilla{L}", 1, 1024, 16, 64, L, 0, n_layers, 1, "bf16", 0.02,
                       3100 + L, d_inner=4096)
    log(f"[case] vanilla window L={L}, {n_layers} full layers, M=0")
    wl = synth.make_workload(cfg)
    dl = DeviceLayers(wl)
    shp = dl.shape()
    ws = workspace(txl.txl_segment_workspace_bytes(shp, n_layers, cfg.d_inner))
    h = to_dev(wl.segments[0], "bf16")
    out = torch.full_like(h, float("nan"))
    start = txl.txl_segment_step(shp, n_layers, cfg.d_inner, dl.layer_structs(), dl.R, h, out, 0,
                                 ws)
    torch.cuda.synchronize()
    assert start == 0
    R = oracle.sinusoid(L, cfg.d_pos)
    log("  oracle")
    want, _, _, per_layer = oracle.segment_step(wl.segments[0], wl.layers, wl.mem, 0, wl.u, wl.v,
                                                R, cfg.n_heads, cfg.d_head)
    assert_close(from_dev(out), want, "bf16", f"window {L}")
