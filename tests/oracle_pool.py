"""Run the CPU oracle over batch rows in worker processes (test infrastructure).

Batch rows never mix in the method (test_oracle.test_batch_independence pins
this for the oracle), so a full-batch oracle result is the concatenation of
per-row results, and batch-summed gradients are sums of per-row gradients.
Workers are started with the "spawn" method: each is a fresh interpreter that
imports only numpy, synth and the oracle (never torch or the GPU library) and
regenerates its inputs from the seeded workload configuration.
"""
from __future__ import annotations

import multiprocessing
import os

import numpy as np

import synth


def _workers(n_items: int, cap: int = 8) -> int:
    return max(1, min(cap, n_items, len(os.sched_getaffinity(0))))


def _pool_map(fn, jobs, cap=8, threads=2):
    """Map fn over jobs in spawned workers with `threads` BLAS threads each."""
    if len(jobs) == 1:
        return [fn(*jobs[0])]
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    for k in keys:
        os.environ[k] = str(threads)
    try:
        ctx = multiprocessing.get_context("spawn")
        with ctx.Pool(_workers(len(jobs), cap)) as pool:
            return pool.starmap(fn, jobs)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


# ------------------------------------------------------------ forward stream
def _fwd_rows(cfg, n_seg, rows, scale):
    import oracle
    wl = synth.make_workload(cfg, n_segments=n_seg)
    R = oracle.sinusoid(cfg.n_pos, cfg.d_pos)
    mems = [m[rows] for m in wl.mem]
    start = 0
    outs, layer_outs = [], []
    for s in range(n_seg):
        y, mems, start, per_layer = oracle.segment_step(wl.segments[s][rows], wl.layers, mems,
                                                        start, wl.u, wl.v, R, cfg.n_heads,
                                                        cfg.d_head, scale)
        outs.append(y)
        layer_outs.append(per_layer)
    return outs, layer_outs, mems, start


def oracle_stream_rows(cfg, n_seg, b_idx=None, scale=None, chunk=None, cap=8):
    """oracle.segment_step over n_seg segments for the batch rows b_idx (all
    by default), split into row chunks run in parallel.  Returns (outputs per
    segment [rows, L, d_out], per-layer outputs per segment, final physical
    rings per layer (ring start 0 at the first segment), final start)."""
    b_idx = np.arange(cfg.batch) if b_idx is None else np.asarray(b_idx)
    if chunk is None:
        chunk = max(1, -(-len(b_idx) // _workers(len(b_idx), cap)))
    parts = [b_idx[i:i + chunk] for i in range(0, len(b_idx), chunk)]
    res = _pool_map(_fwd_rows, [(cfg, n_seg, p, scale) for p in parts], cap)
    outs = [np.concatenate([r[0][s] for r in res]) for s in range(n_seg)]
    layer_outs = [[np.concatenate([r[1][s][n] for r in res]) for n in range(cfg.n_layers)]
                  for s in range(n_seg)]
    mems = [np.concatenate([r[2][n] for r in res]) for n in range(cfg.n_layers)]
    return outs, layer_outs, mems, res[0][3]


# ------------------------------------------------------------------ backward
def _bwd_rows(cfg, rows, g_seed, rk_seed_std):
    import oracle
    wl = synth.make_workload(cfg, n_segments=1)
    c = cfg
    H, dh, L, M, B = c.n_heads, c.d_head, c.seg_len, c.mem_len, c.batch
    rng = np.random.default_rng(g_seed)
    G = synth.round_to(rng.normal(0.0, 1.0, (B, L, H * dh)), "bf16")
    Rk = None
    if rk_seed_std:
        Rk = synth.round_to(rng.normal(0.0, rk_seed_std, (M + L, H, dh)), "bf16")
    lay = wl.layers[0]
    return oracle.backward.rel_attn_bwd(wl.segments[0][rows], wl.mem[0][rows], lay.W_q,
                                        lay.W_kE, lay.W_kR, lay.W_v, wl.u, wl.v,
                                        oracle.sinusoid(M + L, c.d_pos), H, dh,
                                        1.0 / np.sqrt(dh), G[rows], Rk=Rk)


def oracle_bwd_rows(cfg, g_seed, rk_std=0.0, cap=8):
    """oracle.backward.rel_attn_bwd over every batch row of cfg, one row per
    job; per-row gradients are concatenated, batch-summed ones added in row
    order.  The output gradient G and (if rk_std) the caller's position keys
    are drawn exactly as the backward tests draw them."""
    jobs = [(cfg, np.array([b]), g_seed, rk_std) for b in range(cfg.batch)]
    res = _pool_map(_bwd_rows, jobs, cap, threads=1)
    out = {}
    for key in res[0]:
        if key in ("q", "k", "val"):
            out[key] = np.concatenate([r[key] for r in res])
        else:
            acc = np.zeros_like(res[0][key])
            for r in res:
                acc = acc + r[key]
            out[key] = acc
    return out
