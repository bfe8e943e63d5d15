"""GPU parity of the carried projected-K/V ring (txl_kv_ring_init +
txl_rel_attn_fwd_kv) against the CPU oracle, which keeps the hidden-state
memory and recomputes keys and values from [memory ; segment] every segment
(Sec. 3.3).  Tolerance as for the bf16 path: max|gpu - oracle| <=
2e-2 * max|oracle|.  Where the memory length is a multiple of 32 the ring step
runs the same attention blocks as txl_rel_attn_fwd, and the two outputs must
agree bit for bit."""
import numpy as np
import pytest

import synth
from gpu_helpers import (DeviceLayers, assert_close, from_dev, log, oracle_stream,
                         nan_empty, run_attn_stream, tdtype, to_dev, txl_dtype, workspace)
from oracle_pool import oracle_stream_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def txl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_xl_relative_attn_amd as mod
    return mod


def run_ring_stream(wl, n_seg, mem_start=0, use_rk=False):
    """Stream n_seg segments through the K/V ring (single layer).  Returns the
    outputs per segment (float64) and the ring starts seen."""
    import torch
    import transformer_xl_relative_attn_amd as txl
    c = wl.cfg
    dl = DeviceLayers(wl)
    mem = dl.mem[0] if c.mem_len else None
    if mem_start and c.mem_len:
        mem = torch.roll(mem, shifts=mem_start, dims=1).contiguous()
    shp = dl.shape()
    ring = workspace(txl.txl_kv_ring_bytes(shp))
    ws = workspace(txl.txl_kv_ring_workspace_bytes(shp))
    w = dl.W[0]
    Rk = None
    if use_rk:
        Rk = nan_empty((c.n_pos, c.n_heads, c.d_head), dtype=tdtype(c.dtype), device="cuda")
        pws = workspace(txl.txl_rel_proj_workspace_bytes(c.n_pos, c.d_pos, c.n_heads, c.d_head,
                                                         txl_dtype(c.dtype)))
        txl.txl_rel_proj(dl.R, w["W_kR"], Rk, c.n_pos, c.d_pos, c.n_heads, c.d_head,
                         txl_dtype(c.dtype), pws)
    start = txl.txl_kv_ring_init(shp, mem, mem_start, w["W_kE"], w["W_v"], ring, ws)
    assert start == 0
    C = txl.txl_kv_ring_slots(shp)
    outs, starts = [], []
    for s in range(n_seg):
        h = to_dev(wl.segments[s], c.dtype)
        out = nan_empty((c.batch, c.seg_len, c.n_heads * c.d_head), dtype=tdtype(c.dtype),
                          device="cuda")
        starts.append(start)
        new = txl.txl_rel_attn_fwd_kv(shp, h, w["W_q"], w["W_kE"], w["W_kR"], w["W_v"], dl.u,
                                      dl.v, dl.R, Rk, ring, start, out, ws)
        assert new == (start + c.seg_len) % C
        start = new
        torch.cuda.synchronize()
        outs.append(from_dev(out))
    return outs, starts


def _ring_case(txl, cfg, n_seg, b_idx, mem_start=0, use_rk=False, bitwise_vs_plain=False):
    log(f"[case] kv-ring {cfg.name} B={cfg.batch} L={cfg.seg_len} M={cfg.mem_len} "
        f"H={cfg.n_heads} dh={cfg.d_head} d={cfg.d_model} segs={n_seg} mem_start={mem_start} "
        f"rk={use_rk}")
    wl = synth.make_workload(cfg, n_segments=n_seg)
    outs, starts = run_ring_stream(wl, n_seg, mem_start=mem_start, use_rk=use_rk)
    log(f"  ring starts {starts}")
    o_outs, _, _ = oracle_stream(wl, n_seg, b_idx)
    for s in range(n_seg):
        assert_close(outs[s][b_idx], o_outs[s], cfg.dtype, f"segment {s}")
    if bitwise_vs_plain:
        plain, _, _ = run_attn_stream(wl, n_seg)
        for s in range(n_seg):
            assert np.array_equal(outs[s], plain[s]), f"segment {s}: ring != plain path"
    return starts


def test_ring_eval_shaped(txl):
    """Eval-shaped layer (memory 1600 = 50 tiles): parity with the oracle over 4
    segments, and bit-identical to the hidden-state path."""
    cfg = synth.get_config("eval_l128_m1600")
    _ring_case(txl, cfg, 4, np.array([0, 5]), bitwise_vs_plain=True)


def test_ring_eval_cached_rk(txl):
    cfg = synth.get_config("eval_l128_m1600", batch=2)
    _ring_case(txl, cfg, 2, np.array([1]), use_rk=True)


def test_ring_ghost_keys_odd_head(txl):
    """Memory 150 (10 ghost slots), d_model 410 (rows repacked), d_head 41."""
    cfg = synth.Config("ring_odd", 2, 410, 10, 41, 64, 150, 1, 3, "bf16", 0.02, 1002)
    _ring_case(txl, cfg, 3, np.arange(2))


def test_ring_wraps(txl):
    """C = 96 + 64 = 160 slots: the fourth segment's rows wrap around the ring."""
    cfg = synth.Config("ring_wrap", 2, 128, 2, 64, 64, 70, 1, 3, "bf16", 0.05, 31)
    starts = _ring_case(txl, cfg, 5, np.arange(2))
    assert any((s + 96) % 160 + 64 > 160 for s in starts), starts


def test_ring_rotated_hidden_memory(txl):
    """The initial projection reads the hidden-state ring through mem_start."""
    cfg = synth.Config("ring_rot", 2, 128, 2, 64, 32, 100, 1, 3, "bf16", 0.05, 99)
    _ring_case(txl, cfg, 3, np.arange(2), mem_start=37)


@pytest.mark.parametrize("case", [
    ("no_memory", 2, 128, 2, 64, 64, 0),
    ("L_gt_M", 2, 128, 2, 64, 96, 20),
    ("many_splits", 1, 64, 1, 64, 32, 3000),
    ("two_groups", 1, 64, 2, 32, 256, 33),
], ids=lambda c: c[0])
def test_ring_edges(txl, case):
    name, B, d, H, dh, L, M = case
    cfg = synth.Config(name, B, d, H, dh, L, M, 1, 3, "bf16", 0.05, 4242)
    _ring_case(txl, cfg, 3, np.arange(B))


def run_segment_ring_stream(wl, n_seg):
    """Stream n_seg segments through txl_segment_step_kv (rings initialised from
    each layer's memory).  Returns the outputs per segment (float64)."""
    import torch
    import transformer_xl_relative_attn_amd as txl
    c = wl.cfg
    dl = DeviceLayers(wl)
    shp = dl.shape()
    ws = workspace(txl.txl_segment_kv_workspace_bytes(shp, c.n_layers, c.d_inner))
    rings = []
    for n, w in enumerate(dl.W):
        ring = workspace(txl.txl_kv_ring_bytes(shp))
        assert txl.txl_kv_ring_init(shp, dl.mem[n] if c.mem_len else None, 0, w["W_kE"],
                                    w["W_v"], ring, ws) == 0
        rings.append(ring)
    layers = dl.layer_structs()
    d_out = c.d_model if c.d_inner else c.n_heads * c.d_head
    start, outs = 0, []
    for s in range(n_seg):
        h = to_dev(wl.segments[s], c.dtype)
        out = nan_empty((c.batch, c.seg_len, d_out), dtype=tdtype(c.dtype), device="cuda")
        start = txl.txl_segment_step_kv(shp, c.n_layers, c.d_inner, layers, rings, dl.R, h, out,
                                        start, ws)
        torch.cuda.synchronize()
        outs.append(from_dev(out))
    return outs


def test_segment_ring_small_stack(txl):
    """Two full layers (W_o, LayerNorm, ReLU FFN), memory 72 (24 ghost slots)."""
    cfg = synth.Config("ring_stack2", 2, 128, 2, 64, 32, 72, 2, 3, "bf16", 0.02, 1234,
                       d_inner=256)
    log("[case] kv-ring small stack")
    wl = synth.make_workload(cfg)
    outs = run_segment_ring_stream(wl, 3)
    b_idx = np.arange(2)
    o_outs, _, _ = oracle_stream(wl, 3, b_idx)
    for s in range(3):
        assert_close(outs[s][b_idx], o_outs[s], "bf16", f"segment {s}")


def test_segment_ring_matches_hidden_state_step(txl):
    """Memory a multiple of 32: the ring step equals txl_segment_step bit for bit."""
    from gpu_helpers import run_segment_stream
    cfg = synth.Config("ring_stack_eq", 2, 128, 2, 64, 64, 96, 2, 3, "bf16", 0.02, 555,
                       d_inner=256)
    log("[case] kv-ring stack vs hidden-state stack")
    wl = synth.make_workload(cfg)
    ring_outs = run_segment_ring_stream(wl, 3)
    plain, _, _ = run_segment_stream(wl, 3)
    for s in range(3):
        assert np.array_equal(ring_outs[s], plain[s]), f"segment {s}"


def test_segment_ring_stack_16_layers(txl):
    """16-layer stack with the 3,800-state memory (8 ghost slots per ring)."""
    cfg = synth.get_config("stack16_l128_m3800")
    log("[case] kv-ring 16-layer stack, 4 segments")
    wl = synth.make_workload(cfg)
    outs = run_segment_ring_stream(wl, 4)
    b_idx = np.arange(cfg.batch)
    log(f"  oracle on {cfg.batch} rows in worker processes")
    o_outs, _, _, _ = oracle_stream_rows(cfg, 4, b_idx, chunk=1)
    for s in range(4):
        assert_close(outs[s][b_idx], o_outs[s], "bf16", f"segment {s}")
