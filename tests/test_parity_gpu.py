"""GPU parity: libtxl (through its C entry points) against the CPU oracle.

Tolerances: max|gpu - oracle| <= 1e-4 * max|oracle| on the fp32 path and
<= 2e-2 * max|oracle| on the bf16-in / fp32-accumulate path.  Memory rings
after an update are compared bit for bit (they are copies of the inputs).
Every workload is compared on all of its batch rows; the larger ones run the
oracle's rows in parallel worker processes (rows never mix, see
test_oracle.test_batch_independence).
"""
import numpy as np
import pytest

import synth
from gpu_helpers import (DeviceLayers, TOL, assert_close, bf16_bits_of, from_dev, log,
                         oracle_stream, run_attn_stream, run_segment_stream, tdtype, to_dev,
                         txl_dtype, nan_empty, workspace)
from oracle_pool import oracle_stream_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def txl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_xl_relative_attn_amd as mod
    return mod


def _check_ring(dl, wl, mems_oracle, start_o, start_g, b_idx, layer=0, exact=True):
    import oracle
    assert start_g == start_o
    c = wl.cfg
    if not c.mem_len:
        return
    if c.dtype == "bf16":
        got_bits = bf16_bits_of(dl.mem[layer][b_idx])
        want_bits = synth.bf16_bits(mems_oracle[layer])
        if exact:
            assert np.array_equal(got_bits, want_bits), "memory ring differs"
        else:
            got = synth.bits_to_f64(got_bits)
            assert_close(got, mems_oracle[layer], "bf16", f"ring layer {layer}")
    else:
        got = from_dev(dl.mem[layer][b_idx])
        if exact:
            assert np.array_equal(got, mems_oracle[layer].astype(np.float32).astype(np.float64))
        else:
            assert_close(got, mems_oracle[layer], "f32", f"ring layer {layer}")
    _ = oracle


# ------------------------------------------------------------------ R / Rk
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sinusoid(txl, dtype):
    import torch
    import oracle
    n, d = 3928, 1024
    R = nan_empty((n, d), dtype=tdtype(dtype), device="cuda")
    txl.txl_sinusoid_pos(R, n, d, txl_dtype(dtype))
    torch.cuda.synchronize()
    want = oracle.sinusoid(n, d)
    got = from_dev(R)
    if dtype == "f32":
        assert np.max(np.abs(got - want)) <= 1e-7
    else:
        # One rounding of the fp64 value to the nearest bf16 (ties to even),
        # computed here exactly in float64: the two bf16 neighbours of x and
        # their midpoint are exact float64 numbers.  Values within 1e-9 of a
        # midpoint are exempt (fp64 sin/cos may differ in the last bits).
        lo = _bf16_toward_zero(want)
        ulp = _bf16_ulp(lo)
        hi = lo + np.sign(want) * ulp
        mid = (lo + hi) / 2
        away = np.abs(want) > np.abs(mid)
        tie = want == mid
        lo_even = (synth.bf16_bits(lo) & 1) == 0
        rne = np.where(away | (tie & ~lo_even), hi, lo)
        ambiguous = np.abs(want - mid) <= 1e-9 * np.abs(want)
        bad = (got != rne) & ~ambiguous
        assert not np.any(bad), f"{np.sum(bad)} values not correctly rounded"
        assert np.all(np.abs(got - want) <= ulp / 2 + 1e-300)


def _bf16_toward_zero(x):
    """Largest-magnitude bf16 value not above |x| in magnitude (normal range)."""
    bits = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    sign = bits >> np.uint64(63)
    exp = (bits >> np.uint64(52)) & np.uint64(0x7FF)
    man = (bits >> np.uint64(45)) & np.uint64(0x7F)          # top 7 fraction bits
    val = (1.0 + man.astype(np.float64) / 128.0) * np.exp2(exp.astype(np.float64) - 1023.0)
    val = np.where(exp == 0, 0.0, val)
    return np.where(sign == 1, -val, val)


def _bf16_ulp(v):
    """Spacing of bf16 numbers at the (normal, nonzero) bf16 value v."""
    e = np.floor(np.log2(np.where(v == 0, 1.0, np.abs(v))))
    return np.where(v == 0, 2.0 ** -133, np.exp2(e - 7))


@pytest.mark.parametrize("dtype,n_pos,d_pos,H,dh", [
    ("f32", 16, 16, 1, 16), ("bf16", 300, 410, 10, 41), ("bf16", 1728, 1024, 16, 64),
    ("bf16", 77, 128, 3, 24)])
def test_rel_proj(txl, dtype, n_pos, d_pos, H, dh):
    import torch
    import oracle
    rng = np.random.default_rng(5)
    W = synth.round_to(rng.normal(0, 0.02, (H * dh, d_pos)), dtype)
    Rw = oracle.sinusoid(n_pos, d_pos)
    R = to_dev(synth.round_to(Rw, dtype), dtype)
    Rk = nan_empty((n_pos, H, dh), dtype=tdtype(dtype), device="cuda")
    ws = workspace(txl.txl_rel_proj_workspace_bytes(n_pos, d_pos, H, dh, txl_dtype(dtype)))
    txl.txl_rel_proj(R, to_dev(W, dtype), Rk, n_pos, d_pos, H, dh, txl_dtype(dtype), ws)
    torch.cuda.synchronize()
    want = oracle.rel_proj(synth.round_to(Rw, dtype), W, H, dh)
    assert_close(from_dev(Rk), want, dtype, f"Rk {n_pos}x{d_pos}")


# --------------------------------------------------- single layer workloads
def _stream_case(txl, cfg, n_seg, b_idx, start=0, use_rk=False, scale=0.0, parallel=False):
    log(f"[case] {cfg.name} B={cfg.batch} L={cfg.seg_len} M={cfg.mem_len} H={cfg.n_heads} "
        f"dh={cfg.d_head} d={cfg.d_model} {cfg.dtype} segs={n_seg} start={start} rk={use_rk}")
    wl = synth.make_workload(cfg, n_segments=n_seg)
    outs, dl, start_g = run_attn_stream(wl, n_seg, scale=scale, start=start, use_rk=use_rk)
    # the oracle sees the same logical memory (with a rotated GPU ring too); its
    # own ring starts at 0
    if parallel:
        log(f"  oracle on {len(b_idx)} rows in worker processes")
        o_outs, _, o_mems, start_o = oracle_stream_rows(cfg, n_seg, b_idx,
                                                        scale if scale > 0 else None)
    else:
        o_outs, o_mems, start_o = oracle_stream(wl, n_seg, b_idx, scale if scale > 0 else None)
    for s in range(n_seg):
        assert_close(outs[s][b_idx], o_outs[s], cfg.dtype, f"segment {s}")
    if not start:
        _check_ring(dl, wl, o_mems, start_o, start_g, b_idx)
    return outs


def test_tiny_fp32_two_segments(txl):
    cfg = synth.get_config("tiny_f32")
    _stream_case(txl, cfg, 2, np.arange(cfg.batch))


def test_odd_head_dim(txl):
    cfg = synth.get_config("odd_head41")
    _stream_case(txl, cfg, 1, np.arange(cfg.batch), parallel=True)


def test_train_shaped(txl):
    cfg = synth.get_config("train_l512_m512")
    _stream_case(txl, cfg, 4, np.arange(cfg.batch), parallel=True)


def test_eval_shaped(txl):
    cfg = synth.get_config("eval_l128_m1600")
    _stream_case(txl, cfg, 8, np.arange(cfg.batch), parallel=True)


def test_eval_with_cached_rk(txl):
    cfg = synth.get_config("eval_l128_m1600")
    _stream_case(txl, cfg, 2, np.array([3]), use_rk=True)


def test_fp32_path_odd_head_shape(txl):
    cfg = synth.get_config("odd_head41", dtype="f32", batch=2)
    _stream_case(txl, cfg, 2, np.array([0, 1]))


def test_literal_scale_one(txl):
    """scale = 1 (the summary equations applied literally)."""
    cfg = synth.get_config("tiny_f32", seed=77)
    _stream_case(txl, cfg, 2, np.arange(cfg.batch), scale=1.0)


# ------------------------------------------------------------------ edges
EDGE = [
    # (name, B, d, H, dh, L, M, dtype)
    ("no_memory", 2, 128, 2, 64, 70, 0, "bf16"),
    ("L_gt_M", 2, 128, 2, 64, 100, 40, "bf16"),
    ("L_eq_1", 3, 64, 1, 64, 1, 200, "bf16"),
    ("ragged_pack", 2, 96, 3, 24, 37, 45, "bf16"),
    ("many_splits", 1, 64, 1, 64, 33, 3000, "bf16"),
    ("L_257", 1, 64, 1, 32, 257, 31, "bf16"),
    ("fp32_ragged", 2, 24, 3, 8, 13, 7, "f32"),
    ("fp32_no_memory", 1, 16, 2, 8, 9, 0, "f32"),
]


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(txl, case):
    name, B, d, H, dh, L, M, dtype = case
    w = 0.1 if dtype == "f32" else 0.05
    cfg = synth.Config(name, B, d, H, dh, L, M, 1, 3, dtype, w, 4242)
    _stream_case(txl, cfg, 3, np.arange(B))


def test_ring_start_rotation(txl):
    """A rotated physical ring (mem_start != 0) holding the same logical memory
    gives the same result as the oracle on that logical memory."""
    cfg = synth.Config("rot", 2, 128, 2, 64, 24, 100, 1, 3, "bf16", 0.05, 99)
    _stream_case(txl, cfg, 3, np.arange(2), start=37)


def test_deterministic(txl):
    import torch
    cfg = synth.get_config("eval_l128_m1600", batch=2)
    wl = synth.make_workload(cfg, n_segments=1)
    a, _, _ = run_attn_stream(wl, 1)
    b, _, _ = run_attn_stream(wl, 1)
    assert np.array_equal(a[0], b[0])
    _ = torch


# ------------------------------------------------------- segment step
def test_segment_step_single_layer_eval(txl):
    cfg = synth.get_config("eval_l128_m1600")
    log("[case] segment_step eval layer, 8 segments")
    wl = synth.make_workload(cfg, n_segments=8)
    outs, dl, start = run_segment_stream(wl, 8)
    b_idx = np.arange(cfg.batch)
    o_outs, _, o_mems, start_o = oracle_stream_rows(cfg, 8, b_idx)
    for s in range(8):
        assert_close(outs[s][b_idx], o_outs[s], "bf16", f"segment {s}")
    _check_ring(dl, wl, o_mems, start_o, start, b_idx)


@pytest.mark.parametrize("L,M,n_seg", [(150, 150, 3), (40, 100, 4)], ids=["L_ge_M", "L_lt_M_wrap"])
def test_segment_step_packed_rows(txl, L, M, n_seg):
    """d_model 410 (rows repacked to 448 columns, 820-byte rows): the packing
    launch also applies the memory update, so the ring is checked bit for bit
    after every segment, with L >= M and with L < M wrapping around the ring."""
    cfg = synth.Config(f"packed_{L}_{M}", 4 if L >= M else 2, 410, 10, 41, L, M, 1, n_seg, "bf16",
                       0.02, 5150 + L)
    log(f"[case] segment step with packed rows L={L} M={M}")
    wl = synth.make_workload(cfg)
    import torch
    import oracle
    dl = DeviceLayers(wl)
    shp = dl.shape()
    ws = workspace(txl.txl_segment_workspace_bytes(shp, 1, 0))
    layers = dl.layer_structs()
    R = oracle.sinusoid(cfg.n_pos, cfg.d_pos)
    mems = [m.copy() for m in wl.mem]
    start = start_o = 0
    for s in range(n_seg):
        h = to_dev(wl.segments[s], "bf16")
        out = nan_empty((cfg.batch, L, cfg.n_heads * cfg.d_head), dtype=torch.bfloat16,
                          device="cuda")
        start = txl.txl_segment_step(shp, 1, 0, layers, dl.R, h, out, start, ws)
        torch.cuda.synchronize()
        want, mems, start_o, _ = oracle.segment_step(wl.segments[s], wl.layers, mems, start_o,
                                                     wl.u, wl.v, R, cfg.n_heads, cfg.d_head)
        assert_close(from_dev(out), want, "bf16", f"segment {s}")
        assert start == start_o
        assert np.array_equal(bf16_bits_of(dl.mem[0]), synth.bf16_bits(mems[0])), \
            f"segment {s}: memory ring differs"


def test_segment_step_stack_small(txl):
    """Two full layers (W_o, LayerNorm, ReLU FFN) on a small shape."""
    cfg = synth.Config("stack2", 2, 128, 2, 64, 40, 72, 2, 3, "bf16", 0.02, 1234, d_inner=256)
    log("[case] small stack")
    wl = synth.make_workload(cfg)
    outs, dl, start = run_segment_stream(wl, 3)
    b_idx = np.arange(2)
    o_outs, o_mems, start_o = oracle_stream(wl, 3, b_idx)
    for s in range(3):
        assert_close(outs[s][b_idx], o_outs[s], "bf16", f"segment {s}")
    _check_ring(dl, wl, o_mems, start_o, start, b_idx, layer=0, exact=True)
    _check_ring(dl, wl, o_mems, start_o, start, b_idx, layer=1, exact=False)


@pytest.mark.parametrize("d, H, dh", [(50, 2, 25), (64, 2, 32)], ids=["d50_odd_width", "d64"])
def test_segment_step_stack_f32(txl, d, H, dh):
    """Two full fp32 layers: the fp32 GEMM with the ReLU epilogue, no split-K,
    and the LayerNorm on rows of d % 4 != 0 (element path) and d % 4 == 0
    (float4 path, fp32 low copy)."""
    cfg = synth.Config(f"stack2_f32_d{d}", 2, d, H, dh, 12, 20, 2, 3, "f32", 0.05, 77 + d,
                       d_inner=70)
    log(f"[case] fp32 small stack d={d}")
    wl = synth.make_workload(cfg)
    outs, dl, start = run_segment_stream(wl, 3)
    b_idx = np.arange(2)
    o_outs, o_mems, start_o = oracle_stream(wl, 3, b_idx)
    for s in range(3):
        assert_close(outs[s][b_idx], o_outs[s], "f32", f"segment {s}")
    _check_ring(dl, wl, o_mems, start_o, start, b_idx, layer=0, exact=True)
    _check_ring(dl, wl, o_mems, start_o, start, b_idx, layer=1, exact=False)


def test_stack_16_layers(txl):
    """The 16-layer stack over 4 segments, all batch rows, against the oracle.
    Per-layer outputs: the same stream is run a second time one layer per
    txl_segment_step call (fresh memories, the shared ring start passed to each
    layer's call), and every layer's output of that chain is compared with the
    oracle's output of the same layer.  (The chain hands bf16 outputs from call
    to call, while one 16-layer call keeps the LayerNorm output in fp32 for the
    next residual, so the two agree to rounding, not bit for bit.)"""
    import torch
    import transformer_xl_relative_attn_amd as txl_mod
    cfg = synth.get_config("stack16_l128_m3800")
    log("[case] 16-layer stack, 4 segments")
    wl = synth.make_workload(cfg)
    outs, dl, start = run_segment_stream(wl, 4)
    log("  one layer per call")
    dl1 = DeviceLayers(wl)
    shp = dl1.shape()
    ws = workspace(txl_mod.txl_segment_workspace_bytes(shp, 1, cfg.d_inner))
    layers = dl1.layer_structs()
    st = 0
    per_layer = []
    for s in range(4):
        x = to_dev(wl.segments[s], "bf16")
        ys = []
        new_st = st
        for n in range(cfg.n_layers):
            y = torch.full_like(x, float("nan"))
            new_st = txl_mod.txl_segment_step(shp, 1, cfg.d_inner, [layers[n]], dl1.R, x, y, st,
                                              ws)
            ys.append(y)
            x = y
        st = new_st
        torch.cuda.synchronize()
        per_layer.append([from_dev(y) for y in ys])
    assert st == start
    b_idx = np.arange(cfg.batch)
    log(f"  oracle on {cfg.batch} rows in worker processes")
    o_outs, o_layers, o_mems, start_o = oracle_stream_rows(cfg, 4, b_idx, chunk=1)
    for s in range(4):
        for n in range(cfg.n_layers):
            assert_close(per_layer[s][n], o_layers[s][n], "bf16", f"segment {s} layer {n}")
        assert_close(outs[s], o_outs[s], "bf16", f"segment {s}")
        assert_close(per_layer[s][-1], outs[s], "bf16", f"segment {s}: chain vs 16-layer call")
    _check_ring(dl, wl, o_mems, start_o, start, b_idx, layer=0, exact=True)
    for n in range(1, cfg.n_layers):
        _check_ring(dl, wl, o_mems, start_o, start, b_idx, layer=n, exact=False)


def test_segment_step_in_place(txl):
    """h_out may be the same buffer as h_in: the memory must still receive the
    layer input, not the attention output."""
    import torch
    cfg = synth.Config("inplace", 2, 128, 2, 64, 40, 72, 1, 3, "bf16", 0.05, 4321)
    log("[case] in-place segment step")
    wl = synth.make_workload(cfg)
    dl = DeviceLayers(wl)
    shp = dl.shape()
    ws = workspace(txl.txl_segment_workspace_bytes(shp, 1, 0))
    layers = dl.layer_structs()
    start = 0
    outs = []
    for s in range(3):
        h = to_dev(wl.segments[s], "bf16")
        start = txl.txl_segment_step(shp, 1, 0, layers, dl.R, h, h, start, ws)
        torch.cuda.synchronize()
        outs.append(from_dev(h))
    b_idx = np.arange(2)
    o_outs, o_mems, start_o = oracle_stream(wl, 3, b_idx)
    for s in range(3):
        assert_close(outs[s], o_outs[s], "bf16", f"segment {s}")
    _check_ring(dl, wl, o_mems, start_o, start, b_idx)


# ------------------------------------------------- Shaw et al. variant
@pytest.mark.parametrize("path", ["hidden_state", "kv_ring"])
def test_shaw_variant(txl, path):
    """Terms (a) + (b) only with a learned table R_hat (the Shaw et al. form
    compared in Sec. 3.3): u = v = 0 and the caller's Rk = R_hat; W_kR and R are
    not passed.  Eval-shaped layer, 3 segments, through the hidden-state memory
    and through the K/V ring."""
    import torch
    import oracle
    cfg = synth.get_config("eval_l128_m1600", batch=2)
    log(f"[case] Shaw variant via {path}")
    wl = synth.make_workload(cfg, n_segments=3)
    rng = np.random.default_rng(2018)
    n_pos = cfg.mem_len + cfg.seg_len
    R_hat = synth.round_to(rng.normal(0.0, 1.0, (n_pos, cfg.n_heads, cfg.d_head)), "bf16")
    zeros = np.zeros((cfg.n_heads, cfg.d_head))
    dl = DeviceLayers(wl)
    zu = to_dev(zeros, "bf16")
    Rk = to_dev(R_hat, "bf16")
    shp = dl.shape()
    w = dl.W[0]
    outs = []
    if path == "hidden_state":
        ws = workspace(txl.txl_rel_attn_workspace_bytes(shp))
        start = 0
        for s in range(3):
            h = to_dev(wl.segments[s], "bf16")
            out = nan_empty((cfg.batch, cfg.seg_len, cfg.n_heads * cfg.d_head),
                              dtype=torch.bfloat16, device="cuda")
            txl.txl_rel_attn_fwd(shp, h, dl.mem[0], start, w["W_q"], w["W_kE"], None, w["W_v"],
                                 zu, zu, None, Rk, out, ws)
            start = txl.txl_mem_update(dl.mem[0], start, h, cfg.batch, cfg.mem_len, cfg.seg_len,
                                       cfg.d_model, txl.TXL_BF16)
            torch.cuda.synchronize()
            outs.append(from_dev(out))
    else:
        ws = workspace(txl.txl_kv_ring_workspace_bytes(shp))
        ring = workspace(txl.txl_kv_ring_bytes(shp))
        start = txl.txl_kv_ring_init(shp, dl.mem[0], 0, w["W_kE"], w["W_v"], ring, ws)
        for s in range(3):
            h = to_dev(wl.segments[s], "bf16")
            out = nan_empty((cfg.batch, cfg.seg_len, cfg.n_heads * cfg.d_head),
                              dtype=torch.bfloat16, device="cuda")
            start = txl.txl_rel_attn_fwd_kv(shp, h, w["W_q"], w["W_kE"], None, w["W_v"], zu, zu,
                                            None, Rk, ring, start, out, ws)
            torch.cuda.synchronize()
            outs.append(from_dev(out))
    mems = [m for m in wl.mem]
    start_o = 0
    for s in range(3):
        want, mems, start_o, _ = oracle.segment_step(wl.segments[s], wl.layers, mems, start_o,
                                                     zeros, zeros, None, cfg.n_heads,
                                                     cfg.d_head, Rks=[R_hat])
        assert_close(outs[s], want, "bf16", f"segment {s}")
