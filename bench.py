#!/usr/bin/env python3
"""Benchmark of the relative-attention layer step on one MI355X.

A step is one txl_segment_step of the eval-shaped layer (batch 8, d_model 1024,
16 heads of 64, segment 128 against a 1,600-state memory, bf16): position keys
Rk = R W_kR^T, projections q / k / val^T over [memory ; segment], the fused
relative attention, and the ring memory update.  Inputs are synthetic and
resident in HBM before timing; every step consumes the next of 8 pre-generated
segments and advances the memory ring.

Printed JSON line: metric value = algorithmic TFLOP/s of the step (projection,
position-key and attention FLOPs over valid query/key pairs only), plus eval
tokens/s, the roofline entry of the dominant kernel (timed live with HIP events
on the launch stream) and the CPU oracle on a bounded sample.  A second leg
("kv_ring") streams the same segments through txl_segment_step_kv, which
carries projected keys and values instead of hidden states (exact with fixed
weights), and reports its tokens/s beside the headline step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def flops(cfg, with_rk=True):
    """Algorithmic FLOPs of one relative-attention forward (one layer, one segment)."""
    B, L, M, d, H, dh = cfg.batch, cfg.seg_len, cfg.mem_len, cfg.d_model, cfg.n_heads, cfg.d_head
    Hd = H * dh
    pairs = L * M + L * (L + 1) // 2          # visible (query, key) pairs per (b, h)
    f_q = 2 * B * L * d * Hd
    f_kv = 2 * 2 * B * (M + L) * d * Hd
    f_rk = 2 * (M + L) * cfg.d_pos * Hd if with_rk else 0
    f_core = B * H * 3 * 2 * pairs * dh       # (q+u).k, (q+v).Rk, p.val
    extra = 0
    if cfg.d_inner:
        extra = 2 * B * L * Hd * d + 2 * 2 * B * L * d * cfg.d_inner
    return dict(q=f_q, kv=f_kv, rk=f_rk, core=f_core, extra=extra,
                total=f_q + f_kv + f_rk + f_core + extra, pairs=pairs)


def flops_kv_ring(cfg, with_rk=True):
    """Executed FLOPs of one step over a carried K/V ring: keys and values are
    projected for the segment's L rows only."""
    f = flops(cfg, with_rk)
    B, L, d, Hd = cfg.batch, cfg.seg_len, cfg.d_model, cfg.n_heads * cfg.d_head
    kv = 2 * 2 * B * L * d * Hd
    return f["total"] - f["kv"] + kv


def attn_bytes(cfg):
    """Algorithmic HBM bytes of the fused attention kernel (bf16 operands read
    once, fp32 q, bf16 output): q + K + V + Rk + out."""
    B, L, M, H, dh = cfg.batch, cfg.seg_len, cfg.mem_len, cfg.n_heads, cfg.d_head
    n = M + L
    return B * H * L * dh * 4 + 2 * B * H * n * dh * 2 + H * n * dh * 2 + B * L * H * dh * 2


def source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "transformer_xl_relative_attn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# where roofline.achieved's launch duration comes from
TIMING_SOURCE = ("mean launch duration from HIP events recorded on the launch stream around "
                 "each launch (no system-scope fence), over --steps steps after the timed region")

KERNEL_SOURCES = {
    "proj_gemm": ["gemm.hip", "dev_common.h", "txl_internal.h"],
    "rel_attn": ["attn.hip", "dev_common.h", "txl_internal.h"],
}


def load_traffic(kernel, workload):
    """HBM traffic per launch measured with rocprofv3 counters, if the kernel
    source has not changed since (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def mfma_probe_leg():
    """Sustained bf16 matrix-core rate on zero and on random N(0,1) operands
    (txl_probe_mfma: 8 waves per compute unit, independent 32x32x16 products),
    with the shader clock the products ran at."""
    import numpy as np
    import torch
    import transformer_xl_relative_attn_amd as txl
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
    units = n_wg * 512 * 24
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261202)
    data = {"zeros": torch.zeros(units * 8, dtype=torch.bfloat16, device="cuda"),
            "random": torch.randn(units * 8, generator=gen, device="cuda").to(torch.bfloat16)}
    clocks = torch.zeros(2 * n_wg + 1, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    out = {"kernel": "txl_probe_mfma", "workgroups": n_wg}
    for name, buf in data.items():
        for label, iters, reps in (("burst", 256, 1), ("sustained", 4096, 3)):
            txl.txl_probe_mfma(buf, n_wg, 64, clocks, stream)
            torch.cuda.synchronize()
            for _ in range(reps):   # the last repetition is reported
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                txl.txl_probe_mfma(buf, n_wg, iters, clocks, stream)
                e1.record(stream)
                torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = clocks[:2 * n_wg].view(n_wg, 2).cpu().numpy().astype(np.float64)
            ghz = float(np.median(c[:, 0] / c[:, 1])) * 0.1
            fl = 2.0 * 32 * 32 * 16 * 16 * iters * 8 * n_wg
            out[f"{name}_{label}"] = {"us": round(ms * 1e3, 1),
                                      "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                                      "clock_ghz": round(ghz, 3)}
    del data, clocks
    return out


def cpu_baseline(cfg, wl, budget_s):
    """Time the fp64 oracle on the host for consecutive segments of the same
    workload until the budget is spent (at least one segment)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        cores = 1
    R = oracle.sinusoid(cfg.n_pos, cfg.d_pos)
    mems = [m for m in wl.mem]
    start = 0
    t0 = time.perf_counter()
    done = 0
    n_pool = len(wl.segments)
    while True:   # consecutive segments of one stream, cycling the input pool
        _, mems, start, _ = oracle.segment_step(wl.segments[done % n_pool], wl.layers, mems,
                                                start, wl.u, wl.v, R, cfg.n_heads, cfg.d_head)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    f = flops(cfg)["total"] * cfg.n_layers
    _ = np
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": f * done / el / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "cpu_model": model, "kind": "oracle",
            "sample": f"{done} consecutive segment(s) of the {cfg.name} workload, all "
                      f"{cfg.batch} batch rows, fp64 numpy oracle, {el:.1f} s",
            "tokens_per_s": cfg.batch * cfg.seg_len * done / el}


TABLE9_PAPER = {3800: 1874, 2800: 1409, 1800: 773, 800: 363}


def table9(args):
    """Evaluation speed of Sec. 4.5 / Table 9 at this library's scale: per-token
    time of the vanilla sliding-window evaluation (Sec. 3.1: every step runs a
    whole window of the attention length from scratch, no memory, and predicts
    only its last position) against the Transformer-XL segment step (128 new
    tokens per step against a memory of the attention length), both on the
    16-layer stack (d_model 1024, 16 heads of 64, FFN 4096, batch 4, bf16).
    The vanilla window runs through the same layers with M = 0 (the pages'
    vanilla model uses absolute positions; the work per window is the same
    shape).  Prints one JSON line."""
    import numpy as np
    import torch

    import synth
    import transformer_xl_relative_attn_amd as txl

    cfg = synth.get_config("stack16_l128_m3800")
    torch.cuda.set_device(0)
    wl = synth.make_workload(cfg, n_segments=2)

    def dev(x):
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    W = [dict(W_q=dev(l.W_q), W_kE=dev(l.W_kE), W_kR=dev(l.W_kR), W_v=dev(l.W_v),
              W_o=dev(l.W_o), W_ff1=dev(l.W_ff1), W_ff2=dev(l.W_ff2)) for l in wl.layers]
    u, v = dev(wl.u), dev(wl.v)
    mems_full = [dev(m) for m in wl.mem]
    segs = [dev(x) for x in wl.segments]
    del wl
    n_pos = cfg.mem_len + cfg.seg_len
    R = torch.empty((n_pos, cfg.d_pos), dtype=torch.bfloat16, device="cuda")
    txl.txl_sinusoid_pos(R, n_pos, cfg.d_pos, txl.TXL_BF16)
    stream = torch.cuda.current_stream()
    B, L, d = cfg.batch, cfg.seg_len, cfg.d_model

    def timed(fn, warm, reps):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return max(e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3) / reps

    def layer_list(mems):
        return [txl.make_layer(w["W_q"], w["W_kE"], w["W_kR"], w["W_v"], u, v,
                               None if mems is None else mems[n], W_o=w["W_o"],
                               W_ff1=w["W_ff1"], W_ff2=w["W_ff2"]) for n, w in enumerate(W)]

    rows = []
    for A in (800, 1800, 2800, 3800):
        # Transformer-XL: segment of 128 against a memory of A states per layer
        mems = [m[:, -A:, :].contiguous() for m in mems_full]
        shp = txl.AttnShape(B, L, A, d, cfg.n_heads, cfg.d_head, cfg.d_pos, txl.TXL_BF16, 0.0)
        ws = torch.empty(txl.txl_segment_workspace_bytes(shp, cfg.n_layers, cfg.d_inner),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((B, L, d), dtype=torch.bfloat16, device="cuda")
        layers = layer_list(mems)
        st = {"start": 0, "i": 0}

        def xl_step():
            st["start"] = txl.txl_segment_step(shp, cfg.n_layers, cfg.d_inner, layers, R,
                                               segs[st["i"] % 2], out, st["start"], ws, stream)
            st["i"] += 1

        ms_xl = timed(xl_step, 2, args.table9_steps)
        # ... and over carried K/V rings
        wsr = torch.empty(txl.txl_segment_kv_workspace_bytes(shp, cfg.n_layers, cfg.d_inner),
                          dtype=torch.uint8, device="cuda")
        rings = []
        for n, w in enumerate(W):
            ring = torch.empty(txl.txl_kv_ring_bytes(shp), dtype=torch.uint8, device="cuda")
            txl.txl_kv_ring_init(shp, mems[n], st["start"], w["W_kE"], w["W_v"], ring, wsr,
                                 stream)
            rings.append(ring)
        rs = {"start": 0, "i": 0}

        def ring_step():
            rs["start"] = txl.txl_segment_step_kv(shp, cfg.n_layers, cfg.d_inner, layers, rings,
                                                  R, segs[rs["i"] % 2], out, rs["start"], wsr,
                                                  stream)
            rs["i"] += 1

        ms_ring = timed(ring_step, 2, args.table9_steps)
        del rings, wsr, ws, mems, layers
        # vanilla: the whole window of A positions from scratch, no memory
        vshp = txl.AttnShape(B, A, 0, d, cfg.n_heads, cfg.d_head, cfg.d_pos, txl.TXL_BF16, 0.0)
        vws = torch.empty(txl.txl_segment_workspace_bytes(vshp, cfg.n_layers, cfg.d_inner),
                          dtype=torch.uint8, device="cuda")
        win = mems_full[0][:, -A:, :].contiguous()
        vout = torch.empty((B, A, d), dtype=torch.bfloat16, device="cuda")
        vlayers = layer_list(None)

        def vanilla_step():
            txl.txl_segment_step(vshp, cfg.n_layers, cfg.d_inner, vlayers, R, win, vout, 0, vws,
                                 stream)

        ms_van = timed(vanilla_step, 1, max(1, args.table9_steps // 2))
        del vws, win, vout
        xl_tok = ms_xl * 1e3 / (B * L)
        ring_tok = ms_ring * 1e3 / (B * L)
        van_tok = ms_van * 1e3 / B        # one prediction per window and batch row
        rows.append({"attn_len": A, "xl_us_per_token": round(xl_tok, 3),
                     "xl_kv_ring_us_per_token": round(ring_tok, 3),
                     "vanilla_us_per_token": round(van_tok, 3),
                     "slowdown_vs_xl": round(van_tok / xl_tok, 1),
                     "slowdown_vs_xl_kv_ring": round(van_tok / ring_tok, 1),
                     "paper_slowdown": TABLE9_PAPER[A]})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    out = {
        "metric": "eval slowdown of the vanilla sliding window vs the XL segment step "
                  "(per-token time, attention length 3800)",
        "value": rows[-1]["slowdown_vs_xl"],
        "unit": "x",
        "n_gpus": 1,
        "steps": args.table9_steps,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "table9: 16-layer stack, d_model 1024, 16x64 heads, FFN 4096, "
                               "batch 4, segment 128, attention lengths 800-3800"},
        "table9": rows,
        "paper_context": "Table 9 ratios are per-token evaluation time on one GPU; the "
                         "pages name neither the GPU, the model size nor the precision",
    }
    print(json.dumps(out), flush=True)


def bwd_flops(cfg):
    """Algorithmic FLOPs of the attention backward over the visible pairs: the
    score recompute ((q+u).k and (q+v).Rk), dP = G val^T, dq's two products,
    dk, dval and dRk (8 products of 2 * pairs * d_head per (b, h)), plus
    dW_kR."""
    f = flops(cfg)
    core = cfg.batch * cfg.n_heads * 8 * 2 * f["pairs"] * cfg.d_head
    wkr = 2 * (cfg.mem_len + cfg.seg_len) * cfg.n_heads * cfg.d_head * cfg.d_pos
    return core, wkr


def bwd_bench(args):
    """Backward of the train-shaped layer (txl_rel_attn_bwd, batch 22, segment
    512, memory 512, 8 heads of 64, d_model 512, bf16 in, fp32 gradients):
    one step = the whole call (projections and forward recomputed inside).
    Prints one JSON line."""
    import numpy as np
    import torch

    import synth
    import transformer_xl_relative_attn_amd as txl

    cfg = synth.get_config(args.bwd_config)
    torch.cuda.set_device(0)
    wl = synth.make_workload(cfg, n_segments=1)

    def dev(x):
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    lay = wl.layers[0]
    W = dict(W_q=dev(lay.W_q), W_kE=dev(lay.W_kE), W_kR=dev(lay.W_kR), W_v=dev(lay.W_v))
    u, v = dev(wl.u), dev(wl.v)
    mem = dev(wl.mem[0])
    h = dev(wl.segments[0])
    B, L, M, H, dh = cfg.batch, cfg.seg_len, cfg.mem_len, cfg.n_heads, cfg.d_head
    P = M + L
    G = dev(np.random.default_rng(cfg.seed + 1).normal(0.0, 1.0, (B, L, H * dh)))
    R = torch.empty((cfg.n_pos, cfg.d_pos), dtype=torch.bfloat16, device="cuda")
    txl.txl_sinusoid_pos(R, cfg.n_pos, cfg.d_pos, txl.TXL_BF16)
    shape = txl.AttnShape(B, L, M, cfg.d_model, H, dh, cfg.d_pos, txl.TXL_BF16, 0.0)
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = dict(d_q=torch.empty((B, L, H, dh), **f32), d_k=torch.empty((B, P, H, dh), **f32),
                d_val=torch.empty((B, P, H, dh), **f32), d_u=torch.empty((H, dh), **f32),
                d_v=torch.empty((H, dh), **f32), d_Rk=torch.empty((P, H, dh), **f32),
                d_W_kR=torch.empty((H * dh, cfg.d_pos), **f32))
    ws = torch.empty(txl.txl_rel_attn_bwd_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        txl.txl_rel_attn_bwd(shape, h, mem, 0, W["W_q"], W["W_kE"], W["W_kR"], W["W_v"], u, v, R,
                             None, G, outs["d_q"], outs["d_k"], outs["d_val"], outs["d_u"],
                             outs["d_v"], outs["d_Rk"], outs["d_W_kR"], ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = max(e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3) / args.steps
    txl.txl_timing_reset()
    txl.txl_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    per = txl.txl_timing_read()
    txl.txl_timing_enable(False)
    kernels = {k: {"launches": c, "avg_us": round(t / c * 1e3, 2), "ms_per_step": round(t / args.steps, 4)}
               for k, (c, t) in per.items() if c}
    # the training pair: forward with its state kept, then the backward from it
    out_fwd = torch.empty((B, L, H, dh), dtype=torch.bfloat16, device="cuda")

    def fwd_train():
        txl.txl_rel_attn_fwd_train(shape, h, mem, 0, W["W_q"], W["W_kE"], W["W_kR"], W["W_v"], u,
                                   v, R, None, out_fwd, ws, stream)

    def bwd_saved():
        txl.txl_rel_attn_bwd_saved(shape, u, v, R, False, out_fwd, G, outs["d_q"], outs["d_k"],
                                   outs["d_val"], outs["d_u"], outs["d_v"], outs["d_Rk"],
                                   outs["d_W_kR"], ws, stream)

    def timed_ms(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return max(e0.elapsed_time(e1), (time.perf_counter() - t1) * 1e3) / args.steps

    fwd_train()
    ms_saved = timed_ms(bwd_saved)
    ms_pair = timed_ms(lambda: (fwd_train(), bwd_saved()))
    core, wkr = bwd_flops(cfg)
    value = (core + wkr) / (ms * 1e-3) / 1e12
    q_us = kernels.get("attn_bwd_q", {}).get("avg_us")
    # the query-side kernel runs 5 of the 8 products of 2 * pairs * d_head
    q_flops = cfg.batch * H * 5 * 2 * flops(cfg)["pairs"] * dh
    roof = None
    if q_us:
        ach = q_flops / (q_us * 1e-6) / 1e12
        roof = {"kernel": "attn_bwd_q", "bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "algorithmic_per_launch": q_flops}
    out = {
        "metric": "rel-attn bwd TFLOP/s (train-shaped layer, algorithmic backward FLOPs)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: backward of one relative-attention layer",
                   "batch": B, "seg_len": L, "mem_len": M, "d_model": cfg.d_model,
                   "n_heads": H, "d_head": dh},
        "gflop_per_step": round((core + wkr) / 1e9, 3),
        "tokens_per_s": round(B * L / (ms * 1e-3), 1),
        "kernels": kernels,
        "roofline": roof,
        "from_saved_forward": {
            "bwd_saved_ms": round(ms_saved, 4),
            "bwd_saved_tflops": round((core + wkr) / (ms_saved * 1e-3) / 1e12, 2),
            "fwd_train_plus_bwd_saved_ms": round(ms_pair, 4)},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="eval_l128_m1600", help="workload name (see synth.CONFIGS); the headline is eval_l128_m1600")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cached-rk", action="store_true",
                    help="pass precomputed position keys (Rk computed once, outside the step)")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip the carried K/V ring leg")
    ap.add_argument("--no-mall", dest="mall", action="store_false",
                    help="skip the cold/warm Infinity Cache leg of the attention kernel")
    ap.add_argument("--no-probe", dest="probe", action="store_false",
                    help="skip the matrix-core probe (sustained bf16 rate on zero/random operands)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--table9", action="store_true",
                    help="instead of the headline, measure the vanilla-vs-XL evaluation "
                         "slowdown at attention lengths 800..3800 (one JSON line)")
    ap.add_argument("--table9-steps", type=int, default=6)
    ap.add_argument("--bwd", action="store_true",
                    help="instead of the headline, time the backward of the train-shaped layer "
                         "(one JSON line)")
    ap.add_argument("--bwd-config", default="train_l512_m512")
    ap.add_argument("--shaw", action="store_true",
                    help="instead of the headline, time the same layer step as the two-term "
                         "variant of Shaw et al.: u = v = 0 and a learned position table R^ "
                         "passed as the position keys (no W_kR product; one JSON line)")
    args = ap.parse_args()
    if args.shaw:
        args.cached_rk = True
        args.no_ring = True

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the relative-attention step has no "
              "multi-GPU path in this library (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.table9:
        table9(args)
        return
    if args.bwd:
        bwd_bench(args)
        return

    import numpy as np
    import torch

    import synth
    import transformer_xl_relative_attn_amd as txl

    cfg = synth.get_config(args.config)
    torch.cuda.set_device(0)
    dt_t = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dt_x = txl.TXL_BF16 if cfg.dtype == "bf16" else txl.TXL_F32
    n_seg_pool = 8

    def dev(x):
        if cfg.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()

    wl = synth.make_workload(cfg, n_segments=n_seg_pool)
    W = []
    for lay in wl.layers:
        w = dict(W_q=dev(lay.W_q), W_kE=dev(lay.W_kE), W_kR=dev(lay.W_kR), W_v=dev(lay.W_v))
        if lay.W_o is not None:
            w.update(W_o=dev(lay.W_o), W_ff1=dev(lay.W_ff1), W_ff2=dev(lay.W_ff2))
        W.append(w)
    u, v = dev(wl.u), dev(wl.v)
    if args.shaw:
        u.zero_()
        v.zero_()
    mems = [dev(m) for m in wl.mem]
    segs = [dev(s) for s in wl.segments]
    R = torch.empty((cfg.n_pos, cfg.d_pos), dtype=dt_t, device="cuda")
    txl.txl_sinusoid_pos(R, cfg.n_pos, cfg.d_pos, dt_x)
    Rks = None
    if args.shaw:
        # the learned table R^ (one row per distance, already per head): synthetic
        rng = np.random.default_rng(cfg.seed + 77)
        Rks = [dev(rng.normal(0.0, 0.5, (cfg.n_pos, cfg.n_heads, cfg.d_head))) for _ in W]
    elif args.cached_rk:
        Rks = []
        for w in W:
            rk = torch.empty((cfg.n_pos, cfg.n_heads, cfg.d_head), dtype=dt_t, device="cuda")
            pws = torch.empty(max(1, txl.txl_rel_proj_workspace_bytes(
                cfg.n_pos, cfg.d_pos, cfg.n_heads, cfg.d_head, dt_x)), dtype=torch.uint8,
                device="cuda")
            txl.txl_rel_proj(R, w["W_kR"], rk, cfg.n_pos, cfg.d_pos, cfg.n_heads, cfg.d_head,
                             dt_x, pws)
            Rks.append(rk)
    layers = [txl.make_layer(w["W_q"], w["W_kE"], w["W_kR"], w["W_v"], u, v,
                             mems[n] if cfg.mem_len else None,
                             Rk=None if Rks is None else Rks[n], W_o=w.get("W_o"),
                             W_ff1=w.get("W_ff1"), W_ff2=w.get("W_ff2"))
              for n, w in enumerate(W)]
    shape = txl.AttnShape(cfg.batch, cfg.seg_len, cfg.mem_len, cfg.d_model, cfg.n_heads,
                          cfg.d_head, cfg.d_pos, dt_x, 0.0)
    ws = torch.empty(txl.txl_segment_workspace_bytes(shape, cfg.n_layers, cfg.d_inner),
                     dtype=torch.uint8, device="cuda")
    d_out = cfg.d_model if cfg.d_inner else cfg.n_heads * cfg.d_head
    h_out = torch.empty((cfg.batch, cfg.seg_len, d_out), dtype=dt_t, device="cuda")
    stream = torch.cuda.current_stream()
    state = {"start": 0, "i": 0}

    def step():
        state["start"] = txl.txl_segment_step(shape, cfg.n_layers, cfg.d_inner, layers, R,
                                              segs[state["i"] % n_seg_pool], h_out,
                                              state["start"], ws, stream)
        state["i"] += 1

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- headline timing (no instrumentation)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps

    # ---- median step time over at least 50 steps, one event between steps
    n_med = max(50, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_med + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for r in range(n_med):
        step()
        evs[r + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [evs[r].elapsed_time(evs[r + 1]) for r in range(n_med)]
    med_ms = float(np.median(step_ms))

    # ---- per-kernel timing with HIP events on the launch stream
    txl.txl_timing_reset()
    txl.txl_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    per = txl.txl_timing_read()
    txl.txl_timing_enable(False)
    kernels = {k: {"launches": c, "avg_us": (ms / c * 1e3) if c else 0.0,
                   "share": 0.0} for k, (c, ms) in per.items() if c}
    tot = sum(ms for (c, ms) in per.values() if c)
    for k, (c, ms) in per.items():
        if c:
            kernels[k]["share"] = ms / tot

    f = flops(cfg, with_rk=not args.cached_rk)
    f_step = f["total"] * cfg.n_layers
    value = f_step / (ms_per_step * 1e-3) / 1e12
    tokens = cfg.batch * cfg.seg_len / (ms_per_step * 1e-3)

    dominant = max(kernels, key=lambda k: kernels[k]["share"])
    roof = None
    wl_name = cfg.name
    if dominant == "proj_gemm":
        fl = f["q"] + f["kv"] + f["rk"]
        ach = fl / (kernels[dominant]["avg_us"] * 1e-6) / 1e12
        roof = {"kernel": "proj_gemm", "bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic("proj_gemm", wl_name),
                "algorithmic_per_launch": fl, "timing": TIMING_SOURCE}
    elif dominant == "rel_attn":
        by = attn_bytes(cfg)
        ach = by / (kernels[dominant]["avg_us"] * 1e-6) / 1e9
        roof = {"kernel": "rel_attn", "bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": load_traffic("rel_attn", wl_name), "algorithmic_per_launch": by,
                "timing": TIMING_SOURCE}
    else:
        roof = {"kernel": dominant, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": None, "traffic": None}
    attn_info = None
    if "rel_attn" in kernels:
        us = kernels["rel_attn"]["avg_us"]
        attn_info = {"avg_us": round(us, 2),
                     "core_tflops": round(f["core"] / (us * 1e-6) / 1e12, 1),
                     "algorithmic_gbs": round(attn_bytes(cfg) / (us * 1e-6) / 1e9, 1)}

    # ---- the same stream of segments over carried K/V rings (evaluation with
    # fixed weights: memory keys and values are not recomputed)
    ring_info = None
    if cfg.dtype == "bf16" and cfg.seg_len % 32 == 0 and not args.no_ring:
        ws_r = torch.empty(txl.txl_segment_kv_workspace_bytes(shape, cfg.n_layers, cfg.d_inner),
                           dtype=torch.uint8, device="cuda")
        rings = []
        for n, w in enumerate(W):
            ring = torch.empty(txl.txl_kv_ring_bytes(shape), dtype=torch.uint8, device="cuda")
            txl.txl_kv_ring_init(shape, mems[n] if cfg.mem_len else None, state["start"],
                                 w["W_kE"], w["W_v"], ring, ws_r, stream)
            rings.append(ring)
        rstate = {"start": 0, "i": 0}

        def ring_step():
            rstate["start"] = txl.txl_segment_step_kv(shape, cfg.n_layers, cfg.d_inner, layers,
                                                      rings, R, segs[rstate["i"] % n_seg_pool],
                                                      h_out, rstate["start"], ws_r, stream)
            rstate["i"] += 1

        for _ in range(args.warmup):
            ring_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            ring_step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall_r = time.perf_counter() - t0
        ms_r = max(ev0.elapsed_time(ev1), wall_r * 1e3) / args.steps
        fr = flops_kv_ring(cfg, with_rk=not args.cached_rk) * cfg.n_layers
        # the same kernel with its inputs in the Infinity Cache (the ring's
        # memory keys and values were written by earlier steps) or flushed
        # from it: a 512 MiB fill (twice the cache) between steps
        mall = None
        if args.mall:
            flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

            def attn_us(flushed):
                txl.txl_timing_reset()
                txl.txl_timing_enable(True)
                for _ in range(args.steps):
                    if flushed:
                        flush.zero_()
                    ring_step()
                torch.cuda.synchronize()
                per_k = txl.txl_timing_read()
                txl.txl_timing_enable(False)
                c, ms = per_k.get("rel_attn", (0, 0.0))
                return ms / c * 1e3 if c else None

            warm, cold = attn_us(False), attn_us(True)
            by = attn_bytes(cfg)
            mall = {"kernel": "rel_attn (K/V-ring step)", "algorithmic_bytes": by,
                    "warm_us": round(warm, 2), "cold_us": round(cold, 2),
                    "warm_gbs": round(by / (warm * 1e-6) / 1e9, 1),
                    "cold_gbs": round(by / (cold * 1e-6) / 1e9, 1),
                    "flush": "512 MiB device fill between steps"}
            del flush
        ring_info = {"ms_per_step": round(ms_r, 4),
                     "attention_infinity_cache": mall,
                     "tokens_per_s": round(cfg.batch * cfg.seg_len / (ms_r * 1e-3), 1),
                     "speedup_vs_hidden_state_memory": round(ms_per_step / ms_r, 3),
                     "executed_gflop_per_step": round(fr / 1e9, 3),
                     "executed_tflops": round(fr / (ms_r * 1e-3) / 1e12, 1)}
        del rings, ws_r

    probe = None
    if args.probe and cfg.dtype == "bf16" and not args.shaw:
        probe = mfma_probe_leg()
        rs = probe["random_sustained"]["tflops"]
        probe["proj_gemm_vs_random_sustained"] = round(roof["achieved"] / rs, 3) \
            if roof and roof.get("kernel") == "proj_gemm" and roof.get("achieved") and rs else None

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, wl, args.cpu_budget)

    if args.shaw:
        out = {"metric": "Shaw-variant layer step TFLOP/s (executed: q, K, V projections + "
                         "two-term attention core)",
               "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": cfg.dtype, "data": "synthetic",
               "config": {"workload": f"{cfg.name}: Shaw et al. two-term layer step (u = v = 0, "
                                      "learned R^ as position keys)",
                          "batch": cfg.batch, "seg_len": cfg.seg_len, "mem_len": cfg.mem_len,
                          "d_model": cfg.d_model, "n_heads": cfg.n_heads, "d_head": cfg.d_head},
               "tokens_per_s": round(tokens, 1), "gflop_per_step": round(f_step / 1e9, 3),
               "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                               for kk, vv in d.items()} for k, d in kernels.items()},
               "attention_kernel": attn_info}
        print(json.dumps(out), flush=True)
        return

    out = {
        "metric": "rel-attn fwd TFLOP/s (% bf16 MFMA peak) + eval tokens/s at L=128,M=1600",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: relative-attention layer step over a cached memory",
                   "batch": cfg.batch, "seg_len": cfg.seg_len, "mem_len": cfg.mem_len,
                   "d_model": cfg.d_model, "n_heads": cfg.n_heads, "d_head": cfg.d_head,
                   "n_layers": cfg.n_layers, "d_inner": cfg.d_inner,
                   "rk": "cached" if args.cached_rk else "computed in step",
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(tokens, 1),
        "median_step": {"ms": round(med_ms, 4), "reps": n_med,
                        "tflops": round(f_step / (med_ms * 1e-3) / 1e12, 2),
                        "tokens_per_s": round(cfg.batch * cfg.seg_len / (med_ms * 1e-3), 1),
                        "p10_p90_max_ms": [round(float(np.percentile(step_ms, 10)), 4),
                                           round(float(np.percentile(step_ms, 90)), 4),
                                           round(float(max(step_ms)), 4)]},
        "headline_clocks_ms": {"gpu_events": round(gpu_ms, 3), "host_wall": round(wall * 1e3, 3)},
        "gflop_per_step": round(f_step / 1e9, 3),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in d.items()} for k, d in kernels.items()},
        "attention_kernel": attn_info,
        "kv_ring": ring_info,
        "roofline": roof,
        "mfma_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
