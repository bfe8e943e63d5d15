"""Helpers for the GPU parity tests: move synth workloads to the device, run the
library through its C entry points, and compare with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray, dtype: str):
    """float64 array holding dtype-exact values -> device tensor of that dtype."""
    torch = torch_mod()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    bits = synth.bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def from_dev(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bf16_bits_of(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def tdtype(dtype: str):
    torch = torch_mod()
    return torch.float32 if dtype == "f32" else torch.bfloat16


def txl_dtype(dtype: str) -> int:
    import transformer_xl_relative_attn_amd as txl
    return txl.TXL_F32 if dtype == "f32" else txl.TXL_BF16


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-300))


def assert_close(got, want, dtype, what):
    err = rel_err(got, want)
    log(f"  {what}: max|gpu-oracle|/max|oracle| = {err:.3e} (tol {TOL[dtype]:.0e})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    assert err <= TOL[dtype], f"{what}: relative error {err:.3e} > {TOL[dtype]}"


class DeviceLayers:
    """Device copies of a workload's weights and memories."""

    def __init__(self, wl: synth.Workload):
        torch = torch_mod()
        c = wl.cfg
        dt = c.dtype
        self.cfg = c
        self.u = to_dev(wl.u, dt)
        self.v = to_dev(wl.v, dt)
        self.W = []
        for lay in wl.layers:
            d = dict(W_q=to_dev(lay.W_q, dt), W_kE=to_dev(lay.W_kE, dt), W_kR=to_dev(lay.W_kR, dt),
                     W_v=to_dev(lay.W_v, dt))
            if lay.W_o is not None:
                d.update(W_o=to_dev(lay.W_o, dt), W_ff1=to_dev(lay.W_ff1, dt),
                         W_ff2=to_dev(lay.W_ff2, dt))
            self.W.append(d)
        self.mem = [to_dev(m, dt) for m in wl.mem]
        self.R = nan_empty((c.n_pos, c.d_pos), dtype=tdtype(dt), device="cuda")
        import transformer_xl_relative_attn_amd as txl
        txl.txl_sinusoid_pos(self.R, c.n_pos, c.d_pos, txl_dtype(dt))

    def shape(self, scale: float = 0.0):
        import transformer_xl_relative_attn_amd as txl
        c = self.cfg
        return txl.AttnShape(c.batch, c.seg_len, c.mem_len, c.d_model, c.n_heads, c.d_head,
                             c.d_pos, txl_dtype(c.dtype), scale)

    def layer_structs(self, Rks=None):
        import transformer_xl_relative_attn_amd as txl
        out = []
        for n, w in enumerate(self.W):
            out.append(txl.make_layer(w["W_q"], w["W_kE"], w["W_kR"], w["W_v"], self.u, self.v,
                                      self.mem[n] if self.cfg.mem_len else None,
                                      Rk=None if Rks is None else Rks[n], W_o=w.get("W_o"),
                                      W_ff1=w.get("W_ff1"), W_ff2=w.get("W_ff2")))
        return out


def workspace(nbytes: int):
    """A device workspace filled with 0xFF bytes (NaN in bf16 and fp32), so that
    a kernel reading workspace memory that no kernel of the call wrote shows up
    as NaN in the compared outputs."""
    torch = torch_mod()
    return torch.full((max(int(nbytes), 1),), 0xFF, dtype=torch.uint8, device="cuda")


def nan_empty(shape, dtype, device="cuda"):
    """torch.empty for output buffers, filled with NaN instead."""
    torch = torch_mod()
    if isinstance(shape, int):
        shape = (shape,)
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def poisoned(shape, dtype):
    """An output buffer filled with NaN: elements the library leaves unwritten fail
    the comparison."""
    torch = torch_mod()
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def run_attn_stream(wl: synth.Workload, n_seg: int, scale: float = 0.0, start: int = 0,
                    use_rk: bool = False):
    """Stream n_seg segments through txl_rel_attn_fwd + txl_mem_update (single
    layer).  Returns (outputs per segment as float64, device layers, final start)."""
    torch = torch_mod()
    import transformer_xl_relative_attn_amd as txl
    c = wl.cfg
    dl = DeviceLayers(wl)
    if start and c.mem_len:
        # physical ring rotated so that logical row p sits at slot (start + p) % M
        dl.mem[0] = torch.roll(dl.mem[0], shifts=start, dims=1).contiguous()
    shp = dl.shape(scale)
    ws = workspace(txl.txl_rel_attn_workspace_bytes(shp))
    w = dl.W[0]
    Rk = None
    if use_rk:
        Rk = nan_empty((c.n_pos, c.n_heads, c.d_head), dtype=tdtype(c.dtype), device="cuda")
        pws = workspace(txl.txl_rel_proj_workspace_bytes(c.n_pos, c.d_pos, c.n_heads, c.d_head,
                                                         txl_dtype(c.dtype)))
        txl.txl_rel_proj(dl.R, w["W_kR"], Rk, c.n_pos, c.d_pos, c.n_heads, c.d_head,
                         txl_dtype(c.dtype), pws)
    outs = []
    for s in range(n_seg):
        h = to_dev(wl.segments[s], c.dtype)
        out = nan_empty((c.batch, c.seg_len, c.n_heads * c.d_head), dtype=tdtype(c.dtype),
                          device="cuda")
        txl.txl_rel_attn_fwd(shp, h, dl.mem[0] if c.mem_len else None, start, w["W_q"],
                             w["W_kE"], w["W_kR"], w["W_v"], dl.u, dl.v, dl.R, Rk, out, ws)
        start = txl.txl_mem_update(dl.mem[0] if c.mem_len else None, start, h, c.batch,
                                   c.mem_len, c.seg_len, c.d_model, txl_dtype(c.dtype))
        torch.cuda.synchronize()
        outs.append(from_dev(out))
    return outs, dl, start


def run_segment_stream(wl: synth.Workload, n_seg: int, scale: float = 0.0):
    """Stream n_seg segments through txl_segment_step.  Returns (outputs, device
    layers, final start)."""
    torch = torch_mod()
    import transformer_xl_relative_attn_amd as txl
    c = wl.cfg
    dl = DeviceLayers(wl)
    shp = dl.shape(scale)
    ws = workspace(txl.txl_segment_workspace_bytes(shp, c.n_layers, c.d_inner))
    layers = dl.layer_structs()
    d_out = c.d_model if c.d_inner else c.n_heads * c.d_head
    start = 0
    outs = []
    for s in range(n_seg):
        h = to_dev(wl.segments[s], c.dtype)
        out = nan_empty((c.batch, c.seg_len, d_out), dtype=tdtype(c.dtype), device="cuda")
        start = txl.txl_segment_step(shp, c.n_layers, c.d_inner, layers, dl.R, h, out, start, ws)
        torch.cuda.synchronize()
        outs.append(from_dev(out))
    return outs, dl, start


def oracle_stream(wl: synth.Workload, n_seg: int, b_idx, scale=None):
    """Oracle outputs for the sampled batch rows (batch rows are independent)."""
    import oracle
    c = wl.cfg
    R = oracle.sinusoid(c.n_pos, c.d_pos)
    mems = [m[b_idx] for m in wl.mem]
    segs = [s[b_idx] for s in wl.segments[:n_seg]]
    outs, mems, start = oracle.segment_stream(segs, wl.layers, mems, wl.u, wl.v, R, c.n_heads,
                                              c.d_head, scale)
    return outs, mems, start


def default_scale(c):
    return 1.0 / math.sqrt(c.d_head)
