"""Seeded synthetic inputs for the Transformer-XL relative-attention workloads.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It draws random numbers and rounds them to the storage dtype; it holds none of
the method's arithmetic (no projection, no score, no softmax, no sinusoid).

The shapes mirror the workloads of Dai et al., "Transformer-XL: Attentive
Language Models Beyond a Fixed-Length Context": memory equal to the segment
length in training (Sec. 3.2), evaluation attention lengths of 1,600
(WikiText-103) and 3,800 (enwik8) with a 128-token segment (Sec. 4.1).  Those
corpora are not available here; the kernels do not depend on token identity, so
Gaussian activations of the stated scale stand in for them.

Draw order (fixed, so every consumer sees identical bits):
  for each layer: W_q, W_kE, W_kR, W_v, then (stack only) W_o, W_ff1, W_ff2;
  then u, v; then the initial memory of each layer; then the segment inputs.
All draws are float64 from ``numpy.random.default_rng(seed)``, then rounded to
the storage dtype with round-to-nearest-even.  ``N(0, s)`` means standard
deviation ``s``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = ["Config", "CONFIGS", "get_config", "round_to", "bf16_bits",
           "bits_to_f64", "Workload", "make_workload"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    d_model: int
    n_heads: int
    d_head: int
    seg_len: int
    mem_len: int
    n_layers: int
    n_segments: int
    dtype: str            # "f32" or "bf16"
    w_std: float          # std of W_* and of u, v
    seed: int
    d_inner: int = 0      # >0: each layer adds W_o, LayerNorm and a ReLU FFN
    act_std: float = 1.0  # std of h and of the initial memory

    @property
    def d_pos(self) -> int:
        return self.d_model

    @property
    def n_pos(self) -> int:
        return self.mem_len + self.seg_len


CONFIGS = {
    # Tiny fp32 single layer, two segments with the memory carried over.
    "tiny_f32": Config("tiny_f32", batch=1, d_model=16, n_heads=1, d_head=16, seg_len=8, mem_len=8,
                 n_layers=1, n_segments=2, dtype="f32", w_std=0.1, seed=1001),
    # Odd head dimension (41): exercises zero padding of the head axis.
    "odd_head41": Config("odd_head41", batch=16, d_model=410, n_heads=10, d_head=41, seg_len=150, mem_len=150,
                 n_layers=1, n_segments=1, dtype="bf16", w_std=0.02, seed=1002),
    # Train-shaped: memory length equals segment length, 4 streamed segments.
    "train_l512_m512": Config("train_l512_m512", batch=22, d_model=512, n_heads=8, d_head=64, seg_len=512, mem_len=512,
                 n_layers=1, n_segments=4, dtype="bf16", w_std=0.02, seed=1003),
    # Eval-shaped: segment 128 against a 1,600-state memory, 8 streamed segments.
    "eval_l128_m1600": Config("eval_l128_m1600", batch=8, d_model=1024, n_heads=16, d_head=64, seg_len=128, mem_len=1600,
                 n_layers=1, n_segments=8, dtype="bf16", w_std=0.02, seed=1004),
    # 16-layer stack with W_o + LayerNorm + ReLU FFN, 3,800-state memory, 4 segments.
    "stack16_l128_m3800": Config("stack16_l128_m3800", batch=4, d_model=1024, n_heads=16, d_head=64, seg_len=128, mem_len=3800,
                 n_layers=16, n_segments=4, dtype="bf16", w_std=0.02, seed=1005, d_inner=4096),
}


def get_config(name: str, **overrides) -> Config:
    return dataclasses.replace(CONFIGS[name], **overrides)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16.  The float64 -> float32 step is itself RNE."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # finite inputs only (the generators never produce NaN/Inf): no overflow in uint32
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 patterns -> exact float64 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Return x rounded to the storage dtype, as float64 (exactly representable)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bits_to_f64(bf16_bits(x))
    raise ValueError(dtype)


@dataclasses.dataclass
class Layer:
    W_q: np.ndarray
    W_kE: np.ndarray
    W_kR: np.ndarray
    W_v: np.ndarray
    W_o: Optional[np.ndarray] = None
    W_ff1: Optional[np.ndarray] = None
    W_ff2: Optional[np.ndarray] = None


@dataclasses.dataclass
class Workload:
    """All inputs of one workload, as float64 arrays holding dtype-exact values.

    ``mem[n]`` is the initial memory of layer n in logical order (oldest first),
    stored physically with ring start 0.  ``segments[s]`` is the input h of
    segment s, shape [batch, seg_len, d_model]."""
    cfg: Config
    layers: List[Layer]
    u: np.ndarray          # [n_heads, d_head]
    v: np.ndarray          # [n_heads, d_head]
    mem: List[np.ndarray]  # per layer [batch, mem_len, d_model]
    segments: List[np.ndarray]


def make_workload(cfg: Config, n_segments: Optional[int] = None) -> Workload:
    rng = np.random.default_rng(cfg.seed)
    d, hd = cfg.d_model, cfg.n_heads * cfg.d_head
    rt = lambda a: round_to(a, cfg.dtype)  # noqa: E731
    layers = []
    for _ in range(cfg.n_layers):
        W_q = rt(rng.normal(0.0, cfg.w_std, (hd, d)))
        W_kE = rt(rng.normal(0.0, cfg.w_std, (hd, d)))
        W_kR = rt(rng.normal(0.0, cfg.w_std, (hd, cfg.d_pos)))
        W_v = rt(rng.normal(0.0, cfg.w_std, (hd, d)))
        lay = Layer(W_q, W_kE, W_kR, W_v)
        if cfg.d_inner:
            lay.W_o = rt(rng.normal(0.0, cfg.w_std, (d, hd)))
            lay.W_ff1 = rt(rng.normal(0.0, cfg.w_std, (cfg.d_inner, d)))
            lay.W_ff2 = rt(rng.normal(0.0, cfg.w_std, (d, cfg.d_inner)))
        layers.append(lay)
    u = rt(rng.normal(0.0, cfg.w_std, (cfg.n_heads, cfg.d_head)))
    v = rt(rng.normal(0.0, cfg.w_std, (cfg.n_heads, cfg.d_head)))
    mem = [rt(rng.normal(0.0, cfg.act_std, (cfg.batch, cfg.mem_len, d)))
           for _ in range(cfg.n_layers)]
    nseg = cfg.n_segments if n_segments is None else n_segments
    segs = [rt(rng.normal(0.0, cfg.act_std, (cfg.batch, cfg.seg_len, d)))
            for _ in range(nseg)]
    return Workload(cfg, layers, u, v, mem, segs)


def random_case(seed: int, batch: int, d_model: int, n_heads: int, d_head: int,
                seg_len: int, mem_len: int, dtype: str = "f32", w_std: float = 0.1,
                n_segments: int = 1, n_layers: int = 1, d_inner: int = 0) -> Workload:
    """A free-shape workload (edge cases, ragged sizes) with the same draw order."""
    cfg = Config(f"rand{seed}", batch, d_model, n_heads, d_head, seg_len, mem_len,
                 n_layers, n_segments, dtype, w_std, seed, d_inner)
    return make_workload(cfg)
