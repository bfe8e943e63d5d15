"""Python binding of libtxl (relative-positional attention over a cached memory,
Dai et al., Transformer-XL, Sec. 3.3) for MI355X / gfx950.

Argument marshalling only: every function forwards to the C entry point of the
same name in ``libtxl.so``.  Tensors are torch tensors that live on the GPU
(torch is used for device memory and streams); each is passed as its data
pointer, and the work is enqueued on torch's current HIP stream unless a
stream is given.  There is no fallback: if the library is missing, importing
this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "TXL_F32", "TXL_BF16", "TxlError", "AttnShape", "Layer", "lib", "lib_path",
    "txl_abi_version", "txl_status_str", "txl_last_error", "txl_sinusoid_pos",
    "txl_rel_proj_workspace_bytes", "txl_rel_proj", "txl_rel_attn_workspace_bytes",
    "txl_rel_attn_fwd", "txl_rel_attn_fwd_static", "TXL_STATIC_SCRATCH_BYTES",
    "txl_mem_update", "txl_segment_workspace_bytes", "txl_segment_step",
    "txl_kv_ring_slots", "txl_kv_ring_bytes", "txl_kv_ring_workspace_bytes", "txl_kv_ring_init",
    "txl_rel_attn_fwd_kv", "txl_segment_kv_workspace_bytes", "txl_segment_step_kv",
    "txl_rel_attn_bwd_workspace_bytes", "txl_rel_attn_bwd", "txl_rel_attn_fwd_train",
    "txl_rel_attn_bwd_saved",
    "txl_timing_enable", "txl_timing_reset", "txl_timing_read", "txl_probe_mfma",
]

TXL_F32 = 0
TXL_BF16 = 1

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtxl.so")
if not os.path.exists(lib_path):
    raise ImportError(f"{lib_path} is missing: build it with "
                      "`python transformer_xl_relative_attn_amd/_build.py`")
lib = ctypes.CDLL(lib_path)

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class AttnShape(ctypes.Structure):
    """txl_attn_shape_t."""
    _fields_ = [("batch", _i32), ("seg_len", _i32), ("mem_len", _i32), ("d_model", _i32),
                ("n_heads", _i32), ("d_head", _i32), ("d_pos", _i32), ("dtype", _i32),
                ("scale", ctypes.c_float)]


class Layer(ctypes.Structure):
    """txl_layer_t (device pointers as integers; 0 = NULL)."""
    _fields_ = [("W_q", _vp), ("W_kE", _vp), ("W_kR", _vp), ("W_v", _vp), ("u", _vp),
                ("v", _vp), ("Rk", _vp), ("W_o", _vp), ("W_ff1", _vp), ("W_ff2", _vp),
                ("mem", _vp)]


def _sig(name, restype, argtypes):
    f = getattr(lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_abi = _sig("txl_abi_version", ctypes.c_int, [])
_status_str = _sig("txl_status_str", ctypes.c_char_p, [ctypes.c_int])
_last_error = _sig("txl_last_error", ctypes.c_char_p, [])
_sinusoid = _sig("txl_sinusoid_pos", ctypes.c_int, [_vp, _i32, _i32, _i32, _vp])
_probe = _sig("txl_probe_mfma", ctypes.c_int, [_vp, _i32, _i32, _vp, _vp])
_proj_ws = _sig("txl_rel_proj_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32])
_proj = _sig("txl_rel_proj", ctypes.c_int,
             [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp])
_attn_ws = _sig("txl_rel_attn_workspace_bytes", _sz, [ctypes.POINTER(AttnShape)])
_attn = _sig("txl_rel_attn_fwd", ctypes.c_int,
             [ctypes.POINTER(AttnShape), _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
              _vp, _vp, _vp, _sz, _vp])
_attn_static = _sig("txl_rel_attn_fwd_static", ctypes.c_int,
                    [ctypes.POINTER(AttnShape), _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                     _vp, _vp, _vp, _vp])
TXL_STATIC_SCRATCH_BYTES = 96 << 20
_memup = _sig("txl_mem_update", ctypes.c_int,
              [_vp, ctypes.POINTER(_i32), _vp, _i32, _i32, _i32, _i32, _i32, _vp])
_seg_ws = _sig("txl_segment_workspace_bytes", _sz, [ctypes.POINTER(AttnShape), _i32, _i32])
_seg = _sig("txl_segment_step", ctypes.c_int,
            [ctypes.POINTER(AttnShape), _i32, _i32, ctypes.POINTER(Layer), _vp, _vp, _vp,
             ctypes.POINTER(_i32), _vp, _sz, _vp])

_ring_slots = _sig("txl_kv_ring_slots", _i32, [ctypes.POINTER(AttnShape)])
_ring_bytes = _sig("txl_kv_ring_bytes", _sz, [ctypes.POINTER(AttnShape)])
_ring_ws = _sig("txl_kv_ring_workspace_bytes", _sz, [ctypes.POINTER(AttnShape)])
_ring_init = _sig("txl_kv_ring_init", ctypes.c_int,
                  [ctypes.POINTER(AttnShape), _vp, _i32, _vp, _vp, _vp, _sz,
                   ctypes.POINTER(_i32), _vp, _sz, _vp])
_attn_kv = _sig("txl_rel_attn_fwd_kv", ctypes.c_int,
                [ctypes.POINTER(AttnShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                 _vp, _sz, ctypes.POINTER(_i32), _vp, _vp, _sz, _vp])
_seg_kv_ws = _sig("txl_segment_kv_workspace_bytes", _sz, [ctypes.POINTER(AttnShape), _i32, _i32])
_seg_kv = _sig("txl_segment_step_kv", ctypes.c_int,
               [ctypes.POINTER(AttnShape), _i32, _i32, ctypes.POINTER(Layer),
                ctypes.POINTER(_vp), _sz, _vp, _vp, _vp, ctypes.POINTER(_i32), _vp, _sz, _vp])

_bwd_ws = _sig("txl_rel_attn_bwd_workspace_bytes", _sz, [ctypes.POINTER(AttnShape)])
_bwd = _sig("txl_rel_attn_bwd", ctypes.c_int,
            [ctypes.POINTER(AttnShape), _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp])

_fwd_train = _sig("txl_rel_attn_fwd_train", ctypes.c_int,
                  [ctypes.POINTER(AttnShape), _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                   _vp, _vp, _vp, _sz, _vp])
_bwd_saved = _sig("txl_rel_attn_bwd_saved", ctypes.c_int,
                  [ctypes.POINTER(AttnShape), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                   _vp, _vp, _vp, _vp, _sz, _vp])

_t_enable = _sig("txl_timing_enable", ctypes.c_int, [_i32])
_t_reset = _sig("txl_timing_reset", None, [])
_t_read = _sig("txl_timing_read", _i32, [_i32, ctypes.POINTER(ctypes.c_char_p),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_double)])


class TxlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _status_str(status).decode()
        detail = _last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


def _check(status: int, where: str):
    if status != 0:
        raise TxlError(status, where)


def _ptr(t) -> Optional[int]:
    """Data pointer of a tensor (None -> NULL, int -> itself)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def txl_abi_version() -> int:
    return _abi()


def txl_status_str(status: int) -> str:
    return _status_str(status).decode()


def txl_last_error() -> str:
    return _last_error().decode()


def txl_sinusoid_pos(R, n_pos: int, d_pos: int, dtype: int, stream=None):
    _check(_sinusoid(_ptr(R), n_pos, d_pos, dtype, _stream(stream)), "txl_sinusoid_pos")


def txl_rel_proj_workspace_bytes(n_pos, d_pos, n_heads, d_head, dtype) -> int:
    return _proj_ws(n_pos, d_pos, n_heads, d_head, dtype)


def txl_rel_proj(R, W_kR, Rk, n_pos, d_pos, n_heads, d_head, dtype, workspace=None, stream=None):
    _check(_proj(_ptr(R), _ptr(W_kR), _ptr(Rk), n_pos, d_pos, n_heads, d_head, dtype,
                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "txl_rel_proj")


def txl_rel_attn_workspace_bytes(shape: AttnShape) -> int:
    return _attn_ws(ctypes.byref(shape))


def txl_rel_attn_fwd(shape: AttnShape, h, mem, mem_start: int, W_q, W_kE, W_kR, W_v, u, v, R, Rk,
                     out, workspace, stream=None):
    _check(_attn(ctypes.byref(shape), _ptr(h), _ptr(mem), mem_start, _ptr(W_q), _ptr(W_kE),
                 _ptr(W_kR), _ptr(W_v), _ptr(u), _ptr(v), _ptr(R), _ptr(Rk), _ptr(out),
                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "txl_rel_attn_fwd")


def txl_rel_attn_fwd_static(shape: AttnShape, h, mem, mem_start: int, W_q, W_kE, W_kR, W_v, u, v,
                            R, Rk, out, stream=None):
    _check(_attn_static(ctypes.byref(shape), _ptr(h), _ptr(mem), mem_start, _ptr(W_q),
                        _ptr(W_kE), _ptr(W_kR), _ptr(W_v), _ptr(u), _ptr(v), _ptr(R), _ptr(Rk),
                        _ptr(out), _stream(stream)), "txl_rel_attn_fwd_static")


def txl_mem_update(mem, mem_start: int, h, batch, mem_len, seg_len, d_model, dtype,
                   stream=None) -> int:
    """Returns the new mem_start."""
    st = _i32(mem_start)
    _check(_memup(_ptr(mem), ctypes.byref(st), _ptr(h), batch, mem_len, seg_len, d_model, dtype,
                  _stream(stream)), "txl_mem_update")
    return st.value


def txl_segment_workspace_bytes(shape: AttnShape, n_layers: int, d_inner: int) -> int:
    return _seg_ws(ctypes.byref(shape), n_layers, d_inner)


def make_layer(W_q, W_kE, W_kR, W_v, u, v, mem, Rk=None, W_o=None, W_ff1=None, W_ff2=None) -> Layer:
    return Layer(_ptr(W_q), _ptr(W_kE), _ptr(W_kR), _ptr(W_v), _ptr(u), _ptr(v), _ptr(Rk),
                 _ptr(W_o), _ptr(W_ff1), _ptr(W_ff2), _ptr(mem))


def txl_segment_step(shape: AttnShape, n_layers: int, d_inner: int, layers: Sequence[Layer], R,
                     h_in, h_out, mem_start: int, workspace, stream=None) -> int:
    """Returns the new mem_start."""
    arr = (Layer * len(layers))(*layers)
    st = _i32(mem_start)
    _check(_seg(ctypes.byref(shape), n_layers, d_inner, arr, _ptr(R), _ptr(h_in), _ptr(h_out),
                ctypes.byref(st), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "txl_segment_step")
    return st.value


def txl_kv_ring_slots(shape: AttnShape) -> int:
    return _ring_slots(ctypes.byref(shape))


def txl_kv_ring_bytes(shape: AttnShape) -> int:
    return _ring_bytes(ctypes.byref(shape))


def txl_kv_ring_workspace_bytes(shape: AttnShape) -> int:
    return _ring_ws(ctypes.byref(shape))


def txl_kv_ring_init(shape: AttnShape, mem, mem_start: int, W_kE, W_v, ring, workspace,
                     stream=None) -> int:
    """Returns the ring start (0)."""
    st = _i32(0)
    _check(_ring_init(ctypes.byref(shape), _ptr(mem), mem_start, _ptr(W_kE), _ptr(W_v),
                      _ptr(ring), _nbytes(ring), ctypes.byref(st), _ptr(workspace),
                      _nbytes(workspace), _stream(stream)), "txl_kv_ring_init")
    return st.value


def txl_rel_attn_fwd_kv(shape: AttnShape, h, W_q, W_kE, W_kR, W_v, u, v, R, Rk, ring,
                        ring_start: int, out, workspace, stream=None) -> int:
    """Returns the new ring start."""
    st = _i32(ring_start)
    _check(_attn_kv(ctypes.byref(shape), _ptr(h), _ptr(W_q), _ptr(W_kE), _ptr(W_kR), _ptr(W_v),
                    _ptr(u), _ptr(v), _ptr(R), _ptr(Rk), _ptr(ring), _nbytes(ring),
                    ctypes.byref(st), _ptr(out), _ptr(workspace), _nbytes(workspace),
                    _stream(stream)), "txl_rel_attn_fwd_kv")
    return st.value


def txl_segment_kv_workspace_bytes(shape: AttnShape, n_layers: int, d_inner: int) -> int:
    return _seg_kv_ws(ctypes.byref(shape), n_layers, d_inner)


def txl_segment_step_kv(shape: AttnShape, n_layers: int, d_inner: int, layers: Sequence[Layer],
                        rings, R, h_in, h_out, ring_start: int, workspace, stream=None) -> int:
    """rings: one equally sized byte tensor per layer.  Returns the new ring start."""
    arr = (Layer * len(layers))(*layers)
    ptrs = (_vp * len(rings))(*[_ptr(r) for r in rings])
    st = _i32(ring_start)
    _check(_seg_kv(ctypes.byref(shape), n_layers, d_inner, arr, ptrs, _nbytes(rings[0]), _ptr(R),
                   _ptr(h_in), _ptr(h_out), ctypes.byref(st), _ptr(workspace),
                   _nbytes(workspace), _stream(stream)), "txl_segment_step_kv")
    return st.value


def txl_rel_attn_bwd_workspace_bytes(shape: AttnShape) -> int:
    return _bwd_ws(ctypes.byref(shape))


def txl_rel_attn_bwd(shape: AttnShape, h, mem, mem_start: int, W_q, W_kE, W_kR, W_v, u, v, R, Rk,
                     d_out, d_q, d_k, d_val, d_u, d_v, d_Rk, d_W_kR, workspace, stream=None):
    _check(_bwd(ctypes.byref(shape), _ptr(h), _ptr(mem), mem_start, _ptr(W_q), _ptr(W_kE),
                _ptr(W_kR), _ptr(W_v), _ptr(u), _ptr(v), _ptr(R), _ptr(Rk), _ptr(d_out),
                _ptr(d_q), _ptr(d_k), _ptr(d_val), _ptr(d_u), _ptr(d_v), _ptr(d_Rk),
                _ptr(d_W_kR), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "txl_rel_attn_bwd")


def txl_rel_attn_fwd_train(shape: AttnShape, h, mem, mem_start: int, W_q, W_kE, W_kR, W_v, u, v,
                           R, Rk, out, workspace, stream=None):
    _check(_fwd_train(ctypes.byref(shape), _ptr(h), _ptr(mem), mem_start, _ptr(W_q), _ptr(W_kE),
                      _ptr(W_kR), _ptr(W_v), _ptr(u), _ptr(v), _ptr(R), _ptr(Rk), _ptr(out),
                      _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "txl_rel_attn_fwd_train")


def txl_rel_attn_bwd_saved(shape: AttnShape, u, v, R, rk_given: bool, out, d_out, d_q, d_k, d_val,
                           d_u, d_v, d_Rk, d_W_kR, workspace, stream=None):
    _check(_bwd_saved(ctypes.byref(shape), _ptr(u), _ptr(v), _ptr(R), 1 if rk_given else 0,
                      _ptr(out), _ptr(d_out), _ptr(d_q), _ptr(d_k), _ptr(d_val), _ptr(d_u),
                      _ptr(d_v), _ptr(d_Rk), _ptr(d_W_kR), _ptr(workspace), _nbytes(workspace),
                      _stream(stream)),
           "txl_rel_attn_bwd_saved")


def txl_timing_enable(on: bool):
    _check(_t_enable(1 if on else 0), "txl_timing_enable")


def txl_timing_reset():
    _t_reset()


def txl_probe_mfma(operands, n_wg: int, iters: int, clocks, stream=None):
    """Matrix-core probe: operands (n_wg * 512 * 24 * 8 bf16 values), clocks
    (2 * n_wg + 1 uint64 entries: per workgroup, shader cycles and 100 MHz ticks)."""
    _check(_probe(_ptr(operands), n_wg, iters, _ptr(clocks), _stream(stream)), "txl_probe_mfma")


def txl_timing_read() -> dict:
    """{kernel kind: (launches, total_ms)} accumulated since the last reset."""
    cap = 32
    names = (ctypes.c_char_p * cap)()
    counts = (ctypes.c_int64 * cap)()
    ms = (ctypes.c_double * cap)()
    n = _t_read(cap, names, counts, ms)
    return {names[i].decode(): (counts[i], ms[i]) for i in range(min(n, cap))}
