"""CPU checks of the C-ABI library: it loads, exports every function the header
declares, and rejects bad arguments before enqueueing anything (no GPU needed:
none of these calls reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "txl.h")


@pytest.fixture(scope="module")
def txl():
    import transformer_xl_relative_attn_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(txl_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(txl):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(txl.lib, n), f"libtxl.so does not export {n}"


def test_abi_version_and_status_text(txl):
    assert txl.txl_abi_version() == 1
    for st in range(7):
        assert txl.txl_status_str(st)
    assert txl.txl_status_str(99) == "unknown status"


def _shape(txl, **kw):
    base = dict(batch=2, seg_len=8, mem_len=16, d_model=64, n_heads=2, d_head=32, d_pos=64,
                dtype=txl.TXL_BF16, scale=0.0)
    base.update(kw)
    return txl.AttnShape(**base)


def _attn(txl, shape, ws_bytes=None, **ptrs):
    p = dict(h=16, mem=32, mem_start=0, W_q=48, W_kE=64, W_kR=80, W_v=96, u=112, v=128, R=144,
             Rk=None, out=160, ws=176)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = txl.txl_rel_attn_workspace_bytes(shape)
    f = txl.lib.txl_rel_attn_fwd
    return f(ctypes.byref(shape), p["h"], p["mem"], p["mem_start"], p["W_q"], p["W_kE"],
             p["W_kR"], p["W_v"], p["u"], p["v"], p["R"], p["Rk"], p["out"], p["ws"], ws_bytes,
             None)


def test_rel_attn_validation(txl):
    s = _shape(txl)
    assert _attn(txl, s, h=None) == 1                     # NULL_ARG
    assert txl.txl_last_error()
    assert _attn(txl, s, mem=None) == 1                   # mem required when M > 0
    assert _attn(txl, s, W_kR=None, R=None) == 1          # neither Rk nor W_kR/R
    assert _attn(txl, s, ws=None) == 1
    assert _attn(txl, s, mem_start=16) == 2               # outside [0, M)
    assert _attn(txl, s, mem_start=-1) == 2
    assert _attn(txl, _shape(txl, seg_len=0)) == 2
    assert _attn(txl, _shape(txl, mem_len=-1)) == 2
    assert _attn(txl, _shape(txl, dtype=7)) == 3
    assert _attn(txl, _shape(txl, d_head=80, n_heads=1)) == 5   # bf16 d_head > 64
    assert _attn(txl, _shape(txl, scale=float("nan"))) == 2
    assert _attn(txl, s, ws_bytes=txl.txl_rel_attn_workspace_bytes(s) - 1) == 4
    assert _attn(txl, s, h=17) == 5                       # unaligned bf16 pointer
    s0 = _shape(txl, mem_len=0)
    assert _attn(txl, s0, mem=None, mem_start=3) == 2     # M == 0 needs start 0


def test_workspace_sizes(txl):
    a = txl.txl_rel_attn_workspace_bytes(_shape(txl, mem_len=16))
    b = txl.txl_rel_attn_workspace_bytes(_shape(txl, mem_len=1600))
    assert 0 < a < b
    assert txl.txl_rel_attn_workspace_bytes(_shape(txl, seg_len=-3)) == 0
    # eval-shaped layer: K, V^T, Rk in bf16 plus fp32 q and split partials
    eval_shape = _shape(txl, batch=8, seg_len=128, mem_len=1600, d_model=1024, n_heads=16, d_head=64,
                d_pos=1024)
    kv = 2 * 8 * 16 * 1728 * 64 * 2
    assert txl.txl_rel_attn_workspace_bytes(eval_shape) >= kv
    assert txl.txl_segment_workspace_bytes(eval_shape, 1, 0) > txl.txl_rel_attn_workspace_bytes(eval_shape)
    assert txl.txl_rel_proj_workspace_bytes(300, 410, 10, 41, txl.TXL_BF16) > 0
    assert txl.txl_rel_proj_workspace_bytes(300, 512, 10, 41, txl.TXL_BF16) == 0
    assert txl.txl_rel_proj_workspace_bytes(300, 410, 10, 41, txl.TXL_F32) == 0


def test_mem_update_validation_keeps_start(txl):
    st = ctypes.c_int32(5)
    f = txl.lib.txl_mem_update
    assert f(16, ctypes.byref(st), None, 2, 16, 8, 64, txl.TXL_BF16, None) == 1
    assert st.value == 5
    st.value = 16
    assert f(16, ctypes.byref(st), 32, 2, 16, 8, 64, txl.TXL_BF16, None) == 2
    assert st.value == 16
    st.value = 3
    assert f(16, ctypes.byref(st), 32, 2, 16, 8, 64, 9, None) == 3
    assert st.value == 3
    # M == 0: nothing to do, succeeds without touching the device
    st.value = 0
    assert f(None, ctypes.byref(st), 32, 2, 0, 8, 64, txl.TXL_BF16, None) == 0
    assert st.value == 0


def test_segment_step_validation(txl):
    s = _shape(txl)
    ws_n = txl.txl_segment_workspace_bytes(s, 2, 0)
    st = ctypes.c_int32(3)
    good = txl.Layer(48, 64, 80, 96, 112, 128, None, None, None, None, 32)
    arr = (txl.Layer * 2)(good, good)
    f = txl.lib.txl_segment_step
    # attention-only layer feeding another layer needs H*d_head == d_model (64 == 64 ok);
    # break it with d_head 16
    bad_shape = _shape(txl, d_head=16)
    assert f(ctypes.byref(bad_shape), 2, 0, arr, 144, 16, 160, ctypes.byref(st), 176,
             txl.txl_segment_workspace_bytes(bad_shape, 2, 0), None) == 2
    assert st.value == 3
    nomem = txl.Layer(48, 64, 80, 96, 112, 128, None, None, None, None, None)
    arr2 = (txl.Layer * 2)(good, nomem)
    assert f(ctypes.byref(s), 2, 0, arr2, 144, 16, 160, ctypes.byref(st), 176, ws_n, None) == 1
    assert "layer 1" in txl.txl_last_error()
    full_missing_ffn = txl.Layer(48, 64, 80, 96, 112, 128, None, 192, None, None, 32)
    arr3 = (txl.Layer * 1)(full_missing_ffn)
    assert f(ctypes.byref(s), 1, 256, arr3, 144, 16, 160, ctypes.byref(st), 176,
             txl.txl_segment_workspace_bytes(s, 1, 256), None) == 1
    assert f(ctypes.byref(s), 0, 0, arr, 144, 16, 160, ctypes.byref(st), 176, ws_n, None) == 2
    assert f(ctypes.byref(s), 2, 0, arr, 144, 16, 160, ctypes.byref(st), 176, ws_n - 1, None) == 4
    assert st.value == 3


def test_rel_proj_and_sinusoid_validation(txl):
    f = txl.lib.txl_rel_proj
    assert f(None, 32, 48, 10, 64, 2, 32, txl.TXL_BF16, None, 0, None) == 1
    assert f(16, 32, 48, 0, 64, 2, 32, txl.TXL_BF16, None, 0, None) == 2
    assert f(16, 32, 48, 10, 410, 2, 32, txl.TXL_BF16, None, 0, None) == 1   # needs workspace
    assert f(16, 32, 48, 10, 410, 2, 32, txl.TXL_BF16, 64, 10, None) == 4
    g = txl.lib.txl_sinusoid_pos
    assert g(None, 4, 4, txl.TXL_F32, None) == 1
    assert g(16, 0, 4, txl.TXL_F32, None) == 2
    assert g(16, 4, 4, 5, None) == 3


def test_probe_mfma_validation(txl):
    f = txl.lib.txl_probe_mfma
    assert f(None, 4, 2, 16, None) == 1          # operands
    assert f(16, 4, 2, None, None) == 1          # clocks
    assert f(16, 0, 2, 16, None) == 2            # n_wg
    assert f(16, 65537, 2, 16, None) == 2
    assert f(16, 4, 3, 16, None) == 2            # iters odd
    assert f(16, 4, 0, 16, None) == 2
    assert f(24, 4, 2, 16, None) == 5            # operands not 16-byte aligned


def test_kv_ring_queries_and_validation(txl):
    # eval-shaped layer: C = round_up(1600, 32) + 128 slots, K and V^T in bf16
    s = _shape(txl, batch=8, seg_len=128, mem_len=1600, d_model=1024, n_heads=16, d_head=64,
               d_pos=1024)
    assert txl.txl_kv_ring_slots(s) == 1728
    assert txl.txl_kv_ring_bytes(s) == 2 * 8 * 16 * 1728 * 64 * 2
    assert txl.txl_kv_ring_workspace_bytes(s) > 0
    # memory not a multiple of 32: ghost slots round it up
    assert txl.txl_kv_ring_slots(_shape(txl, seg_len=64, mem_len=150)) == 160 + 64
    # unsupported: fp32, segment not a multiple of 32
    assert txl.txl_kv_ring_slots(_shape(txl, dtype=txl.TXL_F32, seg_len=32)) == 0
    assert txl.txl_kv_ring_bytes(_shape(txl, seg_len=33)) == 0

    s = _shape(txl, seg_len=32, mem_len=40)
    rb = txl.txl_kv_ring_bytes(s)
    wsb = txl.txl_kv_ring_workspace_bytes(s)
    st = ctypes.c_int32(64)
    f = txl.lib.txl_rel_attn_fwd_kv

    def fwd(shape, ring_bytes=rb, ws_bytes=wsb, **kw):
        p = dict(h=16, W_q=48, W_kE=64, W_kR=80, W_v=96, u=112, v=128, R=144, Rk=None,
                 ring=192, out=160, ws=176)
        p.update(kw)
        return f(ctypes.byref(shape), p["h"], p["W_q"], p["W_kE"], p["W_kR"], p["W_v"], p["u"],
                 p["v"], p["R"], p["Rk"], p["ring"], ring_bytes, ctypes.byref(st), p["out"],
                 p["ws"], ws_bytes, None)

    assert fwd(_shape(txl, seg_len=32, mem_len=40, dtype=txl.TXL_F32)) == 5
    assert fwd(_shape(txl, seg_len=40, mem_len=40)) == 5
    assert fwd(s, h=None) == 1
    assert fwd(s, ring=None) == 1
    assert fwd(s, W_kR=None, R=None) == 1
    assert fwd(s, ring_bytes=rb - 1) == 2
    assert fwd(s, ws_bytes=wsb - 1) == 4
    assert fwd(s, ring=200) == 5                          # unaligned ring
    st.value = 16                                          # not a multiple of 32
    assert fwd(s) == 2 and st.value == 16
    st.value = txl.txl_kv_ring_slots(s)                    # outside [0, C)
    assert fwd(s) == 2 and st.value == txl.txl_kv_ring_slots(s)

    g = txl.lib.txl_kv_ring_init
    st.value = 96

    def init(shape, mem=32, mem_start=0, ring=192, ring_bytes=rb, ws=176, ws_bytes=wsb):
        return g(ctypes.byref(shape), mem, mem_start, 64, 96, ring, ring_bytes, ctypes.byref(st),
                 ws, ws_bytes, None)

    assert init(s, mem=None) == 1
    assert init(s, mem_start=40) == 2
    assert init(s, ring_bytes=rb - 1) == 2
    assert init(s, ws_bytes=wsb - 1) == 4
    assert init(s, ws=None) == 1
    assert init(_shape(txl, seg_len=32, mem_len=40, dtype=txl.TXL_F32)) == 5
    assert st.value == 96


def test_rel_attn_bwd_validation(txl):
    s = _shape(txl)
    wsb = txl.txl_rel_attn_bwd_workspace_bytes(s)
    assert wsb > txl.txl_rel_attn_workspace_bytes(s)
    assert txl.txl_rel_attn_bwd_workspace_bytes(_shape(txl, dtype=txl.TXL_F32)) == 0
    f = txl.lib.txl_rel_attn_bwd

    def bwd(shape, ws_bytes=wsb, **kw):
        p = dict(h=16, mem=32, mem_start=0, W_q=48, W_kE=64, W_kR=80, W_v=96, u=112, v=128,
                 R=144, Rk=None, d_out=160, d_q=176, d_k=192, d_val=208, d_u=224, d_v=240,
                 d_Rk=256, d_W_kR=None, ws=272)
        p.update(kw)
        return f(ctypes.byref(shape), p["h"], p["mem"], p["mem_start"], p["W_q"], p["W_kE"],
                 p["W_kR"], p["W_v"], p["u"], p["v"], p["R"], p["Rk"], p["d_out"], p["d_q"],
                 p["d_k"], p["d_val"], p["d_u"], p["d_v"], p["d_Rk"], p["d_W_kR"], p["ws"],
                 ws_bytes, None)

    assert bwd(_shape(txl, dtype=txl.TXL_F32)) == 5
    assert bwd(s, d_out=None) == 1
    assert bwd(s, d_q=None) == 1
    assert bwd(s, d_Rk=None) == 1
    assert bwd(s, mem=None) == 1
    assert bwd(s, mem_start=16) == 2
    assert bwd(s, Rk=288, d_W_kR=304) == 2          # no W_kR gradient with a caller Rk
    assert bwd(s, ws_bytes=wsb - 1) == 4
    assert bwd(s, ws=None) == 1


def test_rel_attn_training_pair_validation(txl):
    """txl_rel_attn_fwd_train / txl_rel_attn_bwd_saved reject bad arguments
    before anything is enqueued (fake, 16-byte aligned addresses: nothing is
    dereferenced on these paths)."""
    s = _shape(txl)
    wsb = txl.txl_rel_attn_bwd_workspace_bytes(s)
    fwd = txl.lib.txl_rel_attn_fwd_train
    bwd = txl.lib.txl_rel_attn_bwd_saved

    def fwd_call(shape, ws_bytes=wsb, **kw):
        p = dict(h=16, mem=32, mem_start=0, W_q=48, W_kE=64, W_kR=80, W_v=96, u=112, v=128,
                 R=144, Rk=None, out=160, ws=176)
        p.update(kw)
        return fwd(ctypes.byref(shape), p["h"], p["mem"], p["mem_start"], p["W_q"], p["W_kE"],
                   p["W_kR"], p["W_v"], p["u"], p["v"], p["R"], p["Rk"], p["out"], p["ws"],
                   ws_bytes, None)

    def bwd_call(shape, ws_bytes=wsb, **kw):
        p = dict(u=112, v=128, R=144, rk_given=0, out=160, d_out=192, d_q=208, d_k=224,
                 d_val=240, d_u=256, d_v=272, d_Rk=288, d_W_kR=None, ws=176)
        p.update(kw)
        return bwd(ctypes.byref(shape), p["u"], p["v"], p["R"], p["rk_given"], p["out"],
                   p["d_out"], p["d_q"], p["d_k"], p["d_val"], p["d_u"], p["d_v"], p["d_Rk"],
                   p["d_W_kR"], p["ws"], ws_bytes, None)

    assert fwd_call(_shape(txl, dtype=txl.TXL_F32)) == 5
    assert fwd_call(s, out=None) == 1
    assert fwd_call(s, mem=None) == 1
    assert fwd_call(s, mem_start=16) == 2
    assert fwd_call(s, W_kR=None) == 1                 # neither Rk nor W_kR
    assert fwd_call(s, h=24) == 5                      # misaligned bf16 operand
    assert fwd_call(s, ws_bytes=wsb - 1) == 4
    assert fwd_call(s, ws=None) == 1
    assert bwd_call(_shape(txl, dtype=txl.TXL_F32)) == 5
    assert bwd_call(s, u=None) == 1
    assert bwd_call(s, out=None) == 1
    assert bwd_call(s, d_out=None) == 1
    assert bwd_call(s, d_q=None) == 1
    assert bwd_call(s, d_Rk=None) == 1
    assert bwd_call(s, ws=None) == 1
    assert bwd_call(s, rk_given=1, d_W_kR=304) == 2    # no W_kR gradient with a caller Rk
    assert bwd_call(s, R=None, d_W_kR=304) == 2        # d_W_kR needs R
    assert bwd_call(s, d_out=200) == 5                 # misaligned
    assert bwd_call(s, ws_bytes=wsb - 1) == 4
