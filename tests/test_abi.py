"""C-ABI contract tests that need no GPU.

The library must load, export every function include/txl.h declares, size
workspaces, and reject bad arguments with a status code before it touches the
HIP runtime (so these calls are safe without a device: the pointers passed
here are never dereferenced).
"""
import ctypes

import pytest

from transformer_xl_segment_amd import binding as tb


def test_header_functions_are_exported():
    L = tb.lib()
    names = tb.exported_names()
    assert "txl_rel_attn_fwd" in names and "txl_stack_fwd_segments" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in txl.h but not exported"
    assert len(names) >= 10


def test_status_strings():
    L = tb.lib()
    for st in range(5):
        assert L.txl_status_string(st)
    assert L.txl_status_string(99) == b"unknown status"


def test_workspace_sizes():
    L = tb.lib()
    ws = L.txl_workspace_bytes
    a = ws(tb.OP_REL_ATTN, tb.TXL_BF16, 16, 512, 512, 512, 8, 0)
    assert a > 0 and a % 256 == 0
    # a layer needs at least what attention needs; the stack at least the layer
    lay = ws(tb.OP_LAYER, tb.TXL_BF16, 16, 512, 512, 512, 8, 2048)
    stk = ws(tb.OP_STACK, tb.TXL_BF16, 16, 512, 512, 512, 8, 2048)
    assert a < lay < stk
    # fp32 operands take more room than bf16
    assert ws(tb.OP_REL_ATTN, tb.TXL_FP32, 16, 512, 512, 512, 8, 0) > a
    # monotone in the memory capacity
    assert ws(tb.OP_REL_ATTN, tb.TXL_BF16, 16, 512, 1024, 512, 8, 0) > a
    # invalid sizes
    assert ws(tb.OP_REL_ATTN, tb.TXL_BF16, 16, 512, 512, 510, 8, 0) == 0   # D % H
    assert ws(tb.OP_REL_ATTN, tb.TXL_BF16, 0, 512, 512, 512, 8, 0) == 0
    assert ws(tb.OP_LAYER, tb.TXL_BF16, 1, 4, 4, 16, 2, 0) == 0          # F missing
    assert ws(7, tb.TXL_BF16, 1, 4, 4, 16, 2, 0) == 0


FAKE = 1 << 20   # an aligned, never-dereferenced address


def _params():
    return tb._Params(*[FAKE] * len(tb._PARAM_FIELDS))


def _attn(dt=tb.TXL_FP32, B=1, W=4, D=16, H=2, hs=64, mem=None, p=None, R=FAKE, R_len=8,
          out=FAKE, os_=64, ws=None, wsb=0):
    L = tb.lib()
    p = p if p is not None else _params()
    return L.txl_rel_attn_fwd(dt, B, W, D, H, FAKE, hs, ctypes.byref(mem) if mem else None,
                              ctypes.byref(p), R, R_len, out, os_, ws, wsb, None)


def test_rel_attn_rejects_bad_arguments():
    assert _attn(D=18, H=4) == tb.TXL_ERR_ARG            # D % H
    assert _attn(D=15, H=3) == tb.TXL_ERR_ARG            # odd D
    assert _attn(B=0) == tb.TXL_ERR_ARG
    assert _attn(dt=5) == tb.TXL_ERR_UNSUPPORTED
    assert _attn(D=130, H=1, hs=520, os_=520, R_len=8) == tb.TXL_ERR_UNSUPPORTED   # dh > 64
    assert _attn(hs=10) == tb.TXL_ERR_ARG                # batch stride < W*D
    assert _attn(out=FAKE + 2) == tb.TXL_ERR_ARG          # misaligned
    assert _attn(R=None) == tb.TXL_ERR_ARG
    assert _attn(R_len=3) == tb.TXL_ERR_ARG               # R_len < m + W
    p = _params()
    p.WkR = None
    assert _attn(p=p) == tb.TXL_ERR_ARG
    bad_len = tb._Mem(FAKE, 4, 5, 0)                       # len > M
    assert _attn(mem=bad_len) == tb.TXL_ERR_ARG
    bad_head = tb._Mem(FAKE, 4, 2, 4)                      # head >= M
    assert _attn(mem=bad_head) == tb.TXL_ERR_ARG
    ok_mem = tb._Mem(FAKE, 4, 4, 1)
    assert _attn(mem=ok_mem, R_len=7) == tb.TXL_ERR_ARG    # needs 4 + 4 rows
    # everything valid but no workspace
    assert _attn(mem=ok_mem, R_len=8) == tb.TXL_ERR_WORKSPACE
    assert b"workspace" in tb.lib().txl_last_error()


def test_noalloc_rejects_bad_arguments_and_oversized_calls():
    # every check of txl_rel_attn_fwd_noalloc runs before its first device call
    L = tb.lib()
    assert tb.NOALLOC_SCRATCH_BYTES == 64 << 20
    import re
    hdr = open(tb.HEADER_PATH).read()
    assert re.search(r"#define TXL_NOALLOC_SCRATCH_BYTES \(64u << 20\)", hdr)
    p = _params()

    def call(B=1, W=4, D=16, H=2, hs=64, mem=None, R=FAKE, R_len=8, out=FAKE, os_=64, dt=tb.TXL_BF16):
        return L.txl_rel_attn_fwd_noalloc(dt, B, W, D, H, FAKE, hs, ctypes.byref(mem) if mem else None,
                                          ctypes.byref(p), R, R_len, out, os_, None)
    assert call(D=18, H=4) == tb.TXL_ERR_ARG
    assert call(dt=5) == tb.TXL_ERR_UNSUPPORTED
    assert call(R=None) == tb.TXL_ERR_ARG
    assert call(out=FAKE + 2) == tb.TXL_ERR_ARG
    assert call(mem=tb._Mem(FAKE, 4, 5, 0)) == tb.TXL_ERR_ARG
    # the headline shape fits the fixed scratch; twice its batch does not
    ws = L.txl_workspace_bytes
    assert ws(tb.OP_REL_ATTN, tb.TXL_BF16, 16, 512, 512, 512, 8, 0) <= tb.NOALLOC_SCRATCH_BYTES
    assert ws(tb.OP_REL_ATTN, tb.TXL_BF16, 32, 512, 512, 512, 8, 0) > tb.NOALLOC_SCRATCH_BYTES
    big = tb._Mem(FAKE, 512, 512, 0)
    assert call(B=32, W=512, D=512, H=8, hs=512 * 512, os_=512 * 512, mem=big, R_len=1024) == tb.TXL_ERR_WORKSPACE
    assert b"scratch" in L.txl_last_error()


def test_fused_update_rejects_bad_arguments_and_leaves_memory():
    # txl_rel_attn_fwd_update: the checks of txl_rel_attn_fwd plus a non-NULL
    # memory; on any error the ring's len / head stay as they were
    L = tb.lib()
    p = _params()

    def call(mem, B=1, W=4, D=16, H=2, hs=64, R=FAKE, R_len=8, out=FAKE, os_=64, dt=tb.TXL_BF16, ws=None,
             wsb=0):
        return L.txl_rel_attn_fwd_update(dt, B, W, D, H, FAKE, hs, ctypes.byref(mem) if mem else None,
                                         ctypes.byref(p), R, R_len, out, os_, ws, wsb, None)
    assert call(None) == tb.TXL_ERR_ARG
    assert b"NULL" in L.txl_last_error()
    m = tb._Mem(FAKE, 4, 4, 1)
    assert call(m, D=18, H=4) == tb.TXL_ERR_ARG
    assert call(m, R_len=7) == tb.TXL_ERR_ARG                # needs 4 + 4 rows
    assert call(m, out=FAKE + 2) == tb.TXL_ERR_ARG
    assert call(m) == tb.TXL_ERR_WORKSPACE                    # valid, no workspace
    assert (m.len, m.head) == (4, 1)
    bad = tb._Mem(FAKE, 4, 5, 0)
    assert call(bad) == tb.TXL_ERR_ARG
    assert (bad.len, bad.head) == (5, 0)


def test_mem_update_rejects_bad_arguments():
    L = tb.lib()
    m = tb._Mem(FAKE, 4, 0, 0)
    assert L.txl_mem_update(tb.TXL_FP32, 1, 16, None, FAKE, 64, 4, None) == tb.TXL_ERR_ARG
    assert L.txl_mem_update(tb.TXL_FP32, 1, 16, ctypes.byref(m), None, 64, 4, None) == tb.TXL_ERR_ARG
    assert L.txl_mem_update(tb.TXL_FP32, 1, 16, ctypes.byref(m), FAKE, 63, 4, None) == tb.TXL_ERR_ARG
    m.len = 9
    assert L.txl_mem_update(tb.TXL_FP32, 1, 16, ctypes.byref(m), FAKE, 64, 4, None) == tb.TXL_ERR_ARG
    assert (m.len, m.head) == (9, 0)     # untouched on failure


def test_layer_and_stack_reject_bad_arguments():
    L = tb.lib()
    p = _params()
    # missing FFN weight
    q = _params()
    q.W1 = None
    assert L.txl_layer_fwd(tb.TXL_FP32, 1, 4, 16, 2, 32, FAKE, 64, None, ctypes.byref(q), FAKE, 4,
                           FAKE, 64, None, 0, None) == tb.TXL_ERR_ARG
    # odd F
    assert L.txl_layer_fwd(tb.TXL_FP32, 1, 4, 16, 2, 31, FAKE, 64, None, ctypes.byref(p), FAKE, 4,
                           FAKE, 64, None, 0, None) == tb.TXL_ERR_ARG
    # D > 1024 for the LayerNorm kernels
    assert L.txl_layer_fwd(tb.TXL_FP32, 1, 4, 1040, 26, 32, FAKE, 4160, None, ctypes.byref(p), FAKE, 4,
                           FAKE, 4160, None, 0, None) == tb.TXL_ERR_UNSUPPORTED
    assert L.txl_layer_fwd(tb.TXL_FP32, 1, 4, 16, 2, 32, FAKE, 64, None, ctypes.byref(p), FAKE, 4,
                           FAKE, 64, None, 0, None) == tb.TXL_ERR_WORKSPACE
    mems = (tb._Mem * 2)(tb._Mem(FAKE, 4, 0, 0), tb._Mem(FAKE, 8, 0, 0))   # unequal M
    ps = (tb._Params * 2)(_params(), _params())
    assert L.txl_stack_fwd_segments(tb.TXL_FP32, 1, 4, 16, 2, 32, 2, 3, FAKE, mems, ps, FAKE, 16,
                                    FAKE, None, 0, None) == tb.TXL_ERR_ARG
    mems[1].M = 4
    assert L.txl_stack_fwd_segments(tb.TXL_FP32, 1, 4, 16, 2, 32, 2, 3, FAKE, mems, ps, FAKE, 7,
                                    FAKE, None, 0, None) == tb.TXL_ERR_ARG      # R_len < M + W
    assert L.txl_stack_fwd_segments(tb.TXL_FP32, 1, 4, 16, 2, 32, 2, 3, FAKE, mems, ps, FAKE, 8,
                                    FAKE, None, 0, None) == tb.TXL_ERR_WORKSPACE


def test_stack_window_rejects_bad_arguments():
    L = tb.lib()
    ps = (tb._Params * 2)(_params(), _params())
    win = lambda n_layers=2, xs=64, R_len=4, ys=64, F=32, p=ps: L.txl_stack_fwd_window(
        tb.TXL_FP32, 1, 4, 16, 2, F, n_layers, FAKE, xs, p, FAKE, R_len, FAKE + 4096, ys, None, 0, None)
    assert win(n_layers=0) == tb.TXL_ERR_ARG
    assert win(xs=63) == tb.TXL_ERR_ARG                 # x batch stride < W*D
    assert win(ys=32) == tb.TXL_ERR_ARG
    assert win(R_len=3) == tb.TXL_ERR_ARG               # R_len < W
    assert win(F=31) == tb.TXL_ERR_ARG
    assert win(p=None) == tb.TXL_ERR_ARG
    q = (tb._Params * 2)(_params(), _params())
    q[1].ln2_g = None
    assert win(p=q) == tb.TXL_ERR_ARG
    assert win(xs=1 << 20) == tb.TXL_ERR_WORKSPACE      # a window of a longer stream
    # the window needs the stack's workspace with no memory
    ws = L.txl_workspace_bytes(tb.OP_STACK, tb.TXL_FP32, 1, 4, 0, 16, 2, 32)
    assert 0 < ws < L.txl_workspace_bytes(tb.OP_STACK, tb.TXL_FP32, 1, 4, 128, 16, 2, 32)


def test_variants_reject_bad_arguments():
    L = tb.lib()
    p = _params()
    def var(v=tb.POS_SHAW, clip=4, aK=FAKE, aV=FAKE, W=4, hs=64, mem=None, pp=p):
        return L.txl_attn_fwd_variant(tb.TXL_FP32, v, 1, W, 16, 2, FAKE, hs, ctypes.byref(mem) if mem else None,
                                      ctypes.byref(pp) if pp else None, aK, aV, clip, FAKE, 64, None, 0, None)
    assert var(v=0) == tb.TXL_ERR_ARG
    assert var(v=3) == tb.TXL_ERR_ARG
    assert var(clip=-1) == tb.TXL_ERR_UNSUPPORTED
    assert var(clip=129) == tb.TXL_ERR_UNSUPPORTED
    assert var(aK=None) == tb.TXL_ERR_ARG
    assert var(aV=FAKE + 2) == tb.TXL_ERR_ARG
    assert var(hs=10) == tb.TXL_ERR_ARG
    assert var(pp=None) == tb.TXL_ERR_ARG
    q = _params()
    q.Wv = None
    assert var(pp=q) == tb.TXL_ERR_ARG
    q = _params()
    q.WkR = None; q.u = None; q.v = None                 # not read by the variants
    assert var(pp=q) == tb.TXL_ERR_WORKSPACE
    assert var(v=tb.POS_ABSOLUTE, aK=None, aV=None) == tb.TXL_ERR_WORKSPACE
    assert var(mem=tb._Mem(FAKE, 4, 5, 0)) == tb.TXL_ERR_ARG
    # workspace: the attention layout plus one float per query
    a = L.txl_workspace_bytes(tb.OP_REL_ATTN, tb.TXL_BF16, 16, 512, 512, 512, 8, 0)
    v = L.txl_workspace_bytes(tb.OP_ATTN_VARIANT, tb.TXL_BF16, 16, 512, 512, 512, 8, 0)
    assert v == a + 16 * 8 * 512 * 4
    pos = lambda D=16, xs=64, ys=64, pos0=0: L.txl_add_positions(tb.TXL_FP32, 1, 4, D, FAKE, xs, pos0, FAKE, ys, None)
    assert pos(D=15, xs=60, ys=60) == tb.TXL_ERR_ARG
    assert pos(pos0=-1) == tb.TXL_ERR_ARG
    assert pos(xs=63) == tb.TXL_ERR_ARG
    assert L.txl_add_positions(tb.TXL_FP32, 1, 4, 1026, FAKE, 4104, 0, FAKE, 4104, None) == tb.TXL_ERR_UNSUPPORTED
    assert L.txl_add_positions(7, 1, 4, 16, FAKE, 64, 0, FAKE, 64, None) == tb.TXL_ERR_UNSUPPORTED


def test_backward_rejects_bad_arguments():
    L = tb.lib()
    def bwd(m=2, W=4, D=16, H=2, ins=None, outs=None, wsb=0):
        ins = ins or [FAKE] * 7
        outs = outs or [FAKE] * 6
        return L.txl_rel_attn_bwd(tb.TXL_FP32, 1, W, D, H, m, *ins, *outs, None, wsb, None)
    assert bwd(m=-1) == tb.TXL_ERR_ARG
    assert bwd(m=4090, W=8) == tb.TXL_ERR_UNSUPPORTED              # m + W > 4096
    assert bwd(D=130, H=1) == tb.TXL_ERR_UNSUPPORTED               # dh > 64
    assert bwd(ins=[FAKE] * 6 + [None]) == tb.TXL_ERR_ARG          # dO
    assert bwd(outs=[FAKE + 2] + [FAKE] * 5) == tb.TXL_ERR_ARG     # misaligned dq
    assert bwd() == tb.TXL_ERR_WORKSPACE
    ws = L.txl_workspace_bytes(tb.OP_REL_ATTN_BWD, tb.TXL_BF16, 2, 64, 64, 128, 2, 0)
    assert ws > L.txl_workspace_bytes(tb.OP_REL_ATTN, tb.TXL_BF16, 2, 64, 64, 128, 2, 0)
    assert L.txl_workspace_bytes(tb.OP_REL_ATTN_BWD, tb.TXL_BF16, 1, 64, 4096, 128, 2, 0) == 0


def test_kv_cache_capacity_and_workspace():
    L = tb.lib()
    assert L.txl_kv_cache_capacity(512, 512) == 1024
    assert L.txl_kv_cache_capacity(1600, 128) == 1728
    assert L.txl_kv_cache_capacity(8, 8) == 64
    assert L.txl_kv_cache_capacity(0, 64) == 64
    assert L.txl_kv_cache_capacity(-1, 64) == 0 and L.txl_kv_cache_capacity(8, 0) == 0
    ws = L.txl_workspace_bytes
    c = ws(tb.OP_REL_ATTN_CACHED, tb.TXL_BF16, 16, 512, 512, 512, 8, 0)
    # no context keys and values in the workspace: they live in the cache
    assert 0 < c < ws(tb.OP_REL_ATTN, tb.TXL_BF16, 16, 512, 512, 512, 8, 0)


def _cache(M=8, C=64, len_=0, head=0, k=FAKE, vt=FAKE):
    return tb._KV(k, vt, C, M, len_, head)


def _cached(c, dt=tb.TXL_FP32, B=1, W=8, D=16, H=2, R_len=16, wsb=0):
    L = tb.lib()
    p = _params()
    return L.txl_rel_attn_fwd_cached(dt, B, W, D, H, FAKE, W * D, ctypes.byref(c) if c else None,
                                     ctypes.byref(p), FAKE, R_len, FAKE, W * D, None, wsb, None)


def test_kv_cache_calls_reject_bad_arguments():
    assert _cached(None) == tb.TXL_ERR_ARG
    assert _cached(_cache(M=12)) == tb.TXL_ERR_UNSUPPORTED          # M % 8
    assert _cached(_cache(), W=4, R_len=8) == tb.TXL_ERR_UNSUPPORTED  # W % 8
    assert _cached(_cache(C=60)) == tb.TXL_ERR_ARG                   # C % 64
    assert _cached(_cache(M=64, C=64)) == tb.TXL_ERR_ARG             # C < M + W
    assert _cached(_cache(len_=16)) == tb.TXL_ERR_ARG                # len > M
    assert _cached(_cache(len_=4)) == tb.TXL_ERR_ARG                 # len % 8
    assert _cached(_cache(head=64)) == tb.TXL_ERR_ARG                # head >= C
    assert _cached(_cache(head=4)) == tb.TXL_ERR_ARG                 # head % 8
    assert _cached(_cache(k=None)) == tb.TXL_ERR_ARG
    assert _cached(_cache(vt=FAKE + 8)) == tb.TXL_ERR_ARG            # 16-byte alignment
    c = _cache(len_=8, head=56)
    assert _cached(c, R_len=15) == tb.TXL_ERR_ARG                    # R_len < len + W
    assert _cached(c, R_len=16) == tb.TXL_ERR_WORKSPACE
    assert (c.len, c.head) == (8, 56)                                # untouched on failure
    L = tb.lib()
    p = _params()
    app = lambda c, n, xs=128: L.txl_kv_cache_append(tb.TXL_FP32, 1, 16, 2, ctypes.byref(c),
                                                     ctypes.byref(p), FAKE, xs, n, None)
    assert app(_cache(), 0) == tb.TXL_ERR_ARG
    assert app(_cache(), 4, xs=64) == tb.TXL_ERR_UNSUPPORTED         # n % 8
    assert app(_cache(), 8, xs=63) == tb.TXL_ERR_ARG                 # x batch stride
    assert app(_cache(M=16, C=16), 8) == tb.TXL_ERR_ARG              # C % 64


def test_sinusoid_and_profiler_reject_bad_arguments():
    L = tb.lib()
    assert L.txl_sinusoid_table(tb.TXL_FP32, 8, 15, FAKE, None) == tb.TXL_ERR_ARG
    assert L.txl_sinusoid_table(tb.TXL_FP32, 0, 16, FAKE, None) == tb.TXL_ERR_ARG
    assert L.txl_sinusoid_table(3, 8, 16, FAKE, None) == tb.TXL_ERR_UNSUPPORTED
    assert L.txl_profile_begin(0) == tb.TXL_ERR_ARG
    ms, n = ctypes.c_double(), ctypes.c_int()
    assert L.txl_profile_end(ctypes.byref(ms), ctypes.byref(n)) == tb.TXL_ERR_ARG   # not active
    assert L.txl_profile_times(None, 4, ctypes.byref(n)) == tb.TXL_ERR_ARG            # no buffer
    assert L.txl_profile_times(None, -1, ctypes.byref(n)) == tb.TXL_ERR_ARG
    assert L.txl_profile_times(None, 0, ctypes.byref(n)) == tb.TXL_OK and n.value == 0


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(tb, "_lib", None)
    monkeypatch.setattr(tb, "LIB_PATH", str(tmp_path / "libtxl.so"))
    with pytest.raises(RuntimeError, match="missing"):
        tb.lib()
