"""Python access to the C oracle (``txl_oracle.c``), in float64.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the
CPU-baseline leg of the benchmark. The HIP library never imports it.

Every function takes numpy arrays (any float dtype; converted to float64) and
returns float64 arrays. Parameters are dicts with the keys ``Wq, WkE, WkR,
Wv, Wo`` (``[D, D]``, out-major), ``u, v`` (``[D]``) and, for full layers,
``ln1_g, ln1_b, W1 [F, D], b1, W2 [D, F], b2, ln2_g, ln2_b``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "txl_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``.

    Portable flags only (no -march=native): the library is built here and may
    run on another host.
    """
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        L.orc_set_num_threads.restype = ctypes.c_int
        L.orc_sinusoid_table.argtypes = [ctypes.c_int, ctypes.c_int, _dp]
        L.orc_linear.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.orc_layer_norm.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, _dp, _dp]
        L.orc_rel_attn.argtypes = [ctypes.c_int] * 5 + [_dp] * 2 + [_dp] * 7 + [_dp, ctypes.c_int] + [_dp] * 4
        L.orc_layer_fwd.argtypes = [ctypes.c_int] * 6 + [_dp] * 2 + [_dp] * 7 + [_dp] * 8 + [_dp, ctypes.c_int, _dp]
        L.orc_mem_update.argtypes = [ctypes.c_int] * 4 + [_dp, ctypes.c_int, _dp, _dp, _ip]
        L.orc_stack_fwd.argtypes = ([ctypes.c_int] * 9 + [_dp] + [_dp] * 7 + [_dp] * 8
                                    + [_dp, ctypes.c_int, _dp, _dp, _ip, _dp, _ip])
        L.orc_attn_variant.argtypes = [ctypes.c_int] * 6 + [_dp] * 8 + [ctypes.c_int, _dp]
        L.orc_add_positions.argtypes = [ctypes.c_int] * 4 + [_dp, _dp]
        L.orc_rel_attn_bwd.argtypes = [ctypes.c_int] * 5 + [_dp] * 13
        for f in ("orc_sinusoid_table", "orc_linear", "orc_layer_norm", "orc_rel_attn",
                  "orc_layer_fwd", "orc_mem_update", "orc_stack_fwd", "orc_attn_variant",
                  "orc_add_positions", "orc_rel_attn_bwd"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_dp)


def _check(st: int, what: str) -> None:
    if st != 0:
        raise ValueError(f"oracle {what} failed with status {st}")


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> int:
    """Thread count of the oracle's OpenMP loops from now on; returns the count in use."""
    return int(lib().orc_set_num_threads(n))


def sinusoid_table(R_len: int, D: int) -> np.ndarray:
    R = np.empty((R_len, D), dtype=np.float64)
    _check(lib().orc_sinusoid_table(R_len, D, _ptr(R)), "sinusoid_table")
    return R


def linear(x: np.ndarray, Wt: np.ndarray) -> np.ndarray:
    x = _f64(x)
    Wt = _f64(Wt)
    Dout, Din = Wt.shape
    lead = x.shape[:-1]
    xf = x.reshape(-1, Din)
    y = np.empty((xf.shape[0], Dout), dtype=np.float64)
    _check(lib().orc_linear(xf.shape[0], Din, Dout, _ptr(xf), _ptr(Wt), _ptr(y)), "linear")
    return y.reshape(*lead, Dout)


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray) -> np.ndarray:
    x = _f64(x)
    D = x.shape[-1]
    xf = x.reshape(-1, D)
    y = np.empty_like(xf)
    _check(lib().orc_layer_norm(xf.shape[0], D, _ptr(xf), _ptr(_f64(g)), _ptr(_f64(b)), _ptr(y)),
           "layer_norm")
    return y.reshape(x.shape)


_ATTN_KEYS = ("Wq", "WkE", "WkR", "Wv", "Wo", "u", "v")
_LAYER_KEYS = ("ln1_g", "ln1_b", "W1", "b1", "W2", "b2", "ln2_g", "ln2_b")


def rel_attn(h: np.ndarray, mem: Optional[np.ndarray], p: Dict[str, np.ndarray], R: np.ndarray,
             H: int, return_terms: bool = False):
    """Relative attention + output projection of one segment.

    h [B, W, D]; mem [B, m, D] oldest first (None or m == 0 for an empty memory);
    R [R_len, D] with R_len >= m + W. Returns out [B, W, D] and, with
    ``return_terms``, also P, AC, BD as [B, H, W, m+W] arrays.
    """
    h = _f64(h)
    B, W, D = h.shape
    m = 0 if mem is None else mem.shape[1]
    memf = _f64(mem) if m > 0 else None
    R = _f64(R)
    ps = [_f64(p[k]) for k in _ATTN_KEYS]
    out = np.empty((B, W, D), dtype=np.float64)
    K = m + W
    P = AC = BD = None
    if return_terms:
        P = np.empty((B, H, W, K))
        AC = np.empty((B, H, W, K))
        BD = np.empty((B, H, W, K))
    st = lib().orc_rel_attn(B, W, D, H, m, _ptr(h), _ptr(memf), *[_ptr(a) for a in ps],
                            _ptr(R), R.shape[0], _ptr(out), _ptr(P), _ptr(AC), _ptr(BD))
    _check(st, "rel_attn")
    return (out, P, AC, BD) if return_terms else out


POS_SHAW, POS_ABSOLUTE = 1, 2


def attn_variant(mode: int, h: np.ndarray, mem: Optional[np.ndarray], p: Dict[str, np.ndarray], H: int,
                 aK: Optional[np.ndarray] = None, aV: Optional[np.ndarray] = None, clip: int = 0) -> np.ndarray:
    """Attention + output projection with the encodings Transformer-XL is compared
    against: POS_SHAW (clipped learned embeddings aK, aV [clip+1, dh] on keys and
    values) or POS_ABSOLUTE (content attention; positions already in the rows)."""
    h = _f64(h)
    B, W, D = h.shape
    m = 0 if mem is None else mem.shape[1]
    memf = _f64(mem) if m > 0 else None
    ps = [_f64(p[k]) for k in ("Wq", "WkE", "Wv", "Wo")]
    ak = _f64(aK) if aK is not None else None
    av = _f64(aV) if aV is not None else None
    out = np.empty((B, W, D), dtype=np.float64)
    st = lib().orc_attn_variant(mode, B, W, D, H, m, _ptr(h), _ptr(memf), *[_ptr(a) for a in ps],
                                _ptr(ak), _ptr(av), clip, _ptr(out))
    _check(st, "attn_variant")
    return out


def rel_attn_bwd(q: np.ndarray, k: np.ndarray, val: np.ndarray, r: np.ndarray, u: np.ndarray, v: np.ndarray,
                 dO: np.ndarray, H: int) -> Dict[str, np.ndarray]:
    """Gradients of relative attention (before W_o) w.r.t. its projected operands,
    memory behind a stop-gradient. q, dO [B, W, D]; k, val [B, K, D] (memory rows
    first, K = m + W); r [K, D]; u, v [D]. Returns dq, dk, dval, dr, du, dv."""
    q, k, val, r, u, v, dO = (_f64(a) for a in (q, k, val, r, u, v, dO))
    B, W, D = q.shape
    K = k.shape[1]
    out = {"dq": np.empty((B, W, D)), "dk": np.empty((B, K, D)), "dval": np.empty((B, K, D)),
           "dr": np.empty((K, D)), "du": np.empty(D), "dv": np.empty(D)}
    st = lib().orc_rel_attn_bwd(B, W, D, H, K - W, _ptr(q), _ptr(k), _ptr(val), _ptr(r), _ptr(u), _ptr(v),
                                _ptr(dO), *[_ptr(out[n]) for n in ("dq", "dk", "dval", "dr", "du", "dv")])
    _check(st, "rel_attn_bwd")
    return out


def add_positions(x: np.ndarray, pos0: int = 0) -> np.ndarray:
    """x [B, W, D] plus the absolute sinusoid of positions pos0 .. pos0 + W - 1."""
    x = _f64(x)
    B, W, D = x.shape
    y = np.empty_like(x)
    _check(lib().orc_add_positions(B, W, D, pos0, _ptr(x), _ptr(y)), "add_positions")
    return y


def layer_fwd(h: np.ndarray, mem: Optional[np.ndarray], p: Dict[str, np.ndarray], R: np.ndarray,
              H: int) -> np.ndarray:
    h = _f64(h)
    B, W, D = h.shape
    m = 0 if mem is None else mem.shape[1]
    memf = _f64(mem) if m > 0 else None
    R = _f64(R)
    F = p["W1"].shape[0]
    ps = [_f64(p[k]) for k in _ATTN_KEYS]
    ls = [_f64(p[k]) for k in _LAYER_KEYS]
    y = np.empty((B, W, D), dtype=np.float64)
    st = lib().orc_layer_fwd(B, W, D, H, F, m, _ptr(h), _ptr(memf), *[_ptr(a) for a in ps],
                             *[_ptr(a) for a in ls], _ptr(R), R.shape[0], _ptr(y))
    _check(st, "layer_fwd")
    return y


def mem_update(mem: Optional[np.ndarray], h: np.ndarray, M: int) -> np.ndarray:
    """Logical memory after one segment: the last min(M, m+W) rows of [mem; h]."""
    h = _f64(h)
    B, W, D = h.shape
    m = 0 if mem is None else mem.shape[1]
    memf = _f64(mem) if m > 0 else None
    out = np.empty((B, M, D), dtype=np.float64)
    nm = ctypes.c_int(0)
    _check(lib().orc_mem_update(B, M, D, m, _ptr(memf), W, _ptr(h), _ptr(out), ctypes.byref(nm)),
           "mem_update")
    return out[:, :nm.value].copy()


def stack_fwd(x: np.ndarray, params: Sequence[Dict[str, np.ndarray]], R: np.ndarray, H: int,
              W: int, M: int, full_layer: bool,
              mems0: Optional[Sequence[np.ndarray]] = None) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Segment-by-segment forward over the stream x [B, S*W, D].

    ``mems0`` (optional): the logical memory of every layer to start from
    ([B, m_l, D] each, oldest row first, m_l <= M), as returned by an earlier
    call; by default every memory starts empty.

    Returns y [B, S*W, D] (last layer's output per segment) and the final
    logical memory of every layer ([B, m_l, D] each).
    """
    x = _f64(x)
    B, T, D = x.shape
    assert T % W == 0
    S = T // W
    L = len(params)
    F = params[0]["W1"].shape[0] if full_layer else 0

    def stk(k, shape):
        return np.ascontiguousarray(np.stack([_f64(p[k]) for p in params]).reshape(L, *shape))

    arrs = [stk(k, (D, D)) for k in ("Wq", "WkE", "WkR", "Wv", "Wo")]
    arrs += [stk("u", (D,)), stk("v", (D,))]
    if full_layer:
        lay = [stk("ln1_g", (D,)), stk("ln1_b", (D,)), stk("W1", (F, D)), stk("b1", (F,)),
               stk("W2", (D, F)), stk("b2", (D,)), stk("ln2_g", (D,)), stk("ln2_b", (D,))]
    else:
        lay = [None] * 8
    R = _f64(R)
    y = np.empty_like(x)
    mems = np.zeros((L, B, M, D))
    lens = (ctypes.c_int * L)()
    mems_in, lens_in = None, None
    if mems0 is not None:
        assert len(mems0) == L
        mems_in = np.zeros((L, B, M, D))
        lens_in = (ctypes.c_int * L)()
        for l, mm in enumerate(mems0):
            ml = 0 if mm is None else mm.shape[1]
            assert ml <= M
            if ml:
                mems_in[l, :, :ml] = _f64(mm)
            lens_in[l] = ml
    st = lib().orc_stack_fwd(B, W, D, H, F, L, S, M, 1 if full_layer else 0, _ptr(x),
                             *[_ptr(a) for a in arrs], *[_ptr(a) for a in lay],
                             _ptr(R), R.shape[0], _ptr(y), _ptr(mems),
                             ctypes.cast(lens, _ip), _ptr(mems_in),
                             None if lens_in is None else ctypes.cast(lens_in, _ip))
    _check(st, "stack_fwd")
    return y, [mems[l, :, :lens[l]].copy() for l in range(L)]
