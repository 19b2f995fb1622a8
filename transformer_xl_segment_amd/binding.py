"""Thin ctypes binding of libtxl (include/txl.h), with the same entry-point names.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. torch is
imported before the library is loaded so that libtxl binds to the HIP runtime
torch already holds (both ask for the soname libamdhip64.so.7).

If libtxl.so has not been built, every entry point raises: there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch  # noqa: F401  (must precede loading libtxl.so)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtxl.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "txl.h")

TXL_OK, TXL_ERR_ARG, TXL_ERR_UNSUPPORTED, TXL_ERR_WORKSPACE, TXL_ERR_HIP = range(5)
TXL_FP32, TXL_BF16 = 0, 1
OP_REL_ATTN, OP_LAYER, OP_STACK, OP_REL_ATTN_CACHED, OP_ATTN_VARIANT, OP_REL_ATTN_BWD = 0, 1, 2, 3, 4, 5
POS_SHAW, POS_ABSOLUTE = 1, 2

_PARAM_FIELDS = ("Wq", "WkE", "WkR", "Wv", "Wo", "u", "v", "ln1_g", "ln1_b", "W1", "b1",
                 "W2", "b2", "ln2_g", "ln2_b")


class TxlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _PARAM_FIELDS]


class _Mem(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("M", ctypes.c_int), ("len", ctypes.c_int),
                ("head", ctypes.c_int)]


class _KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("vt", ctypes.c_void_p), ("C", ctypes.c_int),
                ("M", ctypes.c_int), ("len", ctypes.c_int), ("head", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtxl.so; raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -m transformer_xl_segment_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i, ll, vp, sz = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_size_t
        P, Mp = ctypes.POINTER(_Params), ctypes.POINTER(_Mem)
        L.txl_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
        L.txl_workspace_bytes.restype = sz
        L.txl_sinusoid_table.argtypes = [i, i, i, vp, vp]
        L.txl_rel_attn_fwd.argtypes = [i, i, i, i, i, vp, ll, Mp, P, vp, i, vp, ll, vp, sz, vp]
        L.txl_rel_attn_fwd_noalloc.argtypes = [i, i, i, i, i, vp, ll, Mp, P, vp, i, vp, ll, vp]
        L.txl_rel_attn_fwd_update.argtypes = [i, i, i, i, i, vp, ll, Mp, P, vp, i, vp, ll, vp, sz, vp]
        L.txl_mem_update.argtypes = [i, i, i, Mp, vp, ll, i, vp]
        L.txl_layer_fwd.argtypes = [i, i, i, i, i, i, vp, ll, Mp, P, vp, i, vp, ll, vp, sz, vp]
        L.txl_stack_fwd_segments.argtypes = [i, i, i, i, i, i, i, i, vp, Mp, P, vp, i, vp, vp, sz, vp]
        L.txl_attn_fwd_variant.argtypes = [i, i, i, i, i, i, vp, ll, Mp, P, vp, vp, i, vp, ll, vp, sz, vp]
        L.txl_add_positions.argtypes = [i, i, i, i, vp, ll, i, vp, ll, vp]
        L.txl_rel_attn_bwd.argtypes = [i, i, i, i, i, i] + [vp] * 7 + [vp] * 6 + [vp, sz, vp]
        L.txl_stack_fwd_window.argtypes = [i, i, i, i, i, i, i, vp, ll, P, vp, i, vp, ll, vp, sz, vp]
        KVp = ctypes.POINTER(_KV)
        L.txl_kv_cache_capacity.argtypes = [i, i]
        L.txl_kv_cache_append.argtypes = [i, i, i, i, KVp, P, vp, ll, i, vp]
        L.txl_rel_attn_fwd_cached.argtypes = [i, i, i, i, i, vp, ll, KVp, P, vp, i, vp, ll, vp, sz, vp]
        L.txl_profile_begin.argtypes = [i]
        L.txl_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
        L.txl_profile_times.argtypes = [ctypes.POINTER(ctypes.c_double), i, ctypes.POINTER(ctypes.c_int)]
        for f in ("txl_sinusoid_table", "txl_rel_attn_fwd", "txl_rel_attn_fwd_noalloc", "txl_rel_attn_fwd_update",
                  "txl_mem_update", "txl_layer_fwd",
                  "txl_stack_fwd_segments", "txl_stack_fwd_window", "txl_kv_cache_capacity",
                  "txl_attn_fwd_variant", "txl_add_positions", "txl_rel_attn_bwd", "txl_kv_cache_append",
                  "txl_rel_attn_fwd_cached", "txl_profile_begin", "txl_profile_end", "txl_profile_times"):
            getattr(L, f).restype = i
        L.txl_status_string.argtypes = [i]
        L.txl_status_string.restype = ctypes.c_char_p
        L.txl_last_error.argtypes = []
        L.txl_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(st: int, what: str) -> None:
    if st != TXL_OK:
        L = lib()
        raise TxlError(st, f"{what}: {L.txl_status_string(st).decode()}: {L.txl_last_error().decode()}")


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return TXL_FP32
    if dt == torch.bfloat16:
        return TXL_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _rows_view(t: torch.Tensor, name: str) -> int:
    """Batch stride of a [B, W, D] view whose rows are contiguous."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [B, W, D] with contiguous rows")
    return t.stride(0)


@dataclass
class MemoryRing:
    """Segment memory of one layer: ring buffer data [B, M, D] plus (len, head)."""
    data: torch.Tensor
    len: int = 0
    head: int = 0

    @classmethod
    def empty(cls, B: int, M: int, D: int, dtype: torch.dtype, device) -> "MemoryRing":
        return cls(torch.zeros(B, M, D, dtype=dtype, device=device))

    @property
    def M(self) -> int:
        return self.data.shape[1]

    def _struct(self) -> _Mem:
        return _Mem(self.data.data_ptr(), self.M, self.len, self.head)

    def _update_from(self, s: _Mem) -> None:
        self.len, self.head = int(s.len), int(s.head)

    def logical(self) -> torch.Tensor:
        """Valid rows in logical order (oldest first), [B, len, D] (a copy)."""
        idx = (torch.arange(self.len, device=self.data.device) + self.head) % self.M
        return self.data[:, idx]


def head_pad(dh: int) -> int:
    """Padded head width of the head-major projected layouts (dh rounded up to 16)."""
    return (dh + 15) // 16 * 16


def kv_cache_capacity(M: int, W: int) -> int:
    return int(lib().txl_kv_cache_capacity(M, W))


@dataclass
class KVCache:
    """Projected key/value cache of one layer: k [B, H, C, dp], vt [B, H, dp, C] plus
    (M, len, head); key j of the window lives in slot (head + j) % C."""
    k: torch.Tensor
    vt: torch.Tensor
    M: int
    len: int = 0
    head: int = 0

    @classmethod
    def empty(cls, B: int, M: int, W: int, D: int, H: int, dtype: torch.dtype, device) -> "KVCache":
        C = kv_cache_capacity(M, W)
        dp = head_pad(D // H)
        return cls(torch.zeros(B, H, C, dp, dtype=dtype, device=device),
                   torch.zeros(B, H, dp, C, dtype=dtype, device=device), M)

    @property
    def C(self) -> int:
        return self.k.shape[2]

    def _struct(self) -> _KV:
        return _KV(self.k.data_ptr(), self.vt.data_ptr(), self.C, self.M, self.len, self.head)

    def _update_from(self, s: _KV) -> None:
        self.len, self.head = int(s.len), int(s.head)

    def logical(self, dh: int):
        """Cached keys and values in logical order: ([B, H, len, dh], [B, H, len, dh])."""
        idx = (torch.arange(self.len, device=self.k.device) + self.head) % self.C
        return self.k[:, :, idx, :dh], self.vt[:, :, :dh, idx].transpose(2, 3)


class LayerParams:
    """One layer's parameter tensors (device, one dtype), by the names of txl.h."""

    def __init__(self, tensors: Dict[str, torch.Tensor]):
        self.tensors = {k: v.contiguous() for k, v in tensors.items()}

    @classmethod
    def from_numpy(cls, p: Dict, dtype: torch.dtype, device) -> "LayerParams":
        return cls({k: torch.as_tensor(v).to(device=device, dtype=dtype) for k, v in p.items()})

    def _struct(self) -> _Params:
        return _Params(*[_ptr(self.tensors.get(n)) for n in _PARAM_FIELDS])


def workspace_bytes(op: int, dtype: torch.dtype, B: int, W: int, M: int, D: int, H: int, F: int = 0) -> int:
    return int(lib().txl_workspace_bytes(op, dtype_code(dtype), B, W, M, D, H, F))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def sinusoid_table(R_len: int, D: int, dtype: torch.dtype, device) -> torch.Tensor:
    R = torch.empty(R_len, D, dtype=dtype, device=device)
    _check(lib().txl_sinusoid_table(dtype_code(dtype), R_len, D, R.data_ptr(), _stream(R.device)),
           "txl_sinusoid_table")
    return R


def rel_attn_fwd(h: torch.Tensor, mem: Optional[MemoryRing], params: LayerParams, R: torch.Tensor,
                 H: int, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    if out is None:
        out = torch.empty(B, W, D, dtype=h.dtype, device=h.device)
    os_ = _rows_view(out, "out")
    M = mem.M if mem is not None else 0
    nbytes = workspace_bytes(OP_REL_ATTN, h.dtype, B, W, M, D, H)
    ws = _workspace(nbytes, h.device, workspace)
    ms = mem._struct() if mem is not None else None
    ps = params._struct()
    _check(lib().txl_rel_attn_fwd(dtype_code(h.dtype), B, W, D, H, h.data_ptr(), hs,
                                  ctypes.byref(ms) if ms is not None else None, ctypes.byref(ps),
                                  R.data_ptr(), R.shape[0], out.data_ptr(), os_, ws.data_ptr(),
                                  ws.numel() * ws.element_size(), _stream(h.device)),
           "txl_rel_attn_fwd")
    return out


def rel_attn_fwd_update(h: torch.Tensor, mem: MemoryRing, params: LayerParams, R: torch.Tensor,
                        H: int, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rel_attn_fwd then mem_update(mem, h) in one call (txl_rel_attn_fwd_update)."""
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    if out is None:
        out = torch.empty(B, W, D, dtype=h.dtype, device=h.device)
    os_ = _rows_view(out, "out")
    nbytes = workspace_bytes(OP_REL_ATTN, h.dtype, B, W, mem.M, D, H)
    ws = _workspace(nbytes, h.device, workspace)
    ms = mem._struct()
    ps = params._struct()
    _check(lib().txl_rel_attn_fwd_update(dtype_code(h.dtype), B, W, D, H, h.data_ptr(), hs, ctypes.byref(ms),
                                         ctypes.byref(ps), R.data_ptr(), R.shape[0], out.data_ptr(), os_,
                                         ws.data_ptr(), ws.numel() * ws.element_size(), _stream(h.device)),
           "txl_rel_attn_fwd_update")
    mem._update_from(ms)
    return out


# TXL_NOALLOC_SCRATCH_BYTES of txl.h: the fixed scratch of txl_rel_attn_fwd_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20


def rel_attn_fwd_noalloc(h: torch.Tensor, mem: Optional[MemoryRing], params: LayerParams, R: torch.Tensor,
                         H: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """txl_rel_attn_fwd with the library's fixed scratch array in place of a
    workspace (pass ``out`` to make the call allocate nothing at all)."""
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    if out is None:
        out = torch.empty(B, W, D, dtype=h.dtype, device=h.device)
    os_ = _rows_view(out, "out")
    ms = mem._struct() if mem is not None else None
    ps = params._struct()
    _check(lib().txl_rel_attn_fwd_noalloc(dtype_code(h.dtype), B, W, D, H, h.data_ptr(), hs,
                                          ctypes.byref(ms) if ms is not None else None, ctypes.byref(ps),
                                          R.data_ptr(), R.shape[0], out.data_ptr(), os_, _stream(h.device)),
           "txl_rel_attn_fwd_noalloc")
    return out


def kv_cache_append(cache: KVCache, params: LayerParams, x: torch.Tensor, H: int) -> None:
    B, n, D = x.shape
    xs = _rows_view(x, "x")
    cs, ps = cache._struct(), params._struct()
    _check(lib().txl_kv_cache_append(dtype_code(x.dtype), B, D, H, ctypes.byref(cs), ctypes.byref(ps),
                                     x.data_ptr(), xs, n, _stream(x.device)), "txl_kv_cache_append")
    cache._update_from(cs)


def rel_attn_fwd_cached(h: torch.Tensor, cache: KVCache, params: LayerParams, R: torch.Tensor,
                        H: int, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    if out is None:
        out = torch.empty(B, W, D, dtype=h.dtype, device=h.device)
    os_ = _rows_view(out, "out")
    nbytes = workspace_bytes(OP_REL_ATTN_CACHED, h.dtype, B, W, cache.M, D, H)
    ws = _workspace(nbytes, h.device, workspace)
    cs, ps = cache._struct(), params._struct()
    _check(lib().txl_rel_attn_fwd_cached(dtype_code(h.dtype), B, W, D, H, h.data_ptr(), hs,
                                         ctypes.byref(cs), ctypes.byref(ps), R.data_ptr(), R.shape[0],
                                         out.data_ptr(), os_, ws.data_ptr(),
                                         ws.numel() * ws.element_size(), _stream(h.device)),
           "txl_rel_attn_fwd_cached")
    cache._update_from(cs)
    return out


def attn_fwd_variant(h: torch.Tensor, mem: Optional[MemoryRing], params: LayerParams, variant: int, H: int,
                     aK: Optional[torch.Tensor] = None, aV: Optional[torch.Tensor] = None, clip: int = 0,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention + output projection with Shaw et al.'s (POS_SHAW, tables aK, aV
    [clip+1, dh]) or absolute-position (POS_ABSOLUTE) encoding."""
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    if out is None:
        out = torch.empty(B, W, D, dtype=h.dtype, device=h.device)
    os_ = _rows_view(out, "out")
    M = mem.M if mem is not None else 0
    ws = _workspace(workspace_bytes(OP_ATTN_VARIANT, h.dtype, B, W, M, D, H), h.device, workspace)
    ms = mem._struct() if mem is not None else None
    ps = params._struct()
    aK = aK.contiguous() if aK is not None else None
    aV = aV.contiguous() if aV is not None else None
    _check(lib().txl_attn_fwd_variant(dtype_code(h.dtype), variant, B, W, D, H, h.data_ptr(), hs,
                                      ctypes.byref(ms) if ms is not None else None, ctypes.byref(ps),
                                      _ptr(aK), _ptr(aV), clip, out.data_ptr(), os_, ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream(h.device)),
           "txl_attn_fwd_variant")
    return out


def add_positions(x: torch.Tensor, pos0: int = 0, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B, W, D] plus the absolute sinusoid of positions pos0 .. pos0 + W - 1."""
    B, W, D = x.shape
    xs = _rows_view(x, "x")
    if y is None:
        y = torch.empty(B, W, D, dtype=x.dtype, device=x.device)
    ys = _rows_view(y, "y")
    _check(lib().txl_add_positions(dtype_code(x.dtype), B, W, D, x.data_ptr(), xs, pos0, y.data_ptr(), ys,
                                   _stream(x.device)), "txl_add_positions")
    return y


def rel_attn_bwd(q: torch.Tensor, k: torch.Tensor, val: torch.Tensor, r: torch.Tensor, u: torch.Tensor,
                 v: torch.Tensor, dO: torch.Tensor, H: int,
                 workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Gradients (fp32) of relative attention w.r.t. its projected operands, the
    memory behind a stop-gradient: q, dO [B, W, D]; k, val [B, K, D]; r [>=K, D]."""
    B, W, D = q.shape
    K = k.shape[1]
    ins = [t.contiguous() for t in (q, k, val, r, u, v, dO)]
    dev = q.device
    f32 = torch.float32
    out = {"dq": torch.empty(B, W, D, dtype=f32, device=dev), "dk": torch.empty(B, K, D, dtype=f32, device=dev),
           "dval": torch.empty(B, K, D, dtype=f32, device=dev), "dr": torch.empty(K, D, dtype=f32, device=dev),
           "du": torch.empty(D, dtype=f32, device=dev), "dv": torch.empty(D, dtype=f32, device=dev)}
    ws = _workspace(workspace_bytes(OP_REL_ATTN_BWD, q.dtype, B, W, K - W, D, H), dev, workspace)
    _check(lib().txl_rel_attn_bwd(dtype_code(q.dtype), B, W, D, H, K - W, *[t.data_ptr() for t in ins],
                                  *[out[n].data_ptr() for n in ("dq", "dk", "dval", "dr", "du", "dv")],
                                  ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev)),
           "txl_rel_attn_bwd")
    return out


def mem_update(mem: MemoryRing, h: torch.Tensor) -> None:
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    ms = mem._struct()
    _check(lib().txl_mem_update(dtype_code(h.dtype), B, D, ctypes.byref(ms), h.data_ptr(), hs, W,
                                _stream(h.device)), "txl_mem_update")
    mem._update_from(ms)


def layer_fwd(h: torch.Tensor, mem: Optional[MemoryRing], params: LayerParams, R: torch.Tensor,
              H: int, F: int, y: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, W, D = h.shape
    hs = _rows_view(h, "h")
    if y is None:
        y = torch.empty(B, W, D, dtype=h.dtype, device=h.device)
    ys = _rows_view(y, "y")
    M = mem.M if mem is not None else 0
    ws = _workspace(workspace_bytes(OP_LAYER, h.dtype, B, W, M, D, H, F), h.device, workspace)
    ms = mem._struct() if mem is not None else None
    ps = params._struct()
    _check(lib().txl_layer_fwd(dtype_code(h.dtype), B, W, D, H, F, h.data_ptr(), hs,
                               ctypes.byref(ms) if ms is not None else None, ctypes.byref(ps),
                               R.data_ptr(), R.shape[0], y.data_ptr(), ys, ws.data_ptr(),
                               ws.numel() * ws.element_size(), _stream(h.device)), "txl_layer_fwd")
    return y


def stack_fwd_segments(x: torch.Tensor, mems: Sequence[MemoryRing], params: Sequence[LayerParams],
                       R: torch.Tensor, H: int, W: int, F: int, y: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, T, D = x.shape
    if T % W:
        raise ValueError("stream length must be a multiple of W")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous [B, n_seg*W, D]")
    if y is None:
        y = torch.empty_like(x)
    L = len(params)
    M = mems[0].M
    ws = _workspace(workspace_bytes(OP_STACK, x.dtype, B, W, M, D, H, F), x.device, workspace)
    ms = (_Mem * L)(*[m._struct() for m in mems])
    ps = (_Params * L)(*[p._struct() for p in params])
    _check(lib().txl_stack_fwd_segments(dtype_code(x.dtype), B, W, D, H, F, L, T // W, x.data_ptr(), ms, ps,
                                        R.data_ptr(), R.shape[0], y.data_ptr(), ws.data_ptr(),
                                        ws.numel() * ws.element_size(), _stream(x.device)),
           "txl_stack_fwd_segments")
    for m, s in zip(mems, ms):
        m._update_from(s)
    return y


def stack_fwd_window(x: torch.Tensor, params: Sequence[LayerParams], R: torch.Tensor, H: int, F: int,
                     y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The stack over one window x [B, W, D] (rows contiguous, any batch stride) with no memory."""
    B, W, D = x.shape
    xs = _rows_view(x, "x")
    if y is None:
        y = torch.empty(B, W, D, dtype=x.dtype, device=x.device)
    ys = _rows_view(y, "y")
    L = len(params)
    ws = _workspace(workspace_bytes(OP_STACK, x.dtype, B, W, 0, D, H, F), x.device, workspace)
    ps = (_Params * L)(*[p._struct() for p in params])
    _check(lib().txl_stack_fwd_window(dtype_code(x.dtype), B, W, D, H, F, L, x.data_ptr(), xs, ps,
                                      R.data_ptr(), R.shape[0], y.data_ptr(), ys, ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream(x.device)),
           "txl_stack_fwd_window")
    return y


def profile_begin(max_launches: int) -> None:
    _check(lib().txl_profile_begin(max_launches), "txl_profile_begin")


def profile_end():
    """(summed attention-kernel milliseconds, number of timed launches)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int(0)
    _check(lib().txl_profile_end(ctypes.byref(ms), ctypes.byref(n)), "txl_profile_end")
    return ms.value, n.value


def profile_times(capacity: int) -> List[float]:
    """Per-launch attention-kernel milliseconds of the last closed profiling window."""
    buf = (ctypes.c_double * max(capacity, 1))()
    n = ctypes.c_int(0)
    _check(lib().txl_profile_times(buf, capacity, ctypes.byref(n)), "txl_profile_times")
    return [buf[i] for i in range(n.value)]


def exported_names() -> List[str]:
    """Function names declared in include/txl.h."""
    import re
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(txl_\w+)\s*\(", text, re.M)))
