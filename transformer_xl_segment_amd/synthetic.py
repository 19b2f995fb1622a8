"""Seeded synthetic workloads for the Transformer-XL relative-attention path.

This module only draws random numbers and stores them in the dtype a workload
asks for. It holds none of the method's arithmetic (no projection, score,
softmax, normalisation or positional encoding), so both the HIP path and the
CPU oracle can take their inputs from it without sharing any computation.

The pages train and evaluate on language-modelling corpora (enwik8, text8,
WikiText-103, One Billion Word, Penn Treebank). Those corpora and trained
weights are not used: seeded Gaussian tensors of the same shapes stand in.
Hidden states are N(0, 1); projection weights and the global biases u, v are
N(0, 0.02), the initialisation scale of the NumPy TransformerXLLayer on
"Implementing Transformer-XL" (mbrenndoerfer.com, the ``__init__`` of the
layer class); FFN biases are zero and LayerNorm gains/offsets are 1/0, as on
that page.

Weights are stored out-major, ``W[d_out, d_in]`` (the torch.nn.Linear layout),
and a projection computes ``y = x @ W.T``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "round_to_bf16", "draw_layer_params",
           "draw_stream", "draw_problem", "Problem"]


@dataclass(frozen=True)
class Workload:
    """One named workload: sizes, storage dtype and which entry point it drives.

    ``op`` is ``"attn"`` (relative attention + output projection, then the memory
    update), ``"layer"`` (attention + residual/LayerNorm/FFN block) or ``"stack"``
    (``layers`` blocks, each with its own memory).
    """
    name: str
    dtype: str          # "fp32" or "bf16"
    B: int
    D: int
    H: int
    W: int
    M: int
    S: int
    layers: int = 1
    F: Optional[int] = None
    op: str = "attn"
    seed_w: int = 0
    seed_x: int = 0
    warm_mem: bool = False   # also draw a full N(0,1) memory of M rows

    @property
    def d_head(self) -> int:
        return self.D // self.H

    def mem_schedule(self) -> List[int]:
        """Valid memory rows m at each segment, starting from an empty memory."""
        m, out = 0, []
        for _ in range(self.S):
            out.append(m)
            m = min(self.M, m + self.W)
        return out


# The five workloads of the relative-attention benchmark suite.
WORKLOADS: Dict[str, Workload] = {
    "tiny_attn_fp32": Workload("tiny_attn_fp32", "fp32", B=1, D=16, H=2, W=4, M=4, S=3,
                               op="attn", seed_w=43, seed_x=124),
    "layer_ffn_fp32": Workload("layer_ffn_fp32", "fp32", B=4, D=128, H=4, W=64, M=64, S=8,
                               F=512, op="layer", seed_w=44, seed_x=125),
    "attn_w512_bf16": Workload("attn_w512_bf16", "bf16", B=16, D=512, H=8, W=512, M=512, S=4,
                               op="attn", seed_w=45, seed_x=126),
    "longmem_m1600_bf16": Workload("longmem_m1600_bf16", "bf16", B=8, D=1024, H=16, W=128,
                                   M=1600, S=6, op="attn", seed_w=46, seed_x=127,
                                   warm_mem=True),
    "stack16_fp32": Workload("stack16_fp32", "fp32", B=32, D=410, H=10, W=150, M=150, S=8,
                             layers=16, F=2100, op="stack", seed_w=47, seed_x=128),
    "stack16_bf16": Workload("stack16_bf16", "bf16", B=32, D=410, H=10, W=150, M=150, S=8,
                             layers=16, F=2100, op="stack", seed_w=47, seed_x=128),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32.

    The returned values are exactly representable in bfloat16, so converting
    them to a bf16 tensor is lossless and both sides see identical inputs.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(a.shape)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_to_bf16(a) if dtype == "bf16" else a


def draw_layer_params(rng: np.random.Generator, D: int, F: Optional[int], dtype: str,
                      affine: bool = False, scale: float = 0.02) -> Dict[str, np.ndarray]:
    """Draw one layer's parameters in the fixed order Wq, WkE, WkR, Wv, Wo, u, v, W1, W2.

    With ``affine`` the FFN biases and LayerNorm gain/offset are drawn too
    (after everything else, so the main draws do not move); otherwise they are
    the constants 0 and 1.
    """
    p: Dict[str, np.ndarray] = {}
    for name in ("Wq", "WkE", "WkR", "Wv", "Wo"):
        p[name] = rng.standard_normal((D, D)) * scale
    p["u"] = rng.standard_normal(D) * scale
    p["v"] = rng.standard_normal(D) * scale
    if F is not None:
        p["W1"] = rng.standard_normal((F, D)) * scale
        p["W2"] = rng.standard_normal((D, F)) * scale
        p["b1"] = np.zeros(F)
        p["b2"] = np.zeros(D)
    p["ln1_g"] = np.ones(D)
    p["ln1_b"] = np.zeros(D)
    p["ln2_g"] = np.ones(D)
    p["ln2_b"] = np.zeros(D)
    if affine:
        if F is not None:
            p["b1"] = rng.standard_normal(F) * scale
            p["b2"] = rng.standard_normal(D) * scale
        p["ln1_g"] = 1.0 + rng.standard_normal(D) * 0.1
        p["ln1_b"] = rng.standard_normal(D) * 0.1
        p["ln2_g"] = 1.0 + rng.standard_normal(D) * 0.1
        p["ln2_b"] = rng.standard_normal(D) * 0.1
    return {k: _store(v, dtype) for k, v in p.items()}


def draw_stream(rng: np.random.Generator, B: int, T: int, D: int, dtype: str,
                scale: float = 1.0) -> np.ndarray:
    """Hidden states ``[B, T, D]`` drawn N(0, scale^2)."""
    return _store(rng.standard_normal((B, T, D)) * scale, dtype)


@dataclass
class Problem:
    wl: Workload
    params: List[Dict[str, np.ndarray]]
    x: np.ndarray                       # [B, S*W, D] stack / segment-stream input
    warm_mem: Optional[np.ndarray] = None   # [B, M, D]
    extra: dict = field(default_factory=dict)


def draw_problem(wl: Workload, affine: bool = False, weight_scale: float = 0.02,
                 batch: Optional[int] = None) -> Problem:
    """All inputs of a workload from its two seeds (weights, then inputs).

    ``batch`` keeps only the first ``batch`` sequences of the input draw (the
    full draw is made first, so every kept row is identical to the full
    workload's).
    """
    rw = np.random.default_rng(wl.seed_w)
    params = [draw_layer_params(rw, wl.D, wl.F, wl.dtype, affine=affine, scale=weight_scale)
              for _ in range(wl.layers)]
    rx = np.random.default_rng(wl.seed_x)
    x = draw_stream(rx, wl.B, wl.S * wl.W, wl.D, wl.dtype)
    warm = draw_stream(rx, wl.B, wl.M, wl.D, wl.dtype) if wl.warm_mem else None
    if batch is not None:
        x = x[:batch].copy()
        warm = None if warm is None else warm[:batch].copy()
    return Problem(wl, params, x, warm)
