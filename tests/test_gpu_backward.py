"""GPU parity of the relative-attention backward (txl_rel_attn_bwd) with the
oracle: every gradient (dq, dk, dval, dr, du, dv) compared element by element,
including the memory rows of dk and dval, over empty, ragged and long memories,
odd head widths, and the headline workload's per-row shape.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import binding as tb
from transformer_xl_segment_amd import synthetic as syn

from gpu_cases import TOL, TDT, dev, host, nan_workspace, rel_err, say

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dval", "dr", "du", "dv")


def _inputs(seed, B, W, m, D, dtype, scale):
    rng = np.random.default_rng(seed)
    K = m + W
    draw = lambda *shape, s=scale: syn._store(rng.standard_normal(shape) * s, dtype)
    return {"q": draw(B, W, D), "k": draw(B, K, D), "val": draw(B, K, D, s=1.0), "r": draw(K, D),
            "u": draw(D), "v": draw(D), "dO": draw(B, W, D, s=1.0)}


def _gpu(x, H, dtype):
    d = {n: dev(a, dtype) for n, a in x.items()}
    B, W, D = x["q"].shape
    ws = nan_workspace(tb.workspace_bytes(tb.OP_REL_ATTN_BWD, TDT[dtype], B, W, x["k"].shape[1] - W, D, H))
    g = tb.rel_attn_bwd(d["q"], d["k"], d["val"], d["r"], d["u"], d["v"], d["dO"], H, workspace=ws)
    torch.cuda.synchronize()
    return {n: host(t) for n, t in g.items()}


CASES = [
    # name, B, D, H, W, m
    ("dh8_no_memory", 1, 16, 2, 4, 0),
    ("dh32_ragged", 2, 64, 2, 37, 50),
    ("dh64_two_qblocks", 2, 128, 2, 130, 70),
    ("dh41_odd", 2, 82, 2, 29, 45),
    ("dh64_long_memory", 1, 64, 1, 20, 200),
    # one query (W = 1: a single lane of one wave carries data)
    ("dh16_one_query", 1, 32, 2, 1, 3),
    # three query blocks, the last wave partly filled
    ("dh48_three_qblocks", 1, 96, 2, 300, 20),
    # K = m + W = 128 exactly: the last distance window reaches past the padded rows
    ("dh64_k_equals_padding", 2, 64, 1, 100, 28),
    # a long memory behind a five-row segment
    ("dh32_short_segment", 1, 64, 2, 5, 300),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_small(dtype, case):
    name, B, D, H, W, m = case
    say(f"backward {name} {dtype}")
    x = _inputs(9000 + len(name), B, W, m, D, dtype, scale=0.7 if dtype == "fp32" else 0.5)
    g = _gpu(x, H, dtype)
    ref = orc.rel_attn_bwd(x["q"], x["k"], x["val"], x["r"], x["u"], x["v"], x["dO"], H)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_sharp_scores(dtype):
    # stress run: sharp softmax rows (score std about 1.4 s^2 for operand scale s: ~11
    # for fp32 at s = 2.8, ~3 for bf16 at s = 1.5, whose q/k rounding moves a score by
    # ~|s| 2^-8), so p and dS come from the log-sum-exp path far from uniform rows
    B, D, H, W, m = 2, 128, 2, 70, 90
    say(f"backward sharp scores {dtype}")
    x = _inputs(9400, B, W, m, D, dtype, scale=2.8 if dtype == "fp32" else 1.5)
    g = _gpu(x, H, dtype)
    ref = orc.rel_attn_bwd(x["q"], x["k"], x["val"], x["r"], x["u"], x["v"], x["dO"], H)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


def test_backward_headline_shape_bf16():
    # attn_w512_bf16's shape per batch row (W = m = 512, D = 512, 8 heads of 64)
    # with two batch rows, so the batch sums of dr, du, dv are exercised too
    B, D, H, W, m = 2, 512, 8, 512, 512
    say("backward headline shape bf16")
    x = _inputs(9100, B, W, m, D, "bf16", scale=0.5)
    g = _gpu(x, H, "bf16")
    ref = orc.rel_attn_bwd(x["q"], x["k"], x["val"], x["r"], x["u"], x["v"], x["dO"], H)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_wide_launch_bf16():
    # 8 batch rows x 8 heads over K = 512 keys: the gradient GEMMs take 768 tiles, enough for
    # their 128 x 64 tile path (the smaller cases run the 128 x 128 one); all six gradients,
    # dr, du and dv summed over every batch row
    B, D, H, W, m = 8, 512, 8, 128, 384
    say("backward wide launch bf16")
    x = _inputs(9500, B, W, m, D, "bf16", scale=0.5)
    g = _gpu(x, H, "bf16")
    ref = orc.rel_attn_bwd(x["q"], x["k"], x["val"], x["r"], x["u"], x["v"], x["dO"], H)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_full_batch_rows_bf16():
    # the full batch of 16: per-row gradients of rows 0 and 15 against the oracle
    # on those rows alone (rows are independent for dq, dk, dval)
    B, D, H, W, m = 16, 512, 8, 512, 512
    say("backward full batch bf16")
    x = _inputs(9200, B, W, m, D, "bf16", scale=0.5)
    g = _gpu(x, H, "bf16")
    sel = [0, B - 1]
    sub = {n: (a[sel] if n in ("q", "k", "val", "dO") else a) for n, a in x.items()}
    ref = orc.rel_attn_bwd(sub["q"], sub["k"], sub["val"], sub["r"], sub["u"], sub["v"], sub["dO"], H)
    errs = {n: rel_err(g[n][sel], ref[n]) for n in ("dq", "dk", "dval")}
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_memory_rows_and_determinism():
    # keys and values of the memory get gradients (they reach W_kE, W_v), and two
    # runs agree bit for bit
    B, D, H, W, m = 2, 64, 2, 24, 40
    x = _inputs(9300, B, W, m, D, "fp32", scale=0.7)
    a, b = _gpu(x, H, "fp32"), _gpu(x, H, "fp32")
    for n in NAMES:
        np.testing.assert_array_equal(a[n], b[n])
    assert np.abs(a["dk"][:, :m]).max() > 0 and np.abs(a["dval"][:, :m]).max() > 0
