"""GPU parity of the encodings Transformer-XL is compared against
(txl_attn_fwd_variant, txl_add_positions) with the oracle.

Shaw et al.: learned clipped-distance embeddings on keys and values, checked
with clips below, inside and beyond the key range (clip 0 sends every distance
to one embedding). Absolute positions: the model adds positions 0 .. W-1 to
every segment's rows, caches those rows, and attends by content only; the
oracle adds the positions itself in float64.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import binding as tb
from transformer_xl_segment_amd import synthetic as syn

from gpu_cases import TOL, TDT, dev, host, nan_workspace, rel_err, say

pytestmark = pytest.mark.gpu


def _tables(rng, clip, dh, dtype, scale):
    aK = syn.round_to_bf16(rng.standard_normal((clip + 1, dh)).astype(np.float32) * scale) if dtype == "bf16" \
        else (rng.standard_normal((clip + 1, dh)) * scale).astype(np.float32)
    aV = syn.round_to_bf16(rng.standard_normal((clip + 1, dh)).astype(np.float32)) if dtype == "bf16" \
        else rng.standard_normal((clip + 1, dh)).astype(np.float32)
    return aK, aV


def _run(variant, dtype, B, D, H, W, M, S, clip, seed, wscale, batch=None, tscale=1.0):
    T = TDT[dtype]
    rng = np.random.default_rng(seed)
    p = syn.draw_layer_params(rng, D, None, dtype, scale=wscale)
    x = syn.draw_stream(rng, B, S * W, D, dtype)
    dh = D // H
    aK, aV = _tables(rng, clip, dh, dtype, tscale) if variant == tb.POS_SHAW else (None, None)
    params = tb.LayerParams.from_numpy(p, T, "cuda")
    ring = tb.MemoryRing.empty(B, M, D, T, "cuda")
    ws = nan_workspace(tb.workspace_bytes(tb.OP_ATTN_VARIANT, T, B, W, M, D, H))
    xd = dev(x, dtype)
    aKd = dev(aK, dtype) if aK is not None else None
    aVd = dev(aV, dtype) if aV is not None else None
    bsel = list(range(B)) if batch is None else batch
    omem, errs = None, {}
    for t in range(S):
        h = xd[:, t * W:(t + 1) * W]
        hn = x[bsel, t * W:(t + 1) * W].astype(np.float64)
        if variant == tb.POS_ABSOLUTE:
            h = tb.add_positions(h, 0)                 # positions 0 .. W-1 in every segment
            hn = orc.add_positions(hn, 0)
        out = tb.attn_fwd_variant(h, ring, params, variant, H, aK=aKd, aV=aVd, clip=clip, workspace=ws)
        tb.mem_update(ring, h)
        torch.cuda.synchronize()
        ref = orc.attn_variant(variant, hn, omem, p, H, aK=aK, aV=aV, clip=clip)
        errs[f"seg{t}"] = rel_err(host(out)[bsel], ref)
        omem = orc.mem_update(omem, hn, M)
    return errs


SHAW_CASES = [
    # name, B, D, H, W, M, S, clip
    ("dh8_clip0", 1, 16, 2, 4, 4, 3, 0),
    ("dh32_clip5_ragged", 2, 64, 2, 37, 50, 3, 5),
    ("dh64_clip64_two_qblocks", 2, 128, 2, 130, 70, 3, 64),
    ("dh41_clip120_beyond_keys", 2, 82, 2, 29, 45, 3, 120),
    ("dh64_clip128_long_mem", 1, 64, 1, 40, 300, 2, 128),
    ("dh64_clip64_key_split", 1, 64, 1, 40, 700, 2, 64),     # 3 key parts, merged log-sum-exp
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", SHAW_CASES, ids=[c[0] for c in SHAW_CASES])
def test_shaw_small(dtype, case):
    name, B, D, H, W, M, S, clip = case
    say(f"shaw {name} {dtype}")
    errs = _run(tb.POS_SHAW, dtype, B, D, H, W, M, S, clip, seed=8000 + len(name),
                wscale=0.3 if dtype == "fp32" else 0.1, tscale=1.0 if dtype == "fp32" else 0.5)
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


ABS_CASES = [
    ("dh8", 1, 16, 2, 4, 4, 3),
    ("dh32_ragged", 2, 64, 2, 37, 50, 3),
    ("dh64_two_qblocks", 2, 128, 2, 130, 70, 3),
    ("dh41", 2, 82, 2, 29, 45, 3),
    ("dh64_key_split", 1, 64, 1, 40, 700, 2),                 # 3 key parts
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", ABS_CASES, ids=[c[0] for c in ABS_CASES])
def test_absolute_small(dtype, case):
    name, B, D, H, W, M, S = case
    say(f"absolute {name} {dtype}")
    errs = _run(tb.POS_ABSOLUTE, dtype, B, D, H, W, M, S, 0, seed=8100 + len(name),
                wscale=0.3 if dtype == "fp32" else 0.1)
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("variant,clip", [(tb.POS_SHAW, 64), (tb.POS_ABSOLUTE, 0)], ids=["shaw", "absolute"])
def test_variants_attn_w512_bf16(variant, clip):
    wl = syn.WORKLOADS["attn_w512_bf16"]
    say(f"variant {variant} {wl.name}")
    errs = _run(variant, "bf16", wl.B, wl.D, wl.H, wl.W, wl.M, 2, clip, seed=8200, wscale=0.02,
                batch=[0, wl.B - 1])
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL["bf16"], errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_add_positions(dtype):
    B, W, D = 3, 77, 410
    x = syn.draw_stream(np.random.default_rng(8300), B, W, D, dtype)
    for pos0 in (0, 1000):
        y = host(tb.add_positions(dev(x, dtype), pos0))
        ref = orc.add_positions(x, pos0)
        # sin/cos rounded to fp32, the fp32 sum rounded once more, then one
        # rounding to the storage type (half an ulp of the result)
        U = np.abs(ref - x)
        bound = (2.0 ** -8 if dtype == "bf16" else 2.0 ** -24) * np.abs(ref) + 2.0 ** -23 * (np.abs(x) + U) + 1e-30
        assert np.all(np.abs(y - ref) <= bound), float(np.max(np.abs(y - ref) / bound))
    # in place
    xd = dev(x, dtype)
    tb.add_positions(xd, 0, y=xd)
    np.testing.assert_array_equal(host(xd), host(tb.add_positions(dev(x, dtype), 0)))
