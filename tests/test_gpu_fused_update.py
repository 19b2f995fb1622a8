"""GPU tests of txl_rel_attn_fwd_update: the attention of a segment and the
memory update (simulator: mem = last M rows of [mem; h]) in one call, the copy
carried by the output projection's launch. Over a stream of segments that
fills, wraps and (W > M) overflows the ring, its outputs and the ring's raw
slots equal those of txl_rel_attn_fwd followed by txl_mem_update bit for bit,
and the outputs stay within tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import binding as tb
from transformer_xl_segment_amd import synthetic as syn

from gpu_cases import TOL, TDT, dev, host, rel_err, say, table

pytestmark = pytest.mark.gpu


def _segments(x, W, misaligned):
    """Segment views of x [B, S*W, D]; misaligned=True re-packs every segment with
    a batch stride that is 4-byte but not 16-byte aligned (the word-wise copy)."""
    B, T, D = x.shape
    out = []
    for t in range(T // W):
        seg = x[:, t * W:(t + 1) * W]
        if misaligned:
            buf = torch.zeros(B, W * D + 2, dtype=x.dtype, device=x.device)
            buf[:, :W * D] = seg.reshape(B, W * D)
            seg = torch.as_strided(buf, (B, W, D), (W * D + 2, D, 1))
        out.append(seg)
    return out


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,W,M,D,H,S,misaligned", [
    (3, 40, 100, 64, 2, 5, False),     # fills, then wraps
    (2, 40, 30, 48, 3, 3, False),      # W > M: only the last M rows enter
    (2, 24, 50, 82, 2, 4, True),       # dword-aligned rows and batch stride
])
def test_fused_update_equals_separate_calls(dtype, B, W, M, D, H, S, misaligned):
    say(f"fused update {dtype} B={B} W={W} M={M} D={D} H={H} misaligned={misaligned}")
    wl = syn.Workload("fused", dtype, B=B, D=D, H=H, W=W, M=M, S=S, op="attn", seed_w=5000 + D, seed_x=6000 + W)
    prob = syn.draw_problem(wl)
    tdt = TDT[dtype]
    x = dev(prob.x, dtype)
    params = tb.LayerParams.from_numpy(prob.params[0], tdt, "cuda")
    R = table(M + W, D, dtype)
    Rd = dev(R, dtype)
    ring_a = tb.MemoryRing.empty(B, M, D, tdt, "cuda")
    ring_b = tb.MemoryRing.empty(B, M, D, tdt, "cuda")
    ring_a.data.zero_()                 # so that the raw slots compare before the ring is full
    ring_b.data.zero_()
    omem = None
    for t, h in enumerate(_segments(x, W, misaligned)):
        a = tb.rel_attn_fwd(h, ring_a, params, Rd, H)
        tb.mem_update(ring_a, h)
        b = tb.rel_attn_fwd_update(h, ring_b, params, Rd, H)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"segment {t}: outputs differ"
        assert (ring_a.len, ring_a.head) == (ring_b.len, ring_b.head)
        assert torch.equal(ring_a.data, ring_b.data), f"segment {t}: ring slots differ"
        hn = prob.x[:, t * W:(t + 1) * W].astype(np.float64)
        ref = orc.rel_attn(hn, omem, prob.params[0], R, H)
        e = rel_err(host(b), ref)
        assert e <= TOL[dtype], (t, e)
        omem = orc.mem_update(omem, hn, M)
        np.testing.assert_array_equal(host(ring_b.logical()), omem)


def test_fused_update_headline_shape():
    # the headline workload (B=16, W=M=512, D=512, H=8, bf16) for three segments:
    # the third starts from a full ring and wraps it
    wl = syn.WORKLOADS["attn_w512_bf16"]
    wl = syn.Workload(**{**wl.__dict__, "S": 3})
    prob = syn.draw_problem(wl)
    B, W, M, D, H = wl.B, wl.W, wl.M, wl.D, wl.H
    say("fused update at the headline shape")
    x = dev(prob.x, "bf16")
    params = tb.LayerParams.from_numpy(prob.params[0], torch.bfloat16, "cuda")
    Rd = tb.sinusoid_table(M + W, D, torch.bfloat16, "cuda")
    ring_a = tb.MemoryRing.empty(B, M, D, torch.bfloat16, "cuda")
    ring_b = tb.MemoryRing.empty(B, M, D, torch.bfloat16, "cuda")
    ring_a.data.zero_()
    ring_b.data.zero_()
    for t, h in enumerate(_segments(x, W, False)):
        a = tb.rel_attn_fwd(h, ring_a, params, Rd, H)
        tb.mem_update(ring_a, h)
        b = tb.rel_attn_fwd_update(h, ring_b, params, Rd, H)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"segment {t}: outputs differ"
        assert (ring_a.len, ring_a.head) == (ring_b.len, ring_b.head)
        assert torch.equal(ring_a.data, ring_b.data), f"segment {t}: ring slots differ"
