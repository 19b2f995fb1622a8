"""txl_rel_attn_fwd_noalloc against txl_rel_attn_fwd through the C ABI.

The no-allocation variant runs the same launches with the library's fixed
device scratch array in place of the caller's workspace. Two calls in a row
(the second smaller, so the array still holds the first call's data) must
give what txl_rel_attn_fwd gives on the same inputs, and both stay within
tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import binding as tb
from transformer_xl_segment_amd import synthetic as syn

from gpu_cases import TOL, TDT, dev, host, nan_workspace, rel_err, say, table

pytestmark = pytest.mark.gpu


def _case(name, dtype, B, D, H, W, M, seed, scale):
    wl = syn.Workload(name, dtype, B=B, D=D, H=H, W=W, M=M, S=2, seed_w=5000 + seed, seed_x=6000 + seed)
    prob = syn.draw_problem(wl, weight_scale=scale)
    tdt = TDT[dtype]
    params = tb.LayerParams.from_numpy(prob.params[0], tdt, "cuda")
    R = table(M + W, D, dtype)
    ring = tb.MemoryRing.empty(B, M, D, tdt, "cuda")
    tb.mem_update(ring, dev(prob.x[:, :W], dtype))       # m = min(M, W) rows of memory
    h = dev(prob.x[:, W:2 * W], dtype)
    return prob, params, R, ring, h


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    # call 1: the headline shape in bf16 (about 60 MB of scratch), a smaller
    # shape in fp32; call 2: a ragged shape over fewer rows, run right after
    big = (16, 512, 8, 512, 512) if dtype == "bf16" else (4, 256, 4, 200, 180)
    small = (2, 128, 2, 70, 50)
    for i, (B, D, H, W, M) in enumerate([big, small]):
        say(f"noalloc {dtype} call {i + 1}: B={B} D={D} H={H} W={W} M={M}")
        prob, params, R, ring, h = _case(f"noalloc{i}", dtype, B, D, H, W, M, seed=i,
                                         scale=0.02 if i == 0 else 0.1)
        Rd = dev(R, dtype)
        out_na = torch.empty_like(h)
        tb.rel_attn_fwd_noalloc(h, ring, params, Rd, H, out=out_na)
        ws = nan_workspace(tb.workspace_bytes(tb.OP_REL_ATTN, TDT[dtype], B, W, M, D, H))
        out_ws = tb.rel_attn_fwd(h, ring, params, Rd, H, workspace=ws)
        torch.cuda.synchronize()
        g_na, g_ws = host(out_na), host(out_ws)
        rows = [0, B - 1]
        m = ring.len
        ref = orc.rel_attn(prob.x[rows, W:2 * W].astype(np.float64),
                           prob.x[rows, W - m:W].astype(np.float64), prob.params[0], R, H)
        errs = {"noalloc_vs_workspace": rel_err(g_na, g_ws), "noalloc_vs_oracle": rel_err(g_na[rows], ref),
                "workspace_vs_oracle": rel_err(g_ws[rows], ref)}
        say(f"  errors {errs}")
        assert max(errs.values()) <= TOL[dtype], errs
        # same launches on the same inputs: the results are identical
        assert np.array_equal(g_na, g_ws)
