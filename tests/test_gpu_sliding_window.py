"""GPU tests of vanilla sliding-window evaluation (txl_stack_fwd_window, and
txl_rel_attn_fwd with no memory over a window), the baseline the pages compare
segment-recurrent evaluation against.

Each window's output is compared with the oracle on that window with an empty
memory. For a single attention layer the memory holds the layer's own input
rows, so the last query of a segment whose memory is full sees exactly the
window of the last M + W rows: there the recurrent output and the window's last
output must agree, which ties the two evaluation procedures together.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import binding as tb
from transformer_xl_segment_amd import synthetic as syn

from gpu_cases import TOL, TDT, dev, host, nan_workspace, rel_err, say, table

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_window_stack_small(dtype):
    B, D, H, F, layers, Lw, T = 2, 82, 2, 130, 3, 45, 120
    say(f"window stack small {dtype}")
    rng = np.random.default_rng(7100)
    params = [syn.draw_layer_params(rng, D, F, dtype, affine=True, scale=0.2 if dtype == "fp32" else 0.1)
              for _ in range(layers)]
    x = syn.draw_stream(np.random.default_rng(7200), B, T, D, dtype)
    R = table(Lw, D, dtype)
    xd, Rd = dev(x, dtype), dev(R, dtype)
    lp = [tb.LayerParams.from_numpy(p, TDT[dtype], "cuda") for p in params]
    ws = nan_workspace(tb.workspace_bytes(tb.OP_STACK, TDT[dtype], B, Lw, 0, D, H, F))
    errs = {}
    for t in (Lw - 1, 77, T - 1):          # window of the Lw rows ending at token t
        win = xd[:, t - Lw + 1:t + 1]       # a view into the stream (batch stride T*D)
        y = tb.stack_fwd_window(win, lp, Rd, H, F, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = orc.stack_fwd(x[:, t - Lw + 1:t + 1], params, R, H, Lw, Lw, True)
        errs[f"t{t}"] = rel_err(host(y), ref)
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


def test_window_stack16_bf16():
    """The 16-layer workload's shape: a window of M + W = 300 rows, every layer
    re-encoded; batch rows 0 and B-1 against the oracle."""
    wl = syn.WORKLOADS["stack16_bf16"]
    say(f"window {wl.name}")
    prob = syn.draw_problem(wl)
    Lw = wl.M + wl.W
    R = table(Lw, wl.D, wl.dtype)
    lp = [tb.LayerParams.from_numpy(p, torch.bfloat16, "cuda") for p in prob.params]
    xd = dev(prob.x, wl.dtype)
    t = 2 * Lw + 37
    y = tb.stack_fwd_window(xd[:, t - Lw + 1:t + 1], lp, dev(R, wl.dtype), wl.H, wl.F,
                            workspace=nan_workspace(tb.workspace_bytes(tb.OP_STACK, torch.bfloat16, wl.B, Lw,
                                                                       0, wl.D, wl.H, wl.F)))
    torch.cuda.synchronize()
    bsel = [0, wl.B - 1]
    ref, _ = orc.stack_fwd(prob.x[bsel, t - Lw + 1:t + 1], prob.params, R, wl.H, Lw, Lw, True)
    e = rel_err(host(y)[bsel], ref)
    say(f"  error {e}")
    assert e <= TOL[wl.dtype]


@pytest.mark.parametrize("dtype,B,D,H,W,M", [("fp32", 2, 64, 2, 24, 40), ("bf16", 2, 128, 2, 64, 136)])
def test_window_attention_equals_recurrent_last_query(dtype, B, D, H, W, M):
    """Single attention layer: the window of the last M + W rows, evaluated with
    no memory, gives at its last row what the recurrent path gives at the last
    query of a segment with a full memory."""
    say(f"window vs recurrent {dtype} W={W} M={M}")
    T = TDT[dtype]
    p = syn.draw_layer_params(np.random.default_rng(7300 + W), D, None, dtype,
                              scale=0.3 if dtype == "fp32" else 0.1)
    S = (M + W - 1) // W + 2
    x = syn.draw_stream(np.random.default_rng(7400 + W), B, S * W, D, dtype)
    Lw = M + W
    R = table(Lw, D, dtype)
    xd, Rd = dev(x, dtype), dev(R, dtype)
    params = tb.LayerParams.from_numpy(p, T, "cuda")
    ring = tb.MemoryRing.empty(B, M, D, T, "cuda")
    checked = 0
    for s in range(S):
        h = xd[:, s * W:(s + 1) * W]
        full = ring.len == M
        out = tb.rel_attn_fwd(h, ring, params, Rd, H)
        tb.mem_update(ring, h)
        if not full:
            continue
        t = (s + 1) * W - 1
        win = tb.rel_attn_fwd(xd[:, t - Lw + 1:t + 1], None, params, Rd, H)
        torch.cuda.synchronize()
        a, b = host(out[:, -1]), host(win[:, -1])
        # the oracle on that one query: m = Lw - 1 memory rows before it
        ref = orc.rel_attn(x[:, t:t + 1].astype(np.float64), x[:, t - Lw + 1:t].astype(np.float64), p, R, H)[:, 0]
        say(f"  t={t}: recurrent {rel_err(a, ref):.2e}, window {rel_err(b, ref):.2e}, "
            f"identical bits: {bool(np.array_equal(a, b))}")
        assert rel_err(a, ref) <= TOL[dtype] and rel_err(b, ref) <= TOL[dtype]
        assert rel_err(b, a) <= TOL[dtype]
        checked += 1
    assert checked >= 2


def test_window_attention_longmem_bf16():
    """The long-memory workload's window (M + W = 1728 keys for the newest
    token), evaluated with no memory, against the oracle on the newest row."""
    wl = syn.WORKLOADS["longmem_m1600_bf16"]
    say(f"window {wl.name}")
    prob = syn.draw_problem(wl)
    Lw = wl.M + wl.W
    stream = np.concatenate([prob.warm_mem, prob.x], axis=1)      # [B, 1600 + 768, D]
    t = stream.shape[1] - 1
    R = table(Lw, wl.D, wl.dtype)
    params = tb.LayerParams.from_numpy(prob.params[0], torch.bfloat16, "cuda")
    sd = dev(stream, wl.dtype)
    win = tb.rel_attn_fwd(sd[:, t - Lw + 1:t + 1], None, params, dev(R, wl.dtype), wl.H)
    torch.cuda.synchronize()
    bsel = [0, wl.B - 1]
    ref = orc.rel_attn(stream[bsel, t:t + 1].astype(np.float64),
                       stream[bsel, t - Lw + 1:t].astype(np.float64), prob.params[0], R, wl.H)[:, 0]
    e = rel_err(host(win[:, -1])[bsel], ref)
    say(f"  error {e}")
    assert e <= TOL[wl.dtype]
