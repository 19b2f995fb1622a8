"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Small cases span several tiles (128-query and 64-key blocks), ragged tails and
every supported head width; the workload cases run the named configurations at
full size, comparing every output of a batch subset (batch rows are
independent, so the subset is exact) and the memory ring bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import binding as tb
from transformer_xl_segment_amd import synthetic as syn

from gpu_cases import TOL, TDT, dev, host, nan_workspace, rel_err, run_attn_segments, say, table

pytestmark = pytest.mark.gpu


def _wl(name, dtype, B, D, H, W, M, S, F=None, layers=1, op="attn", seed=0):
    return syn.Workload(name, dtype, B=B, D=D, H=H, W=W, M=M, S=S, F=F, layers=layers, op=op,
                        seed_w=1000 + seed, seed_x=2000 + seed)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sinusoid_table(dtype):
    say(f"sinusoid {dtype}")
    for R_len, D in [(1, 2), (300, 410), (1728, 1024)]:
        g = host(tb.sinusoid_table(R_len, D, TDT[dtype], "cuda"))
        o = orc.sinusoid_table(R_len, D)
        if dtype == "fp32":
            np.testing.assert_allclose(g, o, rtol=0, atol=1.2e-7)
        else:
            # at most one bf16 step from the correctly rounded value
            ref = syn.round_to_bf16(o.astype(np.float32)).astype(np.float64)
            ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
            assert np.all(np.abs(g - ref) <= ulp + 1e-30)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("W,M", [(4, 4), (3, 7), (9, 4), (5, 10), (64, 64)])
def test_mem_update_bit_exact(dtype, W, M):
    say(f"mem_update {dtype} W={W} M={M}")
    B, D = 3, 18
    rng = np.random.default_rng(W * 100 + M)
    ring = tb.MemoryRing.empty(B, M, D, TDT[dtype], "cuda")
    omem = None
    for t in range(6):
        h = syn.draw_stream(rng, B, W, D, dtype)
        tb.mem_update(ring, dev(h, dtype))
        omem = orc.mem_update(omem, h.astype(np.float64), M)
        torch.cuda.synchronize()
        assert ring.len == omem.shape[1]
        np.testing.assert_array_equal(host(ring.logical()), omem)


ATTN_CASES = [
    # name, B, D, H, W, M, S
    ("dh8_tiny", 1, 16, 2, 4, 4, 3),
    ("dh32_ragged", 2, 64, 2, 37, 50, 3),
    ("dh64_two_qblocks", 2, 128, 2, 130, 70, 3),
    ("dh41_odd", 2, 82, 2, 29, 45, 3),
    ("dh64_wide_mem", 1, 64, 1, 20, 200, 4),
    # few query blocks over many keys: the key range of each query block is
    # split over several workgroups and merged (2, 4 and 4 parts; in the second
    # case the first query block has 3 key blocks for 4 parts, so some parts
    # are empty, and the queries of a wave see none of the last part's keys)
    ("dh64_split_long_mem", 1, 64, 1, 20, 600, 3),
    ("dh64_split_empty_parts", 1, 64, 1, 1024, 16, 2),
    ("dh41_split", 2, 82, 2, 200, 900, 2),
    # bf16 runs 150 queries as two three-wave blocks (96 + 54) and stores only
    # the 48 value rows of d_head 41 padded to 48; the ring wraps in segment 2
    ("dh41_three_wave_blocks", 2, 82, 2, 150, 150, 3),
    # bf16: 320 (b, h) of 150 queries take two rounds as three-wave blocks
    # (640 on 512 slots) but one as two-wave blocks (960 on 1024), so the
    # launch runs 64-query blocks of 64 + 64 + 22 queries, four per CU
    ("dh16_two_wave_grid", 16, 320, 20, 150, 150, 2),
    # fp32 (one four-wave workgroup per CU): 160 (b, h) of 150 queries take two
    # rounds as 320 four-wave blocks, one as 480 two-wave blocks two per CU
    ("dh32_two_wave_grid", 8, 640, 20, 150, 150, 2),
    ("dh64_two_wave_grid", 8, 1280, 20, 150, 150, 2),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_rel_attn_small(dtype, case):
    name, B, D, H, W, M, S = case
    say(f"rel_attn small {name} {dtype}")
    wl = _wl(name, dtype, B, D, H, W, M, S, seed=[c[0] for c in ATTN_CASES].index(name))
    # weights well above the workloads' 0.02 so that every score term matters;
    # bf16 at 5x (score std ~1.3): its q/k rounding moves a score by ~|s| 2^-8,
    # so much sharper rows leave the 2e-2 regime the workloads are held to
    prob = syn.draw_problem(wl, weight_scale=0.3 if dtype == "fp32" else 0.1)
    errs = run_attn_segments(prob, table(M + W, D, dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rel_attn_far_negative_first_scores(dtype):
    # rows near all-ones with q = 5 h and k = -5 h: every score is about
    # -25 dh / sqrt(dh) = -100, i.e. -144 in the kernel's log2 units, so each
    # query's first re-base moves its running maximum far below zero (where
    # 2^-shift overflows); the output must still be the plain softmax average
    say(f"far negative first scores {dtype}")
    B, H, D, W, M, S = 2, 2, 32, 40, 24, 2
    rng = np.random.default_rng(7)
    eye = np.eye(D, dtype=np.float32)
    prm = {"Wq": 5.0 * eye, "WkE": -5.0 * eye, "WkR": np.zeros((D, D), np.float32),
           "Wv": 0.3 * rng.standard_normal((D, D)).astype(np.float32),
           "Wo": 0.3 * rng.standard_normal((D, D)).astype(np.float32),
           "u": np.zeros(D, np.float32), "v": np.zeros(D, np.float32)}
    x = (1.0 + 0.05 * rng.standard_normal((B, S * W, D))).astype(np.float32)
    if dtype == "bf16":
        prm = {k: syn.round_to_bf16(v) for k, v in prm.items()}
        x = syn.round_to_bf16(x)
    wl = syn.Workload("far_negative", dtype, B=B, D=D, H=H, W=W, M=M, S=S, op="attn", seed_w=0, seed_x=0)
    prob = syn.Problem(wl, [prm], x)
    errs = run_attn_segments(prob, table(M + W, D, dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


def test_rel_attn_sharp_scores_bf16():
    # weights x10 over the workloads' scale: sharp attention rows (stress run)
    wl = _wl("sharp", "bf16", 2, 128, 2, 96, 96, 3, seed=5)
    prob = syn.draw_problem(wl, weight_scale=0.2)
    errs = run_attn_segments(prob, table(192, 128, "bf16"))
    say(f"sharp bf16 errors {errs}")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_rel_attn_deterministic():
    wl = _wl("det", "bf16", 2, 128, 2, 130, 70, 1, seed=7)
    prob = syn.draw_problem(wl, weight_scale=0.3)
    x = dev(prob.x, "bf16")
    params = tb.LayerParams.from_numpy(prob.params[0], torch.bfloat16, "cuda")
    R = dev(table(200, 128, "bf16"), "bf16")
    ring = tb.MemoryRing.empty(2, 70, 128, torch.bfloat16, "cuda")
    tb.mem_update(ring, x[:, :70])
    a = tb.rel_attn_fwd(x, ring, params, R, 2)
    b = tb.rel_attn_fwd(x, ring, params, R, 2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _run_block_segments(prob, R, batch=None):
    """Post-LN layer / stack workloads through txl_stack_fwd_segments (or
    txl_layer_fwd for one layer), compared with the oracle's stack driver."""
    wl = prob.wl
    dt = wl.dtype
    B, D, H, W, M, F = prob.x.shape[0], wl.D, wl.H, wl.W, wl.M, wl.F
    x = dev(prob.x, dt)
    params = [tb.LayerParams.from_numpy(p, TDT[dt], "cuda") for p in prob.params]
    Rd = dev(R, dt)
    bsel = list(range(B)) if batch is None else list(batch)
    ref, ref_mems = orc.stack_fwd(prob.x[bsel], prob.params, R, H, W, M, full_layer=True)
    errs = {}
    if len(params) == 1:
        ring = tb.MemoryRing.empty(B, M, D, TDT[dt], "cuda")
        ws = nan_workspace(tb.workspace_bytes(tb.OP_LAYER, TDT[dt], B, W, M, D, H, F))
        outs = []
        for t in range(wl.S):
            h = x[:, t * W:(t + 1) * W]
            outs.append(tb.layer_fwd(h, ring, params[0], Rd, H, F, workspace=ws))
            tb.mem_update(ring, h)
        torch.cuda.synchronize()
        y = torch.cat(outs, dim=1)
        rings = [ring]
    else:
        rings = [tb.MemoryRing.empty(B, M, D, TDT[dt], "cuda") for _ in params]
        ws = nan_workspace(tb.workspace_bytes(tb.OP_STACK, TDT[dt], B, W, M, D, H, F))
        y = tb.stack_fwd_segments(x, rings, params, Rd, H, W, F, workspace=ws)
        torch.cuda.synchronize()
    yh = host(y)[bsel]
    for t in range(wl.S):
        sl = slice(t * W, (t + 1) * W)
        errs[f"seg{t}"] = rel_err(yh[:, sl], ref[:, sl])
    # each ring holds its layer's input rows of the last segments
    for l, r in enumerate(rings):
        assert r.len == ref_mems[l].shape[1]
        e = rel_err(host(r.logical())[bsel], ref_mems[l])
        errs[f"mem{l}"] = e
    return errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("affine", [False, True])
def test_layer_small(dtype, affine):
    say(f"layer small {dtype} affine={affine}")
    wl = _wl("layer_small", dtype, 3, 96, 3, 40, 56, 4, F=160, op="layer", seed=11)
    prob = syn.draw_problem(wl, affine=affine, weight_scale=0.2 if dtype == "fp32" else 0.1)
    errs = _run_block_segments(prob, table(96, 96, dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D,F", [(82, 1100), (96, 2048)])
def test_stack_split_ffn(dtype, D, F):
    # hidden widths of 1024 and more over few row tiles: in fp32 the second FFN
    # product splits its reduction in two at a 64-element boundary (1100 -> 576
    # + 524, 2048 -> 1024 + 1024) and LayerNorm adds the halves (bf16 keeps one
    # reduction); dword-aligned rows (D = 82) and 16-byte aligned ones (D = 96)
    say(f"stack with a split FFN reduction {dtype} D={D} F={F}")
    wl = _wl("stack_split", dtype, 2, D, 2, 24, 30, 3, F=F, layers=2, op="stack", seed=13)
    prob = syn.draw_problem(wl, affine=True, weight_scale=0.2 if dtype == "fp32" else 0.1)
    errs = _run_block_segments(prob, table(54, D, dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_stack_small(dtype):
    say(f"stack small {dtype}")
    wl = _wl("stack_small", dtype, 2, 82, 2, 30, 30, 4, F=130, layers=3, op="stack", seed=12)
    prob = syn.draw_problem(wl, affine=True, weight_scale=0.2 if dtype == "fp32" else 0.1)
    errs = _run_block_segments(prob, table(60, 82, dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[dtype], errs


# ---------------------------------------------------------------------------
# The named workloads at full size.
# ---------------------------------------------------------------------------

def test_workload_tiny_attn_fp32():
    wl = syn.WORKLOADS["tiny_attn_fp32"]
    say(f"workload {wl.name}")
    prob = syn.draw_problem(wl)
    errs = run_attn_segments(prob, table(wl.M + wl.W, wl.D, wl.dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs


def test_workload_layer_ffn_fp32():
    wl = syn.WORKLOADS["layer_ffn_fp32"]
    say(f"workload {wl.name}")
    prob = syn.draw_problem(wl)
    errs = _run_block_segments(prob, table(wl.M + wl.W, wl.D, wl.dtype))
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs


def test_workload_attn_w512_bf16():
    wl = syn.WORKLOADS["attn_w512_bf16"]
    say(f"workload {wl.name}")
    prob = syn.draw_problem(wl)
    errs = run_attn_segments(prob, table(wl.M + wl.W, wl.D, wl.dtype), batch=[0, wl.B - 1])
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs


def test_workload_attn_w512_bf16_library_table():
    # end to end with the distance table the library computes itself
    # (txl_sinusoid_table) on the GPU side; the oracle keeps its own fp64 table
    wl = syn.WORKLOADS["attn_w512_bf16"]
    say(f"workload {wl.name} with the library's sinusoid table")
    prob = syn.draw_problem(wl)
    R_len = wl.M + wl.W
    Rg = tb.sinusoid_table(R_len, wl.D, TDT[wl.dtype], "cuda")
    errs = run_attn_segments(prob, table(R_len, wl.D, wl.dtype), batch=[0, wl.B - 1], R_gpu=Rg)
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs


def test_large_launch_ragged_bf16():
    # enough rows for the projections' 256-row GEMM tiles, with ragged tails in
    # every dimension: 4000 query rows (4000 % 256 = 160), d_model 520 (eight
    # 64-deep k-tiles and one of 8), heads of 52 padded to 64 (640 columns, five
    # 128-column tiles), and a memory that wraps around the ring in segment 2
    wl = _wl("ragged_large", "bf16", B=20, D=520, H=10, W=200, M=300, S=3, seed=77)
    say(f"ragged large launch {wl.B}x{wl.W} D={wl.D} H={wl.H} M={wl.M}")
    prob = syn.draw_problem(wl)
    errs = run_attn_segments(prob, table(wl.M + wl.W, wl.D, wl.dtype), batch=[0, 7, 19])
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs


@pytest.mark.parametrize("warm", [False, True])
def test_workload_longmem_m1600_bf16(warm):
    wl = syn.WORKLOADS["longmem_m1600_bf16"]
    say(f"workload {wl.name} warm={warm}")
    prob = syn.draw_problem(wl)
    if warm:
        wl = syn.Workload(**{**wl.__dict__, "S": 2})
        prob.wl = wl
    errs = run_attn_segments(prob, table(wl.M + wl.W, wl.D, wl.dtype), batch=[0, wl.B - 1], warm=warm)
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs


@pytest.mark.parametrize("name", ["stack16_fp32", "stack16_bf16"])
def test_workload_stack16(name):
    wl = syn.WORKLOADS[name]
    say(f"workload {wl.name}")
    prob = syn.draw_problem(wl)
    # the first and the last batch row: the last one sits at a nonzero batch
    # offset of every operand (d_model 410 rows are only dword-aligned)
    errs = _run_block_segments(prob, table(wl.M + wl.W, wl.D, wl.dtype), batch=[0, wl.B - 1])
    say(f"  errors {errs}")
    assert max(errs.values()) <= TOL[wl.dtype], errs
