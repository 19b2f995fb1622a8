"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here checks the oracle against something other than itself: values
the pages state (fixtures under tests/golden/), closed forms, invariants,
special cases that reduce to a library routine (torch's scaled-dot-product
attention, numpy/torch linear algebra), and brute force over the whole stream
on tiny inputs. None of them needs a GPU.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from transformer_xl_segment_amd import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _params(rng, D, F=None, scale=0.3, affine=False):
    # larger than the workloads' 0.02 so that every term moves the scores visibly
    return syn.draw_layer_params(rng, D, F, "fp32", affine=affine, scale=scale)


def _R(K, D):
    return orc.sinusoid_table(K, D)


# --------------------------------------------------------------------------
# Relative-encoding table: closed forms of the [sin | cos] reading.
# --------------------------------------------------------------------------

def test_sinusoid_closed_forms():
    D, L = 10, 40
    R = _R(L, D)
    half = D // 2
    # distance 0: sin 0 = 0 in the first half, cos 0 = 1 in the second
    assert np.all(R[0, :half] == 0.0) and np.all(R[0, half:] == 1.0)
    # the first frequency is 1: column 0 is sin(d), column D/2 is cos(d)
    d = np.arange(L)
    np.testing.assert_allclose(R[:, 0], np.sin(d), rtol=0, atol=1e-15)
    np.testing.assert_allclose(R[:, half], np.cos(d), rtol=0, atol=1e-15)
    # every (k, D/2 + k) pair lies on the unit circle
    np.testing.assert_allclose(R[:, :half] ** 2 + R[:, half:] ** 2, 1.0, atol=1e-14)
    # the last frequency is 10000^(-(D-2)/D)
    w = 10000.0 ** (-(D - 2) / D)
    np.testing.assert_allclose(R[:, half - 1], np.sin(d * w), atol=1e-15)
    # R is a function of the distance only: a longer table extends a shorter one unchanged
    np.testing.assert_array_equal(_R(L + 17, D)[:L], R)


# --------------------------------------------------------------------------
# Linear maps and LayerNorm.
# --------------------------------------------------------------------------

def test_linear_matches_library_matmul():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 5, 13))
    Wt = rng.standard_normal((11, 13))
    np.testing.assert_allclose(orc.linear(x, Wt), x @ Wt.T, rtol=1e-13, atol=1e-13)


def test_layer_norm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 24)) * 3.0 + 1.5
    g = 1.0 + rng.standard_normal(24) * 0.1
    b = rng.standard_normal(24) * 0.1
    y = orc.layer_norm(x, g, b)
    z = (y - b) / g
    sd = x.std(axis=-1)
    # normalised rows have mean 0 and population std sigma / (sigma + 1e-6)
    np.testing.assert_allclose(z.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(z.std(axis=-1), sd / (sd + 1e-6), rtol=1e-12)
    # a constant row has sigma = 0 and maps to the offset exactly
    yc = orc.layer_norm(np.full((1, 24), 7.25), g, b)
    np.testing.assert_array_equal(yc[0], b)
    # close to torch's LayerNorm (its eps sits under the square root instead)
    yt = torch.nn.functional.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(g),
                                        torch.from_numpy(b), eps=0.0).numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-5, atol=1e-6)


# --------------------------------------------------------------------------
# Relative attention: special cases, invariants, brute force.
# --------------------------------------------------------------------------

def _attn_case(seed=3, B=2, W=5, m=3, D=12, H=3, scale=0.3):
    rng = np.random.default_rng(seed)
    p = _params(rng, D, scale=scale)
    h = rng.standard_normal((B, W, D))
    mem = rng.standard_normal((B, m, D)) if m > 0 else None
    return p, h, mem, _R(m + W, D)


def test_probability_rows_and_mask():
    p, h, mem, R = _attn_case()
    W, m = h.shape[1], mem.shape[1]
    out, P, AC, BD = orc.rel_attn(h, mem, p, R, H=3, return_terms=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    for i in range(W):
        assert np.all(P[:, :, i, m + i + 1:] == 0.0)
        assert np.all(P[:, :, i, :m + i + 1] > 0.0)
        assert np.all(np.isnan(AC[:, :, i, m + i + 1:])) and np.all(np.isnan(BD[:, :, i, m + i + 1:]))


def test_key_counts_match_glossary_loop():
    # tests/golden/key_counts_glossary.txt: 3 segments of 4 tokens, dim 16, 2 heads,
    # empty first memory, the previous segment cached -> 4, 8, 8 keys.
    with open(os.path.join(GOLDEN, "key_counts_glossary.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    meta = dict(kv.split("=") for kv in lines[0].split())
    expect = [int(t) for t in lines[1].split("=")[1].split()]
    W, D, H, S = int(meta["seg_len"]), int(meta["dim"]), int(meta["heads"]), int(meta["segments"])
    rng = np.random.default_rng(7)
    p = _params(rng, D)
    x = rng.standard_normal((1, S * W, D))
    mem = None
    counts = []
    for t in range(S):
        h = x[:, t * W:(t + 1) * W]
        m = 0 if mem is None else mem.shape[1]
        _, P, _, _ = orc.rel_attn(h, mem, p, _R(m + W, D), H, return_terms=True)
        counts.append(P.shape[-1])
        # the last query of the segment sees every key
        assert int((P[0, 0, W - 1] > 0).sum()) == P.shape[-1]
        mem = orc.mem_update(mem, h, M=W)
    assert counts == expect


def test_plain_attention_special_case_matches_sdpa():
    # u = v = 0 and W_kR = 0 remove both distance terms and both biases: the
    # result is causal softmax(Q K^T / sqrt(dh)) V over [mem; h], then W_o.
    B, W, m, D, H = 2, 6, 4, 16, 4
    p, h, mem, R = _attn_case(seed=11, B=B, W=W, m=m, D=D, H=H)
    p = dict(p)
    p["u"] = np.zeros(D)
    p["v"] = np.zeros(D)
    p["WkR"] = np.zeros((D, D))
    out = orc.rel_attn(h, mem, p, R, H)
    ctx = np.concatenate([mem, h], axis=1)
    dh = D // H
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    q = t(h @ p["Wq"].T).reshape(B, W, H, dh).transpose(1, 2)
    k = t(ctx @ p["WkE"].T).reshape(B, m + W, H, dh).transpose(1, 2)
    v = t(ctx @ p["Wv"].T).reshape(B, m + W, H, dh).transpose(1, 2)
    mask = torch.ones(W, m + W, dtype=torch.bool).tril(diagonal=m)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    ref = o.transpose(1, 2).reshape(B, W, D).numpy() @ p["Wo"].T
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_first_query_sees_only_itself_without_memory():
    p, h, _, R = _attn_case(seed=5, m=0)
    out = orc.rel_attn(h, None, p, R[:h.shape[1]], H=3)
    ref = (h[:, 0] @ p["Wv"].T) @ p["Wo"].T
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-12, atol=1e-13)


def test_uniform_scores_give_running_mean():
    # W_q = 0, u = v = 0: every visible score is 0, so query i averages the values
    # of keys 0..m+i.
    p, h, mem, R = _attn_case(seed=6)
    p = dict(p)
    D = h.shape[2]
    p["Wq"] = np.zeros((D, D))
    p["u"] = np.zeros(D)
    p["v"] = np.zeros(D)
    out = orc.rel_attn(h, mem, p, R, H=3)
    ctx = np.concatenate([mem, h], axis=1)
    V = ctx @ p["Wv"].T
    m = mem.shape[1]
    csum = np.cumsum(V, axis=1)
    ref = np.stack([csum[:, m + i] / (m + i + 1) for i in range(h.shape[1])], axis=1) @ p["Wo"].T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_distance_only_scores_ignore_content():
    # W_q = 0 and u = 0: the score is v . r_delta, a function of the distance
    # only, so the probabilities are the same for every batch row and content.
    p, h, mem, R = _attn_case(seed=8, B=3)
    p = dict(p)
    D = h.shape[2]
    p["Wq"] = np.zeros((D, D))
    p["u"] = np.zeros(D)
    _, P1, _, BD1 = orc.rel_attn(h, mem, p, R, H=3, return_terms=True)
    rng = np.random.default_rng(99)
    _, P2, _, _ = orc.rel_attn(rng.standard_normal(h.shape), rng.standard_normal(mem.shape), p, R,
                               H=3, return_terms=True)
    np.testing.assert_array_equal(P1, P2)
    np.testing.assert_array_equal(P1[0], P1[1])
    # and BD is Toeplitz: it depends on i - j only
    W, K = P1.shape[2], P1.shape[3]
    for i in range(W - 1):
        for j in range(K - 1):
            if not np.isnan(BD1[0, 0, i, j]):
                assert BD1[0, 0, i, j] == BD1[0, 0, i + 1, j + 1]


def test_equal_rows_make_scores_toeplitz():
    # with every input row equal, q and k are the same for all positions, AC is a
    # constant and BD depends on the distance only
    B, W, m, D, H = 1, 5, 4, 12, 3
    rng = np.random.default_rng(12)
    p = _params(rng, D)
    row = rng.standard_normal(D)
    h = np.tile(row, (B, W, 1))
    mem = np.tile(row, (B, m, 1))
    _, _, AC, BD = orc.rel_attn(h, mem, p, _R(m + W, D), H, return_terms=True)
    vis = ~np.isnan(AC)
    for hd in range(H):
        a = AC[0, hd][vis[0, hd]]
        assert np.all(a == a[0])
    for i in range(W - 1):
        for j in range(m + W - 1):
            if vis[0, 0, i, j]:
                np.testing.assert_array_equal(BD[0, :, i, j], BD[0, :, i + 1, j + 1])


def test_pair_score_is_translation_invariant():
    # tests/golden/relative_distance_explainer.txt: the pair (5, 3) and the pair
    # (105, 103) have the same distance 2; with the same two tokens at those
    # positions the oracle gives the same score terms, bit for bit.
    with open(os.path.join(GOLDEN, "relative_distance_explainer.txt")) as f:
        pairs = [tuple(int(t) for t in ln.split()) for ln in f if ln.strip() and not ln.startswith("#")]
    (q0, k0, d0), (q1, k1, d1) = pairs
    assert q0 - k0 == d0 and q1 - k1 == d1 and d0 == d1
    D, H, W = 8, 2, 8
    rng = np.random.default_rng(4)
    p = _params(rng, D)
    tok_q, tok_k = rng.standard_normal(D), rng.standard_normal(D)

    def terms(qpos, kpos):
        # the stream holds other random tokens, the two tokens at qpos and kpos;
        # the query's segment starts at a multiple of W and its memory holds the
        # previous W positions
        T = (qpos // W + 1) * W
        x = np.random.default_rng(qpos).standard_normal((1, T, D))
        x[0, qpos], x[0, kpos] = tok_q, tok_k
        s0 = (qpos // W) * W
        mem = x[:, max(0, s0 - W):s0]
        m = mem.shape[1]
        h = x[:, s0:s0 + W]
        _, _, AC, BD = orc.rel_attn(h, mem if m else None, p, _R(m + W, D), H, return_terms=True)
        i, j = qpos - s0, kpos - (s0 - m)
        assert m + i - j == qpos - kpos
        return AC[0, :, i, j], BD[0, :, i, j]

    a0, b0 = terms(q0, k0)
    a1, b1 = terms(q1, k1)
    np.testing.assert_array_equal(a0, a1)
    np.testing.assert_array_equal(b0, b1)


def test_shift_trick_equals_per_pair_loop():
    # The explainer's step 5: score the distance term once against every
    # distance and shift each row into place. Written here in the classic
    # pad-and-reshape form, independently of the oracle's per-pair loop.
    B, W, m, D, H = 2, 7, 5, 12, 3
    p, h, mem, R = _attn_case(seed=9, B=B, W=W, m=m, D=D, H=H)
    _, _, _, BD = orc.rel_attn(h, mem, p, R, H, return_terms=True)
    K, dh = m + W, D // H
    qv = (h @ p["Wq"].T + p["v"]).reshape(B, W, H, dh)
    rk = (R[:K] @ p["WkR"].T).reshape(K, H, dh)
    # columns ordered by decreasing distance: column c holds distance K-1-c
    rk_rev = rk[::-1]
    full = np.einsum("bihc,khc->bhik", qv, rk_rev)          # [B, H, W, K]
    padded = np.concatenate([np.zeros((B, H, W, 1)), full], axis=-1)
    shifted = padded.reshape(B, H, K + 1, W)[:, :, 1:].reshape(B, H, W, K)
    vis = ~np.isnan(BD)
    np.testing.assert_allclose(shifted[vis], BD[vis], rtol=1e-12, atol=1e-13)


def _stream_brute_force(x, p, R, H, W, M):
    """Single-layer attention over the whole stream with the segment window.

    Query t (segment tau = t // W) sees key s iff s <= t and s >= tau*W - m(tau),
    with m(tau) = min(M, tau*W); the distance is t - s in stream positions.
    Pure Python loops over (t, s); numpy only for the projections.
    """
    B, T, D = x.shape
    dh = D // H
    Q = x @ p["Wq"].T
    Kc = x @ p["WkE"].T
    V = x @ p["Wv"].T
    Rk = R @ p["WkR"].T
    out = np.zeros((B, T, D))
    for b in range(B):
        for hd in range(H):
            cs = slice(hd * dh, (hd + 1) * dh)
            for t in range(T):
                tau = t // W
                lo = tau * W - min(M, tau * W)
                keys = list(range(lo, t + 1))
                sc = []
                for s in keys:
                    ac = float(np.dot(Q[b, t, cs] + p["u"][cs], Kc[b, s, cs]))
                    bd = float(np.dot(Q[b, t, cs] + p["v"][cs], Rk[t - s, cs]))
                    sc.append((ac + bd) / math.sqrt(dh))
                mx = max(sc)
                e = [math.exp(z - mx) for z in sc]
                tot = sum(e)
                for s, w in zip(keys, e):
                    out[b, t, cs] += (w / tot) * V[b, s, cs]
    return out @ p["Wo"].T


@pytest.mark.parametrize("W,M", [(3, 5), (4, 4), (4, 2)])
def test_segments_equal_stream_brute_force(W, M):
    B, S, D, H = 2, 4, 8, 2
    rng = np.random.default_rng(20 + W + M)
    p = _params(rng, D)
    x = rng.standard_normal((B, S * W, D))
    R = _R(S * W, D)
    y, _ = orc.stack_fwd(x, [p], R, H, W, M, full_layer=False)
    ref = _stream_brute_force(x, p, R, H, W, M)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_layer_block_composition():
    # post-LN block: LN1(h + attn), then LN2(h1 + FFN(h1)); FFN from torch's
    # linear and relu, the pinned attention and LayerNorm from the oracle.
    B, W, m, D, H, F = 2, 5, 3, 12, 3, 20
    rng = np.random.default_rng(13)
    p = _params(rng, D, F=F, affine=True)
    h = rng.standard_normal((B, W, D))
    mem = rng.standard_normal((B, m, D))
    R = _R(m + W, D)
    y = orc.layer_fwd(h, mem, p, R, H)
    att = orc.rel_attn(h, mem, p, R, H)
    h1 = orc.layer_norm(h + att, p["ln1_g"], p["ln1_b"])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    f = torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(t(h1), t(p["W1"]), t(p["b1"]))),
                                   t(p["W2"]), t(p["b2"])).numpy()
    ref = orc.layer_norm(h1 + f, p["ln2_g"], p["ln2_b"])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_memory_update_keeps_last_rows():
    # rows carry their stream position; after every segment the memory must be
    # the min(M, tau*W) most recent positions, oldest first
    B, D = 2, 3
    for W, M in [(4, 4), (3, 7), (5, 2), (6, 6)]:
        mem = None
        for tau in range(5):
            pos = np.arange(tau * W, (tau + 1) * W, dtype=np.float64)
            h = np.broadcast_to(pos[None, :, None], (B, W, D)).copy()
            mem = orc.mem_update(mem, h, M)
            n = min(M, (tau + 1) * W)
            assert mem.shape == (B, n, D)
            expect = np.arange((tau + 1) * W - n, (tau + 1) * W, dtype=np.float64)
            np.testing.assert_array_equal(mem[0, :, 0], expect)


def test_stack_with_full_memory_equals_one_pass_stack():
    # With M >= stream length nothing is ever dropped: the segment-recurrent stack
    # equals one causal pass of the same stack over the whole stream as one segment.
    B, W, S, D, H, F, L = 1, 3, 4, 8, 2, 16, 2
    rng = np.random.default_rng(31)
    params = [_params(rng, D, F=F, affine=True) for _ in range(L)]
    x = rng.standard_normal((B, S * W, D))
    R = _R(S * W, D)
    y, mems = orc.stack_fwd(x, params, R, H, W, M=S * W, full_layer=True)
    y1, _ = orc.stack_fwd(x, params, R, H, W=S * W, M=S * W, full_layer=True)
    np.testing.assert_allclose(y, y1, rtol=1e-11, atol=1e-12)
    # layer 0's memory holds the stack input, layer 1's holds layer 0's output
    np.testing.assert_array_equal(mems[0], x)


def test_reach_grows_one_segment_per_layer():
    # M = W, two layers: the output at segment tau depends on input segments
    # tau-2..tau only. Perturbing segment 0 changes segments 0..2 and leaves
    # segments 3 and 4 bit-identical.
    B, W, S, D, H, F, L = 1, 3, 5, 8, 2, 16, 2
    rng = np.random.default_rng(32)
    params = [_params(rng, D, F=F) for _ in range(L)]
    x = rng.standard_normal((B, S * W, D))
    R = _R(2 * W, D)
    y, _ = orc.stack_fwd(x, params, R, H, W, M=W, full_layer=True)
    x2 = x.copy()
    x2[:, :W] += 1.0
    y2, _ = orc.stack_fwd(x2, params, R, H, W, M=W, full_layer=True)
    for tau in range(S):
        seg = slice(tau * W, (tau + 1) * W)
        if tau <= L:
            assert np.max(np.abs(y[:, seg] - y2[:, seg])) > 1e-6
        else:
            np.testing.assert_array_equal(y[:, seg], y2[:, seg])


@pytest.mark.parametrize("W,M,k", [(3, 5, 1), (4, 4, 2), (4, 2, 3), (3, 7, 2)])
def test_resume_from_carried_memories_equals_straight_run(W, M, k):
    # "Transformer-XL, explained.", method step 2: a segment sees the past only
    # through the cached memories, which enter as constants. So k segments,
    # then the remaining S - k segments started from the memories the first call
    # left behind, give the straight S-segment run bit for bit (same arithmetic in
    # the same order), outputs and final memories alike.
    B, S, D, H, F, L = 2, 5, 8, 2, 16, 3
    rng = np.random.default_rng(40 + 10 * W + M + k)
    params = [_params(rng, D, F=F, affine=True) for _ in range(L)]
    x = rng.standard_normal((B, S * W, D))
    R = _R(M + W, D)
    y, mems = orc.stack_fwd(x, params, R, H, W, M, full_layer=True)
    ya, mems_a = orc.stack_fwd(x[:, :k * W], params, R, H, W, M, full_layer=True)
    yb, mems_b = orc.stack_fwd(x[:, k * W:], params, R, H, W, M, full_layer=True, mems0=mems_a)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    for l in range(L):
        np.testing.assert_array_equal(mems_b[l], mems[l])
    # layer 0's carried memory is the last min(M, kW) stack input rows; and the
    # resumed part is not the same as a run from empty memories (the carry matters)
    np.testing.assert_array_equal(mems_a[0], x[:, max(0, k * W - M):k * W])
    y0, _ = orc.stack_fwd(x[:, k * W:], params, R, H, W, M, full_layer=True)
    assert np.max(np.abs(y0[:, :W] - yb[:, :W])) > 1e-6


def test_resume_single_layer_matches_stream_brute_force():
    # the resumed attention-only run equals the brute-force stream attention of
    # the whole stream on the segments after the split point
    B, W, M, S, D, H, k = 2, 3, 5, 5, 8, 2, 2
    rng = np.random.default_rng(44)
    p = _params(rng, D)
    x = rng.standard_normal((B, S * W, D))
    R = _R(S * W, D)
    _, mems_a = orc.stack_fwd(x[:, :k * W], [p], R, H, W, M, full_layer=False)
    yb, _ = orc.stack_fwd(x[:, k * W:], [p], R, H, W, M, full_layer=False, mems0=mems_a)
    ref = _stream_brute_force(x, p, R, H, W, M)
    np.testing.assert_allclose(yb, ref[:, k * W:], rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Encodings Transformer-XL is compared against (Shaw et al.; absolute).
# --------------------------------------------------------------------------

def _sdpa_plain(h, mem, p, H):
    """Causal softmax(Q K^T / sqrt(dh)) V over [mem; h], then W_o, by torch."""
    B, W, D = h.shape
    ctx = np.concatenate([mem, h], axis=1) if mem is not None else h
    K, dh = ctx.shape[1], D // H
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    q = t(h @ p["Wq"].T).reshape(B, W, H, dh).transpose(1, 2)
    k = t(ctx @ p["WkE"].T).reshape(B, K, H, dh).transpose(1, 2)
    v = t(ctx @ p["Wv"].T).reshape(B, K, H, dh).transpose(1, 2)
    mask = torch.ones(W, K, dtype=torch.bool).tril(diagonal=K - W)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    return o.transpose(1, 2).reshape(B, W, D).numpy() @ p["Wo"].T


def test_absolute_variant_is_plain_attention():
    p, h, mem, _ = _attn_case(seed=21, B=2, W=6, m=4, D=16, H=4)
    out = orc.attn_variant(orc.POS_ABSOLUTE, h, mem, p, 4)
    np.testing.assert_allclose(out, _sdpa_plain(h, mem, p, 4), rtol=1e-11, atol=1e-12)


def test_shaw_with_zero_tables_is_plain_attention():
    p, h, mem, _ = _attn_case(seed=22, B=2, W=6, m=4, D=16, H=4)
    z = np.zeros((4, 4))
    out = orc.attn_variant(orc.POS_SHAW, h, mem, p, 4, aK=z, aV=z, clip=3)
    np.testing.assert_allclose(out, _sdpa_plain(h, mem, p, 4), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("clip", [0, 2, 5, 40])
def test_shaw_value_term_under_uniform_attention(clip):
    # W_q = 0: every visible key gets the same weight, so o_i is the mean of the
    # visible values plus the mean of aV over the clipped distances 0 .. m + i
    B, W, m, D, H = 2, 7, 5, 12, 3
    p, h, mem, _ = _attn_case(seed=23, B=B, W=W, m=m, D=D, H=H)
    p = dict(p)
    p["Wq"] = np.zeros((D, D))
    p["Wo"] = np.eye(D)
    dh = D // H
    rng = np.random.default_rng(24)
    aK = rng.standard_normal((clip + 1, dh))
    aV = rng.standard_normal((clip + 1, dh))
    out = orc.attn_variant(orc.POS_SHAW, h, mem, p, H, aK=aK, aV=aV, clip=clip)
    val = np.concatenate([mem, h], axis=1) @ p["Wv"].T
    for i in range(W):
        n = m + i + 1
        mean_val = val[:, :n].mean(axis=1)
        deltas = np.minimum(np.arange(n), clip)
        mean_av = np.tile(aV[deltas].mean(axis=0), H)
        np.testing.assert_allclose(out[:, i], mean_val + mean_av, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("clip", [1, 3, 30])
def test_shaw_distance_weights_follow_clipped_distance(clip):
    # All rows equal: content scores are one constant, so with aK[d] = d g the
    # weights are p(delta) ~ exp(beta min(delta, clip)), beta = q.g / sqrt(dh),
    # over delta = 0 .. m + i; with aV[d] = d e the output is val + E[min(delta, clip)] e.
    B, W, m, D, H = 1, 6, 4, 8, 2
    dh = D // H
    rng = np.random.default_rng(25)
    p = _params(rng, D, scale=0.5)
    row = rng.standard_normal(D)
    h = np.tile(row, (B, W, 1))
    mem = np.tile(row, (B, m, 1))
    g = rng.standard_normal(dh)
    d = np.arange(clip + 1, dtype=np.float64)[:, None]
    aK = d * g[None, :]
    aV = d * np.ones((1, dh))
    out = orc.attn_variant(orc.POS_SHAW, h, mem, p, H, aK=aK, aV=aV, clip=clip)
    q = row @ p["Wq"].T
    val = row @ p["Wv"].T
    for i in range(W):
        deltas = np.minimum(np.arange(m + i + 1), clip)
        o = np.empty(D)
        for hd in range(H):
            beta = q[hd * dh:(hd + 1) * dh] @ g / math.sqrt(dh)
            w = np.exp(beta * deltas - np.max(beta * deltas))
            w /= w.sum()
            o[hd * dh:(hd + 1) * dh] = val[hd * dh:(hd + 1) * dh] + (w * deltas).sum()
        np.testing.assert_allclose(out[0, i], o @ p["Wo"].T, rtol=1e-10, atol=1e-12)


def test_shaw_one_head_matches_relative_attention_without_biases():
    # One head, aK[d] = (R W_kR^T)[d] with no clipping inside the window and
    # aV = 0: Shaw's two score terms are Transformer-XL's with u = v = 0.
    B, W, m, D = 2, 5, 6, 8
    p, h, mem, R = _attn_case(seed=26, B=B, W=W, m=m, D=D, H=1)
    p = dict(p)
    p["u"] = np.zeros(D)
    p["v"] = np.zeros(D)
    aK = R @ p["WkR"].T
    out = orc.attn_variant(orc.POS_SHAW, h, mem, p, 1, aK=aK, aV=np.zeros_like(aK), clip=m + W - 1)
    np.testing.assert_allclose(out, orc.rel_attn(h, mem, p, R, 1), rtol=1e-11, atol=1e-12)


def test_absolute_positions_closed_forms():
    B, W, D = 2, 9, 10
    x = np.random.default_rng(27).standard_normal((B, W, D))
    for pos0 in (0, 5):
        y = orc.add_positions(x, pos0)
        U = y - x
        t = np.arange(pos0, pos0 + W, dtype=np.float64)
        # frequency 1 in column 0 (sin) and column D/2 (cos); the slowest pair
        # has frequency 10000^(-(D-2)/D)
        np.testing.assert_allclose(U[:, :, 0], np.broadcast_to(np.sin(t), (B, W)), atol=1e-13)
        np.testing.assert_allclose(U[:, :, D // 2], np.broadcast_to(np.cos(t), (B, W)), atol=1e-13)
        f = 10000.0 ** (-(D - 2) / D)
        np.testing.assert_allclose(U[:, :, D // 2 - 1], np.broadcast_to(np.sin(t * f), (B, W)), atol=1e-13)
        np.testing.assert_allclose(U[:, :, D - 1], np.broadcast_to(np.cos(t * f), (B, W)), atol=1e-13)


# --------------------------------------------------------------------------
# Backward pass with the memory behind a stop-gradient.
# --------------------------------------------------------------------------

def _bwd_case(seed, B=2, W=3, m=2, D=8, H=2, scale=0.5):
    rng = np.random.default_rng(seed)
    p = {n: a.astype(np.float64) for n, a in _params(rng, D, scale=scale).items()}
    p["Wo"] = np.eye(D)                      # the loss reads the attention output o itself
    h = rng.standard_normal((B, W, D))
    mem = rng.standard_normal((B, m, D)) if m > 0 else None
    dO = rng.standard_normal((B, W, D))
    return p, h, mem, _R(m + W, D), dO


def _bwd_through_projections(p, h, mem, R, dO, H):
    """Gradients of L = sum(dO * o) w.r.t. the weights, u, v and the segment rows,
    from the backward oracle and the chain rule through the linear projections."""
    m = 0 if mem is None else mem.shape[1]
    ctx = h if mem is None else np.concatenate([mem, h], axis=1)
    K = ctx.shape[1]
    q, k, val, r = h @ p["Wq"].T, ctx @ p["WkE"].T, ctx @ p["Wv"].T, R[:K] @ p["WkR"].T
    g = orc.rel_attn_bwd(q, k, val, r, p["u"], p["v"], dO, H)
    return {
        "Wq": np.einsum("bto,bti->oi", g["dq"], h),
        "WkE": np.einsum("bjo,bji->oi", g["dk"], ctx),      # memory rows included
        "Wv": np.einsum("bjo,bji->oi", g["dval"], ctx),
        "WkR": g["dr"].T @ R[:K],
        "u": g["du"], "v": g["dv"],
        "h": g["dq"] @ p["Wq"] + g["dk"][:, m:] @ p["WkE"] + g["dval"][:, m:] @ p["Wv"],
    }


@pytest.mark.parametrize("m", [0, 2, 5])
def test_backward_matches_finite_differences(m):
    # central differences of the (separately pinned) forward oracle, in fp64;
    # the memory is held fixed (stop-gradient), every other input is perturbed
    H = 2
    p, h, mem, R, dO = _bwd_case(31 + m, m=m)
    grads = _bwd_through_projections(p, h, mem, R, dO, H)

    def loss(pp, hh):
        return float(np.sum(dO * orc.rel_attn(hh, mem, pp, R, H)))

    eps = 1e-5
    for name in ("Wq", "WkE", "Wv", "WkR", "u", "v", "h"):
        base = h if name == "h" else p[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += eps
            minus[idx] -= eps
            if name == "h":
                fd[idx] = (loss(p, plus) - loss(p, minus)) / (2 * eps)
            else:
                fd[idx] = (loss({**p, name: plus}, h) - loss({**p, name: minus}, h)) / (2 * eps)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_single_key_closed_form():
    # the first query of a segment with no memory sees only itself: p = 1, so
    # its score gradient vanishes (dq_0 = 0) and its value gets dO_0 exactly
    B, W, D, H = 2, 4, 8, 2
    rng = np.random.default_rng(33)
    q, dO = rng.standard_normal((B, W, D)), rng.standard_normal((B, W, D))
    k, val = rng.standard_normal((B, W, D)), rng.standard_normal((B, W, D))
    r, u, v = rng.standard_normal((W, D)), rng.standard_normal(D), rng.standard_normal(D)
    g = orc.rel_attn_bwd(q, k, val, r, u, v, dO, H)
    assert np.all(g["dq"][:, 0] == 0.0)
    # key W-1 is seen only by the last query (weight p), the first key by all
    o_last = orc.rel_attn_bwd(q, k, val, r, u, v, np.zeros_like(dO), H)
    assert all(np.all(o_last[n] == 0.0) for n in o_last)          # linear in dO
    assert np.all(np.abs(g["dval"][:, 0]) > 0)


def test_bad_arguments_are_rejected():
    p, h, mem, R = _attn_case()
    with pytest.raises(ValueError):
        orc.rel_attn(h, mem, p, R[:3], H=3)       # table shorter than m + W
    with pytest.raises(ValueError):
        orc.rel_attn(h, mem, p, R, H=5)           # D % H != 0
