"""Pins of the CPU oracle against facts that the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks it against a
library routine, a closed form, brute force on tiny inputs, an invariant the
pages state, or a hand-worked example (tests/golden/).
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- sigmoid
def test_sigmoid_ulp_bound_over_fp32_range():
    """Strided sweep of every fp32 bit pattern in [-87, 87]: within 3 ulp of
    the fp64 sigmoid (a dropped Taylor term or a wrong split constant fails)."""
    hi = int(np.float32(87.0).view(np.uint32))
    bits = np.arange(0, hi + 1, 977, dtype=np.uint32)
    v = bits.view(np.float32)
    u = np.concatenate([v, -v])
    s = O.sigmoid_f32(u).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-u.astype(np.float64)))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(s - ref) / ulp) <= 3.0


def test_sigmoid_special_values_and_monotone():
    assert O.sigmoid_f32(np.float32([0.0]))[0] == F32(0.5)
    assert O.sigmoid_f32(np.float32([100.0]))[0] == F32(1.0)
    assert O.sigmoid_f32(np.float32([-100.0]))[0] == F32(0.0)
    u = np.sort(np.random.default_rng(0).normal(0, 8, 200000).astype(F32))
    s = O.sigmoid_f32(u)
    assert np.all(np.diff(s) >= 0)
    # symmetry sigma(-u) = 1 - sigma(u), checked in fp64 to a few ulp
    uu = np.linspace(-10, 10, 10001).astype(F32)
    a = O.sigmoid_f32(uu).astype(np.float64) + O.sigmoid_f32(-uu).astype(np.float64)
    assert np.max(np.abs(a - 1.0)) < 4e-7


# ---------------------------------------------------------------- logits
def test_router_logits_exact_on_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-3, 4, (37, 300)).astype(F32)
    w = rng.integers(-3, 4, (19, 300)).astype(F32)
    exact = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(O.router_logits(x, w), exact.astype(F32))


def test_router_logits_matches_fp64_matmul():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(8, 64)).astype(F32)
    w = rng.normal(size=(5, 64)).astype(F32)
    ref = torch.from_numpy(x).double() @ torch.from_numpy(w).double().T
    assert np.array_equal(O.router_logits(x, w), ref.float().numpy())


# ---------------------------------------------------------------- routing
def test_topk_equals_torch_topk_without_bias_or_groups():
    """b = 0, G = 1: sigmoid is monotone, so the selected set is the library
    top-K of the logits."""
    rng = np.random.default_rng(3)
    u = rng.normal(size=(500, 64)).astype(F32)
    rr = O.route(u, np.zeros(64, F32), top_k=6)
    ref = torch.topk(torch.from_numpy(u), 6, dim=1).indices.numpy()
    assert np.array_equal(np.sort(rr.idx, 1), np.sort(ref, 1))
    # slot order is score-descending
    sc = np.take_along_axis(rr.c, rr.idx.astype(np.int64), 1)
    assert np.all(np.diff(sc, axis=1) <= 0)


def _brute_select(c, K, G, M, topn):
    """Exhaustive: best M-subset of groups by total group score (group score =
    best topn-subset sum), then the best K-subset of eligible experts."""
    E = c.shape[0]
    GS = E // G
    if G > 1:
        gsc = []
        for g in range(G):
            vals = c[g * GS:(g + 1) * GS].astype(np.float64)
            gsc.append(max(sum(s) for s in itertools.combinations(vals, topn)))
        best = max(itertools.combinations(range(G), M), key=lambda S: sum(gsc[g] for g in S))
        elig = [e for e in range(E) if e // GS in best]
    else:
        elig = list(range(E))
    bestk = max(itertools.combinations(elig, K), key=lambda S: sum(float(c[e]) for e in S))
    return set(bestk)


@pytest.mark.parametrize("E,K,G,M,topn", [
    (8, 2, 1, 1, 1), (12, 3, 1, 1, 1), (8, 2, 4, 2, 2), (12, 3, 3, 2, 2),
    (12, 2, 4, 1, 3), (12, 3, 2, 1, 1), (10, 3, 2, 2, 2), (12, 3, 4, 3, 2),
])
def test_route_against_brute_force(E, K, G, M, topn):
    rng = np.random.default_rng(E * 1000 + K * 100 + G * 10 + M)
    T = 60
    u = rng.normal(size=(T, E)).astype(F32)
    b = rng.uniform(-0.3, 0.3, E).astype(F32)
    rr = O.route(u, b, K, G, M, topn)
    for t in range(T):
        assert set(rr.idx[t].tolist()) == _brute_select(rr.c[t], K, G, M, topn)


def test_route_invariants_grouped():
    rng = np.random.default_rng(4)
    T, E, K, G, M = 300, 64, 8, 8, 4
    u = rng.normal(size=(T, E)).astype(F32)
    b = rng.uniform(-0.1, 0.1, E).astype(F32)
    rr = O.route(u, b, K, G, M, 2)
    for t in range(T):
        sel = rr.idx[t]
        assert len(set(sel.tolist())) == K                     # K distinct experts
        assert len(set((sel // (E // G)).tolist())) <= M        # inside <= M groups
    gs = rr.gate.astype(np.float64).sum(1)
    assert np.max(np.abs(gs - 1.0)) <= K * 2.0 ** -23          # gates sum to 1


def test_ties_go_to_lower_index():
    u = np.zeros((1, 8), F32)            # every score 0.5 exactly
    rr = O.route(u, np.zeros(8, F32), top_k=3)
    assert rr.idx[0].tolist() == [0, 1, 2]
    assert rr.near_tie[0]
    rr = O.route(u, np.zeros(8, F32), top_k=2, n_groups=4, topk_groups=2, group_topn=1)
    assert rr.idx[0].tolist() == [0, 1]  # groups 0,1 win the tie; experts 0,1


def test_bias_changes_selection_not_gates():
    """The bias enters routing only, never the gate values [GK Q3]."""
    rng = np.random.default_rng(5)
    T, E, K = 200, 32, 4
    u = rng.normal(size=(T, E)).astype(F32)
    b0 = rng.uniform(-0.05, 0.05, E).astype(F32)
    r0 = O.route(u, b0, K)
    # a constant shift of every bias (exact in fp32 here) changes nothing at all
    r1 = O.route(u, (b0 + F32(0.25)).astype(F32), K)
    same = np.all(r1.idx == r0.idx, axis=1)
    assert same.mean() > 0.97   # fp32 rounding of c may flip exact near-ties only
    assert np.array_equal(r1.gate[same], r0.gate[same])
    # zero bias: same selection -> bit-identical gates
    rz = O.route(u, np.zeros(E, F32), K)
    keep = np.all(np.sort(rz.idx, 1) == np.sort(r0.idx, 1), axis=1) & np.all(rz.idx == r0.idx, axis=1)
    assert np.array_equal(rz.gate[keep], r0.gate[keep])
    # a large bias forces expert 7 into every token; its gate is its own
    # unbiased sigmoid over the selected sigmoids (hand computation in fp64)
    bf = np.zeros(E, F32)
    bf[7] = F32(10.0)
    rf = O.route(u, bf, K)
    assert np.all(rf.idx[:, 0] == 7)
    s = 1.0 / (1.0 + np.exp(-u.astype(np.float64)))
    for t in range(T):
        ref = s[t, 7] / s[t, rf.idx[t]].sum()
        assert abs(rf.gate[t, 0] - ref) < 1e-6


def test_golden_hand_worked_routing():
    with open(os.path.join(GOLDEN, "routing_hand_example.json")) as f:
        g = json.load(f)
    rr = O.route(np.float32(g["logits"]), np.float32(g["bias"]), g["top_k"], g["n_groups"],
                 g["topk_groups"], g["group_topn"])
    assert rr.idx.tolist() == g["expected_idx"]
    assert rr.gate.tolist() == g["expected_gate"]
    assert rr.near_tie.tolist() == g["expected_near_tie"]


def test_gate_zero_sum_fallback():
    u = np.full((1, 4), -200.0, F32)     # every sigmoid underflows to 0
    rr = O.route(u, np.zeros(4, F32), 2)
    assert rr.gate.tolist() == [[0.5, 0.5]]


# ---------------------------------------------------------------- permute
def test_permute_equals_stable_argsort():
    rng = np.random.default_rng(6)
    T, E, K = 333, 20, 3
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    pr = O.permute(idx, E)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(pr.perm, (order // K).astype(np.int32))
    assert np.array_equal(pr.counts, np.bincount(flat, minlength=E))
    assert np.array_equal(pr.offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    for t in range(T):
        for k in range(K):
            assert pr.perm[pr.inv[t, k]] == t
            assert flat[order[pr.inv[t, k]]] == idx[t, k]


def test_permute_empty_experts():
    idx = np.array([[3, 1], [3, 0]], np.int32)
    pr = O.permute(idx, 6)
    assert pr.counts.tolist() == [1, 1, 0, 2, 0, 0]
    assert pr.offsets.tolist() == [0, 1, 2, 2, 4, 4, 4]
    assert pr.perm.tolist() == [1, 0, 0, 1]
    assert pr.inv.tolist() == [[2, 1], [3, 0]]


# ---------------------------------------------------------------- bias update
def test_bias_update_direction_and_step():
    """Overloaded -> minus gamma, underloaded -> plus gamma [KY]."""
    T, K, E = 10, 2, 4                     # mean load 5
    counts = np.array([9, 5, 1, 5], np.int32)
    b = np.array([0.0, 0.5, -0.25, 1.0], F32)
    g32 = F32(0.001)
    nb = O.bias_update(b, counts, 0.001, T, K)
    assert nb[0] == F32(0.0) - g32 and nb[2] == F32(-0.25) + g32
    assert nb[1] == b[1] and nb[3] == b[3]
    # balanced loads never move
    assert np.array_equal(O.bias_update(b, np.full(4, 5, np.int32), 0.001, T, K), b)


def test_bias_update_magnitude_and_toward_balance():
    rng = np.random.default_rng(7)
    E, T, K = 64, 1000, 6
    counts = rng.multinomial(T * K, rng.dirichlet(np.ones(E))).astype(np.int32)
    b = rng.uniform(-0.1, 0.1, E).astype(F32)
    nb = O.bias_update(b, counts, 0.001, T, K)
    d = nb.astype(np.float64) - b.astype(np.float64)
    ulp = np.spacing(np.abs(b)).astype(np.float64)
    moved = counts * E != T * K
    assert np.all(np.abs(np.abs(d[moved]) - float(F32(0.001))) <= ulp[moved])
    assert np.all(np.sign(d) == -np.sign(counts.astype(np.int64) * E - T * K))


def test_bias_loop_balances_skewed_load():
    """Replaying the update on a fixed skewed batch drives max/mean load down."""
    rng = np.random.default_rng(8)
    T, E, K = 256, 16, 2
    u = (rng.normal(size=(T, E)) + np.linspace(1.0, -1.0, E)).astype(F32)
    b = np.zeros(E, F32)
    first = None
    for _ in range(400):
        rr = O.route(u, b, K)
        cnt = O.permute(rr.idx, E).counts
        ratio = cnt.max() / (T * K / E)
        first = ratio if first is None else first
        b = O.bias_update(b, cnt, 0.01, T, K)
    assert ratio < 0.6 * first


# ---------------------------------------------------------------- experts
def _torch_swiglu(x, w13, w2):
    x, w13, w2 = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, w13, w2))
    inter = w13.shape[0] // 2
    h = torch.nn.functional.silu(x @ w13[:inter].T) * (x @ w13[inter:].T)
    return (h @ w2.T).numpy()


def test_single_expert_is_dense_swiglu():
    rng = np.random.default_rng(9)
    x = rng.normal(size=(17, 32)).astype(F32)
    w13 = rng.normal(0, 0.2, (2, 48, 32)).astype(F32)[:1].reshape(1, 48, 32)
    w2 = rng.normal(0, 0.2, (1, 32, 24)).astype(F32)
    idx = np.zeros((17, 1), np.int32)
    gate = np.ones((17, 1), F32)
    y = O.layer_output(x, idx, gate, w13, w2)
    np.testing.assert_allclose(y, _torch_swiglu(x, w13[0], w2[0]), rtol=1e-12, atol=1e-12)


def test_k_equals_e_is_dense_mixture():
    rng = np.random.default_rng(10)
    T, d, E, I = 9, 16, 4, 8
    x = rng.normal(size=(T, d)).astype(F32)
    wr = rng.normal(size=(E, d)).astype(F32)
    w13 = rng.normal(0, 0.3, (E, 2 * I, d)).astype(F32)
    w2 = rng.normal(0, 0.3, (E, d, I)).astype(F32)
    ws13 = rng.normal(0, 0.3, (2 * I, d)).astype(F32)
    ws2 = rng.normal(0, 0.3, (d, I)).astype(F32)
    y, rr, _ = O.forward(x, wr, np.zeros(E, F32), w13, w2, ws13, ws2, top_k=E)
    u = x.astype(np.float64) @ wr.astype(np.float64).T
    s = 1.0 / (1.0 + np.exp(-u))
    w = s / s.sum(1, keepdims=True)
    ref = _torch_swiglu(x, ws13, ws2)
    for e in range(E):
        ref = ref + w[:, e:e + 1] * _torch_swiglu(x, w13[e], w2[e])
    np.testing.assert_allclose(y, ref, rtol=1e-5, atol=1e-7)


def test_shared_expert_applies_to_every_token():
    """The shared expert processes every token [MH §1.1]: with the routed
    down-projections zeroed, y is the shared FFN on every row; with the shared
    one zeroed, y is the routed part alone."""
    rng = np.random.default_rng(11)
    T, d, E, I, K = 20, 16, 6, 8, 2
    x = rng.normal(size=(T, d)).astype(F32)
    wr = rng.normal(size=(E, d)).astype(F32)
    w13 = rng.normal(0, 0.3, (E, 2 * I, d)).astype(F32)
    ws13 = rng.normal(0, 0.3, (2 * I, d)).astype(F32)
    ws2 = rng.normal(0, 0.3, (d, I)).astype(F32)
    y, _, _ = O.forward(x, wr, np.zeros(E, F32), w13, np.zeros((E, d, I), F32), ws13, ws2, K)
    np.testing.assert_allclose(y, _torch_swiglu(x, ws13, ws2), rtol=1e-12, atol=1e-12)
    w2 = rng.normal(0, 0.3, (E, d, I)).astype(F32)
    y0, rr, _ = O.forward(x, wr, np.zeros(E, F32), w13, w2, ws13, np.zeros((d, I), F32), K)
    for t in range(T):
        ref = sum(rr.gate[t, k] * _torch_swiglu(x[t:t + 1], w13[rr.idx[t, k]], w2[rr.idx[t, k]])[0]
                  for k in range(K))
        np.testing.assert_allclose(y0[t], ref, rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------- formats
def test_round_bf16_matches_torch():
    rng = np.random.default_rng(12)
    v = (rng.normal(size=100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(F32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.round_bf16(v), ref)


def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3_encode_against_torch_and_saturation():
    rng = np.random.default_rng(13)
    v = (rng.normal(size=200000) * np.exp(rng.uniform(-12, 5, 200000))).astype(F32)
    v = v[np.abs(v) < 440.0]
    mine = O.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    # midpoints between neighbouring codes go to the even code
    vals = O.e4m3_decode(np.arange(1, 126, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(F32)
    got = O.e4m3_encode(mids)
    assert np.all(got % 2 == 0)
    assert O.e4m3_encode(np.float32([1000.0, -449.0, 448.0]) ).tolist() == [0x7E, 0xFE, 0x7E]
    # every finite code round-trips
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_quantization_granularity_and_error_bound():
    """1x128 activation tiles and 128x128 weight blocks with max-abs scales
    [GK Q8; MH §4.1]: the largest element of each group maps to 448, the error
    is bounded by half an e4m3 step, and a zero group stays exactly zero."""
    rng = np.random.default_rng(14)
    X = rng.normal(size=(5, 384)).astype(F32)
    X[2, 128:256] = 0.0
    q, s = O.quantize_rows_1x128(X)
    assert s.shape == (5, 3) and s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    amax = np.abs(X.reshape(5, 3, 128)).max(2)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / F32(448.0)).astype(F32))
    dq = O.dequant_rows_1x128(q, s)
    bound = np.repeat(s.astype(np.float64), 128, 1) * (np.abs(O.e4m3_decode(q)) * 2.0 ** -4 + 2.0 ** -10)
    assert np.all(np.abs(dq - X) <= bound * (1 + 1e-6))
    W = rng.normal(0, 0.02, (256, 384)).astype(F32)
    qw, sw = O.quantize_blocks_128(W)
    assert sw.shape == (2, 3)
    blk = np.abs(W.reshape(2, 128, 3, 128)).max((1, 3))
    assert np.array_equal(sw, (blk / F32(448.0)).astype(F32))
    big = np.abs(O.e4m3_decode(qw)).reshape(2, 128, 3, 128).max((1, 3))
    assert np.all(big == 448.0)


def test_fp8_layer_lossless_when_values_are_on_the_grid():
    """When x and the weights already sit on the e4m3 grid with a 448 in every
    scaling group, quantization is lossless (scale 1); then the FP8 GEMMs equal
    the fp64 ones on those values, except for H's own 1x128 quantization,
    which only the down projection sees."""
    rng = np.random.default_rng(15)
    grid = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    def on_grid(shape, rowblk):
        a = rng.choice(grid[40:100], size=shape) * rng.choice([-1, 1], size=shape)
        a = a.astype(F32)
        if rowblk:
            a[:, ::128] = 448.0
        else:
            a[::128, ::128] = 448.0
        return a
    T, d, I = 4, 128, 128
    x = on_grid((T, d), True)
    w13 = on_grid((2 * I, d), False)
    w2 = np.zeros((d, I), F32)
    w2[:, 0] = 1.0
    w2[::128, ::128] = 448.0
    q13, s13 = O.quantize_blocks_128(w13)
    q2, s2 = O.quantize_blocks_128(w2)
    assert np.all(s13 == 1.0) and np.all(s2 == 1.0)
    idx = np.zeros((T, 1), np.int32)
    g = np.ones((T, 1), F32)
    y8 = O.layer_output_fp8(x, idx, g, [q13], [s13], [q2], [s2])
    # H quantization is the only lossy step; compare the first GEMM via a down
    # projection that picks H[:,0] exactly scaled by s(H row tile)
    h = (O.swiglu_expert(x, w13, np.eye(I)))            # fp64 H, identity down
    hq, hs = O.quantize_rows_1x128(h.astype(F32))
    ref = O.dequant_rows_1x128(hq, hs) @ w2.T.astype(np.float64)
    np.testing.assert_allclose(y8, ref, rtol=0, atol=0)


def test_vectorized_block_quantizer_equals_per_block_rule():
    """The all-blocks-at-once weight quantizer applies _quant_block's rule."""
    rng = np.random.default_rng(16)
    W = rng.normal(0, 0.02, (256, 384)).astype(F32)
    W[:128, 128:256] = 0.0
    W[200, 5] = 7.5
    q, s = O.quantize_blocks_128(W)
    for i in range(2):
        for j in range(3):
            rq, rs = O.moe_oracle._quant_block(W[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])
            assert np.array_equal(q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128], rq)
            assert s[i, j] == rs


def test_e4m3_arithmetic_encoder_equals_table_search():
    """The arithmetic encoder agrees with the nearest-code table search on
    random values across every binade, the subnormals, exact midpoints and
    saturation."""
    rng = np.random.default_rng(17)
    v = (rng.normal(size=300000) * np.exp2(rng.uniform(-14, 10, 300000))).astype(F32)
    vals = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(F32)
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 448.0, 464.0, 1e9, -1e9, 2.0 ** -10])])
    assert np.array_equal(O.e4m3_encode(v), O.e4m3_encode_table(v))


def test_block_dequant_round_trip_with_non_unit_scales():
    """128x128 weight blocks of very different magnitudes [GK Q8; MH §4.1]:
    every block gets its own scale (none of them 1), and dequantizing the
    codes multiplies each decoded code by its block's scale, so every value
    comes back within half an e4m3 step of the original (relative 2^-4 for
    normal codes, 2^-10 of the scale for subnormal ones). Dividing by the
    scale instead, or taking another block's scale, fails this."""
    rng = np.random.default_rng(18)
    W = rng.normal(0, 1.0, (384, 256)).astype(F32)
    mags = np.array([[3e-3, 0.7], [41.0, 5e-5], [2.0, 900.0]])
    W = (W.reshape(3, 128, 2, 128) * mags[:, None, :, None]).reshape(384, 256).astype(F32)
    q, s = O.quantize_blocks_128(W)
    assert s.shape == (3, 2) and np.all(s != 1.0)
    dq = O.dequant_blocks_128(q, s)
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    bound = sc * (np.abs(O.e4m3_decode(q)).astype(np.float64) * 2.0 ** -4 + 2.0 ** -10)
    err = np.abs(dq - W.astype(np.float64))
    assert np.all(err <= bound * (1 + 1e-6))
    # the per-block error is a small fraction of that block's magnitude
    rel = (err.reshape(3, 128, 2, 128).max((1, 3)) /
           np.abs(W).reshape(3, 128, 2, 128).max((1, 3)))
    assert np.all(rel <= 2.0 ** -4)


def _pow2_grid_matrix(rng, rows, cols, exps, grid):
    """Values on the e4m3 grid times 2^k, with k fixed per 128x128 block
    (exps [ceil(rows/128), cols/128]; one row gives 1x128 activation tiles)
    and a 448 * 2^k in every block, so the block's max-abs scale is exactly
    2^k and quantization is lossless."""
    a = rng.choice(grid, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    a[::128, ::128] = 448.0
    k = np.repeat(np.repeat(np.asarray(exps, np.float64), 128, 0), 128, 1)[:rows]
    return (a * np.exp2(k)).astype(F32)


def test_fp8_layer_with_power_of_two_scales_and_shared_expert():
    """FP8 layer on values that sit on the e4m3 grid times per-block powers
    of two (every activation tile and weight block has a scale 2^k != 1), so
    quantizing x and the weights is exact and the dequantized values equal
    the originals. The reference is a dense fp64 SwiGLU of those exact values
    (torch), shared expert included with weight 1 [MH §1.1], routed experts
    weighted by their gates. The down projections are selectors (output j
    reads one H column, times 448 * 2^k), so each output is one value of H,
    and H's own 1x128 re-quantization is the only lossy step: the error is
    within half an e4m3 step of the H values it reads. A dequantization that
    divides by the scale, a dropped shared expert or a transposed down
    projection fails this."""
    rng = np.random.default_rng(19)
    grid = O.e4m3_decode(np.arange(40, 100, dtype=np.uint8)).astype(np.float64)
    T, d, I, E = 6, 256, 128, 3
    xk = rng.integers(-7, -3, size=(T, d // 128))
    x = np.concatenate([_pow2_grid_matrix(rng, 1, d, xk[t:t + 1], grid) for t in range(T)])
    xq, xs = O.quantize_rows_1x128(x)
    assert np.all(xs != 1.0) and np.array_equal(O.dequant_rows_1x128(xq, xs), x.astype(np.float64))

    def expert(seed_shift):
        w13 = _pow2_grid_matrix(rng, 2 * I, d, rng.integers(-9, -5, size=(2, 2)), grid)
        cols = rng.permutation(I)
        sel = np.zeros((d, I), np.float64)
        sel[np.arange(d), np.concatenate([cols, cols[::-1]])] = 1.0
        kk = rng.integers(-8, -4, size=(2, 1))
        w2 = (sel * 448.0 * np.exp2(np.repeat(kk, 128, 0))).astype(F32)
        return w13, w2

    ws = [expert(e) for e in range(E + 1)]
    q13, s13, q2, s2 = [], [], [], []
    for w13, w2 in ws:
        a, b = O.quantize_blocks_128(w13)
        c, e = O.quantize_blocks_128(w2)
        assert np.all(b != 1.0) and np.all(e != 1.0)
        assert np.array_equal(O.dequant_blocks_128(a, b), w13.astype(np.float64))
        assert np.array_equal(O.dequant_blocks_128(c, e), w2.astype(np.float64))
        q13.append(a); s13.append(b); q2.append(c); s2.append(e)
    idx = np.array([[0, 1], [1, 2], [2, 0], [0, 2], [1, 0], [2, 1]], np.int32)
    g = rng.uniform(0.1, 0.9, size=(T, 2)).astype(F32)
    g = (g / g.sum(1, keepdims=True)).astype(F32)
    y8 = O.layer_output_fp8(x, idx, g, q13[:E], s13[:E], q2[:E], s2[:E],
                            q13[E], s13[E], q2[E], s2[E])

    xt = torch.from_numpy(x.astype(np.float64))

    def dense(e):
        w13 = torch.from_numpy(ws[e][0].astype(np.float64))
        w2 = torch.from_numpy(ws[e][1].astype(np.float64))
        h = torch.nn.functional.silu(xt @ w13[:I].T) * (xt @ w13[I:].T)
        return (h @ w2.T).numpy(), h.numpy(), w2.numpy()

    ref = np.zeros((T, d))
    bound = np.zeros((T, d))
    for e in range(E + 1):
        ye, h, w2 = dense(e)
        # half an e4m3 step of each H value, plus the subnormal step of its tile
        amax = np.abs(h).reshape(T, I // 128, 128).max(2)
        hb = np.abs(h) * 2.0 ** -4 + np.repeat(amax / 448.0, 128, 1) * 2.0 ** -10
        wgt = np.ones(T) if e == E else np.where(idx == e, g, 0.0).sum(1)
        ref += wgt[:, None] * ye
        bound += wgt[:, None] * (hb @ np.abs(w2).T)
    err = np.abs(y8 - ref)
    assert np.all(err <= bound * (1 + 1e-5) + 1e-12 * np.abs(ref).max())
    # the shared expert's share is well above the bound: without it most
    # outputs would fail
    ys = dense(E)[0]
    assert np.mean(np.abs(y8 - (ref - ys)) > bound) > 0.5


def test_fp8_layer_threaded_experts_identical():
    """layer_output_fp8 with its experts on threads equals the sequential run."""
    rng = np.random.default_rng(20)
    T, d, I, E, K = 16, 256, 128, 5, 2
    x = rng.normal(size=(T, d)).astype(F32)
    qs = [O.quantize_blocks_128(rng.normal(0, 0.05, (2 * I, d)).astype(F32)) for _ in range(E)]
    q2 = [O.quantize_blocks_128(rng.normal(0, 0.05, (d, I)).astype(F32)) for _ in range(E)]
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    g = rng.uniform(0.2, 0.8, (T, K)).astype(F32)
    args = (x, idx, g, [q[0] for q in qs], [q[1] for q in qs], [q[0] for q in q2],
            [q[1] for q in q2])
    assert np.array_equal(O.layer_output_fp8(*args), O.layer_output_fp8(*args, workers=3))


def test_fp8_layer_experts_take_the_e4m3_activation_tiles(monkeypatch):
    """The FP8 experts multiply the 1x128 E4M3 tiles of x, not x itself
    [GK Q8; MH §4.1]. Row 0 has max-abs 448, so its scale is 1 and its codes
    follow from the format alone (3 mantissa bits, exponent bias 7, steps of
    2^-9 below 2^-6, ties to the even code): 1.0625 lies halfway between 1 and
    1.125 and goes to 1; 3.3 goes to 3.25; -0.01 is 5.12 subnormal steps and
    goes to -5 * 2^-9; 300 lies between 288 and 320 and goes to 288. Every
    expert call must see exactly these values in row 0."""
    seen = []
    orig = O.moe_oracle._fp8_expert
    monkeypatch.setattr(O.moe_oracle, "_fp8_expert",
                        lambda Xd, *a: (seen.append(np.array(Xd)), orig(Xd, *a))[1])
    rng = np.random.default_rng(41)
    T, d, I = 3, 128, 128
    x = rng.normal(size=(T, d)).astype(F32)
    x[0] = 0.0
    x[0, :5] = [448.0, 1.0625, 3.3, -0.01, 300.0]
    want = np.zeros(d)
    want[:5] = [448.0, 1.0, 3.25, -5 * 2.0 ** -9, 288.0]
    w13 = O.quantize_blocks_128(rng.normal(0, 0.05, (2 * I, d)).astype(F32))
    w2 = O.quantize_blocks_128(rng.normal(0, 0.05, (d, I)).astype(F32))
    idx = np.zeros((T, 1), np.int32)
    g = np.ones((T, 1), F32)
    O.layer_output_fp8(x, idx, g, [w13[0]], [w13[1]], [w2[0]], [w2[1]],
                       w13[0], w13[1], w2[0], w2[1])
    assert len(seen) == 2  # the shared expert and expert 0, each on all rows
    for Xd in seen:
        assert np.array_equal(Xd[0], want)
