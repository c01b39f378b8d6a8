"""Pins of the FP8 backward oracle (CPU only).

The E5M2 codec is checked against torch's float8_e5m2 and a table search;
the 128x1 quantizer against the 1x128 one on the transpose and the per-tile
rule; the FP8 expert backward, with every quantizer made exact, against the
fp64 backward (itself pinned by finite differences and autograd), which
checks which operand each GEMM quantizes and along which axis; and the
quantization error against its bound.
"""
import numpy as np
import torch

import oracle as O
import oracle.fp8_backward as FB
import oracle.moe_oracle as MO

F32 = np.float32


def test_e5m2_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref)) and np.isnan(ref).sum() == 6
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])
    assert mine[0x7B] == 57344.0 and mine[0x01] == 2.0 ** -16 and mine[0x04] == 2.0 ** -14
    assert np.isinf(mine[0x7C]) and np.isinf(mine[0xFC])


def test_e5m2_encode_against_torch_table_and_saturation():
    rng = np.random.default_rng(30)
    v = (rng.normal(size=300000) * np.exp2(rng.uniform(-20, 16, 300000))).astype(F32)
    fin = v[np.abs(v) < 57344.0]
    ref = torch.from_numpy(fin).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(O.e5m2_encode(fin), ref)
    vals = O.e5m2_decode(np.arange(0, 124, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(F32)
    w = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 57344.0, 61439.0, 1e30, -1e30])])
    assert np.array_equal(O.e5m2_encode(w), O.e5m2_encode_table(w))
    assert np.all(O.e5m2_encode(mids) % 2 == 0)
    assert O.e5m2_encode(np.float32([1e9, -60000.0])).tolist() == [0x7B, 0xFB]
    codes = np.arange(0, 124, dtype=np.uint8)
    assert np.array_equal(O.e5m2_encode(O.e5m2_decode(codes)), codes)


def test_tile_quantizers_shapes_scales_and_bounds():
    rng = np.random.default_rng(31)
    X = (rng.normal(size=(300, 256)) * np.exp2(rng.integers(-6, 6, size=(1, 256)))).astype(F32)
    X[:, 7] = 0.0
    for fmt, fmax, half in (("e4m3", 448.0, 2.0 ** -4), ("e5m2", 57344.0, 2.0 ** -3)):
        q, s = O.quantize_128x1(X, fmt)
        assert q.shape == X.shape and s.shape == (3, 256)
        assert np.all(s[:, 7] == 1.0) and not q[:, 7].any()
        amax = np.stack([np.abs(X[i * 128:(i + 1) * 128]).max(0) for i in range(3)])
        nz = amax > 0
        assert np.array_equal(s[nz], (amax[nz] / F32(fmax)).astype(F32))
        # full tiles are the 1x128 tiles of the transpose
        qt, st = O.quantize_1x128(X[:256].T.copy(), fmt)
        assert np.array_equal(qt.T, q[:256]) and np.array_equal(st.T, s[:2])
        # the last, 44-row tile has its own scale; error within half a step
        dq = O.dequant_128x1(q, s, fmt)
        dec = O.e5m2_decode(q) if fmt == "e5m2" else O.e4m3_decode(q)
        sc = np.repeat(s.astype(np.float64), 128, 0)[:300]
        tiny = 2.0 ** -17 if fmt == "e5m2" else 2.0 ** -10
        assert np.all(np.abs(dq - X) <= sc * (np.abs(dec) * half + tiny) * (1 + 1e-6))
        q1, s1 = O.quantize_1x128(X, fmt)
        assert s1.shape == (300, 2)
        assert np.all(np.abs(O.dequant_1x128(q1, s1, fmt) - X) <=
                      np.repeat(s1.astype(np.float64), 128, 1) *
                      (np.abs(O.e5m2_decode(q1) if fmt == "e5m2" else O.e4m3_decode(q1)) * half
                       + tiny) * (1 + 1e-6))


def _exact_codecs(monkeypatch):
    """Every quantizer of the FP8 path made exact: codes are the values
    themselves, scales 1 (an FP8 format with unlimited precision), and the
    bf16 storage of the intermediates exact too."""
    ident = lambda X, fmt=None: (np.asarray(X, np.float64), np.ones(1))
    deq = lambda q, s, fmt=None: np.asarray(q, np.float64)
    monkeypatch.setattr(FB, "round_bf16", lambda v: np.asarray(v, np.float64))
    monkeypatch.setattr(FB, "quantize_1x128", ident)
    monkeypatch.setattr(FB, "dequant_1x128", deq)
    monkeypatch.setattr(FB, "quantize_128x1", ident)
    monkeypatch.setattr(FB, "dequant_128x1", deq)
    monkeypatch.setattr(FB, "_dq_blocks", deq)
    monkeypatch.setattr(MO, "quantize_rows_1x128", lambda X: ident(X))
    monkeypatch.setattr(MO, "dequant_rows_1x128", deq)


def test_expert_backward_with_exact_codecs_is_the_fp64_backward(monkeypatch):
    """With exact quantizers the FP8 expert backward is the fp64 SwiGLU
    backward up to its fp32 roundings of a, b, H, dY and [da | db]: a
    transposed operand, a dropped term or an operand taken from the wrong
    GEMM fails this."""
    _exact_codecs(monkeypatch)
    rng = np.random.default_rng(32)
    n, d, inter = 37, 256, 128
    X = rng.normal(size=(n, d)).astype(F32)
    w13 = rng.normal(0, 0.1, (2 * inter, d))
    w2 = rng.normal(0, 0.1, (d, inter))
    dY = rng.normal(size=(n, d))
    got = FB.fp8_expert_backward(X, w13, None, w2, None, dY)
    ref = O.swiglu_expert_backward(X, w13, w2, dY)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=2e-5, atol=2e-5 * np.abs(b).max())


def test_layer_backward_fp8_with_exact_codecs_is_the_fp64_layer_backward(monkeypatch):
    """The same at the layer: gates, router gradient and shared expert wired
    as in the fp64 layer backward."""
    _exact_codecs(monkeypatch)
    rng = np.random.default_rng(33)
    T, d, E, K, inter = 20, 128, 5, 2, 128
    x = rng.normal(size=(T, d)).astype(F32)
    wr = (rng.normal(size=(E, d)) / np.sqrt(d)).astype(F32)
    w13 = rng.normal(0, 0.1, (E, 2 * inter, d))
    w2 = rng.normal(0, 0.1, (E, d, inter))
    ws13 = rng.normal(0, 0.1, (2 * inter, d))
    ws2 = rng.normal(0, 0.1, (d, inter))
    dy = rng.normal(size=(T, d))
    u = O.router_logits(x, wr)
    idx = O.route(u, np.zeros(E, F32), K).idx
    got = O.layer_backward_fp8(x, wr, u, idx, w13, [None] * E, w2, [None] * E, ws13, None, ws2,
                               None, dy, workers=2)
    ref = O.layer_backward(x, wr, u, idx, w13, w2, ws13, ws2, dy)
    for name in ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2", "dg", "du"):
        a, b = getattr(got, name), getattr(ref, name)
        np.testing.assert_allclose(a, b, rtol=2e-5, atol=2e-5 * np.abs(b).max(), err_msg=name)


def test_expert_backward_quantization_error_is_bounded():
    """With the real codecs the FP8 expert backward stays close to the fp64
    backward of the same (dequantized) weights: each GEMM's operands carry at
    most half a step of relative error (2^-4 for E4M3, 2^-3 for E5M2), which
    bounds the error of the products far below a scale or format slip."""
    rng = np.random.default_rng(34)
    n, d, inter = 200, 256, 128
    X = rng.normal(size=(n, d)).astype(F32)
    w13q, w13s = O.quantize_blocks_128(rng.normal(0, 0.05, (2 * inter, d)).astype(F32))
    w2q, w2s = O.quantize_blocks_128(rng.normal(0, 0.05, (d, inter)).astype(F32))
    W13, W2 = O.dequant_blocks_128(w13q, w13s), O.dequant_blocks_128(w2q, w2s)
    dY = rng.normal(size=(n, d))
    dX, dW13, dW2, Y = FB.fp8_expert_backward(X, w13q, w13s, w2q, w2s, dY)
    rX, rW13, rW2, rY = O.swiglu_expert_backward(X, W13, W2, dY)
    rel = lambda a, b: float(np.abs(a - b).max() / np.abs(b).max())
    errs = [rel(dX, rX), rel(dW13, rW13), rel(dW2, rW2), rel(Y, rY)]
    assert max(errs) < 0.1, errs
    assert min(errs[:3]) > 1e-3, errs  # the quantization is really there


def test_formats_and_axes_per_operand(monkeypatch):
    """Gradients go to E5M2 and activations to E4M3 [NW, FP8 paragraph], each
    along its GEMM's contraction axis: dY (n x d) and [da | db] (n x 2I) in
    1x128 tiles along their rows for the input-gradient GEMMs and in 128x1
    tiles down their columns for the weight-gradient GEMMs, H (n x I) and X
    (n x d) in 128x1 tiles for the weight-gradient GEMMs; the quantizers read
    the bf16 copies the layer keeps of a, b, H and [da | db]."""
    calls = []
    q1, q128 = FB.quantize_1x128, FB.quantize_128x1
    monkeypatch.setattr(FB, "quantize_1x128",
                        lambda X, fmt: (calls.append(("1x128", fmt, np.shape(X))), q1(X, fmt))[1])
    monkeypatch.setattr(FB, "quantize_128x1",
                        lambda X, fmt: (calls.append(("128x1", fmt, np.shape(X))), q128(X, fmt))[1])
    rng = np.random.default_rng(35)
    n, d, inter = 40, 256, 128
    X = rng.normal(size=(n, d)).astype(F32)
    w13q, w13s = O.quantize_blocks_128(rng.normal(0, 0.05, (2 * inter, d)).astype(F32))
    w2q, w2s = O.quantize_blocks_128(rng.normal(0, 0.05, (d, inter)).astype(F32))
    rounded = []
    rb = FB.round_bf16
    monkeypatch.setattr(FB, "round_bf16",
                        lambda v: (rounded.append(np.shape(v)), rb(v))[1])
    FB.fp8_expert_backward(X, w13q, w13s, w2q, w2s, rng.normal(size=(n, d)))
    # bf16 copies the layer keeps: a, b, H (saved by the training forward)
    # and [da | db] (the weight-gradient operand)
    assert sorted(rounded) == sorted([(n, inter), (n, inter), (n, inter), (n, 2 * inter)])
    assert sorted(calls) == sorted([
        ("1x128", "e5m2", (n, d)), ("1x128", "e5m2", (n, 2 * inter)),
        ("128x1", "e5m2", (n, d)), ("128x1", "e4m3", (n, inter)),
        ("128x1", "e5m2", (n, 2 * inter)), ("128x1", "e4m3", (n, d))])


def test_input_gradient_takes_the_quantized_gate_gradients(monkeypatch):
    """dX is the product of the E5M2 1x128 tiles of [da | db] with the
    dequantized [W1; W3]: it is linear in that operand, so a quantizer whose
    tiles decode to twice the values must give exactly twice dX (powers of
    two are exact in fp64), while the other outputs stay as they were."""
    rng = np.random.default_rng(36)
    n, d, inter = 24, 384, 128  # d != 2I: the spy must not touch dY's tiles
    X = rng.normal(size=(n, d)).astype(F32)
    w13q, w13s = O.quantize_blocks_128(rng.normal(0, 0.05, (2 * inter, d)).astype(F32))
    w2q, w2s = O.quantize_blocks_128(rng.normal(0, 0.05, (d, inter)).astype(F32))
    dY = rng.normal(size=(n, d))
    base = FB.fp8_expert_backward(X, w13q, w13s, w2q, w2s, dY)
    q1 = FB.quantize_1x128

    def doubled(A, fmt):
        q, s = q1(A, fmt)
        if np.shape(A) == (n, 2 * inter):
            s = (np.asarray(s, F32) * F32(2.0)).astype(F32)
        return q, s

    monkeypatch.setattr(FB, "quantize_1x128", doubled)
    dX, dW13, dW2, Y = FB.fp8_expert_backward(X, w13q, w13s, w2q, w2s, dY)
    assert np.array_equal(dX, 2.0 * base[0])
    assert np.array_equal(dW13, base[1]) and np.array_equal(dW2, base[2])
    assert np.array_equal(Y, base[3])
