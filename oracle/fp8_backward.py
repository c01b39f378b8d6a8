"""FP8 backward of the DeepSeekMoE feed-forward layer, in fp64 on dequantized
operands (CPU).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library.

Sources, cited by tag as in ``moe_oracle``, plus
[NW] DeepSeek-V3 technical-report article (10100.com), FP8 paragraph: the
     forward pass uses E4M3, the backward pass E5M2.
[MH §4.1] fine-grained scaling: activations in 1x128 groups, weights in
     128x128 blocks, max-abs scaling; products accumulated in fp32.

Reading (the pages give only the formats and the group shapes): every GEMM
of the backward contracts FP8 operands that are quantized along that GEMM's
contraction axis, E5M2 for gradients and E4M3 for activations and weights:
  - input-gradient GEMMs (contraction over the output channels): gradient
    rows in 1x128 tiles along the contraction, the forward's E4M3 weight
    blocks (128x128 tiles are tiles of the transposed matrix too);
  - weight-gradient GEMMs (contraction over an expert's tokens): both
    operands in 128x1 tiles, i.e. 128 consecutive rows of the expert's
    segment in one column (the last tile of a segment may be shorter).
E5M2 (OCP): 1 sign, 5 exponent bits (bias 15), 2 mantissa bits; the top
exponent holds infinities and NaNs, so the largest finite value is 57344.
Scaling as for E4M3: scale = amax / 57344, codes of fl32(v * fl32(57344 /
amax)), round to nearest even, saturating at 57344; an all-zero group gets
scale 1 and zero codes.

Precision of what gets quantized: a code is an integer decided by floating
point, so each quantizer reads the values the layer keeps, in the precision
it keeps them (as in the bf16 backward, intermediates are bf16): the gated
output gradient bf16(fl32(g) * dy) with the forward's fp32 gates, the
pre-activations a, b and H in bf16 as the training forward saves them (the
forward itself uses their fp32 values), [da | db] in fp32 for the input
gradient (formed in the down GEMM's epilogue) and in bf16 for the weight
gradient, x in bf16. Everything after the quantizers is fp64.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import (e4m3_decode, e4m3_encode, _silu64, router_logits,  # noqa: F401
                         round_bf16, sigmoid_f32)
from .moe_backward import LayerGrads, _sigmoid64

F32 = np.float32
F64 = np.float64
E4M3_MAX = 448.0
E5M2_MAX = 57344.0

__all__ = ["e5m2_decode", "e5m2_encode", "e5m2_encode_table", "quantize_1x128",
           "quantize_128x1", "dequant_1x128", "dequant_128x1", "fp8_expert_backward",
           "layer_backward_fp8", "E5M2_MAX"]


def _e5m2_value(c: np.ndarray) -> np.ndarray:
    """OCP E5M2: value of a code from the format definition."""
    c = np.asarray(c, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 2) & 0x1F
    mant = c & 0x3
    val = np.where(ex == 0, mant / 4.0 * 2.0 ** -14, (1.0 + mant / 4.0) * np.exp2(ex - 15.0))
    val = np.where(ex == 31, np.where(mant == 0, np.inf, np.nan), val)
    return (sign * val).astype(F32)


_E5M2_VALUES = _e5m2_value(np.arange(256))
_E5M2_POS = _E5M2_VALUES[:124].astype(F64)  # the finite non-negative values, ascending


def e5m2_decode(code) -> np.ndarray:
    return _E5M2_VALUES[np.asarray(code, dtype=np.uint8)]


def e5m2_encode(v) -> np.ndarray:
    """Nearest E5M2 code, ties to the even code, magnitudes beyond 57344
    saturate to 57344; the sign bit follows the input's sign. With
    |v| = 1.f * 2^E, a normal code (E >= -14) counts steps of 2^(E-2), a
    subnormal one steps of 2^-16: code = (E + 15) * 4 + (steps - 4), or steps."""
    v = np.asarray(v, dtype=F32)
    a = np.minimum(np.abs(v), F32(E5M2_MAX))  # fp32: the scalings and rint are exact
    _, e = np.frexp(a)
    E = e - 1
    sub = E < -14
    step_exp = np.where(sub, -16, E - 2)
    steps = np.rint(np.ldexp(a, -step_exp)).astype(np.int32)
    code = np.where(sub, steps, (E + 15) * 4 + (steps - 4))
    code = np.where(a == 0.0, 0, code).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def e5m2_encode_table(v) -> np.ndarray:
    """Reference for e5m2_encode: nearest finite non-negative code by table
    search, ties to the even code, saturating at 57344."""
    v = np.asarray(v, dtype=F32)
    a = np.abs(v).astype(F64)
    hi = np.clip(np.searchsorted(_E5M2_POS, a, side="left"), 0, 123)
    lo = np.clip(hi - 1, 0, 123)
    d_lo = a - _E5M2_POS[lo]
    d_hi = _E5M2_POS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a >= _E5M2_POS[123], 123, code)
    code = np.where(a == _E5M2_POS[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


_FMT = {"e4m3": (E4M3_MAX, e4m3_encode, e4m3_decode),
        "e5m2": (E5M2_MAX, e5m2_encode, e5m2_decode)}


def _quant_groups(G: np.ndarray, fmt: str):
    """G [n_groups, size]: per group amax, scale = amax / max, codes of
    fl32(v * fl32(max / amax)); all-zero groups get scale 1, codes 0."""
    fmax, enc, _ = _FMT[fmt]
    G = np.asarray(G, F32)
    amax = np.abs(G).max(axis=1).astype(F32) if G.shape[1] else np.zeros(G.shape[0], F32)
    zero = amax == F32(0.0)
    safe = np.where(zero, F32(1.0), amax).astype(F32)
    inv = (F32(fmax) / safe).astype(F32)
    q = enc((G * inv[:, None]).astype(F32))
    q = np.where(zero[:, None], np.uint8(0), q).astype(np.uint8)
    s = np.where(zero, F32(1.0), (safe / F32(fmax)).astype(F32)).astype(F32)
    return q, s


def quantize_1x128(X, fmt: str):
    """1 x 128 tiles along each row (the contraction axis of the
    input-gradient GEMMs): X [n, D], D % 128 == 0 -> codes [n, D], scales
    [n, D/128]."""
    X = np.asarray(X, F32)
    n, D = X.shape
    q, s = _quant_groups(X.reshape(n * (D // 128), 128), fmt)
    return q.reshape(n, D), s.reshape(n, D // 128)


def dequant_1x128(q, s, fmt: str) -> np.ndarray:
    return _FMT[fmt][2](q).astype(F64) * np.repeat(np.asarray(s, F64), 128, axis=1)


def quantize_128x1(X, fmt: str):
    """128 x 1 tiles down each column (rows are the tokens of one expert
    segment, the contraction axis of the weight-gradient GEMMs): rows
    128 j .. 128 j + 127 of one column share a scale; the last tile holds the
    remaining rows. X [n, D] -> codes [n, D], scales [ceil(n/128), D]."""
    X = np.asarray(X, F32)
    n, D = X.shape
    nb = (n + 127) // 128
    q = np.zeros((n, D), np.uint8)
    s = np.ones((nb, D), F32)
    for j in range(nb):
        blk = X[j * 128:(j + 1) * 128]
        qj, sj = _quant_groups(blk.T, fmt)
        q[j * 128:(j + 1) * 128] = qj.T
        s[j] = sj
    return q, s


def dequant_128x1(q, s, fmt: str) -> np.ndarray:
    n = q.shape[0]
    return _FMT[fmt][2](q).astype(F64) * np.repeat(np.asarray(s, F64), 128, axis=0)[:n]


def _dq_blocks(q, s) -> np.ndarray:
    sc = np.repeat(np.repeat(np.asarray(s, F64), 128, axis=0), 128, axis=1)
    return e4m3_decode(q).astype(F64) * sc


def fp8_expert_backward(X, w13q, w13s, w2q, w2s, dY, weight_grads: bool = True):
    """Backward of one expert of the FP8 layer on rows X (bf16 values) with
    output gradient dY (the stored bf16 values), for the FP8 forward the
    layer computed: X in E4M3 1x128 tiles, E4M3 128x128 weight blocks, fp32
    pre-activations a, b and H = silu(a) * b. With a16, b16, H16 their bf16
    copies, returns (dX, dW13, dW2, Y) in fp64, where
      dH  = deq(E5M2 1x128 of dY) W2,        (contraction over d)
      da  = fl32(dH * b16 * silu'(a16)),  db = fl32(dH * silu(a16)),
      dX  = deq(E5M2 1x128 of [da | db]) [W1; W3],   (contraction over 2I)
      dW2 = deq(E5M2 128x1 of dY)^T deq(E4M3 128x1 of H16),
      dW13 = deq(E5M2 128x1 of bf16([da | db]))^T deq(E4M3 128x1 of X)
    (weight gradients contract over the rows, in 128-row tiles), and Y is
    the forward output (fp32 H re-quantized in E4M3 1x128 tiles). With
    weight_grads=False the weight gradients are not formed (None)."""
    from .moe_oracle import dequant_rows_1x128, quantize_rows_1x128
    X = np.asarray(X, F32)
    W13 = _dq_blocks(w13q, w13s)
    W2 = _dq_blocks(w2q, w2s)
    inter = W13.shape[0] // 2
    xq, xs = quantize_rows_1x128(X)
    Xd = dequant_rows_1x128(xq, xs)
    a = (Xd @ W13[:inter].T).astype(F32).astype(F64)
    b = (Xd @ W13[inter:].T).astype(F32).astype(F64)
    H = (a * _sigmoid64(a) * b).astype(F32)
    hq, hs = quantize_rows_1x128(H)
    Y = dequant_rows_1x128(hq, hs) @ W2.T
    a16 = round_bf16(a).astype(F64)
    b16 = round_bf16(b).astype(F64)
    H16 = round_bf16(H)
    dY32 = np.asarray(dY, F64).astype(F32)
    dYd = dequant_1x128(*quantize_1x128(dY32, "e5m2"), "e5m2")
    dH = dYd @ W2
    sa = _sigmoid64(a16)
    da = dH * b16 * (sa * (1.0 + a16 * (1.0 - sa)))
    db = dH * a16 * sa
    dG32 = np.concatenate([da, db], axis=1).astype(F32)
    dGd = dequant_1x128(*quantize_1x128(dG32, "e5m2"), "e5m2")
    dX = dGd @ W13
    if not weight_grads:
        return dX, None, None, Y
    dW2 = dequant_128x1(*quantize_128x1(dY32, "e5m2"), "e5m2").T @ \
        dequant_128x1(*quantize_128x1(H16, "e4m3"), "e4m3")
    dW13 = dequant_128x1(*quantize_128x1(round_bf16(dG32), "e5m2"), "e5m2").T @ \
        dequant_128x1(*quantize_128x1(X, "e4m3"), "e4m3")
    return dX, dW13, dW2, Y


def layer_backward_fp8(x, w_router, logits, topk_idx, w13q, w13s, w2q, w2s,
                       ws13q, ws13s, ws2q, ws2s, dy, experts=None, workers=1) -> LayerGrads:
    """Gradients of L = sum <dy, y> for the FP8 layer with the selection
    fixed to ``topk_idx``: as ``layer_backward``, with every expert's backward
    taken by ``fp8_expert_backward`` (routed experts on their rows with the
    gated output gradient bf16(fl32(g) * dy), g the forward's fp32 gates, the
    shared expert on every row with dy).
    The gates, the router and the combine stay in high precision (the gating
    module is kept in high precision [MH §4.1]): dg = <dy, y_e> with the
    expert's FP8 forward output. ``experts`` restricts the stored routed
    weight gradients; with workers > 1 the experts run on threads, their
    results added in the same order."""
    x = np.asarray(x, F32)
    wr = np.asarray(w_router, F64)
    u = np.asarray(logits, F64)
    idx = np.asarray(topk_idx)
    dy = np.asarray(dy, F64)
    T, d = x.shape
    K = idx.shape[1]
    E = wr.shape[0]
    s = _sigmoid64(np.take_along_axis(u, idx, axis=1))
    S = s.sum(axis=1)
    s32 = sigmoid_f32(np.take_along_axis(np.asarray(logits, F32), idx, axis=1))
    S32 = np.zeros(T, F32)
    for k in range(K):
        S32 = (S32 + s32[:, k]).astype(F32)
    safe = S32 > 0
    g = np.where(safe[:, None], s / np.where(safe, S, 1.0)[:, None], 1.0 / K)
    # the forward's fp32 gates: selected fp32 scores over their fp32 sum
    g32 = np.where(safe[:, None], (s32 / np.where(safe, S32, F32(1.0))[:, None]).astype(F32),
                   F32(1.0) / F32(K)).astype(F32)
    dx = np.zeros((T, d), F64)
    dg = np.zeros((T, K), F64)
    inter = np.asarray(w13q[int(idx.flat[0])]).shape[0] // 2 if T > 0 else 0
    dw13 = np.zeros((E, 2 * inter, d), F64)
    dw2 = np.zeros((E, d, inter), F64)
    wanted = None if experts is None else set(int(e) for e in experts)

    def one(e):
        rows, slots = np.nonzero(idx == e)
        dYe = round_bf16((g32[rows, slots][:, None] * dy[rows].astype(F32)).astype(F32))
        keep = wanted is None or e in wanted
        dXe, dW13e, dW2e, Ye = fp8_expert_backward(x[rows], w13q[e], w13s[e], w2q[e], w2s[e],
                                                   dYe, keep)
        return e, rows, slots, dXe, dW13e, dW2e, Ye

    ids = [int(e) for e in np.unique(idx)]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            outs = list(ex.map(one, ids))
    else:
        outs = map(one, ids)
    for e, rows, slots, dXe, dW13e, dW2e, Ye in outs:
        dg[rows, slots] = np.sum(dy[rows] * Ye, axis=1)
        np.add.at(dx, rows, dXe)
        if dW13e is not None:
            dw13[e] = dW13e
            dw2[e] = dW2e
    dws13 = dws2 = None
    if ws13q is not None:
        dXs, dws13, dws2, _ = fp8_expert_backward(x, ws13q, ws13s, ws2q, ws2s, dy)
        dx += dXs
    mean = np.sum(g * dg, axis=1, keepdims=True)
    ds = np.where(safe[:, None], (dg - mean) / np.where(safe, S, 1.0)[:, None], 0.0)
    du = ds * s * (1.0 - s)
    dx += np.einsum("tk,tkd->td", du, wr[idx])
    dw_router = np.zeros((E, d), F64)
    np.add.at(dw_router, idx.reshape(-1), du.reshape(-1)[:, None] * np.repeat(x.astype(F64), K,
                                                                               axis=0))
    return LayerGrads(dx, dw_router, dw13, dw2, dws13, dws2, dg, du)
