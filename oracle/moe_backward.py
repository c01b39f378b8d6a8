"""Backward of the DeepSeekMoE feed-forward layer for a fixed routing, in fp64.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library.

What is differentiated (sources cited by tag as in ``moe_oracle``):
  u = x W_r^T, s = sigmoid(u) [KY, DeepSeekMoE paragraph];
  g[t,k] = s[t, e_tk] / S_t, S_t = sum_k s[t, e_tk] (gates normalise the
  selected affinity scores [KY]);
  y_t = FFN_shared(x_t) + sum_k g[t,k] FFN_{e_tk}(x_t) (one always-on shared
  expert plus the routed ones [MH §1.1]), FFN(v) = W2 (silu(W1 v) * (W3 v)).
The selection e_tk (top-K of s + b inside the allowed groups) is piecewise
constant in every parameter, so for a fixed selection the gradient is that of
the smooth expression above; the bias, which only takes part in the
selection, receives no gradient (it is adjusted by the load rule instead, not
by gradient descent [MH §1.2; GK Q3]). Weight gradients are returned in fp64:
the pages keep weight gradients in high precision [MH §4.1].

The chain rule, written out for one token t with loss L = sum_t <dy_t, y_t>:
  dg[t,k]   = <dy_t, FFN_{e_tk}(x_t)>
  dL/ds_j   = (dg_j - sum_k g_k dg_k) / S_t              (quotient rule)
  du[t,j]   = dL/ds_j * s_j * (1 - s_j)                  (sigmoid')
  dx_t      = dFFN_shared^T dy_t + sum_k dFFN_{e_tk}^T (g_k dy_t)
              + sum_k du[t,k] W_r[e_tk]
  dW_r[e]   = sum over (t,k) with e_tk = e of du[t,k] x_t
and for one expert applied to rows X with output gradient dY:
  a = X W1^T, b = X W3^T, h = silu(a) * b, Y = h W2^T
  dW2 = dY^T h,  dh = dY W2,  da = dh * b * silu'(a),  db = dh * silu(a)
  dW1 = da^T X,  dW3 = db^T X,  dX = da W1 + db W3,
  silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .moe_oracle import sigmoid_f32

F32 = np.float32
F64 = np.float64

__all__ = ["swiglu_expert_backward", "layer_backward", "LayerGrads"]


def _sigmoid64(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def swiglu_expert_backward(X, w13, w2, dY, weight_grads: bool = True):
    """Gradients of Y = (silu(X W1^T) * (X W3^T)) W2^T, with w13 = [W1; W3]
    stacked as [2I, d] and w2 = [d, I], for the output gradient dY.
    Returns (dX [n, d], dW13 [2I, d], dW2 [d, I], Y [n, d]), all fp64; with
    weight_grads=False the two weight gradients are not formed (None)."""
    X = np.asarray(X, F64)
    w13 = np.asarray(w13, F64)
    w2 = np.asarray(w2, F64)
    dY = np.asarray(dY, F64)
    inter = w13.shape[0] // 2
    W1, W3 = w13[:inter], w13[inter:]
    a = X @ W1.T
    b = X @ W3.T
    sa = _sigmoid64(a)
    silu = a * sa
    h = silu * b
    Y = h @ w2.T
    dh = dY @ w2
    da = dh * b * (sa * (1.0 + a * (1.0 - sa)))
    db = dh * silu
    dX = da @ W1 + db @ W3
    if not weight_grads:
        return dX, None, None, Y
    dW2 = dY.T @ h
    dW13 = np.concatenate([da.T @ X, db.T @ X], axis=0)
    return dX, dW13, dW2, Y


@dataclass
class LayerGrads:
    dx: np.ndarray          # [T, d]
    dw_router: np.ndarray   # [E, d]
    dw13: np.ndarray        # [E, 2I, d]
    dw2: np.ndarray         # [E, d, I]
    dws13: np.ndarray | None
    dws2: np.ndarray | None
    dg: np.ndarray          # [T, K] gradient of the gates
    du: np.ndarray          # [T, K] gradient of the selected logits


def layer_backward(x, w_router, logits, topk_idx, w13, w2, ws13, ws2, dy,
                   experts=None, workers=1) -> LayerGrads:
    """Gradients of L = sum <dy, y> for the layer with the selection fixed to
    ``topk_idx`` [T, K]; the gates are recomputed in fp64 from the fp32
    ``logits`` [T, E] (g = s / S over the selected s), except for tokens whose
    fp32 score sum is zero (every selected logit below about -87), where the
    forward's gates are the constant 1/K and the logits get no gradient. ``w13[e]``, ``w2[e]``
    may be lazy containers. ``experts`` (optional) restricts the routed weight
    gradients to those expert ids (the others stay zero); dx, dg and du need
    every routed expert of every token, so it is only for weight-gradient
    spot checks. With workers > 1 the experts' backward passes run on that
    many threads; their results are added in the same order either way."""
    x = np.asarray(x, F64)
    wr = np.asarray(w_router, F64)
    u = np.asarray(logits, F64)
    idx = np.asarray(topk_idx)
    dy = np.asarray(dy, F64)
    T, d = x.shape
    K = idx.shape[1]
    E = wr.shape[0]
    s = _sigmoid64(np.take_along_axis(u, idx, axis=1))   # [T, K] selected scores
    S = s.sum(axis=1)
    # the forward's rule: where the fp32 sum of the fp32 scores (slot order)
    # is zero, the gates are the constant 1/K, so nothing flows to the logits
    s32 = sigmoid_f32(np.take_along_axis(np.asarray(logits, F32), idx, axis=1))
    S32 = np.zeros(T, F32)
    for k in range(K):
        S32 = (S32 + s32[:, k]).astype(F32)
    safe = S32 > 0
    g = np.where(safe[:, None], s / np.where(safe, S, 1.0)[:, None], 1.0 / K)

    dx = np.zeros((T, d), F64)
    dg = np.zeros((T, K), F64)
    inter = np.asarray(w13[int(idx.flat[0])]).shape[0] // 2 if T > 0 else 0
    dw13 = np.zeros((E, 2 * inter, d), F64)
    dw2 = np.zeros((E, d, inter), F64)
    wanted = None if experts is None else set(int(e) for e in experts)

    def one(e):
        rows, slots = np.nonzero(idx == e)
        dYe = g[rows, slots][:, None] * dy[rows]
        keep = wanted is None or e in wanted
        dXe, dW13e, dW2e, Ye = swiglu_expert_backward(x[rows], w13[e], w2[e], dYe, keep)
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
    if ws13 is not None:
        dXs, dws13, dws2, _ = swiglu_expert_backward(x, ws13, ws2, dy)
        dx += dXs
    # router: quotient rule through the normalisation, then sigmoid'
    mean = np.sum(g * dg, axis=1, keepdims=True)
    ds = np.where(safe[:, None], (dg - mean) / np.where(safe, S, 1.0)[:, None], 0.0)
    du = ds * s * (1.0 - s)
    dx += np.einsum("tk,tkd->td", du, wr[idx])
    dw_router = np.zeros((E, d), F64)
    np.add.at(dw_router, idx.reshape(-1), du.reshape(-1)[:, None] * np.repeat(x, K, axis=0))
    return LayerGrads(dx, dw_router, dw13, dw2, dws13, dws2, dg, du)
