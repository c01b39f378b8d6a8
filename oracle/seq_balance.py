"""Sequence-level balance loss of the DeepSeekMoE router and its gradient, in fp64.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library.

What the pages fix: besides the bias-based balancing, DeepSeek-V3 adds a
sequence-level balance loss so that the tokens of one sequence do not
concentrate on a few experts [MH §1.2, "序列级负载均衡"]. The pages give it
in words only; the form below is the plainest one those words support:

For one sequence of L consecutive tokens, with the layer's own selection
e_tk (K routed experts per token) and the fp32 router logits u:
  s[t,i]  = sigmoid(u[t,i]) over all E routed experts;
  s'[t,i] = s[t,i] / S_t,  S_t = sum_i s[t,i]   (1/E for every i when S_t,
            the fp32 sum of the fp32 scores, is zero);
  P_i     = (1/L) sum_t s'[t,i]                 (mean normalized affinity);
  f_i     = E / (K L) * #{(t,k) in the sequence : e_tk = i}
            (share of the sequence's routed slots, 1 at perfect balance);
  loss    = alpha * sum_i f_i P_i.
f_i is piecewise constant in every parameter, so the gradient flows through
P only:
  dloss/ds[t,j] = alpha / (L S_t) * (f_j - F_t),  F_t = sum_i f_i s'[t,i],
  dloss/du[t,j] = dloss/ds[t,j] * s[t,j] (1 - s[t,j]),
and, with u = x W_r^T, dx = du W_r and dW_r = du^T x. The batch of T tokens
holds T / L sequences; the gradient is that of the sum of their losses.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import sigmoid_f32

F32 = np.float32
F64 = np.float64

__all__ = ["seq_balance_loss", "seq_balance_input_grads"]


def _sigmoid64(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def seq_balance_loss(logits, topk_idx, n_experts: int, seq_len: int, alpha: float):
    """Per-sequence losses [T / seq_len] and dloss/du [T, E] (fp64) for the
    router ``logits`` [T, E] (fp32 from the layer; fp64 values are taken as
    they are) and the selection ``topk_idx`` [T, K]."""
    u64 = np.asarray(logits, F64)
    u32 = u64.astype(F32)
    idx = np.asarray(topk_idx)
    T, E = u64.shape
    assert E == n_experts and T % seq_len == 0
    K = idx.shape[1] if idx.ndim == 2 else 0
    L = seq_len
    n_seq = T // L
    s = _sigmoid64(u64)
    # the zero-sum rule is decided on the fp32 scores: their sum is zero
    # exactly when every fp32 score is zero, whatever the order of the sum
    dead = np.all(sigmoid_f32(u32) == 0, axis=1) if T else np.zeros(0, bool)
    S = s.sum(axis=1)
    sn = np.where(dead[:, None], 1.0 / E, s / np.where(dead, 1.0, S)[:, None])
    losses = np.zeros(n_seq, F64)
    du = np.zeros((T, E), F64)
    for q in range(n_seq):
        rows = slice(q * L, (q + 1) * L)
        cnt = np.bincount(idx[rows].reshape(-1), minlength=E).astype(F64)
        f = cnt * E / (K * L)
        P = sn[rows].mean(axis=0)
        losses[q] = alpha * np.sum(f * P)
        F = sn[rows] @ f
        ds = alpha / (L * np.where(dead[rows], 1.0, S[rows]))[:, None] * (f[None, :] - F[:, None])
        ds[dead[rows]] = 0.0
        du[rows] = ds * s[rows] * (1.0 - s[rows])
    return losses, du


def seq_balance_input_grads(x, w_router, du):
    """dx = du W_r [T, d] and dW_r = du^T x [E, d] in fp64 (u = x W_r^T)."""
    du = np.asarray(du, F64)
    return du @ np.asarray(w_router, F64), du.T @ np.asarray(x, F64)
