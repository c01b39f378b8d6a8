"""Pins of the sequence-level balance loss oracle (CPU only).

``oracle.seq_balance`` writes the loss and its hand-derived gradient out
step by step. They are checked against values the definition fixes without
any implementation: uniform scores give exactly alpha whatever the routing,
perfectly balanced routing gives a zero gradient whatever the scores, one
sequence of a batch does not see another; and against central finite
differences and torch autograd of an independently written expression. A
dropped term, a wrong sign, a transposed operand or a wrong normalization
(by K, L or E) fails at least one of them.
"""
import numpy as np
import torch

import oracle

F64 = np.float64


def _case(seed=0, T=12, E=8, K=2, scale=1.0):
    rng = np.random.default_rng(seed)
    u = (rng.normal(size=(T, E)) * scale).astype(np.float32)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    return u, idx


def test_uniform_scores_give_alpha():
    # s' = 1/E for every expert and sum_i f_i = E, so the loss is alpha
    for seed, (T, E, K, L) in enumerate([(12, 8, 2, 6), (30, 16, 4, 10), (7, 5, 3, 7)]):
        _, idx = _case(seed, T, E, K)
        u = np.full((T, E), 0.3, np.float32)
        loss, _ = oracle.seq_balance_loss(u, idx, E, L, 0.25)
        assert np.allclose(loss, 0.25, rtol=0, atol=1e-15)


def test_zero_score_sum_gives_uniform_share_and_no_gradient():
    # every fp32 score underflows: s' is 1/E by the stated rule, so the loss
    # is alpha again and nothing flows back
    _, idx = _case(1, 8, 6, 2)
    u = np.full((8, 6), -120.0, np.float32)
    loss, du = oracle.seq_balance_loss(u, idx, 6, 4, 0.5)
    assert np.allclose(loss, 0.5, atol=1e-15) and not du.any()


def test_perfect_balance_gives_zero_gradient():
    # each expert takes exactly K L / E slots of every sequence: f_i = 1 and
    # F_t = sum_i s'_i = 1, so dloss/ds vanishes for any scores
    E, K, L = 8, 2, 8
    T = 2 * L
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], np.int32)
    u, _ = _case(2, T, E, K, scale=2.0)
    loss, du = oracle.seq_balance_loss(u, idx, E, L, 0.1)
    assert np.max(np.abs(du)) < 1e-17
    # and the loss is alpha * sum_i P_i = alpha
    assert np.allclose(loss, 0.1, atol=1e-15)


def test_single_expert_concentration():
    # K = 1 and every token on expert 0: f = [E, 0, ...], loss = alpha E P_0
    T, E, L = 6, 4, 3
    u, _ = _case(3, T, E, 1)
    idx = np.zeros((T, 1), np.int32)
    loss, _ = oracle.seq_balance_loss(u, idx, E, L, 1.0)
    s = 1.0 / (1.0 + np.exp(-u.astype(F64)))
    sn = s / s.sum(1, keepdims=True)
    for q in range(T // L):
        assert np.isclose(loss[q], E * sn[q * L:(q + 1) * L, 0].mean(), rtol=1e-14)


def test_sequences_are_independent():
    u, idx = _case(4, 24, 8, 2)
    loss, du = oracle.seq_balance_loss(u, idx, 8, 8, 0.3)
    for q in range(3):
        r = slice(8 * q, 8 * q + 8)
        l1, d1 = oracle.seq_balance_loss(u[r], idx[r], 8, 8, 0.3)
        assert l1[0] == loss[q] and np.array_equal(d1, du[r])
    # the single-sequence loss is not the sum of the per-sequence ones
    lall, _ = oracle.seq_balance_loss(u, idx, 8, 24, 0.3)
    assert not np.isclose(lall[0], loss.sum())


def test_gradient_matches_finite_differences():
    u, idx = _case(5, 10, 6, 2)
    L, alpha = 5, 0.7
    _, du = oracle.seq_balance_loss(u, idx, 6, L, alpha)
    u64 = u.astype(F64)
    h = 1e-6
    for t, j in [(0, 0), (3, 5), (7, 2), (9, 1), (4, 4)]:
        up, dn = u64.copy(), u64.copy()
        up[t, j] += h
        dn[t, j] -= h
        lp, _ = oracle.seq_balance_loss(up, idx, 6, L, alpha)
        lm, _ = oracle.seq_balance_loss(dn, idx, 6, L, alpha)
        fd = (lp.sum() - lm.sum()) / (2 * h)
        assert np.isclose(du[t, j], fd, rtol=1e-6, atol=1e-10), (t, j, du[t, j], fd)


def test_gradient_matches_autograd():
    T, E, K, L, alpha = 16, 8, 3, 8, 0.05
    u, idx = _case(6, T, E, K)
    _, du = oracle.seq_balance_loss(u, idx, E, L, alpha)
    ut = torch.tensor(u.astype(F64), requires_grad=True)
    onehot = torch.zeros(T, E, dtype=torch.float64)
    onehot.scatter_(1, torch.tensor(idx, dtype=torch.int64), 1.0)
    total = 0.0
    for q in range(T // L):
        sl = slice(q * L, (q + 1) * L)
        sc = torch.sigmoid(ut[sl])
        P = (sc / sc.sum(1, keepdim=True)).mean(0)
        f = onehot[sl].sum(0) * E / (K * L)
        total = total + alpha * (f * P).sum()
    total.backward()
    assert np.allclose(du, ut.grad.numpy(), rtol=1e-12, atol=1e-16)


def test_input_gradients_are_the_router_chain():
    # u = x W_r^T: finite differences of the loss in x and W_r
    rng = np.random.default_rng(7)
    T, E, K, d, L, alpha = 8, 6, 2, 5, 4, 0.4
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d)) / np.sqrt(d)
    _, idx = _case(7, T, E, K)
    u = x @ wr.T
    _, du = oracle.seq_balance_loss(u, idx, E, L, alpha)
    dx, dwr = oracle.seq_balance_input_grads(x, wr, du)
    h = 1e-6

    def loss_of(xx, ww):
        return oracle.seq_balance_loss(xx @ ww.T, idx, E, L, alpha)[0].sum()

    for (t, j) in [(0, 0), (5, 3), (7, 4)]:
        xp, xm = x.copy(), x.copy()
        xp[t, j] += h
        xm[t, j] -= h
        assert np.isclose(dx[t, j], (loss_of(xp, wr) - loss_of(xm, wr)) / (2 * h), rtol=1e-6,
                          atol=1e-10)
    for (e, j) in [(0, 1), (3, 0), (5, 4)]:
        wp, wm = wr.copy(), wr.copy()
        wp[e, j] += h
        wm[e, j] -= h
        assert np.isclose(dwr[e, j], (loss_of(x, wp) - loss_of(x, wm)) / (2 * h), rtol=1e-6,
                          atol=1e-10)
