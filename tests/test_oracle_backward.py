"""Pins of the backward oracle (CPU only).

The hand-written chain rule in ``oracle.moe_backward`` is checked against
(1) central finite differences of the fp64 forward, (2) torch autograd of a
dense fp64 forward, (3) the scale invariance of the normalised gates and
(4) special cases with a known answer. A dropped term, a wrong sign or a
transposed operand anywhere in the chain fails at least one of these.
"""
import numpy as np
import pytest
import torch

import oracle

F64 = np.float64


def _tiny(seed=0, T=6, d=8, E=6, K=2, inter=4, shared=4, groups=1, topk_groups=1):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d)) / np.sqrt(d)
    bias = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    w13 = rng.normal(size=(E, 2 * inter, d)) * 0.5
    w2 = rng.normal(size=(E, d, inter)) * 0.5
    ws13 = rng.normal(size=(2 * shared, d)) * 0.5 if shared else None
    ws2 = rng.normal(size=(d, shared)) * 0.5 if shared else None
    dy = rng.normal(size=(T, d))
    u32 = oracle.router_logits(x, wr)
    rr = oracle.route(u32, bias, K, groups, topk_groups, 2)
    return dict(x=x, wr=wr, w13=w13, w2=w2, ws13=ws13, ws2=ws2, dy=dy, idx=rr.idx)


def _loss(p, idx):
    """sum <dy, y> with the selection fixed, everything in fp64."""
    x, wr = p["x"], p["wr"]
    u = x @ wr.T
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(u, idx, axis=1)))
    g = s / s.sum(axis=1, keepdims=True)
    y = oracle.layer_output(x, idx, g, p["w13"], p["w2"], p["ws13"], p["ws2"])
    return float(np.sum(p["dy"] * y))


def _grads(p):
    u = p["x"] @ p["wr"].T
    return oracle.layer_backward(p["x"], p["wr"], u, p["idx"], p["w13"], p["w2"], p["ws13"],
                                 p["ws2"], p["dy"])


@pytest.mark.parametrize("groups,topk_groups,K", [(1, 1, 2), (3, 2, 3)])
def test_backward_matches_finite_differences(groups, topk_groups, K):
    p = _tiny(seed=1 + groups, K=K, groups=groups, topk_groups=topk_groups)
    gr = _grads(p)
    rng = np.random.default_rng(7)
    h = 1e-5
    checks = [("x", gr.dx), ("wr", gr.dw_router), ("w13", gr.dw13), ("w2", gr.dw2),
              ("ws13", gr.dws13), ("ws2", gr.dws2)]
    for name, grad in checks:
        arr = p[name]
        for _ in range(6):
            pos = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[pos]
            arr[pos] = old + h
            lp = _loss(p, p["idx"])
            arr[pos] = old - h
            lm = _loss(p, p["idx"])
            arr[pos] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_backward_matches_torch_autograd():
    p = _tiny(seed=3, T=9, d=12, E=8, K=3, inter=6, shared=8)
    gr = _grads(p)
    t = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=True)
         for k in ("x", "wr", "w13", "w2", "ws13", "ws2")}
    idx = torch.tensor(p["idx"], dtype=torch.long)
    inter = p["w13"].shape[1] // 2

    def ffn(v, w13, w2):
        a = v @ w13[:inter].T
        b = v @ w13[inter:].T
        return (torch.nn.functional.silu(a) * b) @ w2.T

    u = t["x"] @ t["wr"].T
    s = torch.sigmoid(torch.gather(u, 1, idx))
    g = s / s.sum(dim=1, keepdim=True)
    shared_inter = p["ws13"].shape[0] // 2
    a = t["x"] @ t["ws13"][:shared_inter].T
    b = t["x"] @ t["ws13"][shared_inter:].T
    y = (torch.nn.functional.silu(a) * b) @ t["ws2"].T
    for tok in range(idx.shape[0]):
        for k in range(idx.shape[1]):
            e = int(idx[tok, k])
            y = y.index_add(0, torch.tensor([tok]),
                            g[tok, k] * ffn(t["x"][tok:tok + 1], t["w13"][e], t["w2"][e]))
    (torch.tensor(p["dy"]) * y).sum().backward()
    for name, ours in [("x", gr.dx), ("wr", gr.dw_router), ("w13", gr.dw13), ("w2", gr.dw2),
                       ("ws13", gr.dws13), ("ws2", gr.dws2)]:
        ref = t[name].grad.numpy()
        assert np.allclose(ours, ref, rtol=1e-10, atol=1e-12), name


def test_gate_gradient_scale_invariance():
    # g = s / S is unchanged when every selected s is scaled alike, so
    # sum_k s_k dL/ds_k = 0, i.e. sum_k du_k / (1 - s_k) = 0 for every token
    p = _tiny(seed=5, T=32, d=16, E=12, K=4, groups=4, topk_groups=2)
    gr = _grads(p)
    u = p["x"] @ p["wr"].T
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(u, p["idx"], axis=1)))
    lhs = np.sum(gr.du / (1.0 - s), axis=1)
    scale = np.max(np.abs(gr.du / (1.0 - s)), axis=1)
    assert np.all(np.abs(lhs) <= 1e-12 * np.maximum(scale, 1.0))
    assert np.max(np.abs(gr.du)) > 1e-3  # not trivially zero


def test_zero_routed_down_projection():
    # routed W2 = 0: the routed outputs vanish, so the gates get no gradient
    # (dg = du = 0, dW_r = 0) and dx is the shared expert's input gradient
    p = _tiny(seed=9, T=10, d=8, E=5, K=2)
    p["w2"][:] = 0.0
    gr = _grads(p)
    assert np.all(gr.dg == 0) and np.all(gr.du == 0) and np.all(gr.dw_router == 0)
    assert np.all(gr.dw13 == 0)
    dXs, dWs13, dWs2, _ = oracle.swiglu_expert_backward(p["x"], p["ws13"], p["ws2"], p["dy"])
    assert np.array_equal(gr.dx, dXs)
    assert np.array_equal(gr.dws13, dWs13) and np.array_equal(gr.dws2, dWs2)
    assert np.max(np.abs(gr.dw2)) > 0  # dW2 = dY^T h does not vanish


def test_single_expert_dense_swiglu_backward():
    # E = K = 1 and no shared expert: g = 1 and the layer is one dense SwiGLU
    # FFN, whose gradient is the textbook one; the router gets none (S = s)
    p = _tiny(seed=11, T=7, d=6, E=1, K=1, inter=5, shared=0)
    gr = _grads(p)
    dX, dW13, dW2, _ = oracle.swiglu_expert_backward(p["x"], p["w13"][0], p["w2"][0], p["dy"])
    assert np.allclose(gr.dx, dX, rtol=0, atol=1e-13)
    assert np.array_equal(gr.dw13[0], dW13) and np.array_equal(gr.dw2[0], dW2)
    assert np.all(np.abs(gr.du) <= 1e-15)


def test_zero_score_sum_gives_constant_gates():
    # every selected logit far below -87: the fp32 scores underflow, the
    # forward's gates are the constant 1/K, so the logits and the router get
    # no gradient while the experts still do (with weight 1/K each)
    p = _tiny(seed=13, T=5, d=8, E=6, K=2)
    u = np.full((5, 6), -120.0)
    gr = oracle.layer_backward(p["x"], p["wr"], u, p["idx"], p["w13"], p["w2"], p["ws13"],
                               p["ws2"], p["dy"])
    assert np.all(gr.du == 0) and np.all(gr.dw_router == 0)
    e = int(p["idx"][0, 0])
    dX, _, _, Y = oracle.swiglu_expert_backward(p["x"][:1], p["w13"][e], p["w2"][e],
                                                 p["dy"][:1] / 2)
    assert np.isclose(gr.dg[0, 0], np.sum(p["dy"][:1] * Y), rtol=1e-12)
    # one logit back in range: the gates are s / S again and gradients flow
    u[:, :] = -120.0
    u[np.arange(5), p["idx"][:, 0]] = 0.5
    gr2 = oracle.layer_backward(p["x"], p["wr"], u, p["idx"], p["w13"], p["w2"], p["ws13"],
                                p["ws2"], p["dy"])
    assert np.max(np.abs(gr2.du)) > 0


def test_threaded_experts_give_identical_results():
    """Running the experts' backward passes on threads changes nothing: the
    results are added in the same order."""
    p = _tiny(seed=9, T=12, E=6, K=3)
    u = p["x"] @ p["wr"].T
    a = oracle.layer_backward(p["x"], p["wr"], u, p["idx"], p["w13"], p["w2"], p["ws13"],
                              p["ws2"], p["dy"])
    b = oracle.layer_backward(p["x"], p["wr"], u, p["idx"], p["w13"], p["w2"], p["ws13"],
                              p["ws2"], p["dy"], workers=4)
    for name in ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2", "dg", "du"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
