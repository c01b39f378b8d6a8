"""GPU parity of the FP8 training path (moe_forward_train with E4M3 weights,
moe_backward_fp8) against the oracle's FP8 backward (oracle.fp8_backward):
every backward GEMM on FP8 operands quantized along its contraction axis,
E5M2 gradients and E4M3 activations and weights (forward E4M3, backward E5M2:
10100.com DeepSeek-V3 technical-report article, FP8 paragraph; 1x128 / 128x128
scaling: mhpq.cn §4.1). The oracle quantizes the bf16 master weights itself.

Tolerance: the stated FP8 bound, 6e-2, with the input gradient compared row
by row and every weight gradient per matrix (as in the bf16 backward)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_gate_amd as M
from sparse_mixture_experts_gate_amd.workloads import CONFIGS, Workload, make_inputs
from parity_util import TOL, host, mat_rel_err, route_args, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))

# ragged rows, 4 groups of 4 experts with 2 allowed, clustered tokens
FP8_SMALL = Workload("fp8_train_small", T=300, d=256, E=16, K=4, I=256, Is=384, G=4, M=2, topn=2,
                     w="fp8", x_kind="clusters", n_clusters=6, bias_kind="uniform", bias_amp=0.05,
                     w_std=0.05, seed=21)
FP8_MED = CONFIGS["small_bf16"].with_(name="fp8_train_med", T=1024, w="fp8")


def _log(msg):
    print(msg, flush=True)


def _dy(wl, T, seed=77):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(T, wl.d, generator=g, device=DEV).to(torch.bfloat16).contiguous()


class _QuantCache:
    """Oracle-side 128x128 E4M3 quantization of a [E, rows, cols] bf16 weight
    tensor, expert by expert (codes, scales)."""

    def __init__(self, t):
        self.t, self.c = t, {}

    def get(self, e):
        e = int(e)
        if e not in self.c:
            self.c[e] = O.quantize_blocks_128(host(self.t[e]))
        return self.c[e]


class _Part:
    def __init__(self, qc, i):
        self.qc, self.i = qc, i

    def __getitem__(self, e):
        return self.qc.get(e)[self.i]


def _oracle(wl, P, sv, dy, rows=None, experts=None):
    q13, q2 = _QuantCache(P["w13"]), _QuantCache(P["w2"])
    sh = (None,) * 4
    if wl.Is:
        sh = (*O.quantize_blocks_128(host(P["ws13"])), *O.quantize_blocks_128(host(P["ws2"])))
    x, lg, idx, d = host(P["x"]), host(sv["logits"]), host(sv["topk_idx"]), host(dy)
    if rows is not None:
        x, lg, idx, d = x[rows], lg[rows], idx[rows], d[rows]
    return O.layer_backward_fp8(x, host(P["w_router"]), lg, idx, _Part(q13, 0), _Part(q13, 1),
                                _Part(q2, 0), _Part(q2, 1), *sh, d, experts=experts,
                                workers=WORKERS)


def _run(wl, T=None):
    P = make_inputs(wl, DEV, T=T)
    layer = M.MoELayer(wl, P)
    y, sv = layer.forward_train(P["x"])
    dy = _dy(wl, P["x"].shape[0])
    dx, gr = layer.backward(P["x"], dy, sv)
    torch.cuda.synchronize()
    return P, layer, y, sv, dy, dx, gr


@pytest.mark.parametrize("name", ["fp8_train_small", "fp8_train_med"])
def test_fp8_backward_parity(name):
    wl = FP8_SMALL if name == "fp8_train_small" else FP8_MED
    _log(f"FP8 backward parity {name} T={wl.T}")
    P, layer, y, sv, dy, dx, gr = _run(wl)
    # the training forward is the FP8 inference forward plus saved tensors
    out = layer.forward(P["x"])
    torch.cuda.synchronize()
    assert torch.equal(y, out["y"])
    rr = O.route(host(sv["logits"]), host(P["bias"]), **route_args(wl))
    assert np.array_equal(host(sv["topk_idx"]), rr.idx)
    ref = _oracle(wl, P, sv, dy)
    tol = TOL["fp8"]
    dw13, dw2 = host(gr["dw13"]), host(gr["dw2"])
    counts = host(sv["counts"])
    used = np.nonzero(counts)[0]
    errs = {"dx": row_rel_err(host(dx), ref.dx),
            "dw_router": mat_rel_err(host(gr["dw_router"]), ref.dw_router),
            "dw13": max(mat_rel_err(dw13[e], ref.dw13[e]) for e in used),
            "dw2": max(mat_rel_err(dw2[e], ref.dw2[e]) for e in used)}
    if wl.Is:
        errs["dws13"] = mat_rel_err(host(gr["dws13"]), ref.dws13)
        errs["dws2"] = mat_rel_err(host(gr["dws2"]), ref.dws2)
    _log("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)
    for e in np.nonzero(counts == 0)[0]:
        assert not dw13[int(e)].any() and not dw2[int(e)].any()


def test_fp8_backward_no_shared_empty_experts():
    wl = FP8_SMALL.with_(name="fp8_noshared", T=77, E=24, K=3, G=1, M=1, Is=0, n_clusters=3)
    _log("FP8 backward: no shared expert, most experts empty")
    P, layer, y, sv, dy, dx, gr = _run(wl)
    ref = _oracle(wl, P, sv, dy)
    tol = TOL["fp8"]
    counts = host(sv["counts"])
    assert (counts == 0).sum() > 0
    dw13, dw2 = host(gr["dw13"]), host(gr["dw2"])
    assert row_rel_err(host(dx), ref.dx) <= tol
    for e in range(wl.E):
        if counts[e]:
            assert mat_rel_err(dw13[e], ref.dw13[e]) <= tol
            assert mat_rel_err(dw2[e], ref.dw2[e]) <= tol
        else:
            assert not dw13[e].any() and not dw2[e].any()


def test_fp8_backward_single_token_zero_tokens_and_large_k():
    """Degenerate sizes of the FP8 backward: one token (every 128x1 tile holds
    one row, padded with zeros), no token (the weight gradients are
    zero-filled, whatever the buffers held), and more than eight experts per
    token (K = 12 of 24, two groups allowed of four)."""
    wl = FP8_SMALL
    _log("FP8 backward: T = 1")
    P, layer, y, sv, dy, dx, gr = _run(wl, T=1)
    ref = _oracle(wl, P, sv, dy)
    tol = TOL["fp8"]
    assert row_rel_err(host(dx), ref.dx) <= tol
    counts = host(sv["counts"])
    dw13, dw2 = host(gr["dw13"]), host(gr["dw2"])
    for e in range(wl.E):
        if counts[e]:
            assert mat_rel_err(dw13[e], ref.dw13[e]) <= tol
            assert mat_rel_err(dw2[e], ref.dw2[e]) <= tol
        else:
            assert not dw13[e].any() and not dw2[e].any()
    assert mat_rel_err(host(gr["dws13"]), ref.dws13) <= tol
    assert mat_rel_err(host(gr["dws2"]), ref.dws2) <= tol
    _log("FP8 backward: T = 0 zero-fills the weight gradients")
    g0 = {k: (None if v is None else torch.full_like(v, 3.0)) for k, v in gr.items()}
    x0 = P["x"][:0]
    sv0 = layer.alloc_saved(0)
    layer.forward_train(x0, sv0)
    dx0, g0 = layer.backward(x0, dy[:0], sv0, grads=g0)
    torch.cuda.synchronize()
    assert dx0.numel() == 0
    for k, v in g0.items():
        if v is not None:
            assert not v.any(), k
    wl = FP8_SMALL.with_(name="fp8_k12", T=200, E=24, K=12, G=4, M=2, n_clusters=4)
    _log("FP8 backward: K = 12")
    P, layer, y, sv, dy, dx, gr = _run(wl)
    ref = _oracle(wl, P, sv, dy)
    assert row_rel_err(host(dx), ref.dx) <= tol
    counts = host(sv["counts"])
    dw13, dw2 = host(gr["dw13"]), host(gr["dw2"])
    errs = [max(mat_rel_err(dw13[e], ref.dw13[e]), mat_rel_err(dw2[e], ref.dw2[e]))
            for e in np.nonzero(counts)[0]]
    _log(f"  dx {row_rel_err(host(dx), ref.dx):.2e} dW max {max(errs):.2e}")
    assert max(errs) <= tol


def test_fp8_backward_v3_sampled():
    """The V3 layer in FP8 (T = 8192, d = 7168, 256 experts of 2048, shared
    expert of 2048) as the benchmark runs it: the input gradients of 256
    tokens whose experts all lie among the 32 most loaded ones, and the
    weight gradients of four experts from the coldest to a hot one."""
    wl = CONFIGS["v3_fp8"]
    _log("FP8 backward V3 sampled: running the layer")
    P, layer, y, sv, dy, dx, gr = _run(wl)
    idx = host(sv["topk_idx"])
    counts = host(sv["counts"])
    by_load = np.argsort(-counts, kind="stable")
    used = by_load[counts[by_load] > 0]
    rng = np.random.default_rng(6)
    inside = np.nonzero(np.isin(idx, by_load[:32]).all(axis=1))[0]
    toks = np.sort(rng.choice(inside, size=min(256, len(inside)), replace=False))
    _log(f"  oracle: input gradients of {len(toks)} tokens ({len(np.unique(idx[toks]))} experts)")
    ref = _oracle(wl, P, sv, dy, rows=toks, experts=())
    e = row_rel_err(host(dx)[toks], ref.dx)
    _log(f"  dx: {e:.2e}")
    assert e <= TOL["fp8"]
    # weight gradients: all tokens of each picked expert (oracle on those rows
    # only, the gates from their logits)
    pick = [int(used[-1]), int(used[-len(used) // 4]), int(used[len(used) // 2]), int(used[8])]
    logits = host(sv["logits"]).astype(np.float64)
    x, dyh = host(P["x"]), host(dy).astype(np.float64)

    def one(e):
        rows, slots = np.nonzero(idx == e)
        s = 1.0 / (1.0 + np.exp(-np.take_along_axis(logits[rows], idx[rows], 1)))
        g = (s / s.sum(1, keepdims=True))[np.arange(len(rows)), slots]
        q13 = O.quantize_blocks_128(host(P["w13"][e]))
        q2 = O.quantize_blocks_128(host(P["w2"][e]))
        _, dW13, dW2, _ = O.fp8_expert_backward(x[rows], *q13, *q2, g[:, None] * dyh[rows])
        return e, len(rows), mat_rel_err(host(gr["dw13"][e]), dW13), \
            mat_rel_err(host(gr["dw2"][e]), dW2)

    with ThreadPoolExecutor(len(pick)) as ex:
        for e, n, e13, e2 in ex.map(one, pick):
            _log(f"  expert {e} ({n} tokens): dw13 {e13:.2e} dw2 {e2:.2e}")
            assert e13 <= TOL["fp8"] and e2 <= TOL["fp8"]
