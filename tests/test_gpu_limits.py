"""GPU parity at the largest calls the descriptor accepts: the kernels address
the gathered activation rows (and, in the backward, the routed rows) with
32-bit byte offsets, so the last tokens and the last permuted rows sit just
below 2^31 bytes; the forward's H is addressed per tile from a 64-bit base and
lies well beyond 2^31 bytes at the forward's limit. The largest T is
found through the library's own validation (moe_workspace_size /
moe_backward_workspace_size), on a layer narrow enough that the oracle checks
the rows near the end one by one: routing bit-exact on every token from the
kernel's logits, outputs of the last tokens and of the tokens behind the last
permuted rows, and, for the backward at its own limit, the input gradients of
the last tokens and the weight gradients of the expert whose rows come last."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_gate_amd as M
from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd.workloads import Workload, make_inputs
from parity_util import TOL, host, mat_rel_err, route_args, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"

WIDE = Workload("limit", T=1, d=1024, E=16, K=2, I=512, Is=512, G=4, M=2, topn=1,
                x_kind="normal", bias_kind="uniform", bias_amp=0.05, w_std=0.03, seed=31)


def _log(msg):
    print(msg, flush=True)


def _largest_T(wl, fn) -> int:
    """Largest T for which the library accepts the descriptor."""
    n = ctypes.c_size_t(0)
    ok = lambda T: fn(ctypes.byref(M.make_desc(wl, T)), ctypes.byref(n)) == 0
    lo, hi = 1, 1 << 24
    assert ok(lo) and not ok(hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if ok(mid) else (lo, mid)
    return lo


def _sample(T, perm, extra=4):
    """The last tokens and the tokens behind the last permuted rows."""
    toks = set(range(T - extra, T)) | {int(t) for t in perm[-extra:]} | {0}
    return np.array(sorted(toks))


def test_forward_at_size_limit():
    wl = WIDE
    T = _largest_T(wl, L.lib().moe_workspace_size)
    # x is the binding limit here: T * d * 2 bytes < 2^31; H (T (K + 1) rows of
    # max(I, Is) bf16) is larger than 2^31 bytes, so its last rows are read
    # through the per-tile resource
    assert T * wl.d * 2 < (1 << 31) and (T + 1) * wl.d * 2 >= (1 << 31) - 1
    assert T * (wl.K + 1) * max(wl.I, wl.Is) * 2 > (1 << 31)
    _log(f"forward at the size limit: T = {T}")
    wl = wl.with_(T=T)
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = layer.forward(P["x"])
    torch.cuda.synchronize()
    logits, idx = host(out["logits"]), host(out["topk_idx"])
    rr = O.route(logits, host(P["bias"]), **route_args(wl))
    assert np.array_equal(idx, rr.idx)
    assert np.array_equal(host(out["topk_gate"]).view(np.uint32), rr.gate.view(np.uint32))
    pr = O.permute(rr.idx, wl.E)
    assert np.array_equal(host(out["counts"]), pr.counts)
    rows = _sample(T, pr.perm)
    x = host(P["x"][torch.as_tensor(rows, device=DEV)])
    ref = O.layer_output(x, rr.idx[rows], rr.gate[rows], host(P["w13"]), host(P["w2"]),
                         host(P["ws13"]), host(P["ws2"]))
    err = row_rel_err(host(out["y"][torch.as_tensor(rows, device=DEV)]), ref)
    _log(f"  tokens {rows.tolist()}: max row-rel err {err:.2e}")
    assert err <= TOL["bf16"]


def _channel_grads(x, w13, w2, dY, chans):
    """Weight gradients of intermediate channels `chans` of one expert over all
    its rows: SwiGLU acts on each intermediate channel alone, so the rows c
    and I + c of dW13 and the column c of dW2 are those of the expert cut down
    to that channel (I = 1). Returns {c: (dW13 rows [2, d], dW2 column [d])}."""
    inter = w13.shape[0] // 2
    out = {}
    for c in chans:
        _, d13, d2, _ = O.swiglu_expert_backward(x, w13[[c, inter + c]], w2[:, [c]], dY)
        out[c] = (d13, d2[:, 0])
    return out


def test_backward_at_size_limit():
    wl = WIDE
    T = _largest_T(wl, L.lib().moe_backward_workspace_size)
    # the shared expert's rows in the weight-gradient GEMMs bind:
    # T * max(d, 2 max(I, Is)) * 2 bytes < 2^31; the routed buffers ([T K, d]
    # gradients, [T (K + 1), 2 max(I, Is)] [da | db]) lie beyond 2^31 bytes
    row = max(wl.d, 2 * max(wl.I, wl.Is)) * 2
    assert T * row < (1 << 31) and (T + 1) * row >= (1 << 31) - 1
    assert T * wl.K * wl.d * 2 > (1 << 31)
    _log(f"backward at the size limit: T = {T}")
    wl = wl.with_(T=T)
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    y, sv = layer.forward_train(P["x"])
    g = torch.Generator(device=DEV)
    g.manual_seed(41)
    dy = torch.randn(T, wl.d, generator=g, device=DEV).to(torch.bfloat16)
    dx, gr = layer.backward(P["x"], dy, sv)
    torch.cuda.synchronize()
    logits, idx, perm = host(sv["logits"]), host(sv["topk_idx"]), host(sv["perm"])
    w13, w2 = host(P["w13"]), host(P["w2"])
    ws13, ws2 = host(P["ws13"]), host(P["ws2"])
    rows = _sample(T, perm)
    t = torch.as_tensor(rows, device=DEV)
    ref = O.layer_backward(host(P["x"][t]), host(P["w_router"]), logits[rows], idx[rows], w13, w2,
                           ws13, ws2, host(dy[t]))
    err = row_rel_err(host(dx[t]), ref.dx)
    _log(f"  tokens {rows.tolist()}: dx max row-rel err {err:.2e}")
    assert err <= TOL["bf16"]
    # weight gradients over all rows, three intermediate channels each: the
    # expert whose rows are last in the permuted buffers, and the shared
    # expert (every token)
    counts = host(sv["counts"])
    e = int(np.nonzero(counts)[0][-1])
    toks, slots = np.nonzero(idx == e)
    s_sel = 1.0 / (1.0 + np.exp(-np.take_along_axis(logits[toks].astype(np.float64),
                                                    idx[toks], 1)))
    gate = s_sel[np.arange(len(toks)), slots] / s_sel.sum(1)
    xe = host(P["x"][torch.as_tensor(toks, device=DEV)])
    dye = host(dy[torch.as_tensor(toks, device=DEV)])
    chans = [0, wl.I // 2 + 1, wl.I - 1]
    dw13, dw2 = host(gr["dw13"][e]), host(gr["dw2"][e])
    for c, (d13, d2) in _channel_grads(xe, w13[e], w2[e], gate[:, None] * dye, chans).items():
        e13 = mat_rel_err(dw13[[c, wl.I + c]], d13)
        e2 = mat_rel_err(dw2[:, c], d2)
        _log(f"  expert {e} ({len(toks)} tokens), channel {c}: dw13 {e13:.2e} dw2 {e2:.2e}")
        assert e13 <= TOL["bf16"] and e2 <= TOL["bf16"]
    x_all, dy_all = host(P["x"]), host(dy)
    dws13, dws2 = host(gr["dws13"]), host(gr["dws2"])
    chans = [0, wl.Is // 3, wl.Is - 1]
    for c, (d13, d2) in _channel_grads(x_all, ws13, ws2, dy_all, chans).items():
        e13 = mat_rel_err(dws13[[c, wl.Is + c]], d13)
        e2 = mat_rel_err(dws2[:, c], d2)
        _log(f"  shared expert ({T} tokens), channel {c}: dw13 {e13:.2e} dw2 {e2:.2e}")
        assert e13 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_fp8_forward_at_size_limit():
    # FP8 weights: H is one byte per element, so x (T * d * 2 bytes) binds
    wl = WIDE.with_(name="limit_fp8", w="fp8")
    T = _largest_T(wl, L.lib().moe_workspace_size)
    assert T * wl.d * 2 < (1 << 31) and (T + 1) * wl.d * 2 >= (1 << 31) - 1
    _log(f"fp8 forward at the size limit: T = {T}")
    wl = wl.with_(T=T)
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = layer.forward(P["x"])
    torch.cuda.synchronize()
    logits, idx = host(out["logits"]), host(out["topk_idx"])
    rr = O.route(logits, host(P["bias"]), **route_args(wl))
    assert np.array_equal(idx, rr.idx)
    pr = O.permute(rr.idx, wl.E)
    rows = _sample(T, pr.perm)
    q13 = [O.quantize_blocks_128(host(P["w13"][e])) for e in range(wl.E)]
    q2 = [O.quantize_blocks_128(host(P["w2"][e])) for e in range(wl.E)]
    ws13q, ws13s = O.quantize_blocks_128(host(P["ws13"]))
    ws2q, ws2s = O.quantize_blocks_128(host(P["ws2"]))
    x = host(P["x"][torch.as_tensor(rows, device=DEV)])
    ref = O.layer_output_fp8(x, rr.idx[rows], rr.gate[rows], [q[0] for q in q13],
                             [q[1] for q in q13], [q[0] for q in q2], [q[1] for q in q2],
                             ws13q, ws13s, ws2q, ws2s)
    err = row_rel_err(host(out["y"][torch.as_tensor(rows, device=DEV)]), ref)
    _log(f"  tokens {rows.tolist()}: max row-rel err {err:.2e}")
    assert err <= TOL["fp8"]
