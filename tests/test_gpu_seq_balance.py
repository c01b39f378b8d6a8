"""GPU parity of the sequence-level balance loss (moe_seq_balance_loss) against
the fp64 oracle, through the C ABI, on the GPU's own logits and selection.

Tolerances: the per-sequence losses and dloss/du are fp32 arithmetic on fp32
logits: 1e-5 (relative for the loss, row metric for dloss/du). dx and dW_r
come from products of bf16 copies of dloss/du and W_r with fp32
accumulation: the bf16 bound, 2e-2 (row metric for dx, whose rows are
tokens; per-matrix metric for dW_r, a sum over tokens)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_gate_amd as M
from sparse_mixture_experts_gate_amd import _lib as L
from sparse_mixture_experts_gate_amd.workloads import CONFIGS, Workload, make_inputs
from parity_util import TOL, host, mat_rel_err, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = Workload("seqbal_small", T=300, d=256, E=16, K=4, I=128, Is=128, G=4, M=2, topn=2,
                 x_kind="clusters", n_clusters=6, bias_kind="uniform", bias_amp=0.05,
                 w_std=0.05, seed=23)


def _log(msg):
    print(msg, flush=True)


def _check(wl, P, out, seq_len, alpha, res, logits=None, idx=None):
    logits = host(out["logits"]) if logits is None else logits
    idx = host(out["topk_idx"]) if idx is None else idx
    loss, du = O.seq_balance_loss(logits, idx, wl.E, seq_len, alpha)
    dx, dwr = O.seq_balance_input_grads(host(P["x"]), host(P["w_router"]), du)
    errs = {"loss": float(np.max(np.abs(host(res["loss"]) - loss) / np.abs(loss))),
            "dlogits": row_rel_err(host(res["dlogits"]), du),
            "dx": row_rel_err(host(res["dx"]), dx),
            "dw_router": mat_rel_err(host(res["dw_router"]), dwr)}
    _log("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert errs["loss"] <= TOL["f32"] and errs["dlogits"] <= TOL["f32"]
    assert errs["dx"] <= TOL["bf16"] and errs["dw_router"] <= TOL["bf16"]
    return loss, du


@pytest.mark.parametrize("seq_len", [300, 150, 60, 1])
def test_seq_balance_parity(seq_len):
    # 300 tokens as 1, 2, 5 or 300 sequences: chunks of 64 tokens inside a
    # sequence, ragged last chunks, one token per sequence
    wl = SMALL
    _log(f"balance loss parity: T={wl.T} seq_len={seq_len}")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = layer.forward(P["x"])
    res = layer.seq_balance_loss(P["x"], out, seq_len, 0.01, want_dlogits=True)
    torch.cuda.synchronize()
    _check(wl, P, out, seq_len, 0.01, res)


def test_seq_balance_odd_sizes():
    # E and T not multiples of 8 (padded bf16 copies), E > 64 (several
    # experts per lane), K = 1
    wl = SMALL.with_(name="seqbal_odd", T=77, E=90, K=1, G=1, M=1, topn=1)
    _log("balance loss parity: T=77 E=90 K=1")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = layer.forward(P["x"])
    res = layer.seq_balance_loss(P["x"], out, 7, 0.5, want_dlogits=True)
    torch.cuda.synchronize()
    _check(wl, P, out, 7, 0.5, res)


def test_seq_balance_special_cases():
    wl = SMALL.with_(name="seqbal_special", T=128, E=8, K=2, G=1, M=1, topn=1)
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = layer.forward(P["x"])
    # uniform scores: the loss is alpha whatever the routing
    _log("balance loss: uniform scores")
    flat = dict(out, logits=torch.full_like(out["logits"], 0.25))
    res = layer.seq_balance_loss(P["x"], flat, 64, 0.3, want_dlogits=True)
    torch.cuda.synchronize()
    assert np.allclose(host(res["loss"]), 0.3, rtol=1e-6)
    # perfect balance: every expert takes K L / E slots of each sequence, so
    # f = 1 and dloss/du vanishes up to the rounding of sum_i s'_i
    _log("balance loss: perfect balance")
    t = torch.arange(wl.T, device=DEV, dtype=torch.int32)
    bal = dict(out, topk_idx=torch.stack([(2 * t) % 8, (2 * t + 1) % 8], 1).contiguous())
    res = layer.seq_balance_loss(P["x"], bal, 32, 0.3, want_dlogits=True)
    torch.cuda.synchronize()
    assert np.allclose(host(res["loss"]), 0.3, rtol=1e-6)
    assert np.abs(host(res["dlogits"])).max() <= 1e-7 * 0.3
    # tokens whose fp32 scores all underflow: s' = 1/E, no gradient
    _log("balance loss: zero score sums")
    dead = out["logits"].clone()
    dead[::3] = -120.0
    dd = dict(out, logits=dead)
    res = layer.seq_balance_loss(P["x"], dd, 64, 0.3, want_dlogits=True)
    torch.cuda.synchronize()
    assert not host(res["dlogits"])[::3].any()
    _check(wl, P, dd, 64, 0.3, res, logits=host(dead))


def test_seq_balance_zero_tokens():
    wl = SMALL.with_(name="seqbal_empty")
    P = make_inputs(wl, DEV, T=1)
    layer = M.MoELayer(wl, P)
    out = {"logits": torch.empty(0, wl.E, device=DEV),
           "topk_idx": torch.empty(0, wl.K, dtype=torch.int32, device=DEV)}
    res = layer.seq_balance_loss(P["x"][:0], out, 4, 0.1)
    torch.cuda.synchronize()
    assert res["loss"].numel() == 0 and not host(res["dw_router"]).any()


def test_seq_balance_v3_shape():
    # the V3-shaped layer, two sequences of 4096 tokens, every output checked
    wl = CONFIGS["v3_prefill_bf16"]
    _log("balance loss parity at the V3 shape: T=8192 E=256 K=8 seq_len=4096")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = layer.forward(P["x"])
    res = layer.seq_balance_loss(P["x"], out, 4096, 1e-4, want_dlogits=True)
    torch.cuda.synchronize()
    loss, _ = _check(wl, P, out, 4096, 1e-4, res)
    _log(f"  losses {loss.tolist()}")


def _synthetic(T, E, K, d, seed):
    """Logits N(0, 4), the top-K of each row as the selection, x and W_r as
    the layer draws them (the entry point takes any logits and selection)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    logits = (2.0 * torch.randn(T, E, generator=g, device=DEV)).contiguous()
    idx = torch.topk(logits, K, dim=1).indices.to(torch.int32).contiguous()
    return logits, idx


def test_seq_balance_max_experts():
    # E = 512: eight experts per lane and the largest transposed tile
    wl = SMALL.with_(name="seqbal_e512", T=256, E=512, K=8, G=1, M=1, topn=1)
    _log("balance loss parity: E=512 K=8 T=256 seq_len=64")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    logits, idx = _synthetic(wl.T, wl.E, wl.K, wl.d, 5)
    out = {"logits": logits, "topk_idx": idx}
    res = layer.seq_balance_loss(P["x"], out, 64, 0.02, want_dlogits=True)
    torch.cuda.synchronize()
    _check(wl, P, out, 64, 0.02, res)


def test_seq_balance_at_size_limit():
    # the largest T the library accepts for d = 1024: dx [T, d] fp32 just
    # below 2^31 bytes. 2^19 - 1 is prime, so it runs as one sequence (16384
    # chunk sums per expert in the reduction). Loss and dloss/du are checked
    # on every token, dW_r in full, dx on the last rows.
    wl = SMALL.with_(name="seqbal_limit", d=1024, E=16, K=2, G=1, M=1, topn=1,
                     x_kind="normal")
    n = ctypes.c_size_t(0)
    ok = lambda T: L.lib().moe_seq_balance_workspace_size(
        ctypes.byref(M.make_desc(wl, T)), 1, ctypes.byref(n)) == 0
    T = (1 << 19) - 1
    assert ok(T) and not ok(T + 1)
    _log(f"balance loss at the size limit: T={T} d={wl.d} one sequence")
    wl = wl.with_(T=T)
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    logits, idx = _synthetic(T, wl.E, wl.K, wl.d, 6)
    out = {"logits": logits, "topk_idx": idx}
    res = layer.seq_balance_loss(P["x"], out, T, 0.05, want_dlogits=True)
    torch.cuda.synchronize()
    loss, du = O.seq_balance_loss(host(logits), host(idx), wl.E, T, 0.05)
    el = float(abs(host(res["loss"])[0] - loss[0]) / abs(loss[0]))
    eu = row_rel_err(host(res["dlogits"]), du)
    x = host(P["x"])
    dwr = du.T @ x.astype(np.float64)
    ew = mat_rel_err(host(res["dw_router"]), dwr)
    rows = np.arange(T - 64, T)
    dx = du[rows] @ host(P["w_router"]).astype(np.float64)
    ex = row_rel_err(host(res["dx"][torch.as_tensor(rows, device=DEV)]), dx)
    _log(f"  loss {el:.2e} dlogits {eu:.2e} dw_router {ew:.2e} dx(last rows) {ex:.2e}")
    assert el <= TOL["f32"] and eu <= TOL["f32"]
    assert ew <= TOL["bf16"] and ex <= TOL["bf16"]
