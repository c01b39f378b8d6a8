"""The allocation-free forward (deepseek_moe_forward_noalloc: workspace in the
library's fixed device array) against deepseek_moe_forward with a caller
workspace, through the C ABI: two calls in a row on each layer, the second
with fewer tokens, every output equal. It runs the same kernels, so the
outputs are compared bit for bit (stricter than the tolerances of the
float outputs)."""
import pytest
import torch

import sparse_mixture_experts_gate_amd as M
from sparse_mixture_experts_gate_amd.workloads import CONFIGS, make_inputs, make_tokens
from test_gpu_sweep import CASES

pytestmark = pytest.mark.gpu
DEV = "cuda"
KEYS = ("y", "topk_idx", "topk_gate", "counts", "near_tie", "logits")


def _poisoned(layer, T):
    out = layer.alloc_outputs(T)
    for v in out.values():
        v.fill_(-7) if v.dtype == torch.int32 else v.fill_(float("nan"))
    return out


def _noalloc(layer, x, out):
    T = x.shape[0]
    M.deepseek_moe_forward_noalloc(layer.desc(T), x, layer.w_router, layer.bias, layer.weights,
                                   out["y"], out["topk_idx"], out["topk_gate"], out["counts"],
                                   out["near_tie"], out["logits"])


def _compare(layer, x, tag):
    ref = layer.forward(x)
    got = _poisoned(layer, x.shape[0])
    _noalloc(layer, x, got)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(got[k], ref[k]), (tag, k)
    print(f"  {tag}: T={x.shape[0]} all outputs equal", flush=True)


@pytest.mark.parametrize("name,T1,T2", [("small_bf16", 1024, 100), ("v3_prefill_bf16", 532, 16),
                                         ("v3_fp8", 552, 64)])
def test_noalloc_forward_matches_workspace_forward(name, T1, T2):
    wl = CONFIGS[name]
    print(f"noalloc forward {name}: T={T1} then T={T2}", flush=True)
    P = make_inputs(wl, DEV, T=T1)
    layer = M.MoELayer(wl, P)
    _compare(layer, P["x"], name)
    x2 = make_tokens(wl, T2, 11, DEV)
    _compare(layer, x2, name)


SWEEP = CASES[:24]


@pytest.mark.parametrize("wl", SWEEP, ids=[w.name for w in SWEEP])
def test_noalloc_forward_sweep(wl):
    """The seeded small shapes of the parity sweep (fp32, bf16 and FP8 layers,
    group limits, ragged T): two calls in a row, the second with a third of
    the tokens, equal bit for bit to the workspace forward."""
    print(f"noalloc sweep {wl}", flush=True)
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    _compare(layer, P["x"], wl.name)
    _compare(layer, P["x"][: max(1, wl.T // 3)].contiguous(), wl.name)


def test_noalloc_forward_rejects_calls_beyond_the_scratch():
    wl = CONFIGS["small_bf16"]
    T = 4096  # 283 MiB of workspace
    P = make_inputs(wl, DEV, T=T)
    layer = M.MoELayer(wl, P)
    out = _poisoned(layer, T)
    with pytest.raises(M.MoeError, match="fixed scratch"):
        _noalloc(layer, P["x"], out)
    torch.cuda.synchronize()
    assert (out["counts"] == -7).all() and torch.isnan(out["y"].float()).all()
