"""GPU parity against the CPU oracle, through the C ABI, on small and medium
layers: routing bit-exact given the kernel's fp32 logits, counting sort and
bias update bit-exact, outputs within the stated tolerance; plus edge cases
(ties, saturated scores, K = E, ragged sizes, empty batch, no shared expert)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_gate_amd as M
from sparse_mixture_experts_gate_amd.workloads import CONFIGS, Workload, make_inputs
from parity_util import TOL, LazyHost, host, route_args, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _log(msg):
    print(msg, flush=True)


def run_gate(wl, P, T=None):
    T = P["x"].shape[0] if T is None else T
    desc = M.make_desc(wl, T)
    ws = torch.empty(M.moe_workspace_size(desc), dtype=torch.uint8, device=DEV)
    out = {"logits": torch.empty(T, wl.E, device=DEV),
           "idx": torch.empty(T, wl.K, dtype=torch.int32, device=DEV),
           "gate": torch.empty(T, wl.K, device=DEV),
           "counts": torch.full((wl.E,), -7, dtype=torch.int32, device=DEV),
           "near": torch.full((1,), -7, dtype=torch.int32, device=DEV)}
    M.moe_gate(desc, P["x"], P["w_router"], P["bias"], out["logits"], out["idx"], out["gate"],
               out["counts"], out["near"], ws)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def check_routing_same_logits(wl, P, g):
    """Oracle routing on the kernel's own logits must match bit for bit."""
    rr = O.route(g["logits"], host(P["bias"]), **route_args(wl))
    assert np.array_equal(g["idx"], rr.idx)
    assert np.array_equal(g["gate"].view(np.uint32), rr.gate.view(np.uint32))
    pr = O.permute(rr.idx, wl.E)
    assert np.array_equal(g["counts"], pr.counts)
    assert int(g["near"][0]) == int(rr.near_tie.sum())
    return rr


# the V3 router (d = 7168, 256 experts in 8 groups of 32, top-4 groups) with
# small experts, so that only the gate's shapes are real
V3_GATE = CONFIGS["v3_decode_bf16"].with_(name="v3_gate", I=64, Is=64)


@pytest.mark.parametrize("name,T", [("tiny_f32", None), ("small_bf16", None), ("small_bf16", 16),
                                    ("small_bf16", 1), ("v3_gate", 32), ("v3_gate", 7)])
def test_gate_bit_exact_and_independent(name, T):
    # T <= 32 with bf16 activations takes the small-batch router kernel
    wl = V3_GATE if name == "v3_gate" else CONFIGS[name]
    _log(f"gate parity {name} T={T}")
    P = make_inputs(wl, DEV, T=T) if T is not None else make_inputs(wl, DEV)
    g = run_gate(wl, P)
    rr = check_routing_same_logits(wl, P, g)
    # independent mode: the oracle's own fp64 router product
    u = O.router_logits(host(P["x"]), host(P["w_router"]))
    assert np.max(np.abs(u - g["logits"])) < 1e-4 * max(1.0, np.abs(u).max())
    ro = O.route(u, host(P["bias"]), **route_args(wl))
    differ = np.any(np.sort(ro.idx, 1) != np.sort(rr.idx, 1), axis=1)
    assert np.all(ro.near_tie[differ] | rr.near_tie[differ])
    assert ro.near_tie.mean() < 1e-3


@pytest.mark.parametrize("T", [1, 7, 32, 33, 64])
def test_router_integer_inputs_exact(T):
    """Integer-valued x and router weights make every dot product exact in
    fp32 whatever the summation order, so the logits of both router paths
    (small batches: fp32 FMA on the VALU; larger: split-bf16 MFMA) must equal
    the integer products bit for bit; counts start from garbage and must be
    cleared. E = 99 leaves the last expert block of the small path half full."""
    wl = Workload("int_router", T=T, d=512, E=99, K=3, I=64, Is=0)
    _log(f"router integer exact T={T}")
    rng = np.random.default_rng(1000 + T)
    xi = rng.integers(-3, 4, (T, wl.d))
    wi = rng.integers(-3, 4, (wl.E, wl.d))
    P = {"x": torch.tensor(xi, dtype=torch.bfloat16, device=DEV),
         "w_router": torch.tensor(wi, dtype=torch.float32, device=DEV),
         "bias": torch.zeros(wl.E, dtype=torch.float32, device=DEV)}
    g = run_gate(wl, P)
    exact = (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float32)
    assert np.array_equal(g["logits"].view(np.uint32), exact.view(np.uint32))
    check_routing_same_logits(wl, P, g)


def test_route_golden_hand_example():
    with open(os.path.join(GOLDEN, "routing_hand_example.json")) as f:
        G = json.load(f)
    wl = Workload("golden", T=3, d=64, E=8, K=2, I=64, Is=0, G=4, M=2, topn=2)
    desc = M.make_desc(wl, 3)
    logits = torch.tensor(G["logits"], dtype=torch.float32, device=DEV)
    bias = torch.tensor(G["bias"], dtype=torch.float32, device=DEV)
    idx = torch.empty(3, 2, dtype=torch.int32, device=DEV)
    gate = torch.empty(3, 2, device=DEV)
    counts = torch.empty(8, dtype=torch.int32, device=DEV)
    near = torch.empty(1, dtype=torch.int32, device=DEV)
    M.moe_route_from_logits(desc, logits, bias, idx, gate, counts, near)
    torch.cuda.synchronize()
    assert idx.tolist() == G["expected_idx"]
    assert gate.tolist() == G["expected_gate"]
    assert int(near[0]) == sum(G["expected_near_tie"])
    assert counts.tolist() == np.bincount(np.array(G["expected_idx"]).ravel(), minlength=8).tolist()


@pytest.mark.parametrize("E,K,G,Mg,topn,T,kind", [
    (16, 2, 1, 1, 2, 300, "ties"), (16, 16, 1, 1, 2, 50, "normal"), (100, 5, 1, 1, 2, 257, "normal"),
    (96, 6, 4, 2, 3, 333, "normal"), (256, 8, 8, 4, 2, 1000, "saturate"),
    (512, 8, 16, 4, 1, 129, "normal"), (64, 6, 8, 3, 2, 1, "normal"), (8, 2, 4, 2, 2, 77, "ties"),
    # the largest routing accepted: top-64 of 512 experts in 64 groups, with
    # exactly K eligible experts (8 groups of 8), with the group scores from
    # the top 8 of each group, and groups of 32 scored from their top 3
    (512, 64, 64, 8, 1, 150, "ties"), (512, 64, 64, 64, 8, 200, "normal"),
    (512, 32, 16, 4, 3, 100, "saturate"),
])
def test_route_from_logits_edge_cases(E, K, G, Mg, topn, T, kind):
    _log(f"route edge E={E} K={K} G={G} M={Mg} topn={topn} T={T} {kind}")
    rng = np.random.default_rng(E * 7 + K)
    if kind == "ties":
        u = rng.integers(-2, 3, (T, E)).astype(np.float32)      # many exact ties
        b = np.zeros(E, np.float32)
    elif kind == "saturate":
        u = rng.choice([-100.0, -30.0, 0.0, 25.0, 100.0], (T, E)).astype(np.float32)
        b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    else:
        u = rng.normal(0, 2, (T, E)).astype(np.float32)
        b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    wl = Workload("edge", T=T, d=64, E=E, K=K, I=64, Is=0, G=G, M=Mg, topn=topn)
    desc = M.make_desc(wl, T)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    gate = torch.empty(T, K, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    near = torch.empty(1, dtype=torch.int32, device=DEV)
    M.moe_route_from_logits(desc, torch.from_numpy(u).to(DEV), torch.from_numpy(b).to(DEV), idx,
                            gate, counts, near)
    torch.cuda.synchronize()
    rr = O.route(u, b, K, G, Mg, topn)
    assert np.array_equal(host(idx), rr.idx)
    assert np.array_equal(host(gate).view(np.uint32), rr.gate.view(np.uint32))
    assert np.array_equal(host(counts), np.bincount(rr.idx.ravel(), minlength=E))
    assert int(host(near)[0]) == int(rr.near_tie.sum())


def test_permute_and_bias_update_bit_exact():
    wl = CONFIGS["small_bf16"]
    _log("permute + bias update small_bf16")
    P = make_inputs(wl, DEV)
    g = run_gate(wl, P)
    T = wl.T
    desc = M.make_desc(wl, T)
    idx = torch.from_numpy(g["idx"]).to(DEV)
    counts = torch.from_numpy(g["counts"]).to(DEV)
    offsets = torch.full((wl.E + 1,), -1, dtype=torch.int32, device=DEV)
    perm = torch.full((T * wl.K,), -1, dtype=torch.int32, device=DEV)
    inv = torch.full((T, wl.K), -1, dtype=torch.int32, device=DEV)
    xp = torch.empty(T * wl.K, wl.d, dtype=torch.bfloat16, device=DEV)
    M.moe_permute(desc, idx, counts, P["x"], offsets, perm, inv, xp)
    torch.cuda.synchronize()
    pr = O.permute(g["idx"], wl.E)
    assert np.array_equal(host(offsets), pr.offsets)
    assert np.array_equal(host(perm), pr.perm)
    assert np.array_equal(host(inv), pr.inv)
    assert torch.equal(xp, P["x"][perm.long()])
    # bias update from these counts, gamma = 0.001
    bias = P["bias"].clone() + torch.linspace(-0.05, 0.05, wl.E, device=DEV)
    b0 = host(bias)
    M.moe_bias_update(desc, counts, 0.001, bias)
    torch.cuda.synchronize()
    ref = O.bias_update(b0, g["counts"], 0.001, T, wl.K)
    assert np.array_equal(host(bias).view(np.uint32), ref.view(np.uint32))


def forward(layer, x):
    out = layer.forward(x)
    torch.cuda.synchronize()
    return out


def oracle_rows(wl, P, rows, idx, gate):
    x = host(P["x"])[rows]
    y = O.layer_output(x, idx[rows], gate[rows], LazyHost(P["w13"]), LazyHost(P["w2"]),
                       host(P["ws13"]) if wl.Is else None, host(P["ws2"]) if wl.Is else None)
    return y


@pytest.mark.parametrize("name,nrows", [("tiny_f32", None), ("small_bf16", None)])
def test_forward_parity(name, nrows):
    wl = CONFIGS[name]
    _log(f"forward parity {name}")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    out = forward(layer, P["x"])
    g = {k: host(v) for k, v in out.items()}
    rr = O.route(g["logits"], host(P["bias"]), **route_args(wl))
    assert np.array_equal(g["topk_idx"], rr.idx)
    assert np.array_equal(g["topk_gate"].view(np.uint32), rr.gate.view(np.uint32))
    assert np.array_equal(g["counts"], O.permute(rr.idx, wl.E).counts)
    T = wl.T
    rows = np.arange(T) if nrows is None else np.random.default_rng(5).choice(T, nrows, replace=False)
    ref = oracle_rows(wl, P, rows, rr.idx, rr.gate)
    if wl.act == "bf16":
        ref = O.round_bf16(ref)
    err = row_rel_err(g["y"][rows], ref)
    _log(f"  {name}: max row-rel err {err:.3e} (tol {TOL[wl.w]})")
    assert err <= TOL[wl.w]


@pytest.mark.parametrize("name,out", [("small_bf16", "f32"), ("tiny_f32", "bf16"),
                                      ("small_fp8", "f32")])
def test_output_dtype(name, out):
    """out_dtype: the combine's fp32 sum stored as is (fp32) or rounded once
    (bf16). The two outputs of one layer agree bit for bit after that rounding,
    and the fp32 output of a bf16 layer is within the bound of the oracle's
    fp64 result without the final rounding."""
    wl = (CONFIGS["small_bf16"].with_(name="small_fp8", w="fp8") if name == "small_fp8"
          else CONFIGS[name]).with_(T=777)
    _log(f"output dtype {out} on {wl.name}")
    P = make_inputs(wl, DEV)
    base = forward(M.MoELayer(wl, P), P["x"])
    other = forward(M.MoELayer(wl.with_(out=out), P), P["x"])
    torch.cuda.synchronize()
    want = torch.float32 if out == "f32" else torch.bfloat16
    assert other["y"].dtype == want
    assert torch.equal(other["topk_idx"], base["topk_idx"])
    if out == "f32":
        assert torch.equal(other["y"].to(torch.bfloat16), base["y"])
        rr = O.route(host(other["logits"]), host(P["bias"]), **route_args(wl))
        rows = np.arange(0, wl.T, 7)
        if wl.w == "fp8":
            ref = O.layer_output_fp8(host(P["x"])[rows], rr.idx[rows], rr.gate[rows],
                                     *_fp8_weights(P, rr.idx[rows]))
        else:
            ref = oracle_rows(wl, P, rows, rr.idx, rr.gate)
        err = row_rel_err(host(other["y"])[rows], ref)
        _log(f"  fp32 output vs the oracle: {err:.2e}")
        assert err <= TOL[wl.w]
    else:
        assert torch.equal(base["y"].to(torch.bfloat16), other["y"])


def _fp8_weights(P, idx):
    """The oracle's own 128x128 E4M3 quantization of the experts in idx and
    of the shared expert, as layer_output_fp8 takes them (dicts by expert)."""
    need = sorted({int(e) for e in np.unique(idx)})
    q13 = {e: O.quantize_blocks_128(host(P["w13"][e])) for e in need}
    q2 = {e: O.quantize_blocks_128(host(P["w2"][e])) for e in need}
    return ({e: q13[e][0] for e in need}, {e: q13[e][1] for e in need},
            {e: q2[e][0] for e in need}, {e: q2[e][1] for e in need},
            *O.quantize_blocks_128(host(P["ws13"])), *O.quantize_blocks_128(host(P["ws2"])))


def test_staged_entry_points_match_fused_forward():
    """moe_gate -> moe_permute (x_perm) -> moe_expert_ffn -> moe_combine gives the
    fused forward's output bit for bit; the gather-in-GEMM path and the
    materialized x_perm path agree bit for bit."""
    wl = CONFIGS["small_bf16"].with_(T=777)
    _log("staged vs fused small_bf16 T=777")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    fused = forward(layer, P["x"])
    T = wl.T
    desc = M.make_desc(wl, T)
    ws = torch.empty(M.moe_workspace_size(desc), dtype=torch.uint8, device=DEV)
    idx = torch.empty(T, wl.K, dtype=torch.int32, device=DEV)
    gate = torch.empty(T, wl.K, device=DEV)
    counts = torch.empty(wl.E, dtype=torch.int32, device=DEV)
    M.moe_gate(desc, P["x"], P["w_router"], P["bias"], None, idx, gate, counts, None, ws)
    offsets = torch.empty(wl.E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * wl.K, dtype=torch.int32, device=DEV)
    inv = torch.empty(T, wl.K, dtype=torch.int32, device=DEV)
    xp = torch.empty(T * wl.K, wl.d, dtype=torch.bfloat16, device=DEV)
    M.moe_permute(desc, idx, counts, P["x"], offsets, perm, inv, xp)
    yp1 = torch.empty(T * wl.K, wl.d, dtype=torch.bfloat16, device=DEV)
    ys1 = torch.empty(T, wl.d, dtype=torch.bfloat16, device=DEV)
    yp2, ys2 = torch.empty_like(yp1), torch.empty_like(ys1)
    M.moe_expert_ffn(desc, layer.weights, P["x"], perm, None, None, offsets, yp1, ys1, ws)
    M.moe_expert_ffn(desc, layer.weights, P["x"], perm, xp, None, offsets, yp2, ys2, ws)
    y = torch.empty(T, wl.d, dtype=torch.bfloat16, device=DEV)
    M.moe_combine(desc, yp1, inv, gate, ys1, y)
    torch.cuda.synchronize()
    assert torch.equal(idx, fused["topk_idx"]) and torch.equal(gate, fused["topk_gate"])
    assert torch.equal(yp1, yp2) and torch.equal(ys1, ys2)
    assert torch.equal(y, fused["y"])


def test_forward_deterministic():
    wl = CONFIGS["small_bf16"].with_(T=1500)
    _log("determinism small_bf16 T=1500")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    a = {k: v.clone() for k, v in forward(layer, P["x"]).items()}
    layer._ws.fill_(0xFF)  # poison the workspace between calls
    b = forward(layer, P["x"])
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("T,d,E,K,I,Is,G,Mg,act", [
    (1, 128, 12, 3, 64, 64, 1, 1, "bf16"), (3, 192, 12, 3, 192, 0, 1, 1, "bf16"),
    (129, 256, 16, 4, 320, 128, 4, 2, "bf16"), (200, 128, 8, 8, 64, 64, 1, 1, "bf16"),
    (37, 128, 10, 2, 64, 0, 1, 1, "f32"), (300, 320, 24, 5, 448, 192, 6, 3, "bf16"),
    (1, 128, 12, 3, 64, 64, 1, 1, "f32"), (129, 256, 16, 4, 320, 128, 4, 2, "f32"),
    (300, 320, 24, 5, 448, 192, 6, 3, "f32"),
])
def test_forward_ragged_shapes(T, d, E, K, I, Is, G, Mg, act):
    wl = Workload("ragged", T=T, d=d, E=E, K=K, I=I, Is=Is, G=G, M=Mg, topn=1, act=act, w=act,
                  x_kind="normal", bias_kind="uniform", bias_amp=0.05, w_std=0.05, seed=T + d)
    _log(f"ragged {wl}")
    P = make_inputs(wl, DEV)
    layer = M.MoELayer(wl, P)
    g = {k: host(v) for k, v in forward(layer, P["x"]).items()}
    rr = O.route(g["logits"], host(P["bias"]), **route_args(wl))
    assert np.array_equal(g["topk_idx"], rr.idx)
    ref = oracle_rows(wl, P, np.arange(T), rr.idx, rr.gate)
    if act == "bf16":
        ref = O.round_bf16(ref)
    err = row_rel_err(g["y"], ref)
    _log(f"  err {err:.3e}")
    assert err <= TOL[act]


def test_empty_batch():
    wl = CONFIGS["small_bf16"].with_(T=0)
    P = make_inputs(wl.with_(T=4), DEV)
    layer = M.MoELayer(wl, P)
    out = layer.alloc_outputs(0)
    out["counts"].fill_(5)
    out["near_tie"].fill_(5)
    layer.forward(P["x"][:0], out)
    torch.cuda.synchronize()
    assert out["counts"].sum().item() == 0 and out["near_tie"].item() == 0


def test_fp8_quantizers_bit_exact():
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    w = (torch.randn(3, 256, 384, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    w[1, :128, :128] = 0.0                                 # an all-zero block
    w[2, 5, 7] = 3.0                                       # an outlier
    q, s = M.quantize_fp8_blocks(w)
    torch.cuda.synchronize()
    wh = host(w)
    for m in range(3):
        rq, rs = O.quantize_blocks_128(wh[m])
        assert np.array_equal(host(q[m]), rq), m
        assert np.array_equal(host(s[m]).view(np.uint32), rs.view(np.uint32)), m
    x = torch.randn(77, 512, generator=g, device=DEV) * 3.0
    x[3, 128:256] = 0.0
    xq = torch.empty(77, 512, dtype=torch.uint8, device=DEV)
    xs = torch.empty(77, 4, device=DEV)
    M.moe_quantize_fp8_rows(x, xq, xs)
    torch.cuda.synchronize()
    rq, rs = O.quantize_rows_1x128(host(x))
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs).view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("w", ["bf16", "fp8"])
def test_all_tokens_on_the_same_experts(w):
    """A bias that outweighs every affinity (sigmoid < 1 < bias) sends all
    tokens to the same K experts: K segments of T rows next to empty experts,
    the extreme of load skew. Routing is checked on the kernel's logits and
    every token's output against the oracle."""
    wl = Workload("skew", T=1500, d=256, E=16, K=4, I=256, Is=128, G=4, M=2, topn=2, act="bf16",
                  w=w, x_kind="normal", bias_kind="uniform", bias_amp=0.05, w_std=0.05, seed=9)
    _log(f"all tokens on experts 0..3, {w}")
    P = make_inputs(wl, DEV)
    P["bias"].zero_()
    P["bias"][: wl.K] = 2.0
    layer = M.MoELayer(wl, P)
    g = {k: host(v) for k, v in forward(layer, P["x"]).items()}
    rr = O.route(g["logits"], host(P["bias"]), **route_args(wl))
    assert np.array_equal(g["topk_idx"], rr.idx)
    assert np.array_equal(g["topk_gate"].view(np.uint32), rr.gate.view(np.uint32))
    assert set(np.unique(rr.idx)) == set(range(wl.K))
    assert np.array_equal(g["counts"][: wl.K], np.full(wl.K, wl.T))
    assert not g["counts"][wl.K:].any()
    x = host(P["x"])
    if w == "bf16":
        ref = oracle_rows(wl, P, np.arange(wl.T), rr.idx, rr.gate)
    else:
        q13 = {e: O.quantize_blocks_128(host(P["w13"][e])) for e in range(wl.K)}
        q2 = {e: O.quantize_blocks_128(host(P["w2"][e])) for e in range(wl.K)}
        s13 = O.quantize_blocks_128(host(P["ws13"]))
        s2 = O.quantize_blocks_128(host(P["ws2"]))
        ref = O.layer_output_fp8(x, rr.idx, rr.gate, {e: v[0] for e, v in q13.items()},
                                 {e: v[1] for e, v in q13.items()}, {e: v[0] for e, v in q2.items()},
                                 {e: v[1] for e, v in q2.items()}, s13[0], s13[1], s2[0], s2[1])
    err = row_rel_err(g["y"], O.round_bf16(ref))
    _log(f"  err {err:.3e}")
    assert err <= TOL[w]
