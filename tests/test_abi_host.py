"""Host-only checks of the C ABI: the library loads, exports every function
include/dsmoe.h declares, and rejects bad arguments with the documented status
before anything reaches a GPU (validation runs on the host first)."""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_mixture_experts_gate_amd", "libdsmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdsmoe.so not built")


@pytest.fixture(scope="module")
def L():
    from sparse_mixture_experts_gate_amd import _lib
    return _lib


def test_exports_every_declared_symbol(L):
    names = L.header_symbols()
    assert set(names) == {
        "moe_workspace_size", "moe_gate", "moe_route_from_logits", "moe_permute",
        "moe_expert_ffn", "moe_combine", "moe_bias_update", "deepseek_moe_forward",
        "moe_quantize_fp8_blocks", "moe_quantize_fp8_rows", "moe_status_string",
        "moe_last_error", "moe_abi_version", "moe_profile_events", "moe_forward_train",
        "moe_backward_workspace_size", "moe_backward", "moe_seq_balance_workspace_size",
        "moe_seq_balance_loss", "deepseek_moe_forward_noalloc", "moe_transpose_fp8_blocks",
        "moe_backward_fp8"}
    so = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(so, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_abi_version_and_strings(L):
    assert L.moe_abi_version() == 2
    assert L.lib().moe_status_string(4) == b"workspace too small"


def _desc(L, **kw):
    base = dict(T=64, d=256, n_experts=16, top_k=2, n_groups=1, topk_groups=1, group_topn=2,
                inter=128, shared_inter=128, act_dtype=L.MOE_DT_BF16, w_dtype=L.MOE_DT_BF16,
                near_tie_eps=1e-6, out_dtype=L.MOE_DT_BF16)
    base.update(kw)
    return L.MoeLayerDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), 1), (dict(d=0), 1), (dict(n_experts=0), 1), (dict(n_experts=600), 2),
    (dict(top_k=0), 1), (dict(top_k=17), 1), (dict(n_groups=3), 1),
    (dict(n_groups=4, topk_groups=5), 1), (dict(n_groups=8, topk_groups=1, top_k=3), 1),
    (dict(n_groups=4, topk_groups=2, group_topn=5), 1), (dict(inter=0), 1),
    (dict(shared_inter=-1), 1), (dict(act_dtype=0), 2), (dict(w_dtype=2, d=192), 2),
    (dict(d=200), 2), (dict(inter=96), 2), (dict(near_tie_eps=float("nan")), 1),
    (dict(out_dtype=2), 2), (dict(out_dtype=-1), 2),
    # 32-bit byte-offset limits: x, H's FP8 scales, one expert's weights, the
    # split router weights
    (dict(T=1 << 22), 2),
    (dict(T=400000, inter=1 << 16, shared_inter=1 << 16, w_dtype=2), 2),
    (dict(inter=1 << 21), 2), (dict(n_experts=512, d=699072), 2),
])
def test_descriptor_validation(L, kw, status):
    n = ctypes.c_size_t(0)
    st = L.lib().moe_workspace_size(ctypes.byref(_desc(L, **kw)), ctypes.byref(n))
    assert st == status, L.lib().moe_last_error()
    assert L.lib().moe_last_error()


def test_h_beyond_2_gib_is_accepted(L):
    """H is addressed per tile from a 64-bit base, so a forward whose H holds
    more than 2^31 bytes is accepted and its workspace holds all of H."""
    n = ctypes.c_size_t(0)
    T, inter = 1 << 20, 1024
    d = _desc(L, T=T, inter=inter, shared_inter=inter)
    assert L.lib().moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0, \
        L.lib().moe_last_error()
    h_bytes = T * (2 + 1) * inter * 2
    assert h_bytes > 1 << 31
    assert n.value >= h_bytes


def test_training_accepts_v3_batches_beyond_32k_tokens(L):
    """The backward's row operands are addressed per tile (input-gradient
    GEMMs) or per group (weight-gradient GEMMs), so at the V3 shape training
    takes batches up to T * max(d, 2 max(I, Is)) * 2 < 2^31 bytes, for bf16
    and FP8 weights."""
    lib = L.lib()
    n = ctypes.c_size_t(0)
    v3 = dict(d=7168, n_experts=256, top_k=8, n_groups=8, topk_groups=4, group_topn=2,
              inter=2048, shared_inter=2048)
    t_max = ((1 << 31) - 1) // (7168 * 2)
    for w in (L.MOE_DT_BF16, L.MOE_DT_FP8_E4M3):
        for T in (32768, 131072, t_max):
            d = _desc(L, T=T, w_dtype=w, **v3)
            assert lib.moe_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0, \
                lib.moe_last_error()
        d = _desc(L, T=t_max + 1, w_dtype=w, **v3)
        assert lib.moe_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 2


def test_valid_descriptor_sizes(L):
    n = ctypes.c_size_t(0)
    d = _desc(L)
    assert L.lib().moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    # at least H and y_perm live in the workspace
    assert n.value >= 64 * 2 * 128 * 2 + 64 * 2 * 256 * 2
    d0 = _desc(L, T=0)
    assert L.lib().moe_workspace_size(ctypes.byref(d0), ctypes.byref(n)) == 0


def test_null_and_misaligned_pointers_rejected_before_launch(L):
    lib = L.lib()
    d = _desc(L)
    P = ctypes.c_void_p
    good = P(4096)
    # moe_gate with a NULL x
    st = lib.moe_gate(ctypes.byref(d), None, good, good, None, good, good, good, None, good, 1 << 30, None)
    assert st == 1 and b"x is NULL" in lib.moe_last_error()
    # misaligned topk_idx
    st = lib.moe_gate(ctypes.byref(d), good, good, good, None, P(4100), good, good, None, good, 1 << 30, None)
    assert st == 3
    # permute without offsets
    st = lib.moe_permute(ctypes.byref(d), good, good, None, None, good, good, None, None, None)
    assert st == 1
    # combine with NULL y
    st = lib.moe_combine(ctypes.byref(d), good, good, good, None, None, None)
    assert st == 1
    # bias update with non-finite gamma
    st = lib.moe_bias_update(ctypes.byref(d), good, ctypes.c_float(float("inf")), good, None)
    assert st == 1
    # expert ffn: missing weights struct
    st = lib.moe_expert_ffn(ctypes.byref(d), None, good, good, None, None, good, good, good, good, 1 << 30, None)
    assert st == 1
    # quantizers: bad shapes / dtypes
    assert lib.moe_quantize_fp8_blocks(good, 1, 1, 100, 128, good, good, None) == 1
    assert lib.moe_quantize_fp8_blocks(good, 2, 1, 128, 128, good, good, None) == 2
    assert lib.moe_quantize_fp8_rows(good, 1, 4, 130, good, good, None) == 1


def test_workspace_too_small_rejected(L):
    lib = L.lib()
    d = _desc(L)
    good = ctypes.c_void_p(4096)
    w = L.MoeWeights(4096, 4096, 4096, 4096, None, None, None, None)
    st = lib.deepseek_moe_forward(ctypes.byref(d), good, good, good, ctypes.byref(w), good, good,
                                  good, good, None, None, good, 16, None)
    assert st == 4 and b"workspace" in lib.moe_last_error()


def test_product_path_has_no_oracle_import():
    """The package must not reach the CPU oracle: no module under it imports it."""
    pkg = os.path.join(ROOT, "sparse_mixture_experts_gate_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn
    code = ("import sys; import sparse_mixture_experts_gate_amd as m; "
            "assert 'oracle' not in sys.modules and not any(k.startswith('oracle.') for k in sys.modules)")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)


def test_training_entry_points_validate_before_launch(L):
    lib = L.lib()
    good = ctypes.c_void_p(4096)
    n = ctypes.c_size_t(0)
    d = _desc(L)
    assert lib.moe_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    # holds at least the gated output gradients [T*K, d] and [da | db] [T*(K+1), 2 max(I, Is)]
    assert n.value >= 64 * 2 * 256 * 2 + 64 * 3 * 256 * 2
    # one expert's fp32 weight gradient must stay below 2^31 bytes: this
    # layer is a valid forward but too large for the backward's epilogue
    big = _desc(L, inter=1 << 20, shared_inter=128)
    assert lib.moe_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0
    assert lib.moe_backward_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 2
    assert b"2*max(I,Is)*d*4" in lib.moe_last_error()
    big = _desc(L, inter=128, shared_inter=(1 << 20) - 128)
    assert lib.moe_backward_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0
    # fp32 layers have no training path; FP8 layers train through moe_backward_fp8
    assert lib.moe_backward_workspace_size(ctypes.byref(_desc(L, act_dtype=0, w_dtype=0)),
                                           ctypes.byref(n)) == 2
    assert lib.moe_backward_workspace_size(ctypes.byref(_desc(L, w_dtype=2)), ctypes.byref(n)) == 0
    w = L.MoeWeights(4096, 4096, 4096, 4096, None, None, None, None)
    sv = L.MoeSaved(*([4096] * 10))
    # forward_train: NULL saved, then a misaligned saved tensor
    st = lib.moe_forward_train(ctypes.byref(d), good, good, good, ctypes.byref(w), good, None,
                               None, good, 1 << 30, None)
    assert st == 1 and b"saved is NULL" in lib.moe_last_error()
    bad = L.MoeSaved(*([4096] * 7 + [4100] + [4096] * 2))
    st = lib.moe_forward_train(ctypes.byref(d), good, good, good, ctypes.byref(w), good,
                               ctypes.byref(bad), None, good, 1 << 30, None)
    assert st == 3 and b"saved.h" in lib.moe_last_error()
    st = lib.moe_forward_train(ctypes.byref(d), good, good, good, ctypes.byref(w), good,
                               ctypes.byref(sv), None, good, 16, None)
    assert st == 4
    # backward: NULL grads, NULL dy, missing shared weights, small workspace
    g = L.MoeGrads(4096, 4096, 4096, 4096, 4096)
    st = lib.moe_backward(ctypes.byref(d), good, good, ctypes.byref(w), ctypes.byref(sv), good,
                          good, None, good, 1 << 30, None)
    assert st == 1 and b"grads is NULL" in lib.moe_last_error()
    st = lib.moe_backward(ctypes.byref(d), good, good, ctypes.byref(w), ctypes.byref(sv), None,
                          good, ctypes.byref(g), good, 1 << 30, None)
    assert st == 1 and b"dy is NULL" in lib.moe_last_error()
    w_noshared = L.MoeWeights(4096, 4096, None, None, None, None, None, None)
    st = lib.moe_backward(ctypes.byref(d), good, good, ctypes.byref(w_noshared), ctypes.byref(sv),
                          good, good, ctypes.byref(g), good, 1 << 30, None)
    assert st == 1 and b"ws13 is NULL" in lib.moe_last_error()
    st = lib.moe_backward(ctypes.byref(d), good, good, ctypes.byref(w), ctypes.byref(sv), good,
                          good, ctypes.byref(g), good, 16, None)
    assert st == 4 and b"workspace" in lib.moe_last_error()


def test_seq_balance_validates_before_launch(L):
    lib = L.lib()
    good = ctypes.c_void_p(4096)
    n = ctypes.c_size_t(0)
    d = _desc(L)
    assert lib.moe_seq_balance_workspace_size(ctypes.byref(d), 16, ctypes.byref(n)) == 0
    # at least the bf16 copies of du (both layouts) and of the router weights
    assert n.value >= 2 * 64 * 16 * 2 + 16 * 256 * 2
    # seq_len must divide T and be positive; fp32 activations are unsupported
    assert lib.moe_seq_balance_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == 1
    assert lib.moe_seq_balance_workspace_size(ctypes.byref(d), 48, ctypes.byref(n)) == 1
    assert b"does not divide" in lib.moe_last_error()
    d32 = _desc(L, act_dtype=0, w_dtype=0)
    assert lib.moe_seq_balance_workspace_size(ctypes.byref(d32), 16, ctypes.byref(n)) == 2
    args = lambda **kw: [kw.get(k, good) for k in ("x", "wr", "u", "idx", "loss", "dl", "dx", "dwr")]
    call = lambda a, alpha=0.01, ws=1 << 30: lib.moe_seq_balance_loss(
        ctypes.byref(d), 16, alpha, *a, good, ws, None)
    assert call(args(), alpha=float("nan")) == 1 and b"alpha" in lib.moe_last_error()
    assert call(args(dwr=None)) == 1 and b"dw_router is NULL" in lib.moe_last_error()
    assert call(args(u=None)) == 1 and b"logits is NULL" in lib.moe_last_error()
    assert call(args(dl=ctypes.c_void_p(4100))) == 3
    assert call(args(), ws=16) == 4 and b"workspace" in lib.moe_last_error()


def test_noalloc_forward_validates_before_touching_the_device(L):
    """The allocation-free forward checks its arguments and that the call's
    workspace fits the fixed scratch before it looks the scratch up or
    launches anything (no GPU is needed to see these errors)."""
    lib = L.lib()
    good = ctypes.c_void_p(4096)
    w = L.MoeWeights(4096, 4096, 4096, 4096, None, None, None, None)
    args = lambda d, x=good: (ctypes.byref(d), x, good, good, ctypes.byref(w), good, good, good,
                              good, None, None, None)
    d = _desc(L)
    assert lib.deepseek_moe_forward_noalloc(*args(d, None)) == 1
    assert b"x is NULL" in lib.moe_last_error()
    assert lib.deepseek_moe_forward_noalloc(*args(d, ctypes.c_void_p(4100))) == 3
    # V3-shaped layer: T = 532 fits the 128 MiB scratch in bf16, T = 533 does not
    v3 = dict(d=7168, n_experts=256, top_k=8, n_groups=8, topk_groups=4, inter=2048,
              shared_inter=2048)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(_desc(L, T=532, **v3)), ctypes.byref(n)) == 0
    assert n.value <= 128 << 20
    big = _desc(L, T=533, **v3)
    assert lib.moe_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0 and n.value > 128 << 20
    assert lib.deepseek_moe_forward_noalloc(*args(big)) == 4
    assert b"fixed scratch" in lib.moe_last_error()


def test_backward_fp8_validation_before_any_launch(L):
    """moe_backward_fp8 checks everything on the host and returns before
    enqueueing: bf16 weights, missing transposed weights and a short
    workspace each give their own status."""
    lib = L.lib()
    good = 4096
    n = ctypes.c_size_t(0)
    d8 = _desc(L, w_dtype=L.MOE_DT_FP8_E4M3)
    assert lib.moe_backward_workspace_size(ctypes.byref(d8), ctypes.byref(n)) == 0
    need = n.value
    w = L.MoeWeights(*([good] * 8))
    sv = L.MoeSaved(*([good] * 10))
    g = L.MoeGrads(*([good] * 5))

    def call(desc, wt, ws_bytes):
        return lib.moe_backward_fp8(ctypes.byref(desc), good, good, ctypes.byref(w),
                                    None if wt is None else ctypes.byref(wt), ctypes.byref(sv),
                                    good, good, ctypes.byref(g), good, ws_bytes, None)

    assert call(_desc(L), w, need) == 2
    assert b"FP8 weights" in lib.moe_last_error()
    assert call(d8, None, need) == 1
    assert b"transposed weights" in lib.moe_last_error()
    assert call(d8, w, need - 1) == 4
    assert b"workspace" in lib.moe_last_error()
    bad = L.MoeWeights(*([good] * 3 + [4100] + [good] * 4))
    assert call(d8, bad, need) == 3
