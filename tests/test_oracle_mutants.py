"""The oracle's pins catch plausible mistakes: each mutant below plants one
slip in a temporary copy of ``oracle/`` (a flipped sign, a dropped term, a
wrong index or operand, a division for a multiplication, a wrong rounding or
format constant, ties the wrong way), and the CPU pin suites, run against that
copy in a subprocess, must fail. An unmutated copy must pass, so a failure
means the pins saw the slip, not that the harness broke.

CPU only; nothing here touches the GPU or the HIP library."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = ["test_oracle_pins.py", "test_oracle_backward.py", "test_oracle_fp8_backward.py",
              "test_oracle_seq_balance.py", "test_gradient_metric.py"]
SUPPORT = ["conftest.py", "parity_util.py", "golden"]

# (id, file under oracle/, text, replacement): each text occurs exactly once
MUTANTS = [
    # routing and sigmoid (routing article §1.2, walkthrough's DeepSeekMoE paragraphs)
    ("sigmoid_of_minus_u", "moe_oracle.py", "    v = -u\n", "    v = u\n"),
    ("exp_series_no_constant", "moe_oracle.py", "for k in range(6, -1, -1):",
     "for k in range(6, 0, -1):"),
    ("cody_waite_sign", "moe_oracle.py", "r = (vm - n * LN2_HI) - n * LN2_LO",
     "r = (vm - n * LN2_HI) + n * LN2_LO"),
    ("bias_ignored_in_selection", "moe_oracle.py", "c = (s + b[None, :]).astype(F32)",
     "c = s.astype(F32)"),
    ("ties_to_higher_id", "moe_oracle.py", "return np.lexsort((ids, -vals))",
     "return np.lexsort((-ids, -vals))"),
    ("group_score_max_only", "moe_oracle.py", "[::-1][:group_topn]", "[::-1][:1]"),
    ("worst_groups_kept", "moe_oracle.py", "allowed = np.sort(gord[:M])",
     "allowed = np.sort(gord[-M:])"),
    ("gates_from_biased_scores", "moe_oracle.py", "gate[t] = (s[t, sel] / ssum).astype(F32)",
     "gate[t] = (c[t, sel] / ssum).astype(F32)"),
    ("permute_tokens_descending", "moe_oracle.py",
     "    for t in range(T):\n        for k in range(K):\n            buckets",
     "    for t in range(T - 1, -1, -1):\n        for k in range(K):\n            buckets"),
    ("bias_step_wrong_sign", "moe_oracle.py", "b[e] = F32(b[e] - g32)", "b[e] = F32(b[e] + g32)"),
    ("balanced_load_without_k", "moe_oracle.py", "total = int(n_tokens) * int(top_k)",
     "total = int(n_tokens)"),
    ("near_tie_strict", "moe_oracle.py",
     "if order.shape[0] > K and F32(ct[order[K - 1]] - ct[order[K]]) <= eps32:",
     "if order.shape[0] > K and F32(ct[order[K - 1]] - ct[order[K]]) < F32(0.0):"),
    ("zero_sum_gates_zero", "moe_oracle.py", "gate[t] = F32(1.0) / F32(K)",
     "gate[t] = F32(0.0)"),
    ("offsets_not_cumulative", "moe_oracle.py", "offsets[e + 1] = offsets[e] + counts[e]",
     "offsets[e + 1] = counts[e]"),
    ("router_product_in_fp16", "moe_oracle.py", "return (x64 @ w64.T).astype(F32)",
     "return (x64 @ w64.T).astype(np.float16).astype(F32)"),
    # experts (§1.1: shared expert always on, routed experts gated)
    ("swiglu_operands_swapped", "moe_oracle.py", "return (_silu64(a) * b) @ w2.T",
     "return (a * _silu64(b)) @ w2.T"),
    ("shared_expert_dropped", "moe_oracle.py", "        y += swiglu_expert(x, ws13, ws2)\n",
     "        y += 0.0\n"),
    ("routed_outputs_ungated", "moe_oracle.py",
     "ye = swiglu_expert(x[rows], w13[int(e)], w2[int(e)])\n        for i in range(rows.shape[0]):\n"
     "            y[rows[i]] += g[rows[i], slots[i]] * ye[i]",
     "ye = swiglu_expert(x[rows], w13[int(e)], w2[int(e)])\n        for i in range(rows.shape[0]):\n"
     "            y[rows[i]] += ye[i]"),
    # number formats and FP8 scaling (§4.1; notes Q8)
    ("bf16_truncates", "moe_oracle.py", "q = np.rint(m * 256.0) / 256.0",
     "q = np.trunc(m * 256.0) / 256.0"),
    ("e4m3_ties_away", "moe_oracle.py",
     "    steps = np.rint(np.ldexp(a, -step_exp)).astype(np.int32)\n    code = np.where(sub, steps, (E + 7)",
     "    steps = np.floor(np.ldexp(a, -step_exp) + 0.5).astype(np.int32)\n"
     "    code = np.where(sub, steps, (E + 7)"),
    ("e4m3_exponent_bias", "moe_oracle.py", "(1.0 + mant / 8.0) * np.exp2(ex - 7.0))",
     "(1.0 + mant / 8.0) * np.exp2(ex - 8.0))"),
    ("row_scale_inverted", "moe_oracle.py", "return q, F32(amax / F32(448.0))",
     "return q, F32(F32(448.0) / amax)"),
    ("row_amax_without_abs", "moe_oracle.py", "amax = F32(np.max(np.abs(vals)))",
     "amax = F32(np.max(vals))"),
    ("block_scale_divides", "moe_oracle.py",
     "    sc = np.repeat(np.repeat(np.asarray(s, F64), 128, axis=0), 128, axis=1)\n    return v * sc",
     "    sc = np.repeat(np.repeat(np.asarray(s, F64), 128, axis=0), 128, axis=1)\n    return v / sc"),
    ("row_scale_divides", "moe_oracle.py",
     "return v * np.repeat(np.asarray(s, F64), 128, axis=1)",
     "return v / np.repeat(np.asarray(s, F64), 128, axis=1)"),
    ("block_scales_transposed", "moe_oracle.py",
     "s = np.where(zero, F32(1.0), (safe / F32(448.0)).astype(F32)).astype(F32)",
     "s = np.where(zero, F32(1.0), (safe / F32(448.0)).astype(F32)).T.astype(F32)"),
    ("fp8_h_not_requantized", "moe_oracle.py",
     "    hq, hs = quantize_rows_1x128(H)\n    return dequant_rows_1x128(hq, hs) @ W2.T",
     "    return H.astype(F64) @ W2.T"),
    ("fp8_shared_dropped", "moe_oracle.py",
     "        y += _fp8_expert(Xd, ws13q, ws13s, ws2q, ws2s)\n", "        y += 0.0\n"),
    ("fp8_x_not_quantized", "moe_oracle.py", "    Xd = dequant_rows_1x128(xq, xs)\n    idx",
     "    Xd = np.asarray(x, F64)\n    idx"),
    # backward (chain rule written out in the backward oracle's header)
    ("silu_derivative_dropped_term", "moe_backward.py",
     "da = dh * b * (sa * (1.0 + a * (1.0 - sa)))", "da = dh * b * sa"),
    ("db_uses_sigmoid_not_silu", "moe_backward.py", "    db = dh * silu\n",
     "    db = dh * sa\n"),
    ("quotient_rule_sign", "moe_backward.py", "(dg - mean) / np.where", "(dg + mean) / np.where"),
    ("sigmoid_derivative_dropped", "moe_backward.py", "du = ds * s * (1.0 - s)", "du = ds * s"),
    ("shared_dx_dropped", "moe_backward.py", "        dx += dXs\n", "        dx += 0.0\n"),
    ("expert_grad_ungated", "moe_backward.py", "dYe = g[rows, slots][:, None] * dy[rows]",
     "dYe = dy[rows]"),
    ("dw2_without_silu", "moe_backward.py", "dW2 = dY.T @ h", "dW2 = dY.T @ (a * b)"),
    ("dw13_gate_up_swapped", "moe_backward.py",
     "dW13 = np.concatenate([da.T @ X, db.T @ X], axis=0)",
     "dW13 = np.concatenate([db.T @ X, da.T @ X], axis=0)"),
    ("router_grad_rows_misaligned", "moe_backward.py",
     "du.reshape(-1)[:, None] * np.repeat(x, K, axis=0))",
     "du.reshape(-1)[:, None] * np.tile(x, (K, 1)))"),
    ("fp8_router_quotient_sign", "fp8_backward.py", "(dg - mean) / np.where",
     "(dg + mean) / np.where"),
    # sequence-level balance loss
    ("balance_f_without_e", "seq_balance.py", "f = cnt * E / (K * L)", "f = cnt / (K * L)"),
    ("balance_grad_sign", "seq_balance.py", "(f[None, :] - F[:, None])",
     "(F[:, None] - f[None, :])"),
    ("balance_affinity_unnormalized", "seq_balance.py",
     "sn = np.where(dead[:, None], 1.0 / E, s / np.where(dead, 1.0, S)[:, None])",
     "sn = np.where(dead[:, None], 1.0 / E, s)"),
    ("balance_sigmoid_derivative_dropped", "seq_balance.py",
     "du[rows] = ds * s[rows] * (1.0 - s[rows])", "du[rows] = ds * s[rows]"),
    # FP8 backward (E5M2 gradients, E4M3 activations and weights)
    ("e5m2_exponent_bias", "fp8_backward.py",
     "(1.0 + mant / 4.0) * np.exp2(ex - 15.0))", "(1.0 + mant / 4.0) * np.exp2(ex - 16.0))"),
    ("e5m2_max", "fp8_backward.py", "E5M2_MAX = 57344.0", "E5M2_MAX = 49152.0"),
    ("fp8_dw2_h_in_e5m2", "fp8_backward.py",
     'dequant_128x1(*quantize_128x1(H16, "e4m3"), "e4m3")',
     'dequant_128x1(*quantize_128x1(H16, "e5m2"), "e5m2")'),
    ("fp8_db_without_sigmoid", "fp8_backward.py", "db = dH * a16 * sa", "db = dH * a16"),
    ("fp8_dx_unquantized_grad", "fp8_backward.py", "    dX = dGd @ W13\n",
     "    dX = dG32.astype(F64) @ W13\n"),
]


def _copy_tree(dst, mutant=None):
    """A scratch checkout: oracle/ (mutated), the pin suites and their
    support files, and the package (symlinked; the suites import its input
    generators only)."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in PIN_SUITES + SUPPORT:
        src = os.path.join(ROOT, "tests", f)
        if os.path.isdir(src):
            shutil.copytree(src, os.path.join(dst, "tests", f))
        else:
            shutil.copy(src, os.path.join(dst, "tests", f))
    os.symlink(os.path.join(ROOT, "sparse_mixture_experts_gate_amd"),
               os.path.join(dst, "sparse_mixture_experts_gate_amd"))
    if mutant is not None:
        _, fname, old, new = mutant
        path = os.path.join(dst, "oracle", fname)
        text = open(path).read()
        assert text.count(old) == 1, (mutant[0], text.count(old))
        open(path, "w").write(text.replace(old, new))


def _run_pins(dst):
    env = dict(os.environ, OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2", MKL_NUM_THREADS="2",
               PYTHONDONTWRITEBYTECODE="1")
    env.pop("PYTHONPATH", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests"],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmutated_copy_passes(tmp_path):
    _copy_tree(str(tmp_path))
    rc, out = _run_pins(str(tmp_path))
    assert rc == 0, out


def test_every_mutant_fails_a_pin(tmp_path):
    def one(m):
        dst = str(tmp_path / m[0])
        os.makedirs(dst)
        _copy_tree(dst, m)
        rc, out = _run_pins(dst)
        return m[0], rc, out

    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(one, MUTANTS))
    survived = [name for name, rc, _ in results if rc == 0]
    broken = [(name, out) for name, rc, out in results if rc not in (0, 1)]
    assert not broken, broken
    assert not survived, f"mutants no pin caught: {survived}"
