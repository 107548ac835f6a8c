"""Mutation audit of the oracle's pins (CPU).

Each case plants one plausible mistake in a scratch copy of the oracle (a dropped term, a
wrong sign, index or operand pairing, a wrong rounding) and runs the pins in
test_oracle_pins.py against it: every case must make them fail.  The shipped oracle is
never modified; the planted copy lives in a temporary directory placed first on the path.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "beam_moe_oracle.py")

MUTATIONS = [
    ("logit bias dropped", "        L = L + np.asarray(logit_bias, dtype=np.float64)[None, :]", "        L = L"),
    ("sigmoid sign", "out[pos] = 1.0 / (1.0 + np.exp(-L[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(L[pos]))"),
    ("group score top-1", "return top[:, :, 0] + (top[:, :, 1] if gs >= 2 else 0.0)", "return top[:, :, 0] + 0.0"),
    ("group score top + min", "return top[:, :, 0] + (top[:, :, 1] if gs >= 2 else 0.0)", "return top[:, :, 0] + (top[:, :, -1] if gs >= 2 else 0.0)"),
    ("group score sum of all", "return top[:, :, 0] + (top[:, :, 1] if gs >= 2 else 0.0)", "return top.sum(axis=2)"),
    ("one group too many", "mask[t, _ranked(GS[t])[:topk_groups]] = True", "mask[t, _ranked(GS[t])[:topk_groups + 1]] = True"),
    ("expert ties to higher id", "order = np.lexsort((c, -S[t, c]))", "order = np.lexsort((-c, -S[t, c]))"),
    ("groups ignored", "cand = np.repeat(group_mask, E // G, axis=1)", "cand = np.ones_like(np.repeat(group_mask, E // G, axis=1))"),
    ("weights not normalised", "return sel / sel.sum(axis=1, keepdims=True) * routed_scaling", "return sel * routed_scaling"),
    ("scaling dropped", "return sel / sel.sum(axis=1, keepdims=True) * routed_scaling", "return sel / sel.sum(axis=1, keepdims=True)"),
    ("weights from biased values", "w = normalised_weights(S, ids, routed_scaling)", "w = normalised_weights(C, ids, routed_scaling)"),
    ("groups ranked on unbiased", "GS = group_scores(C, num_groups)", "GS = group_scores(S, num_groups)"),
    ("selection bias sign", "return S + np.asarray(select_bias, dtype=np.float64)[None, :]", "return S - np.asarray(select_bias, dtype=np.float64)[None, :]"),
    ("fp32 group score top-1", "GS[g] = blk[order[0]] + (blk[order[1]] if gs >= 2 else np.float32(0.0))", "GS[g] = blk[order[0]]"),
    ("margin off", "m[t] = min(m[t], g[topk_groups - 1] - g[topk_groups])", "m[t] = min(m[t], g[0] - g[topk_groups])"),
    ("offsets shifted", "offsets[1:] = np.cumsum(counts)", "offsets[:-1] = np.cumsum(counts)"),
    ("dispatch order", 'slots = np.argsort(flat, kind="stable").astype(np.int32)', 'slots = np.argsort(-flat, kind="stable").astype(np.int32)'),
    ("silu is sigmoid", "return v * sigmoid(v)", "return sigmoid(v)"),
    ("gate/up swapped", "h = silu(g) * u", "h = g * silu(u)"),
    ("combine unweighted", 'return np.einsum("tk,tkh->th", w, y)', 'return np.einsum("tk,tkh->th", np.ones_like(w), y)'),
    ("e4m3 bias 8", "np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3 subnormal exponent", "np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    ("scale per column", "return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]", "return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[None, :]"),
    ("fp8 scales paired wrong", "return dequantize_rows(q_gate, s_gate), dequantize_rows(q_up, s_up), dequantize_rows(q_down, s_down)", "return dequantize_rows(q_gate, s_up), dequantize_rows(q_up, s_gate), dequantize_rows(q_down, s_down)"),
    ("rms uses sum", "r = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)", "r = v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) + eps)"),
    ("eps outside sqrt", "r = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)", "r = v / (np.sqrt(np.mean(v * v, axis=-1, keepdims=True)) + eps)"),
    ("residual weights swapped", "return math.sqrt((k - 1) / k), 1.0 / math.sqrt(k)", "return 1.0 / math.sqrt(k), math.sqrt((k - 1) / k)"),
    ("post-norm missing", 'r["out"] = a * stream + b * rms_norm(r["moe"], norm_out_weight, eps)', 'r["out"] = a * stream + b * r["moe"]'),
    ("pre-norm missing", "x = bf16_round(rms_norm(stream, norm_in_weight, eps))", "x = bf16_round(stream)"),
    ("bf16 truncation", "u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16", "u = u >> 16 << 16"),
    ("bf16 ties away", "u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16", "u = (u + 0x8000) >> 16 << 16"),
]


def _caught(tmp_root, index, name, old, new, base):
    """Run the pins against the oracle with one planted mistake; True if they fail."""
    d = os.path.join(tmp_root, f"m{index}")
    pkg = os.path.join(d, "oracle")
    os.makedirs(pkg)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(pkg, "__init__.py"))
    with open(os.path.join(pkg, "beam_moe_oracle.py"), "w") as f:
        f.write(base.replace(old, new))
    env = dict(os.environ, PYTHONPATH=d + os.pathsep + ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=d, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode == 1  # 1: tests failed (2 and up would be a collection or usage error)


def test_pins_catch_every_planted_mistake(tmp_path):
    base = open(SRC).read()
    for name, old, _ in MUTATIONS:
        assert base.count(old) == 1, f"mutation site for {name!r} not found once"
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        caught = list(pool.map(lambda im: _caught(str(tmp_path), im[0], *im[1], base), enumerate(MUTATIONS)))
    survivors = [m[0] for m, c in zip(MUTATIONS, caught) if not c]
    assert not survivors, f"pins did not catch: {survivors}"
