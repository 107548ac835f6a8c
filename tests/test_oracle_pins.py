"""Pins of the FP64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: integers
printed on the pages, hand-worked examples (tests/golden), exhaustive
enumeration on tiny inputs, closed forms and invariants.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from grouped_top_routing_fp32_amd import synth
from oracle import beam_moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logit(a):
    return math.log(a / (1.0 - a))


# --------------------------------------------------------------------------
# shapes: parameter accounting printed on the pages
# --------------------------------------------------------------------------
def test_parameter_accounting_matches_pages():
    g = {k: v for k, v in _golden("beam_param_counts.json").items() if not k.startswith("_")}
    H, I = g["hidden_size"]["value"], g["moe_intermediate"]["value"]
    E, L = g["num_experts"]["value"], g["moe_layers"]["value"]
    # one expert = W_gate [I,H] + W_up [I,H] + W_down [H,I]; this is the shape swiglu_expert consumes
    x = np.zeros((1, H))
    orc.swiglu_expert(x, np.zeros((I, H)), np.zeros((I, H)), np.zeros((H, I)))
    per_expert = 3 * H * I
    assert per_expert == 39_321_600
    assert abs(per_expert - g["params_per_expert_approx"]["value"]) <= g["params_per_expert_approx"]["rel_tol"] * 39e6
    total = g["total_params"]["value"]
    assert g["bf16_params"]["value"] + g["f32_params"]["value"] == total
    experts = L * E * per_expert
    assert abs(100.0 * experts / total - g["expert_share_pct"]["value"]) <= g["expert_share_pct"]["abs_tol"]
    # the F32 tensors are exactly one fp32 [E,H] router matrix plus one [E] vector per MoE layer
    assert L * (E * H + E) == g["f32_params"]["value"]
    non_expert = total - experts
    assert abs(non_expert * 2 / 1e9 - g["replicated_bf16_gb_approx"]["value"]) <= g["replicated_bf16_gb_approx"]["abs_tol"] + 0.05
    active = non_expert + L * g["routed_per_token"]["value"] * per_expert
    assert abs(active - g["active_params_approx"]["value"]) <= g["active_params_approx"]["rel_tol"] * active
    for n, key in ((16, "per_gpu_gb_16"), (8, "per_gpu_gb_8")):
        gb = (non_expert + experts / n) * 2 / 1e9
        assert abs(gb - g[key]["value"]) <= g[key]["abs_tol"], (n, gb)


def test_workload_dims_match_pages():
    from grouped_top_routing_fp32_amd import synth
    g = _golden("beam_param_counts.json")
    d = synth.BEAM
    assert d.hidden == g["hidden_size"]["value"]
    assert d.intermediate == g["moe_intermediate"]["value"]
    assert d.num_experts == g["num_experts"]["value"]
    assert d.num_groups == g["n_group"]["value"]
    assert d.topk_groups == g["topk_group"]["value"]
    assert d.topk == g["routed_per_token"]["value"]
    assert d.routed_scaling == g["routed_scaling_factor"]["value"]


# --------------------------------------------------------------------------
# routing: the hand-worked example
# --------------------------------------------------------------------------
def _hand():
    h = _golden("routing_hand_example.json")
    s = np.array(h["scores"], dtype=np.float64)
    return h, s


def test_hand_example_through_router_weight():
    h, s = _hand()
    E = h["num_experts"]
    H = 3
    x = np.array([[1.0, 0.0, 0.0]])
    w_r = np.zeros((E, H))
    w_r[:, 0] = [_logit(a) for a in s]
    ids, w, S, GS = orc.route(x, w_r, None, h["num_groups"], h["topk_groups"], h["topk"], h["routed_scaling"])
    np.testing.assert_allclose(S[0], s, rtol=0, atol=1e-14)
    np.testing.assert_allclose(GS[0], h["expected_group_scores"], rtol=0, atol=1e-14)
    assert ids[0].tolist() == h["expected_ids"]
    np.testing.assert_allclose(w[0], h["expected_weights"], rtol=0, atol=1e-14)


def test_hand_example_through_logit_bias():
    # the bias is added to the logit before the sigmoid: with x = 0 the logits are the bias
    h, s = _hand()
    E = h["num_experts"]
    x = np.zeros((1, 4))
    bias = np.array([_logit(a) for a in s])
    ids, w, S, _ = orc.route(x, np.zeros((E, 4)), bias, h["num_groups"], h["topk_groups"], h["topk"],
                             h["routed_scaling"])
    assert ids[0].tolist() == h["expected_ids"]
    np.testing.assert_allclose(w[0], h["expected_weights"], rtol=0, atol=1e-14)


def test_hand_example_fp32_mode():
    h, s = _hand()
    ids, w = orc.select_fp32(s.astype(np.float32)[None, :], h["num_groups"], h["topk_groups"], h["topk"],
                             h["routed_scaling"])
    assert ids[0].tolist() == h["expected_ids"]
    np.testing.assert_allclose(w[0], h["expected_weights"], rtol=0, atol=3e-7)


def test_sigmoid_closed_forms():
    L = np.array([0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0, 40.0])
    np.testing.assert_allclose(orc.sigmoid(L), [0.5, 0.75, 0.25, 1.0, 0.0, 1.0], rtol=0, atol=1e-15)
    # x = 0, no bias: every score is 1/2, all ties: lowest-index groups and experts win, equal weights
    E, G, TG, K = 16, 4, 2, 4
    ids, w, S, _ = orc.route(np.zeros((1, 8)), np.ones((E, 8)), None, G, TG, K, 2.5)
    assert ids[0].tolist() == [0, 1, 2, 3]
    np.testing.assert_allclose(w[0], [2.5 / K] * K, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# selection-only bias (DeepSeek-V3 scheme): moves the choice, not the weights
# --------------------------------------------------------------------------
def _bias_example():
    h = _golden("routing_selection_bias_example.json")
    return h, np.array(h["scores"]), np.array(h["selection_bias"])


def test_selection_bias_hand_example():
    h, s, b = _bias_example()
    E = h["num_experts"]
    x = np.array([[1.0, 0.0]])
    w_r = np.zeros((E, 2))
    w_r[:, 0] = [_logit(a) for a in s]
    ids, w, S, GS = orc.route(x, w_r, None, h["num_groups"], h["topk_groups"], h["topk"], h["routed_scaling"],
                              select_bias=b)
    np.testing.assert_allclose(S[0], s, rtol=0, atol=1e-14)   # scores stay unbiased
    np.testing.assert_allclose(GS[0], h["expected_group_scores"], rtol=0, atol=1e-14)
    assert ids[0].tolist() == h["expected_ids"]
    np.testing.assert_allclose(w[0], h["expected_weights"], rtol=0, atol=1e-14)
    # without the bias: the plain hand example's answer
    ids0, _, _, _ = orc.route(x, w_r, None, h["num_groups"], h["topk_groups"], h["topk"], h["routed_scaling"])
    assert ids0[0].tolist() == _golden("routing_hand_example.json")["expected_ids"]


def test_selection_bias_hand_example_fp32_mode():
    h, s, b = _bias_example()
    ids, w = orc.select_fp32(s.astype(np.float32)[None, :], h["num_groups"], h["topk_groups"], h["topk"],
                             h["routed_scaling"], select_bias=b.astype(np.float32))
    assert ids[0].tolist() == h["expected_ids"]
    np.testing.assert_allclose(w[0], h["expected_weights"], rtol=0, atol=3e-7)


@pytest.mark.parametrize("seed", range(40))
def test_selection_bias_matches_enumeration(seed):
    # the choice is the dominant one under the biased values; the weights keep the
    # ratios of the unbiased scores and sum to the scale
    rng = np.random.default_rng(1000 + seed)
    G, TG, K, E = 4, 2, 4, 16
    S = rng.random((1, E))
    b = rng.normal(0.0, 0.3, E)
    if seed % 4 == 1:
        b = np.round(b * 4) / 4  # coarse: ties among the biased values
        S = np.round(S * 4) / 4
    ids, w, _, _ = orc.route(np.array([[1.0]]), np.array([[_logit(a)] for a in np.clip(S[0], 1e-9, 1 - 1e-9)]),
                             None, G, TG, K, 2.5, select_bias=b)
    Sx = np.clip(S[0], 1e-9, 1 - 1e-9)
    want, _ = _brute_select(Sx + b, G, TG, K)
    assert sorted(ids[0].tolist()) == want
    assert abs(w[0].sum() - 2.5) < 1e-12
    for k in range(1, K):
        assert abs(w[0, k] / w[0, 0] - Sx[ids[0, k]] / Sx[ids[0, 0]]) < 1e-12
    ids32, w32 = orc.select_fp32(Sx.astype(np.float32)[None, :], G, TG, K, 2.5, select_bias=b.astype(np.float32))
    want32, _ = _brute_select((Sx.astype(np.float32) + b.astype(np.float32)).astype(np.float32), G, TG, K)
    assert sorted(ids32[0].tolist()) == want32


def test_selection_bias_closed_forms():
    G, TG, K, E = 4, 2, 4, 16
    # equal scores: the bias alone decides the choice, and every weight is scale / K
    S = np.full((1, E), 0.3)
    b = np.zeros(E)
    b[[13, 2, 14, 3]] = [0.4, 0.3, 0.2, 0.1]  # groups 0 and 3 win; experts by bias
    ids, w = orc.select_fp32(S.astype(np.float32), G, TG, K, 2.5, select_bias=b.astype(np.float32))
    assert ids[0].tolist() == [13, 2, 14, 3]
    np.testing.assert_allclose(w[0], [2.5 / K] * K, rtol=0, atol=1e-7)
    # a zero bias changes nothing; a bias constant over all experts changes no choice
    rng = np.random.default_rng(7)
    S = rng.random((5, E))
    x = np.eye(5)
    w_r = np.array([[_logit(a) for a in S[:, e]] for e in range(E)])
    base = orc.route(x, w_r, None, G, TG, K, 2.5)
    for bb in (np.zeros(E), np.full(E, 0.7)):
        r = orc.route(x, w_r, None, G, TG, K, 2.5, select_bias=bb)
        assert np.array_equal(r[0], base[0])
        np.testing.assert_allclose(r[1], base[1], rtol=0, atol=1e-12)
    m = orc.route_margins(S, G, TG, K, select_bias=np.full(E, 0.7))
    np.testing.assert_allclose(m, orc.route_margins(S, G, TG, K), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# routing: exhaustive enumeration on tiny inputs
# --------------------------------------------------------------------------
def _brute_select(S, G, TG, K):
    """Enumerate every group choice and expert choice; keep the dominant one.

    A choice is valid when nothing left out beats anything taken (group
    scores taken as the best pair sum, itself found over all pairs).  Among
    valid choices the lexicographically smallest index set is the
    lower-index tie rule.
    """
    E = S.shape[0]
    gs = E // G
    GS = []
    for g in range(G):
        blk = S[g * gs:(g + 1) * gs]
        GS.append(max(blk[i] + blk[j] for i, j in itertools.combinations(range(gs), 2)) if gs >= 2 else blk[0])
    best_groups = None
    for gsel in itertools.combinations(range(G), TG):
        rest = [g for g in range(G) if g not in gsel]
        if rest and min(GS[g] for g in gsel) < max(GS[g] for g in rest):
            continue
        best_groups = gsel
        break
    cand = [e for g in best_groups for e in range(g * gs, (g + 1) * gs)]
    for esel in itertools.combinations(cand, K):
        rest = [e for e in cand if e not in esel]
        if rest and min(S[e] for e in esel) < max(S[e] for e in rest):
            continue
        return sorted(esel), GS
    raise AssertionError("no valid choice")


@pytest.mark.parametrize("seed", range(60))
def test_selection_matches_enumeration_random(seed):
    rng = np.random.default_rng(seed)
    G, TG, K = 4, 2, 4
    E = 16
    S = rng.random((1, E))
    if seed % 3 == 1:            # coarse values: many exact ties
        S = np.round(S * 4) / 4
    GSo = orc.group_scores(S, G)
    ids = orc.select_experts(S, orc.kept_groups(GSo, TG), K)
    want, GSb = _brute_select(S[0], G, TG, K)
    np.testing.assert_allclose(GSo[0], GSb, rtol=0, atol=1e-15)
    assert sorted(ids[0].tolist()) == want
    # listed by score descending, then id ascending
    sel = ids[0]
    for a, b in zip(sel[:-1], sel[1:]):
        assert S[0, a] > S[0, b] or (S[0, a] == S[0, b] and a < b)
    ids32, _ = orc.select_fp32(S.astype(np.float32), G, TG, K, 2.5)
    want32, _ = _brute_select(S[0].astype(np.float32), G, TG, K)
    assert sorted(ids32[0].tolist()) == want32


@pytest.mark.parametrize("shape", [(8, 2, 1, 2), (12, 3, 2, 3), (16, 4, 3, 5), (16, 8, 2, 3), (6, 6, 3, 3), (8, 1, 1, 4)])
def test_selection_matches_enumeration_shapes(shape):
    E, G, TG, K = shape
    rng = np.random.default_rng(E * 100 + G * 10 + K)
    for _ in range(30):
        S = rng.random((1, E))
        ids = orc.select_experts(S, orc.kept_groups(orc.group_scores(S, G), TG), K)
        want, _ = _brute_select(S[0], G, TG, K)
        assert sorted(ids[0].tolist()) == want


def test_hand_built_ties():
    G, TG, K = 4, 2, 4
    # two groups tie on their pair sum at the keep boundary: the lower group index is kept
    S = np.array([[0.5, 0.5, 0.0, 0.0,  0.9, 0.8, 0.0, 0.0,  0.6, 0.4, 0.0, 0.0,  0.0, 0.0, 0.0, 0.0]])
    ids = orc.select_experts(S, orc.kept_groups(orc.group_scores(S, G), TG), K)
    assert ids[0].tolist() == [4, 5, 0, 1]
    # experts tie at the k boundary across kept groups: lower id wins
    S = np.array([[0.9, 0.3, 0.0, 0.0,  0.8, 0.3, 0.3, 0.0,  0.1, 0.1, 0.0, 0.0,  0.0, 0.0, 0.0, 0.0]])
    ids = orc.select_experts(S, orc.kept_groups(orc.group_scores(S, G), TG), K)
    assert ids[0].tolist() == [0, 4, 1, 5]


# --------------------------------------------------------------------------
# routing invariants at Beam shapes
# --------------------------------------------------------------------------
def test_routing_invariants_beam_shape():
    rng = np.random.default_rng(7)
    T, H, E, G, TG, K = 64, 128, 256, 8, 4, 8
    x = rng.standard_normal((T, H))
    w_r = rng.standard_normal((E, H)) / math.sqrt(H)
    ids, w, S, GS = orc.route(x, w_r, None, G, TG, K, 2.5)
    gs = E // G
    for t in range(T):
        assert len(set(ids[t].tolist())) == K
        groups = set((ids[t] // gs).tolist())
        kept = set(np.argsort(-GS[t], kind="stable")[:TG].tolist())
        assert groups <= kept
        assert np.all(w[t] > 0)
        assert abs(w[t].sum() - 2.5) <= 1e-12
        # every kept group beats every dropped group on its best pair sum
        for g in range(G):
            blk = S[t, g * gs:(g + 1) * gs]
            pair = max(blk[i] + blk[j] for i, j in itertools.combinations(range(gs), 2))
            assert abs(pair - GS[t, g]) <= 1e-15


def test_margins_bound_the_decision():
    rng = np.random.default_rng(3)
    G, TG, K = 8, 4, 8
    S = rng.random((200, 256))
    m = orc.route_margins(S, G, TG, K)
    base = orc.select_experts(S, orc.kept_groups(orc.group_scores(S, G), TG), K)
    for t in range(S.shape[0]):
        for trial in range(3):
            d = (rng.random(256) * 2 - 1) * 0.24 * m[t]
            St = S[t:t + 1] + d
            ids = orc.select_experts(St, orc.kept_groups(orc.group_scores(St, G), TG), K)
            assert set(ids[0].tolist()) == set(base[t].tolist())


def test_fp32_mode_agrees_with_fp64_away_from_ties():
    rng = np.random.default_rng(11)
    G, TG, K = 8, 4, 8
    S = rng.random((300, 256))
    m = orc.route_margins(S, G, TG, K)
    ids64 = orc.select_experts(S, orc.kept_groups(orc.group_scores(S, G), TG), K)
    w64 = orc.normalised_weights(S, ids64, 2.5)
    ids32, w32 = orc.select_fp32(S.astype(np.float32), G, TG, K, 2.5)
    ok = m > 1e-6
    assert ok.sum() > 290
    assert np.array_equal(ids32[ok], ids64[ok])
    np.testing.assert_allclose(w32[ok], w64[ok], rtol=0, atol=2e-6)
    assert np.all(np.abs(w32.astype(np.float64).sum(1) - 2.5) <= 8 * 2.5 * 2.0 ** -23)


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["uniform", "skewed", "one_expert", "single_token", "empty"])
def test_dispatch_by_counting(case):
    rng = np.random.default_rng(5)
    E, K = 32, 4
    T = {"uniform": 50, "skewed": 40, "one_expert": 10, "single_token": 1, "empty": 0}[case]
    if case == "uniform":
        ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    elif case == "skewed":
        ids = np.stack([np.concatenate([[3], rng.choice(np.arange(4, 8), K - 1, replace=False)]) for _ in range(T)])
    elif case == "one_expert":
        ids = np.full((T, K), 7)
    elif case == "single_token":
        ids = np.array([[9, 2, 30, 4]])
    else:
        ids = np.zeros((0, K), dtype=np.int32)
    counts, offsets, slots = orc.dispatch(ids, E)
    flat = [int(v) for v in ids.reshape(-1)]
    # counting by hand, then placing each pair in a bucket in the order it is met
    want_counts = [0] * E
    for v in flat:
        want_counts[v] += 1
    buckets = [[] for _ in range(E)]
    for i, v in enumerate(flat):
        buckets[v].append(i)
    want_slots = [i for b in buckets for i in b]
    assert counts.tolist() == want_counts
    assert offsets[0] == 0 and offsets[-1] == len(flat)
    assert all(offsets[e + 1] - offsets[e] == want_counts[e] for e in range(E))
    assert slots.tolist() == want_slots
    assert sorted(slots.tolist()) == list(range(len(flat)))


# --------------------------------------------------------------------------
# experts and combine
# --------------------------------------------------------------------------
def test_swiglu_hand_example():
    h = _golden("swiglu_hand_example.json")
    y = orc.swiglu_expert(np.array([h["x"]]), np.array(h["w_gate"]), np.array(h["w_up"]), np.array(h["w_down"]))
    np.testing.assert_allclose(y[0], h["expected_y"], rtol=0, atol=1e-14)


def test_silu_closed_forms():
    v = np.array([0.0, 50.0, -50.0, 1.5, -1.5])
    s = orc.silu(v)
    assert s[0] == 0.0
    assert abs(s[1] - 50.0) < 1e-15 and abs(s[2]) < 1e-15
    # silu(-v) = silu(v) - v
    assert abs(s[4] - (s[3] - 1.5)) < 1e-15


def _tiny_problem(seed, T=12, H=32, I=16, E=16, G=4, TG=2, K=4, identical=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w_r = rng.standard_normal((E, H)) / math.sqrt(H)
    ws = [(rng.standard_normal((I, H)) * 0.2, rng.standard_normal((I, H)) * 0.2, rng.standard_normal((H, I)) * 0.2)
          for _ in range(E)]
    if identical:
        ws = [ws[0]] * E
    return x, w_r, ws, (G, TG, K)


def test_identical_experts_reduce_to_dense_swiglu():
    x, w_r, ws, (G, TG, K) = _tiny_problem(1, identical=True)
    r = orc.moe_forward(x, w_r, None, lambda e: ws[e], G, TG, K, 2.5)
    dense = orc.swiglu_expert(x, *ws[0])
    np.testing.assert_allclose(r["out"], 2.5 * dense, rtol=1e-12, atol=1e-12)


def test_single_expert_block_is_dense_swiglu():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 8))
    w = (rng.standard_normal((4, 8)), rng.standard_normal((4, 8)), rng.standard_normal((8, 4)))
    r = orc.moe_forward(x, rng.standard_normal((1, 8)), None, lambda e: w, 1, 1, 1, 2.5)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 2.5)
    np.testing.assert_allclose(r["out"], 2.5 * orc.swiglu_expert(x, *w), rtol=1e-13, atol=1e-13)


def test_combine_is_the_weighted_sum_of_the_chosen_experts():
    x, w_r, ws, (G, TG, K) = _tiny_problem(4)
    r = orc.moe_forward(x, w_r, None, lambda e: ws[e], G, TG, K, 2.5)
    for t in range(x.shape[0]):
        acc = np.zeros(x.shape[1])
        for k in range(K):
            acc += r["w"][t, k] * orc.swiglu_expert(x[t:t + 1], *ws[r["ids"][t, k]])[0]
        np.testing.assert_allclose(r["out"][t], acc, rtol=1e-12, atol=1e-12)


def test_linear_in_down_projection_and_token_permutation():
    x, w_r, ws, (G, TG, K) = _tiny_problem(9)
    r = orc.moe_forward(x, w_r, None, lambda e: ws[e], G, TG, K, 2.5)
    ws3 = [(a, b, 3.0 * c) for a, b, c in ws]
    r3 = orc.moe_forward(x, w_r, None, lambda e: ws3[e], G, TG, K, 2.5)
    np.testing.assert_allclose(r3["out"], 3.0 * r["out"], rtol=1e-12, atol=1e-12)
    perm = np.random.default_rng(0).permutation(x.shape[0])
    rp = orc.moe_forward(x[perm], w_r, None, lambda e: ws[e], G, TG, K, 2.5)
    np.testing.assert_allclose(rp["out"], r["out"][perm], rtol=1e-12, atol=1e-12)
    assert np.array_equal(rp["ids"], r["ids"][perm])


# --------------------------------------------------------------------------
# residual sublayer: what the blog's residual-stream section fixes
# --------------------------------------------------------------------------
def test_residual_weights_keep_the_stream_scale():
    # the two weights of every step have squares summing to one
    for k in range(2, 200):
        a, b = orc.residual_weights(k)
        assert abs(a * a + b * b - 1.0) < 1e-15


def test_residual_weights_equalise_after_104_additions():
    # embedding = step 1; 104 further additions (52 layers x 2 sublayers): the embedding and
    # every sublayer output end with the same weight, 1/sqrt(105)
    n = 105
    coef = np.zeros(n)        # coef[j]: weight of the term added at step j + 1 (j = 0: embedding)
    coef[0] = 1.0
    for k in range(2, n + 1):
        a, b = orc.residual_weights(k)
        coef[:k - 1] *= a
        coef[k - 1] = b
    np.testing.assert_allclose(coef, np.full(n, 1.0 / math.sqrt(n)), rtol=0, atol=1e-14)


def test_rms_norm_closed_forms():
    v = np.array([[3.0, -3.0, 3.0, -3.0], [1.0, 2.0, 2.0, 4.0]])
    r = orc.rms_norm(v, eps=0.0)
    np.testing.assert_allclose(r[0], [1.0, -1.0, 1.0, -1.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r[1], np.array([1.0, 2.0, 2.0, 4.0]) / math.sqrt(25.0 / 4.0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(np.mean(orc.rms_norm(v * 7.5, eps=0.0) ** 2, axis=1), [1.0, 1.0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(orc.rms_norm(v, [2.0, 1.0, 0.5, 0.0], eps=0.0)[0], [2.0, -1.0, 0.5, 0.0], atol=1e-15)
    # eps: a zero row stays zero; a tiny row is damped
    np.testing.assert_allclose(orc.rms_norm(np.zeros((1, 4))), 0.0)
    assert abs(orc.rms_norm(np.full((1, 4), 1e-3))[0, 0] - 1e-3 / math.sqrt(1e-6 + 1e-6)) < 1e-12


def test_bf16_rounding():
    # exact values pass; halfway cases go to the even neighbour; others to the nearest
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1.0 + 2 ** -7 + 2 ** -10])
    want = np.array([1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5, 1.0 + 2 ** -7])
    np.testing.assert_array_equal(orc.bf16_round(vals), want)


def test_residual_step_special_cases():
    # identical experts: the block is 2.5 * SwiGLU(x) whatever the routing, so the step is
    # a * stream + b * norm(2.5 * SwiGLU(bf16(norm(stream))))
    rng = np.random.default_rng(3)
    E, G, TG, K, H, I = 16, 4, 2, 4, 8, 6
    wg, wu, wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    stream = rng.standard_normal((5, H)) * 3.0
    w_r = rng.standard_normal((E, H))
    k = 7
    r = orc.moe_residual_step(stream, k, w_r, None, lambda e: (wg, wu, wd), G, TG, K, 2.5)
    x = orc.bf16_round(orc.rms_norm(stream))
    dense = orc.swiglu_expert(x, wg, wu, wd)
    a, b = math.sqrt(6 / 7), 1 / math.sqrt(7)
    np.testing.assert_allclose(r["moe"], 2.5 * dense, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["out"], a * stream + b * orc.rms_norm(2.5 * dense), rtol=0, atol=1e-12)
    # the block's input is the normalised stream: scaling the stream changes only the kept part
    r2 = orc.moe_residual_step(stream * 4.0, k, w_r, None, lambda e: (wg, wu, wd), G, TG, K, 2.5)
    np.testing.assert_allclose(r2["out"] - a * stream * 4.0, r["out"] - a * stream, rtol=0, atol=1e-12)


def test_residual_step_norm_weights_act_where_named():
    # the pre-norm weight scales the block's input, the post-norm weight only the added term
    # (identical experts, so the block is 2.5 * SwiGLU whatever the routing): g_out = 2 doubles
    # the added term and leaves the block's output alone; g_in = 2 doubles the block's input
    # (exactly: a power of two commutes with the bf16 rounding) and so changes its output
    rng = np.random.default_rng(5)
    E, G, TG, K, H, I = 16, 4, 2, 4, 8, 6
    wg, wu, wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    stream = rng.standard_normal((4, H))
    w_r = rng.standard_normal((E, H))
    k = 3
    a, b = math.sqrt(2 / 3), 1 / math.sqrt(3)
    ex = lambda e: (wg, wu, wd)  # noqa: E731
    base = orc.moe_residual_step(stream, k, w_r, None, ex, G, TG, K, 2.5)
    two = np.full(H, 2.0)
    r_out = orc.moe_residual_step(stream, k, w_r, None, ex, G, TG, K, 2.5, norm_out_weight=two)
    np.testing.assert_allclose(r_out["moe"], base["moe"], rtol=0, atol=0)
    np.testing.assert_allclose(r_out["out"] - a * stream, 2.0 * (base["out"] - a * stream), rtol=0, atol=1e-12)
    r_in = orc.moe_residual_step(stream, k, w_r, None, ex, G, TG, K, 2.5, norm_in_weight=two)
    np.testing.assert_allclose(r_in["x"], 2.0 * base["x"], rtol=0, atol=0)
    np.testing.assert_allclose(r_in["moe"], 2.5 * orc.swiglu_expert(2.0 * base["x"], wg, wu, wd), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r_in["out"], a * stream + b * orc.rms_norm(r_in["moe"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# FP8 (E4M3) expert weights
# --------------------------------------------------------------------------
def test_e4m3_decode_known_values():
    # values fixed by the OCP 8-bit floating point specification (E4M3, bias 7, no infinities)
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert orc.e4m3_decode(np.array([c]))[0] == v, hex(c)
    assert np.isnan(orc.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    z = orc.e4m3_decode(np.array([0x80]))[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_e4m3_decode_matches_torch_float8():
    # an independent implementation: torch's float8_e4m3fn dtype
    codes = np.arange(256)
    mine = orc.e4m3_decode(codes)
    lib = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])


def test_e4m3_decode_order_and_symmetry():
    pos = orc.e4m3_decode(np.arange(0, 127))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(orc.e4m3_decode(np.arange(128, 255)), -pos)
    # relative spacing of the normal range is 2^-3 (three mantissa bits)
    normal = pos[8:]
    assert np.max(np.diff(normal) / normal[:-1]) == 0.125


def test_dequantize_rows_scales_each_row():
    codes = np.array([[0x38, 0x40], [0xB8, 0x30]])
    w = orc.dequantize_rows(codes, [2.0, 0.5])
    assert np.array_equal(w, [[2.0, 4.0], [-0.5, 0.25]])


def test_fp8_expert_hand_example():
    # H = 2, I = 1; W_gate = [[2, 2]], W_up = [[1, 0]], W_down = [[1], [-3]]; x = [1, 1]:
    # g = 4, u = 1, h = silu(4), y = [h, -3h].  Pairing a scale with the wrong matrix
    # (gate <-> up) gives g = 1, u = 4, another value.
    qg, sg = np.array([[0x38, 0x38]]), [2.0]
    qu, su = np.array([[0x40, 0x00]]), [0.5]
    qd, sd = np.array([[0x38], [0xB8]]), [1.0, 3.0]
    wg, wu, wd = orc.fp8_expert(qg, sg, qu, su, qd, sd)
    y = orc.swiglu_expert(np.array([[1.0, 1.0]]), wg, wu, wd)
    h = 4.0 / (1.0 + math.exp(-4.0))
    np.testing.assert_allclose(y[0], [h, -3.0 * h], rtol=1e-15)
    wg2, wu2, wd2 = orc.fp8_expert(qg, su, qu, sg, qd, sd)
    y2 = orc.swiglu_expert(np.array([[1.0, 1.0]]), wg2, wu2, wd2)
    assert abs(y2[0, 0] - h) > 0.1


def test_fp8_generator_codes_are_finite_and_scaled():
    wl = synth.WORKLOADS["tiny"]
    qg, sg, qu, su, qd, sd = synth.expert_weights_fp8(wl, 0)
    for q in (qg, qu, qd):
        v = orc.e4m3_decode(q.numpy())
        assert not np.isnan(v).any() and np.abs(v).max() <= 448.0
    for s in (sg, su, sd):
        assert (s > 0).all()
    w = orc.dequantize_rows(qd.numpy(), sd.numpy())
    assert 0.015 < w.std() < 0.025
