"""Plain, slow FP64 CPU oracle for the forward pass of one Beam MoE block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module; only the tests, the smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP path.

Source of every step: the Hugging Face post on Beam in its Chinese
translation, 「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」 (section
专家混合模型 / mixture of experts, and section 残差流 / residual stream for the
FP32 policy); the bilingual excerpt of the English original, "Welcome Beam: a
501B open model you can own, customize, and scale" (its mixture-of-experts
paragraph); the tech.fxxz.com rewrite (section 混合专家系统); and the
config.json fields quoted in 「Reflection 放出 501B 的 Beam 权重：四套精度、
滑动窗口和一场榜单落差」 (section "config.json 里还有六处能直接抄的细节":
n_group 8, topk_group 4, norm_topk_prob true, routed_scaling_factor 2.5).
In the function notes below, "blog" means that Chinese translation.  What
those passages fix:

* router: a sigmoid score for every expert (blog, MoE section);
* experts are split into n_group groups; a group is ranked by the sum of the
  two highest scores inside it; the topk_group best groups are kept; the top-k
  experts are taken from inside the kept groups; there is no shared expert;
* the k expert outputs are combined with the normalised router weights and
  multiplied by 2.5 (norm_topk_prob, routed_scaling_factor);
* every expert is a SwiGLU MLP (hidden 5120, intermediate 2560);
* the router and the SwiGLU product are computed in FP32.

Readings where the pages are silent (each one is repeated where it is used):

* groups are contiguous blocks of E / n_group expert indices;
* ties are broken towards the lower index (groups and experts), and the k
  selected ids are listed by score descending, then id ascending;
* a group of a single expert scores that expert alone (top-2 of one value);
* SwiGLU is silu(x W_gate^T) * (x W_up^T), followed by W_down, with no
  biases, weights in the [out, in] layout;
* no normalisation epsilon, no capacity limit, no token dropping;
* an optional selection-only per-expert bias (DeepSeek-V3 scheme, which the
  blog's MoE section names; the pages show no such vector in use) is added to
  the scores for ranking groups and choosing experts, never for the weights.

All arithmetic is float64 on float64 copies of the given (bf16-rounded or
fp32) inputs, except :func:`select_fp32`, which follows a fixed FP32
evaluation order on purpose (see there).
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------
def router_logits(x, w_router, logit_bias=None):
    """L[t, e] = sum_h x[t, h] * W_r[e, h] (+ b[e]), in FP64.

    Blog, MoE section: every expert gets a router score; residual-stream
    section: the router runs in FP32 (here FP64, which contains it).
    """
    X = np.asarray(x, dtype=np.float64)
    W = np.asarray(w_router, dtype=np.float64)
    L = X @ W.T
    if logit_bias is not None:
        L = L + np.asarray(logit_bias, dtype=np.float64)[None, :]
    return L


def sigmoid(L):
    """1 / (1 + exp(-L)), evaluated without overflow for either sign."""
    L = np.asarray(L, dtype=np.float64)
    out = np.empty_like(L)
    pos = L >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-L[pos]))
    ex = np.exp(L[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def _ranked(values):
    """Indices of a 1-D array ordered by value descending, index ascending."""
    v = np.asarray(values)
    return np.lexsort((np.arange(v.shape[0]), -v))


def group_scores(S, num_groups):
    """GS[t, g] = largest + second-largest score of group g (contiguous blocks).

    Blog, MoE section: groups are ranked by the sum of their two best experts.
    A group of one expert scores that expert alone.
    """
    S = np.asarray(S, dtype=np.float64)
    T, E = S.shape
    gs = E // num_groups
    blocks = S.reshape(T, num_groups, gs)
    top = -np.sort(-blocks, axis=2)
    return top[:, :, 0] + (top[:, :, 1] if gs >= 2 else 0.0)


def kept_groups(GS, topk_groups):
    """Boolean mask [T, G] of the topk_group groups with the largest group score."""
    GS = np.asarray(GS)
    T, G = GS.shape
    mask = np.zeros((T, G), dtype=bool)
    for t in range(T):
        mask[t, _ranked(GS[t])[:topk_groups]] = True
    return mask


def select_experts(S, group_mask, topk):
    """ids[t, :] = the topk experts with the highest score among the kept groups."""
    S = np.asarray(S)
    T, E = S.shape
    G = group_mask.shape[1]
    cand = np.repeat(group_mask, E // G, axis=1)
    ids = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        c = np.nonzero(cand[t])[0]
        order = np.lexsort((c, -S[t, c]))
        ids[t] = c[order[:topk]]
    return ids


def normalised_weights(S, ids, routed_scaling):
    """w[t, k] = S[t, id_k] / sum_j S[t, id_j] * routed_scaling (norm_topk_prob, x2.5)."""
    sel = np.take_along_axis(np.asarray(S, dtype=np.float64), ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True) * routed_scaling


def selection_values(S, select_bias=None):
    """C = S + b: the values groups and experts are ranked by.

    With no bias C = S.  A selection-only bias (the DeepSeek-V3 scheme the
    blog's MoE section names) moves the choice, never the weights, which stay
    the normalised unbiased scores.
    """
    S = np.asarray(S, dtype=np.float64)
    if select_bias is None:
        return S
    return S + np.asarray(select_bias, dtype=np.float64)[None, :]


def route(x, w_router, logit_bias, num_groups, topk_groups, topk, routed_scaling, select_bias=None):
    """Router + group-limited selection + weights, all FP64.

    Returns (ids [T,K] int32, w [T,K] f64, S [T,E] f64, GS [T,G] f64); GS is
    taken over the selection values (S, or S + select_bias).
    """
    S = sigmoid(router_logits(x, w_router, logit_bias))
    C = selection_values(S, select_bias)
    GS = group_scores(C, num_groups)
    ids = select_experts(C, kept_groups(GS, topk_groups), topk)
    w = normalised_weights(S, ids, routed_scaling)
    return ids, w, S, GS


def route_margins(S, num_groups, topk_groups, topk, select_bias=None):
    """Per-token distance from a routing decision flip, in FP64.

    m_t = min(GS_(TG) - GS_(TG+1), C_(K) - C_(K+1) over the kept groups'
    candidates), with (j) the j-th largest and C the selection values.  A
    missing (TG+1)-th group or (K+1)-th candidate contributes +inf.
    """
    S = selection_values(S, select_bias)
    T, E = S.shape
    GS = group_scores(S, num_groups)
    mask = kept_groups(GS, topk_groups)
    cand = np.repeat(mask, E // num_groups, axis=1)
    m = np.full(T, np.inf)
    for t in range(T):
        g = -np.sort(-GS[t])
        if num_groups > topk_groups:
            m[t] = min(m[t], g[topk_groups - 1] - g[topk_groups])
        c = -np.sort(-S[t, cand[t]])
        if c.shape[0] > topk:
            m[t] = min(m[t], c[topk - 1] - c[topk])
    return m


def select_fp32(scores, num_groups, topk_groups, topk, routed_scaling, select_bias=None):
    """Selection on caller-supplied FP32 scores with a fixed FP32 evaluation order.

    Same rule as :func:`route` after the sigmoid, but every floating-point
    value that decides or forms an output is an IEEE FP32 result:

    * C = fl32(S + b) with a selection bias b, else C = S;
    * GS = fl32(first + second) of the group's two largest values of C;
    * ids: the K largest C among the kept groups, C descending, id ascending;
    * sum = fl32 running sum of the selected unbiased scores in output order
      (((S_0 + S_1) + S_2) + ...);
    * w_k = fl32(fl32(S_k / sum) * fl32(routed_scaling)).

    This is the supplied-scores mode: ids and weights are meant to agree bit
    for bit with any implementation that states the same FP32 order.
    """
    S = np.asarray(scores, dtype=np.float32)
    T, E = S.shape
    C = S if select_bias is None else (S + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)
    gs = E // num_groups
    scale = np.float32(routed_scaling)
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float32)
    for t in range(T):
        GS = np.empty(num_groups, dtype=np.float32)
        for g in range(num_groups):
            blk = C[t, g * gs:(g + 1) * gs]
            order = _ranked(blk)
            GS[g] = blk[order[0]] + (blk[order[1]] if gs >= 2 else np.float32(0.0))
        keep = _ranked(GS)[:topk_groups]
        cand = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in sorted(keep)])
        order = np.lexsort((cand, -C[t, cand]))
        sel = cand[order[:topk]]
        ids[t] = sel
        total = np.float32(0.0)
        for e in sel:
            total = np.float32(total + S[t, e])
        for k, e in enumerate(sel):
            w[t, k] = np.float32(np.float32(S[t, e] / total) * scale)
    return ids, w


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------
def dispatch(ids, num_experts):
    """Counting sort of the T*K (token, slot) pairs by expert.

    counts[e] = #{i : ids.flat[i] == e}; offsets = exclusive prefix sum with
    offsets[E] = T*K; sorted_slots = the indices i = t*K + k in ascending
    expert order, ascending i inside an expert (a stable sort, hence unique).
    Every token runs exactly K experts (blog, MoE section); no capacity limit.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    slots = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, slots


# --------------------------------------------------------------------------
# experts and combine
# --------------------------------------------------------------------------
def silu(v):
    return v * sigmoid(v)


def swiglu_expert(x_rows, w_gate, w_up, w_down):
    """y = (silu(x W_gate^T) * (x W_up^T)) W_down^T for each row, FP64.

    Blog, MoE section: each expert is a SwiGLU MLP with intermediate size
    2560; the SwiGLU product is FP32 on the pages (FP64 here).
    """
    X = np.asarray(x_rows, dtype=np.float64)
    g = X @ np.asarray(w_gate, dtype=np.float64).T
    u = X @ np.asarray(w_up, dtype=np.float64).T
    h = silu(g) * u
    return h @ np.asarray(w_down, dtype=np.float64).T


def combine(y, w):
    """out[t] = sum_k w[t, k] * y[t, k, :] (blog, MoE section: weighted combine)."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return np.einsum("tk,tkh->th", w, y)


def expert_outputs(x, ids, expert_weights):
    """y[t, k, :] = expert ids[t, k] applied to x[t] (FP64).

    expert_weights(e) -> (W_gate [I,H], W_up [I,H], W_down [H,I]); it is called
    once for every expert some row uses, in ascending expert order.
    """
    ids = np.asarray(ids)
    X = np.asarray(x, dtype=np.float64)
    T, K = ids.shape
    y = np.zeros((T, K, X.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        rows, ks = np.nonzero(ids == e)
        wg, wu, wd = expert_weights(int(e))
        y[rows, ks] = swiglu_expert(X[rows], wg, wu, wd)
    return y


def moe_forward(x, w_router, logit_bias, expert_weights, num_groups, topk_groups, topk,
                routed_scaling, select_bias=None):
    """Whole block for the given token rows: route, dispatch, experts, combine.

    Routing is per token, so any subset of a batch's rows may be passed; the
    dispatch by-products then describe that subset.  Returns a dict with ids,
    w, S, GS, counts, offsets, slots and out [T, H] (FP64).
    """
    ids, w, S, GS = route(x, w_router, logit_bias, num_groups, topk_groups, topk, routed_scaling, select_bias)
    counts, offsets, slots = dispatch(ids, np.asarray(w_router).shape[0])
    y = expert_outputs(x, ids, expert_weights)
    out = combine(y, w)
    return dict(ids=ids, w=w, S=S, GS=GS, counts=counts, offsets=offsets, slots=slots, out=out)


def route_only(x, w_router, logit_bias, num_groups, topk_groups, topk, routed_scaling, select_bias=None):
    """Router, selection and dispatch, without the experts."""
    ids, w, S, GS = route(x, w_router, logit_bias, num_groups, topk_groups, topk, routed_scaling, select_bias)
    counts, offsets, slots = dispatch(ids, w_router.shape[0])
    return dict(ids=ids, w=w, S=S, GS=GS, counts=counts, offsets=offsets, slots=slots)


# --------------------------------------------------------------------------
# FP8 (E4M3) expert weights
# --------------------------------------------------------------------------
# 「Reflection 放出 501B 的 Beam 权重：四套精度、滑动窗口和一场榜单落差」, the
# parameter-precision listing of the FP8 repository and the remarks under it:
# every expert weight is stored as F8_E4M3 (the router, embedding and LM head
# are kept out of the quantisation), a plain dynamic FP8 quantisation of the
# BF16 weights.  The pages give no scale granularity; read here as one FP32
# scale per output row (per channel): W[r, :] = decode(q[r, :]) * scale[r].
def e4m3_decode(codes):
    """Values of OCP FP8 E4M3 codes (the "fn" variant: no infinities, S.1111.111 is NaN).

    Sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0:
    normal (e > 0):  (-1)^s * 2^(e - 7) * (1 + m / 8);
    subnormal (e = 0): (-1)^s * 2^-6 * (m / 8).
    """
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def dequantize_rows(codes, scales):
    """W[r, :] = e4m3_decode(codes[r, :]) * scales[r] (FP64; one scale per output row)."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def fp8_expert(q_gate, s_gate, q_up, s_up, q_down, s_down):
    """(W_gate, W_up, W_down) in FP64 from E4M3 codes and per-row scales.

    q_gate, q_up [I, H] with s_gate, s_up [I]; q_down [H, I] with s_down [H].
    Any function returning these can serve as ``expert_weights`` of
    :func:`moe_forward`: the block itself is unchanged.
    """
    return dequantize_rows(q_gate, s_gate), dequantize_rows(q_up, s_up), dequantize_rows(q_down, s_down)


# --------------------------------------------------------------------------
# the block as a residual sublayer (pre-norm, post-norm, scaled update)
# --------------------------------------------------------------------------
# Blog, section 残差流 (residual stream): the input embedding is step 1; at
# step k a sublayer's output is added with weight 1/sqrt(k) while the stream
# is kept with weight sqrt((k-1)/k); every sublayer is normalised before and
# after; normalisation runs in FP32.  The pages name neither the norm's form
# nor its weights or epsilon: read as RMSNorm, unit weights unless given,
# eps = 1e-6.
NORM_EPS = 1e-6


def rms_norm(v, weight=None, eps=NORM_EPS):
    """v / sqrt(mean(v^2) + eps) * weight, per row, FP64."""
    v = np.asarray(v, dtype=np.float64)
    r = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return r if weight is None else r * np.asarray(weight, dtype=np.float64)


def residual_weights(k):
    """(stream weight, sublayer weight) of step k >= 2: (sqrt((k-1)/k), 1/sqrt(k))."""
    return math.sqrt((k - 1) / k), 1.0 / math.sqrt(k)


def bf16_round(v):
    """Round to the nearest bf16 value (ties to even), returned as float64."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def moe_residual_step(stream, k, w_router, logit_bias, expert_weights, num_groups, topk_groups, topk,
                      routed_scaling, select_bias=None, norm_in_weight=None, norm_out_weight=None, eps=NORM_EPS):
    """stream' = sqrt((k-1)/k) * stream + 1/sqrt(k) * norm(MoE(bf16(norm(stream)))).

    The block's input is the pre-norm of the stream rounded to bf16 (the
    precision the block takes its hidden states in); everything else FP64.
    Returns dict(x=bf16 input, moe=block output, out=new stream, plus the
    routing by-products of moe_forward).
    """
    stream = np.asarray(stream, dtype=np.float64)
    x = bf16_round(rms_norm(stream, norm_in_weight, eps))
    r = moe_forward(x, w_router, logit_bias, expert_weights, num_groups, topk_groups, topk, routed_scaling,
                    select_bias)
    a, b = residual_weights(k)
    r["x"] = x
    r["moe"] = r["out"]
    r["out"] = a * stream + b * rms_norm(r["moe"], norm_out_weight, eps)
    return r
