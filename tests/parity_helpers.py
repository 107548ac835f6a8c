"""Shared helpers of the GPU parity tests: input generation on the device,
oracle evaluation on the CPU, and the comparison rules.

Comparison rules (acceptance criteria of the block):
* routing decided in FP32 on both sides (beam_moe_select vs the oracle's
  supplied-scores mode): ids and weights bit for bit;
* end-to-end routing (GPU FP32 router vs FP64 oracle): tokens whose oracle
  margin is below 1e-5 are counted and excluded from the id comparison; for
  them the GPU choice is checked to be valid within that margin; other tokens
  must select the same expert set, with weights within 1e-5;
* block output: per token, max |gpu - oracle| <= 1e-2 * RMS(oracle row).
"""
from __future__ import annotations

import numpy as np
import torch

from grouped_top_routing_fp32_amd import synth
from oracle import beam_moe_oracle as orc

MARGIN = 1e-5
OUT_TOL = 1e-2
W_TOL = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Problem:
    """Inputs of one workload, generated on the device with the shared generator."""

    def __init__(self, wl: synth.Workload, device="cuda", experts=None, select_bias=None, fp8=False):
        self.wl = wl
        self.dims = wl.dims
        self.x = synth.make_x(wl, device)
        self.wr = synth.make_router(wl, device)
        self.bias = synth.make_bias(wl, device)
        self.select_bias = select_bias  # fp32 [E] device tensor or None
        self.fp8 = fp8
        if fp8:
            # (q_gate, s_gate, q_up, s_up, q_down, s_down) of every expert
            self.q = experts if experts is not None else synth.make_experts_fp8(wl, device)
            experts = None
        elif experts is None and not wl.router_only:
            experts = synth.make_experts(wl, device)
        self.wg, self.wu, self.wd = experts if experts is not None else (None, None, None)
        self._cache = {}

    def expert_f64(self, e: int):
        if e not in self._cache:
            if self.fp8:
                qg, sg, qu, su, qd, sd = (t[e].cpu().numpy() for t in self.q)
                self._cache[e] = orc.fp8_expert(qg, sg, qu, su, qd, sd)
            else:
                self._cache[e] = (f64(self.wg[e]), f64(self.wu[e]), f64(self.wd[e]))
        return self._cache[e]

    def route_oracle(self, tokens=None):
        """(X, ids, w, C, GS, margins) of the oracle; C = the selection values (S, or S + select_bias)."""
        d = self.dims
        if tokens is not None:
            # checked on the host: an index past the batch would trip the device-side gather's assert
            tok = np.asarray(tokens)
            if tok.size and (tok.min() < 0 or tok.max() >= self.x.shape[0]):
                raise IndexError(f"token sample {tok.tolist()} outside a batch of {self.x.shape[0]}")
        X = f64(self.x if tokens is None else self.x[torch.as_tensor(tokens, device=self.x.device)])
        bias = None if self.bias is None else f64(self.bias)
        sb = None if self.select_bias is None else f64(self.select_bias)
        ids, w, S, GS = orc.route(X, f64(self.wr), bias, d.num_groups, d.topk_groups, d.topk, d.routed_scaling,
                                  select_bias=sb)
        m = orc.route_margins(S, d.num_groups, d.topk_groups, d.topk, select_bias=sb)
        return X, ids, w, orc.selection_values(S, sb), GS, m


def valid_near_tie(ids_gpu_row, S_row, d: synth.Dims, slack=2 * MARGIN) -> bool:
    """The GPU's choice for a near-tie token is optimal up to `slack` under FP64 scores."""
    E, G, TG, K = d.num_experts, d.num_groups, d.topk_groups, d.topk
    ids = [int(v) for v in ids_gpu_row]
    if len(set(ids)) != K or min(ids) < 0 or max(ids) >= E:
        return False
    gs = E // G
    GS = orc.group_scores(S_row[None, :], G)[0]
    gth = np.sort(GS)[::-1][TG - 1]
    groups = {e // gs for e in ids}
    if len(groups) > TG or any(GS[g] < gth - slack for g in groups):
        return False
    cand = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in groups])
    kth = np.sort(S_row[cand])[::-1][K - 1]
    return all(S_row[e] >= kth - slack for e in ids)


def compare_routing(ids_gpu, w_gpu, ids_o, w_o, S_o, m, d: synth.Dims):
    """Returns the number of excluded (near-tie) tokens; asserts the rest."""
    excluded = 0
    for t in range(ids_o.shape[0]):
        if m[t] < MARGIN:
            excluded += 1
            assert valid_near_tie(ids_gpu[t], S_o[t], d), (t, ids_gpu[t], ids_o[t], m[t])
            continue
        assert sorted(ids_gpu[t].tolist()) == sorted(ids_o[t].tolist()), (t, ids_gpu[t], ids_o[t], m[t])
        wg = dict(zip(ids_gpu[t].tolist(), w_gpu[t].tolist()))
        for e, wv in zip(ids_o[t].tolist(), w_o[t].tolist()):
            assert abs(wg[e] - wv) <= W_TOL, (t, e, wg[e], wv)
    return excluded


def check_dispatch_valid(ids_gpu: np.ndarray, counts, offsets, slots, E: int):
    """Properties that make the dispatch the unique stable counting sort of ids_gpu."""
    flat = ids_gpu.reshape(-1).astype(np.int64)
    n = flat.shape[0]
    assert counts.shape == (E,) and offsets.shape == (E + 1,) and slots.shape == (n,)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[E] == n
    assert np.array_equal(np.sort(slots), np.arange(n))
    for e in range(E):
        seg = slots[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)


def compare_outputs(out_gpu: np.ndarray, out_o: np.ndarray, keep: np.ndarray):
    """Per-token max-abs error against 1e-2 x RMS of the oracle row; returns worst ratio."""
    worst = 0.0
    for t in np.nonzero(keep)[0]:
        rms = float(np.sqrt(np.mean(out_o[t] ** 2)))
        err = float(np.max(np.abs(out_gpu[t] - out_o[t])))
        ratio = err / (OUT_TOL * rms)
        worst = max(worst, ratio)
        assert err <= OUT_TOL * rms, (t, err, rms)
    return worst


def forward_parity(p: Problem, bufs, tokens=None):
    """Compare one beam_moe_forward result with the oracle on the listed tokens (default all).

    Returns (excluded tokens, worst error ratio)."""
    d = p.dims
    T = p.x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    X, ids_o, w_o, S_o, GS_o, m = p.route_oracle(tokens)
    ids_g = bufs.ids.cpu().numpy()
    w_g = bufs.w.cpu().numpy()
    excluded = compare_routing(ids_g[tokens], w_g[tokens], ids_o, w_o, S_o, m, d)
    check_dispatch_valid(ids_g, bufs.counts.cpu().numpy(), bufs.offsets.cpu().numpy(), bufs.slots.cpu().numpy(),
                         d.num_experts)
    keep = m >= MARGIN
    y = orc.expert_outputs(X[keep], ids_o[keep], p.expert_f64)
    out_o = np.zeros((len(tokens), d.hidden))
    out_o[keep] = orc.combine(y, w_o[keep])
    out_g = bufs.out[torch.as_tensor(tokens, device=bufs.out.device)].cpu().numpy().astype(np.float64)
    worst = compare_outputs(out_g, out_o, keep)
    return excluded, worst


def residual_parity(p: Problem, stream: torch.Tensor, step: int, bufs, tokens=None, g_in=None, g_out=None,
                    eps=orc.NORM_EPS):
    """Compare one beam_moe_residual_forward result (new stream in bufs.out) with the oracle.

    Two output checks per kept token: the new stream within 1e-2 x its RMS, and
    the sublayer's contribution recovered from it, (new - a * stream) / b, within
    1e-2 x the RMS of the oracle's norm(out) * g_out, which the stream term
    would otherwise mask at large stream scales.  Returns (excluded, worst ratio)."""
    d = p.dims
    T = stream.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    S = f64(stream)[tokens]
    sb = None if p.select_bias is None else f64(p.select_bias)
    bias = None if p.bias is None else f64(p.bias)
    r = orc.moe_residual_step(S, step, f64(p.wr), bias, p.expert_f64, d.num_groups, d.topk_groups, d.topk,
                              d.routed_scaling, select_bias=sb,
                              norm_in_weight=None if g_in is None else f64(g_in),
                              norm_out_weight=None if g_out is None else f64(g_out), eps=eps)
    m = orc.route_margins(r["S"], d.num_groups, d.topk_groups, d.topk, select_bias=sb)
    ids_g = bufs.ids.cpu().numpy()
    w_g = bufs.w.cpu().numpy()
    excluded = compare_routing(ids_g[tokens], w_g[tokens], r["ids"], r["w"], orc.selection_values(r["S"], sb), m,
                               d)
    check_dispatch_valid(ids_g, bufs.counts.cpu().numpy(), bufs.offsets.cpu().numpy(), bufs.slots.cpu().numpy(),
                         d.num_experts)
    keep = m >= MARGIN
    new_g = bufs.out.cpu().numpy().astype(np.float64)[tokens]
    worst = compare_outputs(new_g, r["out"], keep)
    a, b = orc.residual_weights(step)
    term_o = orc.rms_norm(r["moe"], None if g_out is None else f64(g_out), eps)
    term_g = (new_g - a * S) / b
    worst = max(worst, compare_outputs(term_g, term_o, keep))
    return excluded, worst
