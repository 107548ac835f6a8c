"""Shared helpers of the GPU parity tests: input generation on the device,
oracle evaluation on the CPU, and the comparison rules.

Comparison rules (acceptance criteria of the block):
* routing decided in FP32 on both sides (beam_moe_select vs the oracle's
  supplied-scores mode): ids and weights bit for bit;
* end-to-end routing (GPU FP32 router vs FP64 oracle): tokens whose oracle
  margin is below 1e-5 are counted and excluded from the id comparison; for
  them the GPU choice is checked to be valid within that margin and its
  weights to be the normalised FP64 scores of the ids it chose; other tokens
  must select the same expert set, with weights within 1e-5;
* block output, for every compared token: max |gpu - oracle| <= 1e-2 *
  RMS(oracle row).  For a near-tie token the oracle output is the expert path
  re-run in FP64 on the GPU's ids and weights, so its GEMMs and combine are
  still checked although its choice of experts is not unique.
"""
from __future__ import annotations

import os
from collections import OrderedDict

import numpy as np
import torch

from grouped_top_routing_fp32_amd import synth
from oracle import beam_moe_oracle as orc

MARGIN = 1e-5
OUT_TOL = 1e-2
W_TOL = 1e-5
# expert weights held as FP64 host copies by one Problem (an expert at Beam dims is 315 MB)
CACHE_BYTES = 8 << 30


# (test, tokens compared, near-ties among them, worst error / tolerance) of every output
# comparison in this session; tests/conftest.py prints them when the session ends
RECORDS = []


def _record(tokens, near, worst):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0].split("::")[-1]
    RECORDS.append((test, int(tokens), int(near), float(worst)))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


_E4M3 = None


def fp8_expert_lookup(q_gate, s_gate, q_up, s_up, q_down, s_down):
    """orc.fp8_expert with the oracle's decode of each of the 256 codes looked up per
    element: the same FP64 values, without decoding millions of codes one at a time."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = orc.e4m3_decode(np.arange(256, dtype=np.int64))
    return tuple(_E4M3[q] * np.asarray(sc, dtype=np.float64)[:, None]
                 for q, sc in ((q_gate, s_gate), (q_up, s_up), (q_down, s_down)))


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
        self._cache = OrderedDict()

    def expert_f64(self, e: int):
        if e in self._cache:
            self._cache.move_to_end(e)
            return self._cache[e]
        if self.fp8:
            w = fp8_expert_lookup(*(t[e].cpu().numpy() for t in self.q))
        else:
            w = (f64(self.wg[e]), f64(self.wu[e]), f64(self.wd[e]))
        per = sum(a.nbytes for a in w)
        while self._cache and (len(self._cache) + 1) * per > CACHE_BYTES:
            self._cache.popitem(last=False)
        self._cache[e] = w
        return w

    def route_oracle(self, tokens=None):
        """(X, ids, w, C, GS, margins) of the oracle; C = the selection values (S, or S + select_bias)."""
        X, ids, w, S, C, GS, m = self.route_oracle_full(tokens)
        return X, ids, w, C, GS, m

    def route_oracle_full(self, tokens=None):
        """(X, ids, w, S, C, GS, margins): as route_oracle, plus the unbiased scores S."""
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
        return X, ids, w, S, orc.selection_values(S, sb), GS, m


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


def compare_routing(ids_gpu, w_gpu, ids_o, w_o, C_o, m, d: synth.Dims, S_o=None):
    """Returns the number of excluded (near-tie) tokens; asserts the rest.

    C_o: the oracle's selection values (what groups and experts are ranked by);
    S_o: its unbiased scores (what weights are formed from; defaults to C_o).
    A near-tie token's ids must be a valid choice under C_o, and its weights
    the normalised S_o of the ids it chose, within 1e-5."""
    S_o = C_o if S_o is None else S_o
    excluded = 0
    for t in range(ids_o.shape[0]):
        if m[t] < MARGIN:
            excluded += 1
            assert valid_near_tie(ids_gpu[t], C_o[t], d), (t, ids_gpu[t], ids_o[t], m[t])
            w_want = orc.normalised_weights(S_o[t:t + 1], np.asarray(ids_gpu[t:t + 1]), d.routed_scaling)[0]
            assert np.max(np.abs(np.asarray(w_gpu[t], dtype=np.float64) - w_want)) <= W_TOL, (t, w_gpu[t], w_want)
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


def compare_outputs(out_gpu: np.ndarray, out_o: np.ndarray, keep=None):
    """Per-token max-abs error against 1e-2 x RMS of the oracle row; returns worst ratio.

    keep: optional boolean mask of the rows to compare (default every row)."""
    worst = 0.0
    rows = range(out_o.shape[0]) if keep is None else np.nonzero(keep)[0]
    for t in rows:
        rms = float(np.sqrt(np.mean(out_o[t] ** 2)))
        err = float(np.max(np.abs(out_gpu[t] - out_o[t])))
        ratio = err / (OUT_TOL * rms)
        worst = max(worst, ratio)
        assert err <= OUT_TOL * rms, (t, err, rms)
    return worst


def oracle_outputs(X, ids_o, w_o, m, ids_g, w_g, expert_weights):
    """The oracle's block output for the compared tokens: on its own routing where
    the margin is at least 1e-5, on the GPU's ids and weights below it."""
    near = m < MARGIN
    ids = np.where(near[:, None], ids_g, ids_o)
    w = np.where(near[:, None], np.asarray(w_g, dtype=np.float64), w_o)
    return orc.combine(orc.expert_outputs(X, ids, expert_weights), w)


def forward_parity(p: Problem, bufs, tokens=None, label=""):
    """Compare one beam_moe_forward result with the oracle on the listed tokens (default all).

    Returns (near-tie tokens, worst error ratio); near-tie tokens are left out of the
    id comparison only: their outputs are checked on the GPU's routing."""
    d = p.dims
    T = p.x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    X, ids_o, w_o, S_o, C_o, GS_o, m = p.route_oracle_full(tokens)
    ids_all = bufs.ids.cpu().numpy()
    w_all = bufs.w.cpu().numpy()
    ids_g, w_g = ids_all[tokens], w_all[tokens]
    excluded = compare_routing(ids_g, w_g, ids_o, w_o, C_o, m, d, S_o=S_o)
    check_dispatch_valid(ids_all, bufs.counts.cpu().numpy(), bufs.offsets.cpu().numpy(), bufs.slots.cpu().numpy(),
                         d.num_experts)
    out_o = oracle_outputs(X, ids_o, w_o, m, ids_g, w_g, p.expert_f64)
    out_g = bufs.out[torch.as_tensor(tokens, device=bufs.out.device)].cpu().numpy().astype(np.float64)
    worst = compare_outputs(out_g, out_o)
    _record(len(tokens), excluded, worst)
    print(f"  {label}outputs of {len(tokens)} tokens compared, {excluded} of them near-ties "
          f"(margin < {MARGIN:g}: ids not compared, outputs checked on the GPU's routing)", flush=True)
    return excluded, worst


def residual_parity(p: Problem, stream: torch.Tensor, step: int, bufs, tokens=None, g_in=None, g_out=None,
                    eps=orc.NORM_EPS):
    """Compare one beam_moe_residual_forward result (new stream in bufs.out) with the oracle.

    Two output checks per token: the new stream within 1e-2 x its RMS, and
    the sublayer's contribution recovered from it, (new - a * stream) / b, within
    1e-2 x the RMS of the oracle's norm(out) * g_out, which the stream term
    would otherwise mask at large stream scales.  Near-tie tokens are checked on
    the GPU's routing.  Returns (near-tie tokens, worst ratio)."""
    d = p.dims
    T = stream.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    S = f64(stream)[tokens]
    sb = None if p.select_bias is None else f64(p.select_bias)
    bias = None if p.bias is None else f64(p.bias)
    gi = None if g_in is None else f64(g_in)
    go = None if g_out is None else f64(g_out)
    r = orc.moe_residual_step(S, step, f64(p.wr), bias, p.expert_f64, d.num_groups, d.topk_groups, d.topk,
                              d.routed_scaling, select_bias=sb, norm_in_weight=gi, norm_out_weight=go, eps=eps)
    m = orc.route_margins(r["S"], d.num_groups, d.topk_groups, d.topk, select_bias=sb)
    ids_all = bufs.ids.cpu().numpy()
    w_all = bufs.w.cpu().numpy()
    ids_g, w_g = ids_all[tokens], w_all[tokens]
    excluded = compare_routing(ids_g, w_g, r["ids"], r["w"], orc.selection_values(r["S"], sb), m, d, S_o=r["S"])
    check_dispatch_valid(ids_all, bufs.counts.cpu().numpy(), bufs.offsets.cpu().numpy(), bufs.slots.cpu().numpy(),
                         d.num_experts)
    a, b = orc.residual_weights(step)
    moe = r["moe"].copy()
    near = m < MARGIN
    if near.any():
        moe[near] = oracle_outputs(r["x"][near], r["ids"][near], r["w"][near], m[near], ids_g[near], w_g[near],
                                   p.expert_f64)
    term_o = orc.rms_norm(moe, go, eps)
    new_o = a * S + b * term_o
    new_g = bufs.out.cpu().numpy().astype(np.float64)[tokens]
    worst = compare_outputs(new_g, new_o)
    term_g = (new_g - a * S) / b
    worst = max(worst, compare_outputs(term_g, term_o))
    _record(len(tokens), excluded, worst)
    print(f"  new stream of {len(tokens)} tokens compared, {excluded} of them near-ties "
          f"(outputs checked on the GPU's routing)", flush=True)
    return excluded, worst


# --------------------------------------------------------------------------
# token samples at large batch sizes, chosen from the dispatch result
# --------------------------------------------------------------------------
TILE_ROWS = 256     # rows of a grouped-GEMM tile
LEVEL_ROWS = 64     # rows of one row level of a grouped-GEMM tile
MERGE_ROWS = 64     # a last grouped-GEMM tile of at most this many rows joins the tile before it


def tile_samples(counts, offsets, slots, topk, per_kind=2, stream_rows=0):
    """Tokens whose routed rows fall in each part of the expert kernels' tiling.

    Grouped GEMMs (stream_rows = 0): an expert's rows (expert-sorted order) are
    cut into tiles of 256 rows, and a last tile of at most 64 rows is merged into
    the tile before it as a fifth 64-row level.  Stream kernels (stream_rows = R):
    tiles of at most R rows, in 16-row fragments, nothing merged.  Returns
    [(label, token)]: rows in each level (fragment) of a full tile, the fifth
    level of merged tiles (its first and last row), the last row of partial
    tiles, the first and last row of the hottest expert and of its last tile, and
    the last row of an expert with very few rows."""
    counts = np.asarray(counts)
    offsets = np.asarray(offsets)
    slots = np.asarray(slots)
    tile = stream_rows or TILE_ROWS
    level = 16 if stream_rows else LEVEL_ROWS
    merge = 0 if stream_rows else MERGE_ROWS
    out = []

    def add(label, e, r):
        out.append((label, int(slots[offsets[e] + r]) // topk))

    order = np.argsort(-counts, kind="stable")
    full = [e for e in order if counts[e] >= tile]
    for e in full[:1]:
        for lev in range(tile // level):
            add(f"expert {e} ({counts[e]} rows) tile 0 level {lev}", e, lev * level + (17 * lev + 5) % level)
    merged = [e for e in order if merge and counts[e] > tile and 0 < counts[e] % tile <= merge]
    for e in merged[:per_kind]:
        c = int(counts[e])
        first5 = c - c % tile
        add(f"expert {e} ({c} rows) merged fifth level, first row", e, first5)
        add(f"expert {e} ({c} rows) merged fifth level, last row", e, c - 1)
    partial = [e for e in order if counts[e] % tile > merge]
    for e in partial[:per_kind]:
        c = int(counts[e])
        add(f"expert {e} ({c} rows) partial last tile ({c % tile} rows), last row", e, c - 1)
    if counts.max() > 0:
        e = int(order[0])
        c = int(counts[e])
        add(f"hottest expert {e} ({c} rows), first row", e, 0)
        last_tile = (c - 1) // tile * tile
        if merge and c > tile and c % tile and c % tile <= merge:
            last_tile -= tile
        add(f"hottest expert {e} ({c} rows), first row of its last tile", e, last_tile)
        add(f"hottest expert {e} ({c} rows), last row", e, c - 1)
    small = [e for e in order[::-1] if 0 < counts[e] <= min(level, tile)]
    for e in small[:1]:
        add(f"expert {e} ({counts[e]} rows, one level), last row", e, int(counts[e]) - 1)
    return out


def print_samples(samples):
    for label, t in samples:
        print(f"    token {t}: {label}", flush=True)
