"""Host-side checks of the GPU parity helpers (CPU only)."""
import itertools
import types

import numpy as np
import pytest
import torch

from grouped_top_routing_fp32_amd import synth
from oracle import beam_moe_oracle as orc
from parity_helpers import (MARGIN, Problem, compare_outputs, forward_parity, fp8_expert_lookup, residual_parity,
                            tile_samples)


def test_route_oracle_rejects_tokens_outside_the_batch():
    # the helper gathers the sampled rows on the tensors' device; a sample past the batch
    # must fail on the host rather than reach a device-side gather
    p = Problem(synth.with_tokens(synth.WORKLOADS["tiny"], 1), "cpu")
    with pytest.raises(IndexError):
        p.route_oracle([0, 1])
    X, ids, w, C, GS, m = p.route_oracle([0])
    assert X.shape == (1, p.dims.hidden) and ids.shape == (1, p.dims.topk) and np.isfinite(m).all()


def _tied_problem():
    """The tiny workload with two experts of one group given the same router row, so
    that every token scores them exactly alike; returns (problem, a, b, tied tokens),
    where the tied tokens select exactly one of a < b at the top-k boundary."""
    d = synth.WORKLOADS["tiny"].dims
    gs = d.num_experts // d.num_groups
    for g in range(d.num_groups):
        for a, b in itertools.combinations(range(g * gs, (g + 1) * gs), 2):
            p = Problem(synth.WORKLOADS["tiny"], "cpu")
            wr = p.wr.clone()
            wr[b] = wr[a]
            p.wr = wr
            X, ids, w, S, C, GS, m = p.route_oracle_full()
            tied = [t for t in range(ids.shape[0]) if (a in ids[t]) != (b in ids[t])]
            if tied:
                assert all(m[t] < MARGIN for t in tied)
                return p, a, b, tied
    raise AssertionError("no boundary tie found")


def _fake_bufs(p, ids_g):
    """What a correct GPU run that broke the ties the other way would return."""
    d = p.dims
    X, ids_o, w_o, S, C, GS, m = p.route_oracle_full()
    w_g = orc.normalised_weights(S, ids_g, d.routed_scaling).astype(np.float32)
    out = orc.combine(orc.expert_outputs(X, ids_g, p.expert_f64), w_g)
    c, o, s = orc.dispatch(ids_g, d.num_experts)
    return types.SimpleNamespace(ids=torch.from_numpy(ids_g.astype(np.int32)), w=torch.from_numpy(w_g),
                                 out=torch.from_numpy(out.astype(np.float32)), counts=torch.from_numpy(c),
                                 offsets=torch.from_numpy(o), slots=torch.from_numpy(s))


def _swap_ties(ids, a, b, tied):
    ids_g = ids.copy()
    for t in tied:
        ids_g[t] = np.where(ids_g[t] == a, b, ids_g[t])  # the oracle takes the lower id on a tie
    return ids_g


def test_near_tie_outputs_are_checked_on_the_gpu_routing():
    p, a, b, tied = _tied_problem()
    X, ids_o, w_o, S, C, GS, m = p.route_oracle_full()
    ids_g = _swap_ties(ids_o, a, b, tied)
    bufs = _fake_bufs(p, ids_g)
    # the other expert changes the output: the oracle's own routing would reject it
    out_o = orc.combine(orc.expert_outputs(X, ids_o, p.expert_f64), w_o)
    with pytest.raises(AssertionError):
        compare_outputs(bufs.out.numpy().astype(np.float64)[tied], out_o[tied])
    excluded, worst = forward_parity(p, bufs)
    assert excluded >= len(tied) and worst < 1e-3


@pytest.mark.parametrize("what", ["output", "weight"])
def test_near_tie_mistakes_fail(what):
    p, a, b, tied = _tied_problem()
    X, ids_o, w_o, S, C, GS, m = p.route_oracle_full()
    bufs = _fake_bufs(p, _swap_ties(ids_o, a, b, tied))
    t = tied[0]
    if what == "output":
        rms = float(bufs.out[t].pow(2).mean().sqrt())
        bufs.out[t, 3] += 0.05 * rms
    else:
        bufs.w[t, 0] += 1e-4
    with pytest.raises(AssertionError):
        forward_parity(p, bufs)


def test_near_tie_residual_outputs_are_checked_on_the_gpu_routing():
    p, a, b, tied0 = _tied_problem()
    d = p.dims
    wl = p.wl
    stream = synth.make_stream(wl, "cpu")
    r = orc.moe_residual_step(stream.double().numpy(), 3, p.wr.double().numpy(), None, p.expert_f64,
                              d.num_groups, d.topk_groups, d.topk, d.routed_scaling)
    tied = [t for t in range(wl.tokens) if (a in r["ids"][t]) != (b in r["ids"][t])]
    if not tied:
        pytest.skip("the normalised stream puts no token at the tie boundary")
    ids_g = _swap_ties(r["ids"], a, b, tied)
    w_g = orc.normalised_weights(r["S"], ids_g, d.routed_scaling)
    moe = orc.combine(orc.expert_outputs(r["x"], ids_g, p.expert_f64), w_g)
    aw, bw = orc.residual_weights(3)
    new = aw * stream.double().numpy() + bw * orc.rms_norm(moe)
    c, o, s = orc.dispatch(ids_g, d.num_experts)
    bufs = types.SimpleNamespace(ids=torch.from_numpy(ids_g.astype(np.int32)),
                                 w=torch.from_numpy(w_g.astype(np.float32)), out=torch.from_numpy(new),
                                 counts=torch.from_numpy(c), offsets=torch.from_numpy(o), slots=torch.from_numpy(s))
    excluded, worst = residual_parity(p, stream, 3, bufs)
    assert excluded >= len(tied) and worst < 1e-3
    bufs.out[tied[0], 0] += 0.2
    with pytest.raises(AssertionError):
        residual_parity(p, stream, 3, bufs)


def test_tile_samples_land_where_labelled():
    K = 4
    counts = np.array([560, 700, 40, 512, 0, 300], dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(offsets[-1])
    slots = np.random.default_rng(0).permutation(n).astype(np.int32)
    got = tile_samples(counts, offsets, slots, K)
    labels = [lab for lab, _ in got]

    def row_of(t, e):
        rows = [r for r in range(counts[e]) if slots[offsets[e] + r] // K == t]
        return rows

    def find(prefix):
        return [t for lab, t in got if lab.startswith(prefix)]

    # the hottest expert (700 rows: tiles 256, 256, 188) is expert 1
    assert any("hottest expert 1 (700 rows), first row of its last tile" in lab for lab in labels)
    assert 512 in row_of(find("hottest expert 1 (700 rows), first row of its last tile")[0], 1)
    # merged fifth levels: 560 = 256 + 304 and 300 = 256 + 44
    for e, c in ((0, 560), (5, 300)):
        first = find(f"expert {e} ({c} rows) merged fifth level, first row")[0]
        last = find(f"expert {e} ({c} rows) merged fifth level, last row")[0]
        assert c - c % 256 in row_of(first, e) and c - 1 in row_of(last, e)
    assert 699 in row_of(find("expert 1 (700 rows) partial last tile")[0], 1)
    assert 39 in row_of(find("expert 2 (40 rows, one level)")[0], 2)
    levels = [t for lab, t in got if "tile 0 level" in lab]
    assert len(levels) == 4


def test_fp8_lookup_equals_the_oracle_decode():
    wl = synth.Workload("f8", 4, synth.Dims(256, 128, 2, 1, 1, 1))
    q = synth.expert_weights_fp8(wl, 1, "cpu")
    args = [t.numpy() for t in q]
    args[0][0, :4] = [0x7E, 0xFE, 0x01, 0x80]  # 448, -448, the smallest subnormal, -0
    for a, b in zip(fp8_expert_lookup(*args), orc.fp8_expert(*args)):
        assert np.array_equal(a, b)


def test_tile_samples_on_stream_tiles():
    K, R = 8, 32
    counts = np.array([100, 7, 64, 0, 33], dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    slots = np.arange(int(offsets[-1]), dtype=np.int32)   # token of row r of expert e: (offsets[e] + r) // K
    got = dict((lab, t) for lab, t in tile_samples(counts, offsets, slots, K, stream_rows=R))
    assert not any("merged" in lab for lab in got)        # the stream path merges nothing
    assert got["hottest expert 0 (100 rows), first row of its last tile"] == (0 + 96) // K
    assert got["expert 0 (100 rows) partial last tile (4 rows), last row"] == 99 // K
    assert sum("tile 0 level" in lab for lab in got) == R // 16
    assert got["expert 1 (7 rows, one level), last row"] == (100 + 6) // K
