"""GPU parity of the HIP path (through the C ABI) against the FP64 oracle.

Every case prints its name before touching the GPU, so that a failing run
names it.  Sizes: small cases run the oracle on every token and span several
tiles with a ragged tail; the Beam-size cases (decode T=64, prefill T=16384,
skewed T=8192) run the exact launch configuration of the benchmark and check
sampled tokens against the oracle, and the dispatch of every token by its
defining properties.
"""
import math

import numpy as np
import pytest
import torch

from grouped_top_routing_fp32_amd import binding, synth
from oracle import beam_moe_oracle as orc
from parity_helpers import (Problem, check_dispatch_valid, compare_outputs, compare_routing, f64, forward_parity,
                            print_samples, residual_parity, tile_samples)

pytestmark = pytest.mark.gpu

DEV = "cuda"
TINY = synth.WORKLOADS["tiny"].dims


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.fixture(scope="module")
def beam_experts_fp8():
    _announce("generate Beam FP8 expert weights on the device")
    ex = synth.make_experts_fp8(synth.WORKLOADS["decode"], DEV)
    torch.cuda.synchronize()
    return ex


@pytest.fixture(scope="module")
def beam_experts():
    _announce("generate Beam expert weights on the device")
    wl = synth.WORKLOADS["decode"]
    ex = synth.make_experts(wl, DEV)
    torch.cuda.synchronize()
    return ex


# --------------------------------------------------------------------------
# shared generator: identical bits on CPU and GPU
# --------------------------------------------------------------------------
def test_generator_bits_match_cpu():
    _announce("generator cpu vs gpu")
    wl = synth.WORKLOADS["decode"]
    a = synth.normal((2560, 5120), 0.02, 0, synth.TENSOR_GATE, 3, torch.bfloat16, DEV).cpu()
    b = synth.normal((2560, 5120), 0.02, 0, synth.TENSOR_GATE, 3, torch.bfloat16, "cpu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    xr = synth.x_rows(wl, [0, 17, 63], DEV).cpu()
    assert torch.equal(xr.view(torch.int16), synth.x_rows(wl, [0, 17, 63], "cpu").view(torch.int16))
    wr = synth.make_router(wl, DEV).cpu()
    assert torch.equal(wr.view(torch.int32), synth.make_router(wl, "cpu").view(torch.int32))


# --------------------------------------------------------------------------
# selection on supplied FP32 scores: bit-exact
# --------------------------------------------------------------------------
def _select_case(d, scores_np):
    scores = torch.from_numpy(scores_np.astype(np.float32)).to(DEV)
    ids, w = binding.beam_moe_select(d, scores)
    ids_o, w_o = orc.select_fp32(scores_np.astype(np.float32), d.num_groups, d.topk_groups, d.topk,
                                 d.routed_scaling)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.int32), w_o.view(np.int32))


@pytest.mark.parametrize("kind", ["uniform", "coarse_ties", "group_sum_ties", "boundary_ties", "all_equal"])
def test_select_bit_exact_beam(kind):
    _announce(f"select beam {kind}")
    rng = np.random.default_rng(["uniform", "coarse_ties", "group_sum_ties", "boundary_ties", "all_equal"].index(kind))
    T, E = 333, 256
    if kind == "uniform":
        s = rng.random((T, E))
    elif kind == "coarse_ties":
        s = np.floor(rng.random((T, E)) * 8) / 8 + 0.0625
    elif kind == "group_sum_ties":
        # every group holds the pair (a, b) or (b, a) or (a + d, b - d) with equal sums
        s = rng.random((T, E)) * 0.25
        for t in range(T):
            for g in range(8):
                i, j = rng.choice(32, 2, replace=False)
                s[t, g * 32 + i], s[t, g * 32 + j] = (0.75, 0.5) if g % 2 else (0.5, 0.75)
    elif kind == "boundary_ties":
        s = rng.random((T, E)) * 0.5
        for t in range(T):
            hot = rng.choice(E, 12, replace=False)
            s[t, hot] = 0.875
    else:
        s = np.full((T, E), 0.5)
    _select_case(synth.BEAM, s)


def test_select_bit_exact_router_scores():
    _announce("select on oracle scores (router_dispatch, 512 tokens)")
    wl = synth.with_tokens(synth.WORKLOADS["router_dispatch"], 512)
    X = f64(synth.make_x(wl))
    S = orc.sigmoid(orc.router_logits(X, f64(synth.make_router(wl))))
    _select_case(wl.dims, S)


@pytest.mark.parametrize("dims", [TINY, synth.Dims(256, 128, 64, 8, 3, 6), synth.Dims(256, 128, 200, 8, 8, 16),
                                  synth.Dims(256, 128, 8, 1, 1, 8), synth.Dims(256, 128, 32, 32, 5, 5),
                                  synth.Dims(256, 128, 1, 1, 1, 1)])
def test_select_bit_exact_shapes(dims):
    _announce(f"select shapes {dims}")
    rng = np.random.default_rng(dims.num_experts)
    # scores in (0, 1): sigmoid outputs are positive, so a token's weight sum is never 0
    s = rng.random((77, dims.num_experts)) * 0.99 + 0.005
    s[::3] = (np.floor(s[::3] * 4) + 0.5) / 4   # coarse values: exact ties between experts and groups
    assert np.all(s > 0)
    _select_case(dims, s)


def test_hand_example_on_gpu():
    _announce("hand-worked routing example")
    import json
    import os
    h = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "routing_hand_example.json")))
    d = synth.Dims(256, 128, h["num_experts"], h["num_groups"], h["topk_groups"], h["topk"], h["routed_scaling"])
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV)
    x[0, 0] = 1.0
    wr = torch.zeros((16, 256), dtype=torch.float32, device=DEV)
    wr[:, 0] = torch.tensor([math.log(a / (1 - a)) for a in h["scores"]], dtype=torch.float32)
    ids, w, s = binding.beam_moe_route(d, x, wr, want_scores=True)
    assert ids.cpu().tolist()[0] == h["expected_ids"]
    np.testing.assert_allclose(w.cpu().numpy()[0], h["expected_weights"], rtol=0, atol=2e-6)
    np.testing.assert_allclose(s.cpu().numpy()[0], h["scores"], rtol=0, atol=2e-7)


# --------------------------------------------------------------------------
# dispatch: bit-exact on oracle ids
# --------------------------------------------------------------------------
def _dispatch_case(d, ids_np):
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
    c, o, s = binding.beam_moe_dispatch(d, ids)
    c2, o2, s2 = binding.beam_moe_dispatch(d, ids)
    co, oo, so = orc.dispatch(ids_np, d.num_experts)
    assert np.array_equal(c.cpu().numpy(), co)
    assert np.array_equal(o.cpu().numpy(), oo)
    assert np.array_equal(s.cpu().numpy(), so)
    assert torch.equal(c, c2) and torch.equal(o, o2) and torch.equal(s, s2)


@pytest.mark.parametrize("case", ["uniform", "skewed", "one_expert", "single_token", "ragged", "large"])
def test_dispatch_bit_exact(case):
    _announce(f"dispatch {case}")
    d = synth.BEAM
    rng = np.random.default_rng(1)
    T = {"uniform": 300, "skewed": 999, "one_expert": 40, "single_token": 1, "ragged": 37, "large": 16384}[case]
    if case == "one_expert":
        d = synth.Dims(5120, 2560, 256, 8, 4, 1)
        ids = np.full((T, 1), 200)
    elif case == "skewed":
        p = np.arange(1, 257, dtype=np.float64) ** -1.2
        p /= p.sum()
        ids = np.stack([rng.choice(256, 8, replace=False, p=p) for _ in range(T)])
    else:
        ids = np.stack([rng.choice(256, 8, replace=False) for _ in range(T)])
    _dispatch_case(d, ids)


def test_dispatch_on_router_ids():
    _announce("dispatch on oracle router ids (router_dispatch, T=4096)")
    wl = synth.WORKLOADS["router_dispatch"]
    d = wl.dims
    p = Problem(wl, DEV)
    X, ids_o, w_o, S_o, GS_o, m = p.route_oracle()
    _dispatch_case(d, ids_o)


# --------------------------------------------------------------------------
# router end to end (FP32 on the GPU vs FP64 oracle)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,T", [("tiny", 16), ("router_dispatch", 4096), ("skewed", 1000),
                                    ("router_dispatch", 16384)])
def test_route_end_to_end(name, T):
    _announce(f"route e2e {name} T={T}")
    wl = synth.with_tokens(synth.WORKLOADS[name], T)
    d = wl.dims
    p = Problem(wl, DEV, experts=(None, None, None))
    ids, w, s = binding.beam_moe_route(d, p.x, p.wr, p.bias, want_scores=True)
    X, ids_o, w_o, S_o, GS_o, m = p.route_oracle()
    np.testing.assert_allclose(s.cpu().numpy(), S_o, rtol=0, atol=2e-6)
    excluded = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_o, w_o, S_o, m, d)
    print(f"  excluded near-tie tokens: {excluded} of {T}")
    assert excluded <= max(2, T // 200)
    ids2, w2, s2 = binding.beam_moe_route(d, p.x, p.wr, p.bias, want_scores=True)
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(s, s2)
    c, o, sl = binding.beam_moe_dispatch(d, ids)
    check_dispatch_valid(ids.cpu().numpy(), c.cpu().numpy(), o.cpu().numpy(), sl.cpu().numpy(), d.num_experts)


# --------------------------------------------------------------------------
# whole block
# --------------------------------------------------------------------------
# Each case names the expert path it covers: R > 0 for the stream kernels on tiles of at most R
# rows (the smallest of 8 .. 128 at least twice the average rows per expert), 0 for the grouped
# GEMMs (more than 64 average rows per expert); the library's choice is asserted first.
MID = {
    # stream path, 8-row tiles, several column blocks; experts with more than one tile
    "mid_stream": (synth.Workload("mid_stream", 40, synth.Dims(512, 384, 64, 8, 4, 6), router_sigma=0.06), 8),
    # grouped path, 16 experts, ~225 rows each: full and ragged 256-row tiles
    "mid_tiled": (synth.Workload("mid_tiled", 900, synth.Dims(512, 384, 16, 4, 2, 4), router_sigma=0.06), 0),
    # grouped path with Beam's expert count: one partial tile (about 69 rows, two levels) per expert
    "mid_tiled_e256": (synth.Workload("mid_tiled_e256", 2200, synth.Dims(768, 256, 256, 8, 4, 8), router_sigma=0.04),
                       0),
    # stream path with skewed bias: some experts get several 8-row tiles
    "mid_stream_skew": (synth.Workload("mid_stream_skew", 60, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06,
                                       zipf_s=1.2), 8),
    # stream path, I/32 not a multiple of 8
    "mid_stream_i384": (synth.Workload("mid_stream_i384", 40, synth.Dims(512, 384, 64, 8, 4, 4),
                                       router_sigma=0.06), 8),
    # large activations (expert weights N(0, 10^2)): the SwiGLU activations and the expert
    # outputs exceed 2^15 and travel to the next step with a power-of-two scale
    "mid_stream_big": (synth.Workload("mid_stream_big", 40, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06,
                                      expert_sigma=10.0), 8),
    "mid_tiled_big": (synth.Workload("mid_tiled_big", 900, synth.Dims(512, 384, 16, 4, 2, 4), router_sigma=0.06,
                                     expert_sigma=10.0), 0),
    # huge activations (expert weights N(0, 200^2)): SwiGLU activations near 2^24 and expert
    # outputs near 2^36, so h and y carry scales 2^-s with s >= 9.  The down projection keeps
    # its accumulators in units of 2^s and never scales its weights: weights times 2^s would
    # pass fp16's 65504 here
    "mid_stream_huge": (synth.Workload("mid_stream_huge", 40, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06,
                                       expert_sigma=200.0), 8),
    "mid_tiled_huge": (synth.Workload("mid_tiled_huge", 900, synth.Dims(512, 384, 16, 4, 2, 4), router_sigma=0.06,
                                      expert_sigma=200.0), 0),
    # grouped path with skew (75 rows per expert on average): hot experts with several tiles,
    # many nearly empty tiles, whose idle waves copy no activations
    "mid_grouped_skew": (synth.Workload("mid_grouped_skew", 1200, synth.Dims(512, 256, 64, 8, 4, 4),
                                        router_sigma=0.06, zipf_s=1.2), 0),
    # stream path on every wider tile: 16, 32 and 64 rows (one to four row fragments per wave;
    # the down kernel with two column fragments per wave from 32 rows), partial tiles, and skewed
    # batches whose hot experts take several tiles
    "mid_stream_r16": (synth.Workload("mid_stream_r16", 100, synth.Dims(512, 384, 64, 8, 4, 4), router_sigma=0.06),
                       16),
    "mid_stream_r32": (synth.Workload("mid_stream_r32", 200, synth.Dims(512, 384, 64, 8, 4, 4), router_sigma=0.06),
                       32),
    "mid_stream_r32_skew": (synth.Workload("mid_stream_r32_skew", 200, synth.Dims(512, 384, 64, 8, 4, 4),
                                           router_sigma=0.06, zipf_s=1.2), 32),
    "mid_stream_r64": (synth.Workload("mid_stream_r64", 400, synth.Dims(512, 384, 64, 8, 4, 4), router_sigma=0.06),
                       64),
    "mid_stream_r64_skew": (synth.Workload("mid_stream_r64_skew", 400, synth.Dims(512, 384, 64, 8, 4, 4),
                                           router_sigma=0.06, zipf_s=1.2), 64),
    # just past the stream path (50 rows per expert on average): grouped GEMMs, one partial tile each
    "mid_grouped_r50": (synth.Workload("mid_grouped_r50", 800, synth.Dims(512, 384, 64, 8, 4, 4),
                                       router_sigma=0.06), 0),
    "mid_stream_r64_big": (synth.Workload("mid_stream_r64_big", 400, synth.Dims(512, 256, 64, 8, 4, 4),
                                          router_sigma=0.06, expert_sigma=10.0), 64),
}


def _expect_path(wl, rows, fp8=False):
    got = binding.beam_moe_stream_rows(wl.dims, wl.tokens, fp8)
    assert got == rows, f"{wl.name}: the library takes {got} (0 = grouped GEMMs), the case covers {rows}"


def test_forward_tiny():
    _announce("forward tiny (all tokens)")
    p = Problem(synth.WORKLOADS["tiny"], DEV)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    excluded, worst = forward_parity(p, bufs)
    print(f"  worst error / tolerance {worst:.3f}")


@pytest.mark.parametrize("name", list(MID))
def test_forward_mid(name):
    _announce(f"forward {name} (all tokens)")
    wl, rows = MID[name]
    _expect_path(wl, rows)
    p = Problem(wl, DEV)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    excluded, worst = forward_parity(p, bufs)
    print(f"  worst error / tolerance {worst:.3f}")
    out1 = bufs.out.clone()
    binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd, bufs=bufs)
    assert torch.equal(out1, bufs.out)


def _beam_forward(name, beam_experts, sample):
    return _beam_forward_wl(synth.WORKLOADS[name], beam_experts, sample)


def _samples(p, bufs, fixed):
    """Fixed tokens plus tokens whose routed rows land in each part of the expert kernels'
    tiling (row levels, merged fifth levels, partial tiles, the hottest expert), chosen
    from this run's dispatch and the path the library takes; prints which."""
    rows = binding.beam_moe_stream_rows(p.dims, p.x.shape[0], p.fp8)
    print(f"    expert path: {'stream kernels, tiles of %d rows' % rows if rows else 'grouped GEMMs'}", flush=True)
    picks = tile_samples(bufs.counts.cpu().numpy(), bufs.offsets.cpu().numpy(), bufs.slots.cpu().numpy(),
                         p.dims.topk, stream_rows=rows)
    print_samples(picks)
    return sorted(set(int(t) for t in fixed) | {t for _, t in picks})


def _beam_forward_wl(wl, beam_experts, sample):
    """sample: token list, or None for all tokens, or "tiles" for tile-aware samples."""
    p = Problem(wl, DEV, experts=beam_experts)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    torch.cuda.synchronize()
    T = wl.tokens
    if isinstance(sample, str):
        sample = _samples(p, bufs, (0, T // 2, T - 1))
    excluded, worst = forward_parity(p, bufs, sample)
    print(f"  worst error / tolerance {worst:.3f}")
    out1 = bufs.out.clone()
    ids1 = bufs.ids.clone()
    slots1 = bufs.slots.clone()
    binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd, bufs=bufs)
    assert torch.equal(out1, bufs.out) and torch.equal(ids1, bufs.ids) and torch.equal(slots1, bufs.slots)
    return p, bufs


def test_forward_decode(beam_experts):
    _announce("forward decode T=64 (all tokens)")
    _beam_forward("decode", beam_experts, None)


def test_forward_prefill(beam_experts):
    _announce("forward prefill T=16384 (tile-aware sample)")
    _beam_forward("prefill", beam_experts, "tiles")


def test_forward_skewed(beam_experts):
    _announce("forward skewed T=8192 (tile-aware sample)")
    p, bufs = _beam_forward("skewed", beam_experts, "tiles")
    counts = bufs.counts.cpu().numpy()
    assert counts.max() >= 20 * counts.mean()


# Beam dims across the batch sizes where the expert path changes form: T <= 1024
# stream kernels (T = 1: two-slot rings, every workgroup resident at once; T = 128:
# experts with more than one 8-row tile; 256 .. 1024: 16-, 32- and 64-row tiles); from
# T = 2048 the grouped GEMMs: tiles of at most two levels (three activation and three
# weight stages), of three (T = 4096, 6144: two and three), four-level tiles with small
# merged fifth levels (T = 8192), full tiles followed by short ones (T = 12288), and
# T = 32768, twice the prefill batch: about 1024 rows, four tiles, per expert.
@pytest.mark.parametrize("T", [1, 8, 128, 160, 256, 512, 1024, 2048, 4096, 6144, 8192, 12288, 32768])
def test_forward_beam_sizes(beam_experts, T):
    _announce(f"forward Beam T={T}")
    wl = synth.with_tokens(synth.WORKLOADS["decode"], T)
    _beam_forward_wl(wl, beam_experts, None if T <= 8 else "tiles")


# The largest batch tried: 2,097,152 routed rows, so the expert outputs y [n, H] hold 1.07e10
# elements and every offset past 2^31 must be formed in 64 bits; the last token's rows sit at
# the highest offsets.  (About 70 GB of device memory with the experts.)
def test_forward_beam_offsets_past_2_31(beam_experts):
    T = 262144
    _announce(f"forward Beam T={T}")
    wl = synth.with_tokens(synth.WORKLOADS["decode"], T)
    _beam_forward_wl(wl, beam_experts, [0, 1, T // 2, T - 2, T - 1])


# Degenerate and extreme shapes of the method through the whole block (all tokens).
EDGE = {
    # one expert, one group, top-1: the block is 2.5 x a dense SwiGLU (stream path, then grouped
    # with three tiles of 256, 256 and 88 rows)
    "dense_stream": synth.Workload("dense_stream", 3, synth.Dims(256, 128, 1, 1, 1, 1), router_sigma=0.06),
    "dense_grouped": synth.Workload("dense_grouped", 600, synth.Dims(256, 128, 1, 1, 1, 1), router_sigma=0.06),
    # a last tile of at most 64 rows joins the tile before it (256 + 48 = 304 rows, five levels) in
    # both projections; large weights, so h and y carry non-zero power-of-two scales
    "dense_merged_big": synth.Workload("dense_merged_big", 560, synth.Dims(256, 128, 1, 1, 1, 1), router_sigma=0.06,
                                       expert_sigma=10.0),
    # merged fifth levels: a tail of one 16-row fragment (5 rows), of two (17 rows: the second
    # holds one row), and a full one (64 rows: 320 rows, the kernel's no-level-test loop), with
    # non-zero scales
    "dense_tail1": synth.Workload("dense_tail1", 261, synth.Dims(256, 128, 1, 1, 1, 1), router_sigma=0.06,
                                  expert_sigma=10.0),
    "dense_tail2": synth.Workload("dense_tail2", 273, synth.Dims(256, 128, 1, 1, 1, 1), router_sigma=0.06,
                                  expert_sigma=10.0),
    "dense_tail_full": synth.Workload("dense_tail_full", 320, synth.Dims(256, 128, 1, 1, 1, 1), router_sigma=0.06,
                                      expert_sigma=10.0),
    # about 300 rows per expert: some experts' tails are merged (<= 64 rows), others are not
    "merged_tails_big": synth.Workload("merged_tails_big", 1200, synth.Dims(512, 256, 8, 2, 1, 2), router_sigma=0.06,
                                       expert_sigma=10.0),
    # the largest top-k, on both paths
    "topk16_stream": synth.Workload("topk16_stream", 16, synth.Dims(256, 128, 64, 8, 8, 16), router_sigma=0.06),
    "topk16_grouped": synth.Workload("topk16_grouped", 300, synth.Dims(256, 128, 64, 8, 8, 16), router_sigma=0.06),
    # no grouping (one group), every group kept (plain top-k), one expert per group
    "one_group": synth.Workload("one_group", 24, synth.Dims(256, 128, 64, 1, 1, 8), router_sigma=0.06),
    "all_groups": synth.Workload("all_groups", 24, synth.Dims(256, 128, 64, 8, 8, 8), router_sigma=0.06),
    "group_of_one": synth.Workload("group_of_one", 24, synth.Dims(256, 128, 16, 16, 6, 4), router_sigma=0.06),
    # the largest intermediate size the library takes, with a wide hidden size
    "wide": synth.Workload("wide", 12, synth.Dims(2048, 32768, 2, 1, 1, 1), router_sigma=0.03),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_forward_edge_dims(name):
    _announce(f"forward {name} (all tokens)")
    p = Problem(EDGE[name], DEV)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    excluded, worst = forward_parity(p, bufs)
    print(f"  worst error / tolerance {worst:.3f}")


def test_forward_dense_is_scaled_swiglu():
    # with one expert every token takes it with weight 2.5: out = 2.5 * SwiGLU(x), checked
    # against the oracle's dense expert directly (no routing step)
    _announce("forward dense = 2.5 x SwiGLU")
    p = Problem(EDGE["dense_grouped"], DEV)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    assert torch.all(bufs.ids == 0) and torch.all(bufs.w == 2.5)
    want = 2.5 * orc.swiglu_expert(f64(p.x), *p.expert_f64(0))
    compare_outputs(bufs.out.cpu().numpy().astype(np.float64), want, np.ones(want.shape[0], dtype=bool))


def test_forward_empty_batch():
    _announce("forward T=0")
    wl = synth.with_tokens(synth.WORKLOADS["tiny"], 0)
    p = Problem(wl, DEV)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    assert bufs.out.shape == (0, p.dims.hidden) and bufs.ids.shape == (0, p.dims.topk)


# --------------------------------------------------------------------------
# selection-only bias: ranks groups and experts, never forms the weights
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["normal", "coarse"])
@pytest.mark.parametrize("dims", [TINY, synth.BEAM, synth.Dims(256, 128, 64, 8, 3, 6)])
def test_select_with_selection_bias_bit_exact(dims, kind):
    _announce(f"select with selection bias {kind} {dims}")
    E = dims.num_experts
    rng = np.random.default_rng(E + (7 if kind == "coarse" else 0))
    s = rng.random((129, E)).astype(np.float32)
    b = rng.normal(0.0, 0.05, E).astype(np.float32)
    if kind == "coarse":   # exact ties among the biased values
        s = (np.round(s * 8) / 8).astype(np.float32)
        b = (np.round(b * 16) / 16).astype(np.float32)
    ids, w = binding.beam_moe_select(dims, torch.from_numpy(s).to(DEV), select_bias=torch.from_numpy(b).to(DEV))
    ids_o, w_o = orc.select_fp32(s, dims.num_groups, dims.topk_groups, dims.topk, dims.routed_scaling,
                                 select_bias=b)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.int32), w_o.view(np.int32))


def test_hand_example_selection_bias_on_gpu():
    _announce("hand-worked selection-bias example")
    import json
    import os
    h = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "routing_selection_bias_example.json")))
    d = synth.Dims(256, 128, h["num_experts"], h["num_groups"], h["topk_groups"], h["topk"], h["routed_scaling"])
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV)
    x[0, 0] = 1.0
    wr = torch.zeros((16, 256), dtype=torch.float32, device=DEV)
    wr[:, 0] = torch.tensor([math.log(a / (1 - a)) for a in h["scores"]], dtype=torch.float32)
    sb = torch.tensor(h["selection_bias"], dtype=torch.float32, device=DEV)
    ids, w, s = binding.beam_moe_route(d, x, wr, select_bias=sb, want_scores=True)
    assert ids.cpu().tolist()[0] == h["expected_ids"]
    np.testing.assert_allclose(w.cpu().numpy()[0], h["expected_weights"], rtol=0, atol=2e-6)
    np.testing.assert_allclose(s.cpu().numpy()[0], h["scores"], rtol=0, atol=2e-7)  # scores stay unbiased


def test_route_with_selection_bias_e2e():
    _announce("route with selection bias, T=4096 at Beam scale")
    wl = synth.WORKLOADS["router_dispatch"]
    d = wl.dims
    sb = torch.from_numpy(np.random.default_rng(5).normal(0.0, 0.05, d.num_experts).astype(np.float32)).to(DEV)
    p = Problem(wl, DEV, select_bias=sb)
    ids, w, _ = binding.beam_moe_route(d, p.x, p.wr, p.bias, select_bias=sb)
    X, ids_o, w_o, S_o, C_o, GS_o, m = p.route_oracle_full()
    excluded = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_o, w_o, C_o, m, d, S_o=S_o)
    print(f"  excluded near-tie tokens: {excluded} of {wl.tokens}")
    assert excluded <= max(2, wl.tokens // 200)
    # the bias moved the choice of a good share of tokens
    ids0, _, _ = binding.beam_moe_route(d, p.x, p.wr, p.bias)
    moved = (np.sort(ids.cpu().numpy(), 1) != np.sort(ids0.cpu().numpy(), 1)).any(1).mean()
    print(f"  tokens whose experts the bias changed: {moved:.1%}")
    assert moved > 0.05


@pytest.mark.parametrize("name", ["tiny", "mid_stream", "mid_tiled_e256"])
def test_forward_with_selection_bias(name):
    _announce(f"forward {name} with selection bias")
    wl = synth.WORKLOADS[name] if name in synth.WORKLOADS else MID[name][0]
    E = wl.dims.num_experts
    sb = torch.from_numpy(np.random.default_rng(E).normal(0.0, 0.05, E).astype(np.float32)).to(DEV)
    p = Problem(wl, DEV, select_bias=sb)
    bufs = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd, select_bias=sb)
    excluded, worst = forward_parity(p, bufs)
    print(f"  worst error / tolerance {worst:.3f}")
    out1 = bufs.out.clone()
    binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd, select_bias=sb, bufs=bufs)
    assert torch.equal(out1, bufs.out)


# --------------------------------------------------------------------------
# the block as a residual sublayer: pre-norm, block, post-norm, scaled update
# --------------------------------------------------------------------------
def _residual_case(wl, step, weights, experts=None, select_bias=None):
    p = Problem(wl, DEV, experts=experts, select_bias=select_bias)
    stream = synth.make_stream(wl, DEV)
    g_in, g_out = synth.make_norm_weights(wl, DEV) if weights else (None, None)
    bufs = binding.beam_moe_residual_forward(p.dims, stream, step, p.wr, p.bias, p.wg, p.wu, p.wd,
                                             select_bias=select_bias, norm_in_weight=g_in, norm_out_weight=g_out)
    torch.cuda.synchronize()
    return p, stream, g_in, g_out, bufs


@pytest.mark.parametrize("step,weights", [(2, False), (3, True), (105, True)])
def test_residual_tiny(step, weights):
    _announce(f"residual tiny step={step} weights={weights}")
    p, stream, g_in, g_out, bufs = _residual_case(synth.WORKLOADS["tiny"], step, weights)
    excluded, worst = residual_parity(p, stream, step, bufs, g_in=g_in, g_out=g_out)
    print(f"  worst error / tolerance {worst:.3f}")


@pytest.mark.parametrize("name", ["mid_stream", "mid_tiled", "mid_stream_skew", "mid_stream_r64"])
def test_residual_mid(name):
    _announce(f"residual {name} (all tokens)")
    wl, rows = MID[name]
    _expect_path(wl, rows)
    p, stream, g_in, g_out, bufs = _residual_case(wl, 4, True)
    excluded, worst = residual_parity(p, stream, 4, bufs, g_in=g_in, g_out=g_out)
    print(f"  worst error / tolerance {worst:.3f}")
    # in place (stream_out is stream_in) gives the same bits, and so does a second call
    new1 = bufs.out.clone()
    inplace = stream.clone()
    binding.beam_moe_residual_forward(p.dims, inplace, 4, p.wr, p.bias, p.wg, p.wu, p.wd, norm_in_weight=g_in,
                                      norm_out_weight=g_out, stream_out=inplace, bufs=bufs)
    assert torch.equal(inplace, new1)
    # stream_out is per call: the buffers keep their own out, untouched by that call
    assert bufs.out.data_ptr() != inplace.data_ptr() and torch.equal(bufs.out, new1)
    binding.beam_moe_residual_forward(p.dims, stream, 4, p.wr, p.bias, p.wg, p.wu, p.wd, norm_in_weight=g_in,
                                      norm_out_weight=g_out, bufs=bufs)
    assert torch.equal(bufs.out, new1)


def test_residual_selection_bias():
    _announce("residual mid_tiled with selection bias")
    wl, _ = MID["mid_tiled"]
    sb = synth.normal((wl.dims.num_experts,), 0.05, 11, 0, device=DEV)
    p, stream, g_in, g_out, bufs = _residual_case(wl, 6, True, select_bias=sb)
    excluded, worst = residual_parity(p, stream, 6, bufs, g_in=g_in, g_out=g_out)
    print(f"  worst error / tolerance {worst:.3f}")


# the three batches the residual entry point is timed on (decode, prefill and the skewed
# batch), plus one in between
@pytest.mark.parametrize("name,T", [("decode", 64), ("decode", 1024), ("prefill", 16384), ("skewed", 8192)])
def test_residual_beam(beam_experts, name, T):
    _announce(f"residual Beam {name} T={T}")
    wl = synth.with_tokens(synth.WORKLOADS[name], T)
    p, stream, g_in, g_out, bufs = _residual_case(wl, 3, True, experts=beam_experts)
    fixed = [t for t in (0, 1, 2, 3, T // 2, T - 1) if t < T]
    sample = None if T <= 64 else _samples(p, bufs, fixed)
    excluded, worst = residual_parity(p, stream, 3, bufs, sample, g_in=g_in, g_out=g_out)
    print(f"  worst error / tolerance {worst:.3f}")


# --------------------------------------------------------------------------
# FP8 (E4M3) expert weights with per-row scales
# --------------------------------------------------------------------------
def test_fp8_generator_bits_match_cpu():
    _announce("fp8 generator cpu vs gpu")
    wl = synth.WORKLOADS["decode"]
    g = synth.expert_weights_fp8(wl, 5, DEV)
    c = synth.expert_weights_fp8(wl, 5, "cpu")
    for a, b in zip(g, c):
        assert torch.equal(a.cpu(), b)


FP8 = {
    "f8_small": synth.Workload("f8_small", 16, synth.Dims(256, 256, 16, 4, 2, 4), router_sigma=1.0 / 16.0),
    # several column blocks, experts with more than one 8-row pass
    "f8_stream": synth.Workload("f8_stream", 40, synth.Dims(512, 512, 64, 8, 4, 6), router_sigma=0.06),
    # skewed routing: hot experts run many passes
    "f8_skew": synth.Workload("f8_skew", 60, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06, zipf_s=1.2),
    # large activations: h and y travel with power-of-two scales, codes are converted times 2^s
    "f8_big": synth.Workload("f8_big", 40, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06, expert_sigma=10.0),
    # grouped GEMMs with E4M3 weights: about 75 rows per expert (full and ragged tiles), Beam's
    # expert count with one partial tile each, skewed routing just above the stream threshold,
    # and large activations
    "f8_grouped": synth.Workload("f8_grouped", 300, synth.Dims(512, 256, 16, 4, 2, 4), router_sigma=0.06),
    "f8_grouped_e256": synth.Workload("f8_grouped_e256", 1100, synth.Dims(768, 256, 256, 8, 4, 8),
                                      router_sigma=0.04),
    "f8_grouped_skew": synth.Workload("f8_grouped_skew", 1200, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06,
                                      zipf_s=1.2),
    # FP8 stream kernels on wider tiles (16, 32, 64 rows), with skew at 32 and 64
    "f8_stream_r16": synth.Workload("f8_stream_r16", 100, synth.Dims(512, 512, 64, 8, 4, 4), router_sigma=0.06),
    "f8_stream_r32": synth.Workload("f8_stream_r32", 200, synth.Dims(512, 512, 64, 8, 4, 4), router_sigma=0.06),
    "f8_stream_r32_skew": synth.Workload("f8_stream_r32_skew", 200, synth.Dims(512, 512, 64, 8, 4, 4),
                                         router_sigma=0.06, zipf_s=1.2),
    "f8_stream_r64": synth.Workload("f8_stream_r64", 400, synth.Dims(512, 512, 64, 8, 4, 4), router_sigma=0.06),
    "f8_stream_r64_skew": synth.Workload("f8_stream_r64_skew", 400, synth.Dims(512, 512, 64, 8, 4, 4),
                                         router_sigma=0.06, zipf_s=1.2),
    "f8_stream_r64_huge": synth.Workload("f8_stream_r64_huge", 400, synth.Dims(512, 512, 64, 8, 4, 4),
                                         router_sigma=0.06, expert_sigma=200.0),
    "f8_grouped_big": synth.Workload("f8_grouped_big", 900, synth.Dims(512, 512, 16, 4, 2, 4), router_sigma=0.06,
                                     expert_sigma=10.0),
    # huge activations (near 2^24, scales 2^-s with s >= 9): E4M3 values up to 448 times 2^s would
    # pass fp16's range if the down weights carried the scale; the accumulators carry it instead
    "f8_huge": synth.Workload("f8_huge", 40, synth.Dims(512, 256, 64, 8, 4, 4), router_sigma=0.06,
                              expert_sigma=200.0),
    "f8_grouped_huge": synth.Workload("f8_grouped_huge", 900, synth.Dims(512, 512, 16, 4, 2, 4), router_sigma=0.06,
                                      expert_sigma=200.0),
    # merged tails (a last tile of at most 64 rows joins the tile before it) with large activations
    "f8_dense_merged_big": synth.Workload("f8_dense_merged_big", 560, synth.Dims(256, 256, 1, 1, 1, 1),
                                          router_sigma=0.06, expert_sigma=10.0),
    "f8_merged_tails_big": synth.Workload("f8_merged_tails_big", 1200, synth.Dims(512, 256, 8, 2, 1, 2),
                                          router_sigma=0.06, expert_sigma=10.0),
    # merged fifth levels of one fragment and of four (full), on the register-path kernels
    "f8_dense_tail1": synth.Workload("f8_dense_tail1", 261, synth.Dims(256, 256, 1, 1, 1, 1), router_sigma=0.06,
                                     expert_sigma=10.0),
    "f8_dense_tail_full": synth.Workload("f8_dense_tail_full", 320, synth.Dims(256, 256, 1, 1, 1, 1),
                                         router_sigma=0.06, expert_sigma=10.0),
}


# the expert path each FP8 case covers (R of the stream tiles, or 0 for the grouped GEMMs)
FP8_PATH = {"f8_small": 8, "f8_stream": 8, "f8_skew": 8, "f8_big": 8, "f8_huge": 8, "f8_grouped": 0,
            "f8_grouped_e256": 0, "f8_grouped_skew": 0, "f8_grouped_big": 0, "f8_grouped_huge": 0,
            "f8_stream_r16": 16, "f8_stream_r32": 32, "f8_stream_r32_skew": 32, "f8_stream_r64": 64,
            "f8_stream_r64_skew": 64, "f8_stream_r64_huge": 64, "f8_dense_merged_big": 0, "f8_merged_tails_big": 0,
            "f8_dense_tail1": 0, "f8_dense_tail_full": 0}


@pytest.mark.parametrize("name", list(FP8))
def test_forward_fp8(name):
    _announce(f"forward fp8 {name} (all tokens)")
    _expect_path(FP8[name], FP8_PATH[name], fp8=True)
    p = Problem(FP8[name], DEV, fp8=True)
    bufs = binding.beam_moe_forward_fp8(p.dims, p.x, p.wr, p.bias, *p.q)
    excluded, worst = forward_parity(p, bufs)
    print(f"  worst error / tolerance {worst:.3f}")
    out1 = bufs.out.clone()
    binding.beam_moe_forward_fp8(p.dims, p.x, p.wr, p.bias, *p.q, bufs=bufs)
    assert torch.equal(out1, bufs.out)


def test_forward_fp8_routing_matches_bf16_entry():
    # the router does not see the expert weights: both entry points route and dispatch alike
    _announce("fp8 and bf16 entry points route alike")
    wl = FP8["f8_stream"]
    p = Problem(wl, DEV, fp8=True)
    wg, wu, wd = synth.make_experts(wl, DEV)
    b16 = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, wg, wu, wd)
    b8 = binding.beam_moe_forward_fp8(p.dims, p.x, p.wr, p.bias, *p.q)
    for name in ("ids", "w", "counts", "offsets", "slots"):
        assert torch.equal(getattr(b16, name), getattr(b8, name)), name


def test_forward_fp8_rejects_unsupported_intermediate():
    wl = MID["mid_stream"][0]  # intermediate 384: not a whole number of 256-value stages
    d = wl.dims
    x = synth.make_x(wl, DEV)
    wr = synth.make_router(wl, DEV)
    E, I, H = d.num_experts, d.intermediate, d.hidden
    q = (torch.zeros((E, I, H), dtype=torch.uint8, device=DEV), torch.ones((E, I), device=DEV),
         torch.zeros((E, I, H), dtype=torch.uint8, device=DEV), torch.ones((E, I), device=DEV),
         torch.zeros((E, H, I), dtype=torch.uint8, device=DEV), torch.ones((E, H), device=DEV))
    with pytest.raises(binding.BeamMoeError) as ei:
        binding.beam_moe_forward_fp8(d, x, wr, None, *q)
    assert ei.value.status == binding.BEAM_MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("T", [1, 64, 256, 512, 1024, 2048, 4096, 8192, 16384])
def test_forward_fp8_beam(beam_experts_fp8, T):
    _announce(f"forward fp8 Beam T={T}")
    wl = synth.with_tokens(synth.WORKLOADS["decode"], T)
    p = Problem(wl, DEV, experts=beam_experts_fp8, fp8=True)
    bufs = binding.beam_moe_forward_fp8(p.dims, p.x, p.wr, p.bias, *p.q)
    torch.cuda.synchronize()
    # every token of the decode batch and below; tile-aware samples of larger batches
    sample = None if T <= 64 else _samples(p, bufs, (0, 1, T // 3, T // 2, T - 1))
    excluded, worst = forward_parity(p, bufs, sample)
    print(f"  worst error / tolerance {worst:.3f}")
    out1 = bufs.out.clone()
    binding.beam_moe_forward_fp8(p.dims, p.x, p.wr, p.bias, *p.q, bufs=bufs)
    assert torch.equal(out1, bufs.out)


@pytest.mark.parametrize("name", ["f8_stream", "f8_stream_r32", "f8_grouped"])
def test_residual_fp8(name):
    _announce(f"residual fp8 {name} (all tokens)")
    wl = FP8[name]
    p = Problem(wl, DEV, fp8=True)
    stream = synth.make_stream(wl, DEV)
    g_in, g_out = synth.make_norm_weights(wl, DEV)
    bufs = binding.beam_moe_residual_forward_fp8(p.dims, stream, 5, p.wr, p.bias, *p.q, norm_in_weight=g_in,
                                                 norm_out_weight=g_out)
    excluded, worst = residual_parity(p, stream, 5, bufs, g_in=g_in, g_out=g_out)
    print(f"  worst error / tolerance {worst:.3f}")
    new1 = bufs.out.clone()
    inplace = stream.clone()
    binding.beam_moe_residual_forward_fp8(p.dims, inplace, 5, p.wr, p.bias, *p.q, norm_in_weight=g_in,
                                          norm_out_weight=g_out, stream_out=inplace)
    assert torch.equal(inplace, new1)


def test_residual_fp8_beam(beam_experts_fp8):
    _announce("residual fp8 Beam T=64")
    wl = synth.with_tokens(synth.WORKLOADS["decode"], 64)
    p = Problem(wl, DEV, experts=beam_experts_fp8, fp8=True)
    stream = synth.make_stream(wl, DEV)
    bufs = binding.beam_moe_residual_forward_fp8(p.dims, stream, 2, p.wr, p.bias, *p.q)
    torch.cuda.synchronize()
    excluded, worst = residual_parity(p, stream, 2, bufs)
    print(f"  worst error / tolerance {worst:.3f}")


# --------------------------------------------------------------------------
# graph capture: every call is stream-ordered and allocation-free, so a captured
# forward replays to the eager bits (outputs overwritten by eager work in between)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,fp8", [("mid_stream", False), ("mid_tiled", False), ("mid_stream_r64", False),
                                      ("f8_stream", True), ("f8_grouped", True), ("f8_stream_r32", True)])
def test_forward_graph_replay(name, fp8):
    _announce(f"graph replay {name}")
    wl = FP8[name] if fp8 else MID[name][0]
    p = Problem(wl, DEV, fp8=fp8)
    if fp8:
        run = lambda b: binding.beam_moe_forward_fp8(p.dims, p.x, p.wr, p.bias, *p.q, bufs=b)  # noqa: E731
    else:
        run = lambda b: binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd, bufs=b)  # noqa: E731
    names = ("out", "ids", "w", "counts", "offsets", "slots")
    eager = binding.ForwardBuffers(p.dims, wl.tokens, DEV)
    run(eager)
    torch.cuda.synchronize()
    ref = {k: getattr(eager, k).clone() for k in names}
    bufs = binding.ForwardBuffers(p.dims, wl.tokens, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(bufs)
    for i in range(3):
        bufs.out.fill_(float("nan"))
        bufs.ids.fill_(-1)
        bufs.slots.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(getattr(bufs, k), ref[k]), (i, k)


# --------------------------------------------------------------------------
# W_down packed to fp16 once (beam_moe_pack_weights): the same conversion the down kernels apply
# to bf16 weights as they read them, so the packed forward gives the bf16 forward's bits
# --------------------------------------------------------------------------
PACKED = {
    "mid_stream": MID["mid_stream"][0],           # stream kernels, 8-row tiles
    "mid_stream_r64": MID["mid_stream_r64"][0],   # stream kernels, 64-row tiles, two column fragments per wave
    "mid_tiled": MID["mid_tiled"][0],             # grouped GEMMs, full and ragged tiles
    "mid_tiled_huge": MID["mid_tiled_huge"][0],   # accumulator rescaling between activation blocks
    "dense_merged_big": EDGE["dense_merged_big"],  # a merged five-level tile with non-zero scales
    "dense_tail1": EDGE["dense_tail1"],            # a fifth level of one fragment
}


def _packed_equals_bf16(p):
    wdp = binding.beam_moe_pack_weights(p.dims, p.wd)
    ref = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    got = binding.beam_moe_forward_packed(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, wdp)
    torch.cuda.synchronize()
    for k in ("out", "ids", "w", "counts", "offsets", "slots"):
        assert torch.equal(getattr(ref, k), getattr(got, k)), k
    return wdp


@pytest.mark.parametrize("name", list(PACKED))
def test_forward_packed_matches_bf16_bits(name):
    _announce(f"forward packed {name}")
    p = Problem(PACKED[name], DEV)
    wdp = _packed_equals_bf16(p)
    # the packed weights are the bf16 ones, exactly where fp16 represents them
    w32 = p.wd.float()
    normal = w32.abs() >= 2.0 ** -14
    assert torch.equal(wdp.float()[normal], w32[normal])


# 4096: every grouped tile has two or three levels, so packed down runs the three-stage ring
# (three activation stages at two levels, two at three) against bf16 down's two stages
@pytest.mark.parametrize("T", [64, 4096, 16384])
def test_forward_packed_beam(beam_experts, T):
    _announce(f"forward packed Beam T={T}")
    wl = synth.with_tokens(synth.WORKLOADS["decode"], T)
    p = Problem(wl, DEV, experts=beam_experts)
    _packed_equals_bf16(p)
