"""GPU: beam_moe_forward_noalloc (scratch in the library's static device array)
against beam_moe_forward (caller workspace) on the same inputs: every output
bit for bit, over consecutive calls whose second batch is smaller than the
first, so that nothing a call reads can come from what an earlier call left in
the shared scratch."""
import pytest
import torch

from grouped_top_routing_fp32_amd import binding, synth
from parity_helpers import Problem

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("out", "ids", "w", "counts", "offsets", "slots")

# grouped GEMMs (about 225 rows per expert), then the stream kernels (few rows per expert)
GROUPED = synth.Workload("noalloc_grouped", 900, synth.Dims(512, 384, 16, 4, 2, 4), router_sigma=0.06)
STREAM = synth.Workload("noalloc_stream", 40, synth.Dims(512, 384, 64, 8, 4, 6), router_sigma=0.06)


def _announce(name):
    print(f"\n[case] {name}", flush=True)


def _same_as_forward(p):
    ref = binding.beam_moe_forward(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    got = binding.beam_moe_forward_noalloc(p.dims, p.x, p.wr, p.bias, p.wg, p.wu, p.wd)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(getattr(ref, k), getattr(got, k)), k


def test_noalloc_matches_forward_then_smaller_batch():
    _announce("noalloc: grouped T=900, then stream T=40, then grouped again")
    big = Problem(GROUPED, DEV)
    small = Problem(STREAM, DEV)
    _same_as_forward(big)
    _same_as_forward(small)
    _same_as_forward(big)


def test_noalloc_beam_decode_then_smaller_batch():
    _announce("noalloc: Beam T=64, then T=8")
    experts = synth.make_experts(synth.WORKLOADS["decode"], DEV)
    for T in (64, 8):
        p = Problem(synth.with_tokens(synth.WORKLOADS["decode"], T), DEV, experts=experts)
        _same_as_forward(p)
