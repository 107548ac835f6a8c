"""Host-side checks of the GPU parity helpers (CPU only)."""
import numpy as np
import pytest

from grouped_top_routing_fp32_amd import synth
from parity_helpers import Problem


def test_route_oracle_rejects_tokens_outside_the_batch():
    # the helper gathers the sampled rows on the tensors' device; a sample past the batch
    # must fail on the host rather than reach a device-side gather
    p = Problem(synth.with_tokens(synth.WORKLOADS["tiny"], 1), "cpu")
    with pytest.raises(IndexError):
        p.route_oracle([0, 1])
    X, ids, w, C, GS, m = p.route_oracle([0])
    assert X.shape == (1, p.dims.hidden) and ids.shape == (1, p.dims.topk) and np.isfinite(m).all()
