"""Seeded synthetic inputs for the Beam MoE block.

This module is shared by both sides of every parity check: the FP64 oracle
and the HIP path receive tensors generated here and nothing else.  It holds
none of the block's arithmetic (no routing, no GEMM, no SwiGLU); it only
draws numbers.

Generator.  Every tensor element is a pure function of
(seed, tensor id, expert, flat element index), so any slice (a few token rows,
one expert) can be regenerated on its own, on the CPU or on the GPU, with
identical bits:

* the counter is hashed to 32 bits with two rounds of the MurmurHash3 32-bit
  finaliser ("fmix32", Austin Appleby), keyed by the stream;
* the top 16 bits select one of 65,536 equiprobable atoms of a discretised
  standard normal (the quantiles Phi^-1((j + 1/2) / 65536), mirrored so the
  table is exactly symmetric and rescaled so its variance is exactly 1);
* the atom is multiplied by sigma in FP32 and, for bf16 tensors, rounded to
  bfloat16 with round-to-nearest-even.

Only integer operations, a table lookup, one IEEE FP32 multiply and an RNE
conversion are involved, so torch on the CPU and torch on the GPU produce the
same bits (a GPU test checks this).  The normal law is the one the Beam MoE
workloads are stated in (x ~ N(0,1), router ~ N(0, 1/sqrt(H)),
experts ~ N(0, 0.02), second argument a standard deviation); the 16-bit
discretisation is finer than the bf16 grid the values are rounded to, and
truncates the tails at about 4.3 sigma.

Tensor ids: x = 0, router weight = 1, gate = 2, up = 3, down = 4,
bias permutation = 5.
"""
from __future__ import annotations

import dataclasses
import math
import statistics
from typing import Optional

import numpy as np
import torch

M32 = 0xFFFFFFFF

(TENSOR_X, TENSOR_ROUTER, TENSOR_GATE, TENSOR_UP, TENSOR_DOWN, TENSOR_PERM, TENSOR_STREAM, TENSOR_NORM,
 TENSOR_GATE_SCALE, TENSOR_UP_SCALE, TENSOR_DOWN_SCALE) = range(11)


# --------------------------------------------------------------------------
# counter-based hash (MurmurHash3 fmix32), exact in int64 on CPU and GPU
# --------------------------------------------------------------------------
def _fmix32_int(h: int) -> int:
    h &= M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & M32
    h ^= h >> 16
    return h


def _mul32(h: torch.Tensor, c: int) -> torch.Tensor:
    """(h * c) mod 2**32 for 0 <= h < 2**32, without int64 overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (h * lo + ((h * hi) & 0xFFFF) * 65536) & M32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def stream_keys(seed: int, tensor_id: int, expert: int = 0) -> tuple[int, int]:
    k0 = _fmix32_int((seed * 0x9E3779B1 + tensor_id * 0x85EBCA77 + expert * 0xC2B2AE3D + 0x27D4EB2F) & M32)
    k1 = _fmix32_int(k0 ^ 0x165667B1 ^ ((expert * 0x27D4EB2F + tensor_id) & M32))
    return k0, k1


def hash32(counter: torch.Tensor, keys: tuple[int, int]) -> torch.Tensor:
    """32-bit hash of int64 counters in [0, 2**32)."""
    k0, k1 = keys
    return _fmix32(_fmix32(counter ^ k0) ^ k1)


# --------------------------------------------------------------------------
# discretised standard normal
# --------------------------------------------------------------------------
_TABLE_CACHE: dict = {}


def normal_table(device="cpu") -> torch.Tensor:
    dev = torch.device(device)
    key = str(dev)
    if key not in _TABLE_CACHE:
        if "cpu" not in _TABLE_CACHE:
            nd = statistics.NormalDist()
            half = np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(32768)], dtype=np.float64)
            q = np.concatenate([half, -half[::-1]])
            q = q / math.sqrt(float(np.mean(q * q)))
            _TABLE_CACHE["cpu"] = torch.from_numpy(q.astype(np.float32))
        _TABLE_CACHE[key] = _TABLE_CACHE["cpu"].to(dev)
    return _TABLE_CACHE[key]


def normal_at(counter: torch.Tensor, keys: tuple[int, int], sigma: float,
              dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Values of one stream at the given int64 counters (any shape)."""
    u = hash32(counter, keys)
    z = normal_table(counter.device)[(u >> 16)]
    v = z * torch.tensor(sigma, dtype=torch.float32, device=counter.device)
    return v if dtype == torch.float32 else v.to(dtype)


def normal(shape, sigma: float, seed: int, tensor_id: int, expert: int = 0,
           dtype: torch.dtype = torch.float32, device="cpu",
           out: Optional[torch.Tensor] = None, chunk: int = 1 << 24) -> torch.Tensor:
    """A whole tensor of one stream, element (i0, i1, ...) at its row-major flat index."""
    n = int(np.prod(shape)) if len(shape) else 1
    if n >= (1 << 32):
        raise ValueError("a single stream holds at most 2**32 elements")
    keys = stream_keys(seed, tensor_id, expert)
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(s, e, dtype=torch.int64, device=flat.device)
        flat[s:e] = normal_at(idx, keys, sigma, dtype)
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    intermediate: int
    num_experts: int
    num_groups: int
    topk_groups: int
    topk: int
    routed_scaling: float = 2.5


BEAM = Dims(hidden=5120, intermediate=2560, num_experts=256, num_groups=8, topk_groups=4, topk=8,
            routed_scaling=2.5)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    dims: Dims
    x_sigma: float = 1.0
    router_sigma: Optional[float] = None     # default 1/sqrt(hidden)
    expert_sigma: float = 0.02
    zipf_s: Optional[float] = None           # per-expert router-logit bias when set
    seed: int = 0
    router_only: bool = False

    @property
    def wr_sigma(self) -> float:
        return self.router_sigma if self.router_sigma is not None else 1.0 / math.sqrt(self.dims.hidden)


WORKLOADS = {
    # oracle bring-up: 16 experts in 4 groups of 4, keep 2 groups, pick 4
    "tiny": Workload("tiny", 16, Dims(256, 128, 16, 4, 2, 4, 2.5), router_sigma=1.0 / 16.0),
    # router + dispatch only at Beam scale
    "router_dispatch": Workload("router_dispatch", 4096, BEAM, router_only=True),
    # full layer, decode-sized and prefill-sized batches
    "decode": Workload("decode", 64, BEAM),
    "prefill": Workload("prefill", 16384, BEAM),
    # full layer with a Zipf(1.2) router-logit bias over a seeded expert permutation
    "skewed": Workload("skewed", 8192, BEAM, zipf_s=1.2),
}


def with_tokens(wl: Workload, tokens: int) -> Workload:
    return dataclasses.replace(wl, tokens=tokens)


def x_rows(wl: Workload, rows, device="cpu") -> torch.Tensor:
    """bf16 hidden states x[rows, :] of the workload (rows: iterable of token indices)."""
    H = wl.dims.hidden
    r = torch.as_tensor(list(rows) if not torch.is_tensor(rows) else rows, dtype=torch.int64, device=device)
    idx = r[:, None] * H + torch.arange(H, dtype=torch.int64, device=device)[None, :]
    return normal_at(idx, stream_keys(wl.seed, TENSOR_X), wl.x_sigma, torch.bfloat16)


def make_x(wl: Workload, device="cpu") -> torch.Tensor:
    return normal((wl.tokens, wl.dims.hidden), wl.x_sigma, wl.seed, TENSOR_X, dtype=torch.bfloat16, device=device)


def make_stream(wl: Workload, device="cpu") -> torch.Tensor:
    """fp32 residual stream [T, H]: unit normals, token t scaled by 2^((t mod 7) - 3) so
    that the token RMS spans 1/8 .. 8 (exact scaling, powers of two)."""
    T, H = wl.tokens, wl.dims.hidden
    z = normal((T, H), 1.0, wl.seed, TENSOR_STREAM, dtype=torch.float32, device=device)
    e = (torch.arange(T, dtype=torch.int64, device=device) % 7 - 3).to(torch.float32)
    return z * torch.exp2(e)[:, None]


def make_norm_weights(wl: Workload, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """fp32 norm weights (g_in, g_out) [H] each: 1 + N(0, 0.1^2)."""
    H = wl.dims.hidden
    g = normal((2, H), 0.1, wl.seed, TENSOR_NORM, dtype=torch.float32, device=device) + 1.0
    return g[0].contiguous(), g[1].contiguous()


def make_router(wl: Workload, device="cpu") -> torch.Tensor:
    d = wl.dims
    return normal((d.num_experts, d.hidden), wl.wr_sigma, wl.seed, TENSOR_ROUTER, dtype=torch.float32, device=device)


def zipf_bias(wl: Workload) -> Optional[np.ndarray]:
    """b[pi(r)] = ln(E * p_r), p_r = r^-s / sum_r' r'^-s, r = 1..E, pi a seeded permutation (fp32)."""
    if wl.zipf_s is None:
        return None
    E = wl.dims.num_experts
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-wl.zipf_s)
    p /= p.sum()
    vals = np.log(E * p)
    keys = hash32(torch.arange(E, dtype=torch.int64), stream_keys(wl.seed, TENSOR_PERM)).numpy()
    perm = np.lexsort((np.arange(E), keys))         # pi(r) = perm[r-1]
    b = np.zeros(E, dtype=np.float64)
    b[perm] = vals
    return b.astype(np.float32)


def make_bias(wl: Workload, device="cpu") -> Optional[torch.Tensor]:
    b = zipf_bias(wl)
    return None if b is None else torch.from_numpy(b).to(device)


def expert_weights(wl: Workload, e: int, device="cpu"):
    """(W_gate[e] [I,H], W_up[e] [I,H], W_down[e] [H,I]) in bf16, Linear [out, in] layout."""
    d = wl.dims
    s = wl.expert_sigma
    wg = normal((d.intermediate, d.hidden), s, wl.seed, TENSOR_GATE, e, torch.bfloat16, device)
    wu = normal((d.intermediate, d.hidden), s, wl.seed, TENSOR_UP, e, torch.bfloat16, device)
    wd = normal((d.hidden, d.intermediate), s, wl.seed, TENSOR_DOWN, e, torch.bfloat16, device)
    return wg, wu, wd


def make_experts(wl: Workload, device="cpu", experts=None):
    """Stacked bf16 expert weights [E,I,H], [E,I,H], [E,H,I], generated expert by expert in place."""
    d = wl.dims
    E, I, H = d.num_experts, d.intermediate, d.hidden
    wg = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
    wu = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
    wd = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
    s = wl.expert_sigma
    for e in (range(E) if experts is None else experts):
        normal((I, H), s, wl.seed, TENSOR_GATE, e, torch.bfloat16, out=wg[e])
        normal((I, H), s, wl.seed, TENSOR_UP, e, torch.bfloat16, out=wu[e])
        normal((H, I), s, wl.seed, TENSOR_DOWN, e, torch.bfloat16, out=wd[e])
    return wg, wu, wd


# --------------------------------------------------------------------------
# FP8 (E4M3) expert weights: codes and one fp32 scale per output row
# --------------------------------------------------------------------------
FP8_CODE_SIGMA = 100.0  # codes ~ N(0, 100^2) rounded to E4M3; the table's tails (|z| < 4.4) stay below 448


def fp8_codes(shape, seed: int, tensor_id: int, expert: int, device="cpu", out=None) -> torch.Tensor:
    """uint8 E4M3 codes: unit normals times FP8_CODE_SIGMA (fp32), rounded by torch's float8_e4m3fn cast."""
    z = normal(shape, FP8_CODE_SIGMA, seed, tensor_id, expert, torch.float32, device)
    q = z.to(torch.float8_e4m3fn).view(torch.uint8)
    if out is None:
        return q
    out.copy_(q)
    return out


def fp8_scales(n: int, sigma: float, seed: int, tensor_id: int, expert: int, device="cpu") -> torch.Tensor:
    """fp32 per-row scales (sigma / FP8_CODE_SIGMA) * (1 + 0.2 z), z a unit normal (|z| < 4.4: positive)."""
    z = normal((n,), 1.0, seed, tensor_id, expert, torch.float32, device)
    f32 = lambda v: torch.tensor(v, dtype=torch.float32, device=z.device)  # noqa: E731
    return (z * f32(0.2) + f32(1.0)) * f32(sigma / FP8_CODE_SIGMA)


def expert_weights_fp8(wl: Workload, e: int, device="cpu"):
    """(q_gate [I,H], s_gate [I], q_up [I,H], s_up [I], q_down [H,I], s_down [H]) of expert e;
    dequantised rows have standard deviation about expert_sigma."""
    d = wl.dims
    s = wl.expert_sigma
    I, H = d.intermediate, d.hidden
    return (fp8_codes((I, H), wl.seed, TENSOR_GATE, e, device), fp8_scales(I, s, wl.seed, TENSOR_GATE_SCALE, e, device),
            fp8_codes((I, H), wl.seed, TENSOR_UP, e, device), fp8_scales(I, s, wl.seed, TENSOR_UP_SCALE, e, device),
            fp8_codes((H, I), wl.seed, TENSOR_DOWN, e, device), fp8_scales(H, s, wl.seed, TENSOR_DOWN_SCALE, e, device))


def make_experts_fp8(wl: Workload, device="cpu"):
    """Stacked FP8 experts: codes [E,I,H], [E,I,H], [E,H,I] (uint8) and scales [E,I], [E,I], [E,H] (fp32)."""
    d = wl.dims
    E, I, H = d.num_experts, d.intermediate, d.hidden
    qg = torch.empty((E, I, H), dtype=torch.uint8, device=device)
    qu = torch.empty((E, I, H), dtype=torch.uint8, device=device)
    qd = torch.empty((E, H, I), dtype=torch.uint8, device=device)
    sg = torch.empty((E, I), dtype=torch.float32, device=device)
    su = torch.empty((E, I), dtype=torch.float32, device=device)
    sd = torch.empty((E, H), dtype=torch.float32, device=device)
    s = wl.expert_sigma
    for e in range(E):
        fp8_codes((I, H), wl.seed, TENSOR_GATE, e, device, out=qg[e])
        fp8_codes((I, H), wl.seed, TENSOR_UP, e, device, out=qu[e])
        fp8_codes((H, I), wl.seed, TENSOR_DOWN, e, device, out=qd[e])
        sg[e] = fp8_scales(I, s, wl.seed, TENSOR_GATE_SCALE, e, device)
        su[e] = fp8_scales(I, s, wl.seed, TENSOR_UP_SCALE, e, device)
        sd[e] = fp8_scales(H, s, wl.seed, TENSOR_DOWN_SCALE, e, device)
    return qg, sg, qu, su, qd, sd
