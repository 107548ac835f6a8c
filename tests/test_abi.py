"""The C-ABI library loads, exports every declared symbol and validates its
arguments on the host (no device work: every call here returns before any
launch).  CPU only."""
import ctypes
import os
import re

import pytest

from grouped_top_routing_fp32_amd import binding
from grouped_top_routing_fp32_amd.synth import BEAM, Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")

TINY = Dims(256, 128, 16, 4, 2, 4, 2.5)
FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: validation fails or T == 0 first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_symbols_are_plain_c():
    # nm shows the exported names unmangled
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared_functions():
        assert name in names, name


def test_status_strings():
    lib = binding.load_library()
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.beam_moe_status_str(st)
    assert b"unknown" in lib.beam_moe_status_str(7)


def test_workspace_bytes():
    n64 = binding.beam_moe_workspace_bytes(BEAM, 64)
    n16k = binding.beam_moe_workspace_bytes(BEAM, 16384)
    assert 0 < n64 < n16k
    # dominated by the fp16 activations h [T*K, I] and expert outputs y [T*K, H], plus the bf16 input x [T, H]
    per_token = 8 * (2560 * 2 + 5120 * 2) + 5120 * 2
    assert n16k >= 16384 * per_token
    assert n16k < 16384 * per_token * 1.1
    assert binding.beam_moe_workspace_bytes(TINY, 0) >= 0


@pytest.mark.parametrize("T", [1, 64, 4096, 16384, 262144])
def test_route_and_dispatch_workspace_sizes(T):
    """Route and dispatch need only their own scratch (split-K partial logits, unit
    histograms), and the forward workspace is always enough for either."""
    full = binding.beam_moe_workspace_bytes(BEAM, T)
    route = binding.beam_moe_route_workspace_bytes(BEAM, T)
    disp = binding.beam_moe_dispatch_workspace_bytes(BEAM, T)
    E, K = BEAM.num_experts, BEAM.topk
    assert T * E * 4 <= route <= 16 * T * E * 4 and route <= full
    assert disp == -(-T * K // 1024) * E * 4 and disp <= full
    if T >= 4096:
        # one split per token tile: T * E * 4 bytes, far below the forward's ~132 KB per token
        assert route == T * E * 4 and route * 100 < full


def test_stream_rows_rule():
    """The expert path the library reports: stream tiles of R rows (the smallest of 8 .. 64 at
    least twice the average rows per expert), else 0."""
    got = {T: (binding.beam_moe_stream_rows(BEAM, T), binding.beam_moe_stream_rows(BEAM, T, True))
           for T in (1, 64, 128, 129, 256, 257, 512, 1024, 1025, 2048, 2049, 16384)}
    assert got == {1: (8, 8), 64: (8, 8), 128: (8, 8), 129: (16, 16), 256: (16, 16), 257: (32, 32), 512: (32, 32),
                   1024: (64, 64), 1025: (0, 0), 2048: (0, 0), 2049: (0, 0), 16384: (0, 0)}
    lib = binding.load_library()
    bad = binding._cdims(Dims(5120, 2560, 256, 7, 4, 8))
    assert lib.beam_moe_stream_rows(ctypes.byref(bad), 64, 0) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert lib.beam_moe_stream_rows(ctypes.byref(binding._cdims(BEAM)), -1, 0) == binding.BEAM_MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("K", [1, 8])
def test_routed_pair_limit(K):
    """T * K <= 2^28 is accepted; one token more is UNSUPPORTED before any pointer is read."""
    lib = binding.load_library()
    cd = binding._cdims(Dims(256, 128, 16, 4, 2, K))
    T = (1 << 28) // K
    for fn in (lib.beam_moe_workspace_bytes, lib.beam_moe_route_workspace_bytes,
               lib.beam_moe_dispatch_workspace_bytes):
        assert fn(ctypes.byref(cd), T) != binding.SIZE_MAX
        assert fn(ctypes.byref(cd), T + 1) == binding.SIZE_MAX
    # at the limit validation reaches the pointers (NULL x: INVALID_ARG); past it, dims fail first
    args = [None] + [FAKE] * 13
    assert lib.beam_moe_forward(ctypes.byref(cd), T, *args, 1 << 40, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_forward(ctypes.byref(cd), T + 1, *args, 1 << 40, None) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert lib.beam_moe_dispatch(ctypes.byref(cd), T, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == \
        binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_dispatch(ctypes.byref(cd), T + 1, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == \
        binding.BEAM_MOE_ERR_UNSUPPORTED
    assert lib.beam_moe_select(ctypes.byref(cd), T + 1, FAKE, None, FAKE, FAKE, None) == \
        binding.BEAM_MOE_ERR_UNSUPPORTED
    assert lib.beam_moe_route(ctypes.byref(cd), T + 1, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, 1 << 40,
                              None) == binding.BEAM_MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("bad", [
    Dims(5120, 2560, 256, 7, 4, 8),      # E % G != 0
    Dims(5120, 2560, 512, 8, 4, 8),      # E > 256
    Dims(5120, 2560, 256, 8, 9, 8),      # TG > G
    Dims(5120, 2560, 256, 8, 1, 33),     # K > candidates
    Dims(5120, 2560, 256, 8, 4, 17),     # K > 16
    Dims(5000, 2560, 256, 8, 4, 8),      # H % 256
    Dims(5120, 2500, 256, 8, 4, 8),      # I % 128
    Dims(5120, 2560, 256, 8, 4, 0),      # K = 0
    Dims(5120, 2560, 256, 8, 4, 8, float("inf")),
])
def test_unsupported_dims(bad):
    lib = binding.load_library()
    cd = binding._cdims(bad)
    assert lib.beam_moe_workspace_bytes(ctypes.byref(cd), 64) == binding.SIZE_MAX
    st = lib.beam_moe_forward(ctypes.byref(cd), 64, *([FAKE] * 14), 1 << 40, None)
    assert st == binding.BEAM_MOE_ERR_UNSUPPORTED
    st = lib.beam_moe_select(ctypes.byref(cd), 64, FAKE, None, FAKE, FAKE, None)
    assert st == binding.BEAM_MOE_ERR_UNSUPPORTED


def test_invalid_arguments_rejected_before_launch():
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    ok = [FAKE] * 14
    # negative T
    assert lib.beam_moe_forward(ctypes.byref(cd), -1, *ok, 1 << 40, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    # each required pointer of forward: NULL and misaligned
    required = [0, 1, 4, 5, 6, 7, 8, 9, 10, 11, 12]  # x, w_router, gate, up, down, out, ids, w, counts, offsets, slots
    for i in required:
        args = list(ok)
        args[i] = None
        assert lib.beam_moe_forward(ctypes.byref(cd), 64, *args, 1 << 40, None) == binding.BEAM_MOE_ERR_INVALID_ARG
        args[i] = ctypes.c_void_p((1 << 20) + 8)
        assert lib.beam_moe_forward(ctypes.byref(cd), 64, *args, 1 << 40, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    # the optional biases may be NULL but not misaligned
    for i in (2, 3):
        args = list(ok)
        args[i] = ctypes.c_void_p((1 << 20) + 4)
        assert lib.beam_moe_forward(ctypes.byref(cd), 64, *args, 1 << 40, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_select(ctypes.byref(cd), 4, FAKE, ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, None) == \
        binding.BEAM_MOE_ERR_INVALID_ARG
    # select / dispatch / route null pointers
    assert lib.beam_moe_select(ctypes.byref(cd), 4, None, None, FAKE, FAKE, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_dispatch(ctypes.byref(cd), 4, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == \
        binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_route(ctypes.byref(cd), 4, None, FAKE, None, None, FAKE, FAKE, None, FAKE, 1 << 40, None) == \
        binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_forward(None, 4, *ok, 1 << 40, None) == binding.BEAM_MOE_ERR_INVALID_ARG


def test_short_or_missing_workspace_rejected():
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    need = lib.beam_moe_workspace_bytes(ctypes.byref(cd), 64)
    ok = [FAKE] * 14
    assert lib.beam_moe_forward(ctypes.byref(cd), 64, *ok, need - 1, None) == binding.BEAM_MOE_ERR_WORKSPACE
    args = list(ok)
    args[13] = None
    assert lib.beam_moe_forward(ctypes.byref(cd), 64, *args, need, None) == binding.BEAM_MOE_ERR_WORKSPACE
    need_d = lib.beam_moe_dispatch_workspace_bytes(ctypes.byref(cd), 64)
    need_r = lib.beam_moe_route_workspace_bytes(ctypes.byref(cd), 64)
    assert lib.beam_moe_dispatch(ctypes.byref(cd), 64, FAKE, FAKE, FAKE, FAKE, FAKE, need_d - 1, None) == \
        binding.BEAM_MOE_ERR_WORKSPACE
    assert lib.beam_moe_dispatch(ctypes.byref(cd), 64, FAKE, FAKE, FAKE, FAKE, None, need_d, None) == \
        binding.BEAM_MOE_ERR_WORKSPACE
    assert lib.beam_moe_route(ctypes.byref(cd), 64, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, need_r - 1,
                              None) == binding.BEAM_MOE_ERR_WORKSPACE
    assert lib.beam_moe_route(ctypes.byref(cd), 64, FAKE, FAKE, None, None, FAKE, FAKE, None, None, need_r,
                              None) == binding.BEAM_MOE_ERR_WORKSPACE


def test_zero_tokens_is_a_no_op():
    lib = binding.load_library()
    cd = binding._cdims(TINY)
    assert lib.beam_moe_forward(ctypes.byref(cd), 0, *([None] * 14), 0, None) == binding.BEAM_MOE_OK
    assert lib.beam_moe_route(ctypes.byref(cd), 0, *([None] * 8), 0, None) == binding.BEAM_MOE_OK
    assert lib.beam_moe_select(ctypes.byref(cd), 0, None, None, None, None, None) == binding.BEAM_MOE_OK
    assert lib.beam_moe_dispatch(ctypes.byref(cd), 0, *([None] * 5), 0, None) == binding.BEAM_MOE_OK


def _residual(lib, cd, T, step=2, eps=1e-6, ptrs=None, ws_bytes=1 << 40):
    # dims, T, stream_in, step, g_in, g_out, eps, w_router, logit_bias, select_bias, gate, up, down,
    # stream_out, ids, w, counts, offsets, slots, ws, ws_bytes, stream
    p = ptrs if ptrs is not None else {}
    g = lambda k, dflt=FAKE: p.get(k, dflt)  # noqa: E731
    return lib.beam_moe_residual_forward(ctypes.byref(cd), T, g("stream_in"), step, g("g_in", None),
                                         g("g_out", None), eps, g("w_router"), g("logit_bias", None),
                                         g("select_bias", None), g("gate"), g("up"), g("down"), g("stream_out"),
                                         g("ids"), g("w"), g("counts"), g("offsets"), g("slots"), g("ws"), ws_bytes,
                                         None)


def test_residual_forward_validation():
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    assert _residual(lib, cd, 64, step=1) == binding.BEAM_MOE_ERR_INVALID_ARG       # step 1 is the embedding
    assert _residual(lib, cd, 64, eps=-1.0) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert _residual(lib, cd, 64, eps=float("nan")) == binding.BEAM_MOE_ERR_INVALID_ARG
    for name in ("stream_in", "w_router", "gate", "up", "down", "stream_out", "ids", "w", "counts", "offsets",
                 "slots"):
        assert _residual(lib, cd, 64, ptrs={name: None}) == binding.BEAM_MOE_ERR_INVALID_ARG, name
    for name in ("g_in", "g_out", "logit_bias", "select_bias"):
        assert _residual(lib, cd, 64, ptrs={name: ctypes.c_void_p((1 << 20) + 4)}) == \
            binding.BEAM_MOE_ERR_INVALID_ARG, name
    need = lib.beam_moe_workspace_bytes(ctypes.byref(cd), 64)
    assert _residual(lib, cd, 64, ws_bytes=need - 1) == binding.BEAM_MOE_ERR_WORKSPACE
    wide = binding._cdims(Dims(8448, 2560, 256, 8, 4, 8))   # H > 8192
    assert _residual(lib, wide, 64) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert _residual(lib, binding._cdims(TINY), 0, ptrs={k: None for k in ("stream_in", "w_router", "gate", "up",
                     "down", "stream_out", "ids", "w", "counts", "offsets", "slots", "ws")}, ws_bytes=0) == \
        binding.BEAM_MOE_OK


_FP8_PTRS = ("x", "w_router", "logit_bias", "select_bias", "q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down",
             "out", "ids", "w", "counts", "offsets", "slots", "ws")
_FP8_OPTIONAL = ("logit_bias", "select_bias")


def _fp8(lib, cd, T, ptrs=None, ws_bytes=1 << 40):
    p = ptrs if ptrs is not None else {}
    args = [p.get(k, None if k in _FP8_OPTIONAL else FAKE) for k in _FP8_PTRS]
    return lib.beam_moe_forward_fp8(ctypes.byref(cd), T, *args[:16], args[16], ws_bytes, None)


def test_forward_fp8_validation():
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    for name in _FP8_PTRS[:-1]:
        if name in _FP8_OPTIONAL:
            assert _fp8(lib, cd, 64, ptrs={name: ctypes.c_void_p((1 << 20) + 4)}) == \
                binding.BEAM_MOE_ERR_INVALID_ARG, name
        else:
            assert _fp8(lib, cd, 64, ptrs={name: None}) == binding.BEAM_MOE_ERR_INVALID_ARG, name
            assert _fp8(lib, cd, 64, ptrs={name: ctypes.c_void_p((1 << 20) + 8)}) == \
                binding.BEAM_MOE_ERR_INVALID_ARG, name
    assert _fp8(lib, cd, 64, ws_bytes=1) == binding.BEAM_MOE_ERR_WORKSPACE
    assert _fp8(lib, cd, 64, ptrs={"ws": None}) == binding.BEAM_MOE_ERR_WORKSPACE
    # K of each projection must be whole 256-value stages
    assert _fp8(lib, binding._cdims(Dims(5120, 2432, 256, 8, 4, 8)), 64) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert _fp8(lib, binding._cdims(Dims(256, 128, 16, 4, 2, 4)), 64) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert _fp8(lib, cd, -1) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert _fp8(lib, cd, 0, ptrs={k: None for k in _FP8_PTRS}, ws_bytes=0) == binding.BEAM_MOE_OK


_RES8_PTRS = ("stream_in", "g_in", "g_out", "w_router", "logit_bias", "select_bias", "q_gate", "s_gate", "q_up",
              "s_up", "q_down", "s_down", "stream_out", "ids", "w", "counts", "offsets", "slots", "ws")
_RES8_OPTIONAL = ("g_in", "g_out", "logit_bias", "select_bias")


def _res8(lib, cd, T, step=2, eps=1e-6, ptrs=None, ws_bytes=1 << 40):
    p = ptrs if ptrs is not None else {}
    v = {k: p.get(k, None if k in _RES8_OPTIONAL else FAKE) for k in _RES8_PTRS}
    return lib.beam_moe_residual_forward_fp8(ctypes.byref(cd), T, v["stream_in"], step, v["g_in"], v["g_out"], eps,
                                             *[v[k] for k in _RES8_PTRS[3:]], ws_bytes, None)


def test_residual_forward_fp8_validation():
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    assert _res8(lib, cd, 64, step=1) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert _res8(lib, cd, 64, eps=float("inf")) == binding.BEAM_MOE_ERR_INVALID_ARG
    for name in _RES8_PTRS[:-1]:
        if name in _RES8_OPTIONAL:
            assert _res8(lib, cd, 64, ptrs={name: ctypes.c_void_p((1 << 20) + 4)}) == \
                binding.BEAM_MOE_ERR_INVALID_ARG, name
        else:
            assert _res8(lib, cd, 64, ptrs={name: None}) == binding.BEAM_MOE_ERR_INVALID_ARG, name
    assert _res8(lib, cd, 64, ws_bytes=1) == binding.BEAM_MOE_ERR_WORKSPACE
    assert _res8(lib, binding._cdims(Dims(5120, 2432, 256, 8, 4, 8)), 64) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert _res8(lib, binding._cdims(Dims(8448, 2560, 256, 8, 4, 8)), 64) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert _res8(lib, cd, 0, ptrs={k: None for k in _RES8_PTRS}, ws_bytes=0) == binding.BEAM_MOE_OK


def test_forward_noalloc_validation():
    """Every rejection returns before any device call (no GPU is touched here)."""
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    ok = [FAKE] * 13
    assert lib.beam_moe_workspace_bytes(ctypes.byref(cd), 472) > binding.SCRATCH_BYTES
    assert lib.beam_moe_forward_noalloc(ctypes.byref(cd), 472, *ok, None) == binding.BEAM_MOE_ERR_SCRATCH
    assert lib.beam_moe_forward_noalloc(ctypes.byref(cd), 1 << 20, *ok, None) == binding.BEAM_MOE_ERR_SCRATCH
    for i in range(13):
        if i in (2, 3):   # the optional biases: NULL allowed, misaligned not
            args = list(ok)
            args[i] = ctypes.c_void_p((1 << 20) + 4)
        else:
            args = list(ok)
            args[i] = None
        assert lib.beam_moe_forward_noalloc(ctypes.byref(cd), 64, *args, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_forward_noalloc(ctypes.byref(cd), -1, *ok, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    bad = binding._cdims(Dims(5120, 2560, 256, 7, 4, 8))
    assert lib.beam_moe_forward_noalloc(ctypes.byref(bad), 64, *ok, None) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert lib.beam_moe_forward_noalloc(ctypes.byref(cd), 0, *([None] * 13), None) == binding.BEAM_MOE_OK


def test_pack_and_forward_packed_validation():
    """Rejections of the packed entry points return before any device call."""
    lib = binding.load_library()
    cd = binding._cdims(BEAM)
    other = ctypes.c_void_p(2 << 20)
    assert lib.beam_moe_pack_weights(ctypes.byref(cd), None, FAKE, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_pack_weights(ctypes.byref(cd), FAKE, None, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_pack_weights(ctypes.byref(cd), FAKE, ctypes.c_void_p((2 << 20) + 8), None) == \
        binding.BEAM_MOE_ERR_INVALID_ARG
    assert lib.beam_moe_pack_weights(ctypes.byref(cd), FAKE, FAKE, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    bad = binding._cdims(Dims(5120, 2560, 256, 7, 4, 8))
    assert lib.beam_moe_pack_weights(ctypes.byref(bad), FAKE, other, None) == binding.BEAM_MOE_ERR_UNSUPPORTED
    assert lib.beam_moe_pack_weights(None, FAKE, other, None) == binding.BEAM_MOE_ERR_INVALID_ARG
    ok = [FAKE] * 14
    for i in (0, 1, 4, 5, 6, 7, 8, 9, 10, 11, 12):
        args = list(ok)
        args[i] = None
        assert lib.beam_moe_forward_packed(ctypes.byref(cd), 64, *args, 1 << 40, None) == \
            binding.BEAM_MOE_ERR_INVALID_ARG
    need = lib.beam_moe_workspace_bytes(ctypes.byref(cd), 64)
    assert lib.beam_moe_forward_packed(ctypes.byref(cd), 64, *ok, need - 1, None) == binding.BEAM_MOE_ERR_WORKSPACE
    assert lib.beam_moe_forward_packed(ctypes.byref(cd), 0, *([None] * 14), 0, None) == binding.BEAM_MOE_OK
