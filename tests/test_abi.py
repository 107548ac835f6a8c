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
    return sorted(set(re.findall(r"\b(beam_moe_[a-z_]+)\s*\(", text)))


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
    for st in (0, -1, -2, -3, -4):
        assert lib.beam_moe_status_str(st)
    assert b"unknown" in lib.beam_moe_status_str(7)


def test_workspace_bytes():
    n64 = binding.beam_moe_workspace_bytes(BEAM, 64)
    n16k = binding.beam_moe_workspace_bytes(BEAM, 16384)
    assert 0 < n64 < n16k
    # dominated by the fp16 activations h [T*K, I] and expert outputs y [T*K, H]
    assert n16k >= 16384 * 8 * (2560 * 2 + 5120 * 2)
    assert n16k < 16384 * 8 * (2560 * 2 + 5120 * 2) * 1.1
    assert binding.beam_moe_workspace_bytes(TINY, 0) >= 0


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
    assert lib.beam_moe_dispatch(ctypes.byref(cd), 64, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        binding.BEAM_MOE_ERR_WORKSPACE
    assert lib.beam_moe_route(ctypes.byref(cd), 64, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, need - 1,
                              None) == binding.BEAM_MOE_ERR_WORKSPACE


def test_zero_tokens_is_a_no_op():
    lib = binding.load_library()
    cd = binding._cdims(TINY)
    assert lib.beam_moe_forward(ctypes.byref(cd), 0, *([None] * 14), 0, None) == binding.BEAM_MOE_OK
    assert lib.beam_moe_route(ctypes.byref(cd), 0, *([None] * 8), 0, None) == binding.BEAM_MOE_OK
    assert lib.beam_moe_select(ctypes.byref(cd), 0, None, None, None, None, None) == binding.BEAM_MOE_OK
    assert lib.beam_moe_dispatch(ctypes.byref(cd), 0, *([None] * 5), 0, None) == binding.BEAM_MOE_OK
