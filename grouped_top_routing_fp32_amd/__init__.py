"""Beam MoE block forward on MI355X (gfx950): group-limited sigmoid router,
counting-sort dispatch, grouped bf16 SwiGLU expert GEMMs and a deterministic
combine, behind the C-ABI library ``libbeam_moe.so``.

The binding is loaded lazily: ``from grouped_top_routing_fp32_amd import
binding`` (or any of the ``beam_moe_*`` names below) loads the built library
and fails loudly when it is missing.
"""

_EXPORTS = ("beam_moe_route", "beam_moe_select", "beam_moe_dispatch", "beam_moe_forward", "beam_moe_forward_fp8",
            "beam_moe_residual_forward", "beam_moe_residual_forward_fp8", "beam_moe_workspace_bytes",
            "beam_moe_status_str", "Dims", "BeamMoeError", "load_library")


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
