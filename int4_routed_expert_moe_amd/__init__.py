"""MI355X-native int4 routed-expert MoE layer.

The compute path is the C-ABI library ``libmoe_int4.so`` (hand-written HIP for
gfx950, declared in ``include/moe_int4.h``); ``int4_routed_expert_moe_amd.moe``
is its thin Python binding and ``int4_routed_expert_moe_amd.layer`` composes the
calls into one layer forward.  Importing this package loads nothing; importing
the binding loads the library and fails loudly when it is not built.
"""
__all__ = ["synthetic"]
