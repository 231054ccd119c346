"""MI355X-native int4 routed-expert MoE layer (Flint, fwht128-rotated int4 experts).

    from int4_routed_expert_amd import moe_w4     # the Python binding of libmoe_w4.so
    python -m int4_routed_expert_amd.build        # builds libmoe_w4.so for gfx950

Importing the binding raises ImportError when the library is not built.
"""
