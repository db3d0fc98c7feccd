"""MI355X-native single-token routed-expert MoE decode layer (HIP, gfx950).

The compute path is the C-ABI library ``libmoe_decode.so`` built from
``csrc/``; the Python functions exported here only marshal tensors into it.
"""
