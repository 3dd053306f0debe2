"""MI355X-native forward pass of the Step-3.5-Flash sparse MoE FFN layer.

The compute path is the C-ABI library `libsmoe_gfx950.so` (hand-written HIP
kernels for gfx950); `binding` marshals torch device tensors into it.
"""
__all__ = ["binding", "inputs"]
