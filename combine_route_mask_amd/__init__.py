"""MI355X (gfx950) MoE expert-parallel dispatch / combine exchange.

The exchange runs in hand-written HIP kernels behind the C ABI of
``include/moe_ep.h`` (``libmoe_ep.so``); ``combine_route_mask_amd.moe_ep``
is its thin Python binding.  Build with ``combine_route_mask_amd.build``.
"""
