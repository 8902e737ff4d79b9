"""MoE dispatch and combine for AMD MI355X (gfx950), hand-written HIP.

The device entry points live in ``api`` (a thin ctypes binding over the C-ABI
library ``libmoe_dispatch.so``); importing them loads the library and fails
loudly when it has not been built.  ``inputs`` holds the seeded workload
generators and does not need the library.
"""
_API = ("moe_route_topk", "moe_route_topk_grouped", "moe_dispatch", "moe_combine", "moe_expert_scale",
        "moe_recv_rows", "Shape", "Layout", "MoeError")


def __getattr__(name):
    if name in _API:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
