"""MI355X (gfx950) MoE routing path: fused router, counting-sort dispatch,
weighted combine.

The compute lives in libmoe.so (HIP kernels behind the C ABI in
include/moe.h).  ``moe_token_routing_router_amd._lib`` is its ctypes binding;
the names below are re-exported lazily so that importing the package (for
example for the input generator) does not load torch or the library.
"""
_BINDING = ("moe_route", "moe_dispatch", "moe_route_dispatch", "moe_combine",
            "moe_route_workspace_size", "moe_dispatch_workspace_size",
            "moe_route_dispatch_workspace_size", "route", "dispatch", "route_dispatch",
            "combine", "MoeError", "library")

__all__ = list(_BINDING)


def __getattr__(name):
    if name in _BINDING:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
