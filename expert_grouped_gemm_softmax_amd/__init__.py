"""One MI355X's share of a routed sparse mixture-of-experts feed-forward layer.

The computation lives in libmoe_mi355x.so (hand-written HIP for gfx950, C ABI in include/moe.h);
this package only binds it to torch tensors:

  ops.route, ops.pack_routing, ops.permute, ops.grouped_gemm, ops.combine  -- the five C calls
  layer.MoELayer                                                        -- the calls composed
  workloads                                                             -- seeded synthetic inputs
"""
from . import workloads  # noqa: F401  (numpy only)

__all__ = ["workloads", "ops", "layer", "load_library"]


def load_library():
    from ._abi import load
    return load()


def __getattr__(name):
    if name in ("ops", "layer"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
