"""ThriftAttention forward pass for AMD MI355X (gfx950).

The product is the C-ABI library libthrift.so (include/thrift.h); this
package holds its HIP sources (csrc/), the build script, a thin ctypes/torch
binding (api.py) and the seeded workload generator (workloads.py).  The
binding is imported lazily so that the generator can be used without a GPU.
"""
import importlib


def __getattr__(name):
    if name.startswith("_") or name in ("api", "workloads", "build"):
        raise AttributeError(name)
    api = importlib.import_module(__name__ + ".api")
    if hasattr(api, name):
        return getattr(api, name)
    raise AttributeError(name)
