"""Block-quantized MoE expert layer for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libmoe_quant.so`` (C ABI declared in
``include/moe_quant.h``).  This package is a thin ctypes binding over it plus
the seeded synthetic-input generators.  Importing the package does not load the
library; constructing a :class:`Layer` does, and raises if it is missing.
"""
from .binding import (  # noqa: F401
    FORMATS,
    Layer,
    MoeQuantError,
    import_expert,
    library_path,
    load_library,
    router_logits,
)

__all__ = ["FORMATS", "Layer", "MoeQuantError", "import_expert", "library_path", "load_library",
           "router_logits"]
