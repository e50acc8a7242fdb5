"""MI355X (gfx950) GPTQ layer-quantization hot path.

The kernels live in libgptq_mi355x.so (C ABI in include/gptq.h); this package
holds the in-tree build script, a ctypes binding with the same entry-point
names, and the seeded synthetic layer generator.
"""

from . import synthetic  # noqa: F401
from .gptq import (accumulate_hessian, load_library, pack_codes, prepare_hinv,  # noqa: F401
                   quantize, quantize_layer, workspace_bytes)
