"""MI355X (gfx950) quantized expert-FFN MoE layer: a C-ABI HIP library
(libmoe.so, declared in include/moe.h) and its thin Python binding."""
from . import binding  # noqa: F401
