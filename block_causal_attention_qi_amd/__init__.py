"""MI355X (gfx950) single-stream DiT denoising step with block-causal attention
and exact text-K/V reuse.

The compute path is the HIP library libqi.so (C ABI in include/qi.h); this
package is its Python binding (argument marshalling) plus the build step and
the algorithmic FLOP/byte model used to report roofline fractions."""
from . import _lib  # noqa: F401
from .qi import *  # noqa: F401,F403

__version__ = "0.1.0"
