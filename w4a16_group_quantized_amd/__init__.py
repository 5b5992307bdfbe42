"""W4A16 group-quantized linear layer (AWQ inference hot path) for MI355X.

The compute lives in hand-written HIP kernels for gfx950, built into the C-ABI
library ``libawq.so`` (entry points declared in ``include/awq.h``).  This
package only marshals arguments to it (``binding``), builds it (``build``) and
draws seeded synthetic inputs (``synth``).  Importing the package loads
nothing; the first call through ``binding`` loads the library and raises if it
is missing.
"""

__all__ = ["binding", "build", "synth"]
