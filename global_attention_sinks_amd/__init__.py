"""MiMo-V2.6-Flash attention hot path on MI355X (gfx950).

The compute lives in libmimo_attn.so (hand-written HIP behind a C ABI,
include/mimo_attn.h); `binding` marshals torch tensors into it.  Importing the
package loads nothing: the binding loads the library on first use and raises if
it is missing.
"""

__all__ = ["binding", "inputs", "build"]
