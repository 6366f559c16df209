"""MI355X-native PagedAttention decode.

The compute path is the HIP library ``libpagedattn.so`` (gfx950 kernels
behind the C-ABI declared in ``include/paged_attn.h``); :mod:`.binding` is a
thin ctypes layer over it that only marshals torch tensors into pointers and
sizes.  :mod:`.inputs` builds seeded synthetic workloads and
:mod:`.accounting` counts algorithmic bytes.  Importing the package loads no
native code; the binding loads the library on first use and raises if it is
missing.
"""

__all__ = ["inputs", "accounting", "binding"]
