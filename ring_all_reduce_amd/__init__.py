"""Ring all-reduce-mean (+ synchronous SGD) for data-parallel training on MI355X.

The work happens in the HIP library ``librar.so`` (C ABI declared in
include/rar.h).  This package is its thin Python binding: ``api`` marshals
arguments to the C entry points of the same names, ``synth`` draws seeded
synthetic inputs.  Nothing here computes any step of the all-reduce; if the
library is missing, the first call raises.
"""
__all__ = ["api", "synth"]
