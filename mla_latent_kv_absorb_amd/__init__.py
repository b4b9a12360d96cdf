"""MI355X (gfx950) weight-absorbed MLA decode over a paged latent KV cache.

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libmla_absorb.so``, declared in ``include/mla_absorb.h``).  The Python layer
only marshals arguments: ``binding`` loads the library (raising if it is not
built) and passes device pointers and the current stream.  ``inputs`` draws
seeded synthetic workloads.
"""
__all__ = ["binding", "inputs"]
