"""MI355X-native paged MLA decode (gfx950 HIP kernels behind a C ABI).

The compute path lives in ``libmla_decode.so`` (built from ``csrc/``); this
package only marshals arguments to it (``binding``) and makes seeded synthetic
inputs (``synth``).  Importing the package does not load the library; the
first call into ``binding`` does, and raises if the library is missing.
"""

__all__ = ["binding", "synth"]
