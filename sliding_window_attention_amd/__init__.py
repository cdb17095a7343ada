"""MI355X-native sliding-window attention: HIP kernels behind a C ABI.

The compute path is ``libswa.so`` (built from ``csrc/`` for gfx950).  The Python
binding in ``binding.py`` only marshals tensors to pointers and the current HIP
stream; importing this package does not load the library (``inputs`` is usable
on a machine without the extension).
"""

__all__ = ["binding", "inputs"]
