"""MI355X-native hybrid window-softmax attention (VDN-H3 form).

The compute path is the C-ABI library ``libhwa.so`` built from ``csrc/``
(HIP kernels for gfx950); :mod:`.hwa` is its thin ctypes binding and
:mod:`.inputs` the seeded synthetic input generator. Importing the package
does not load the library; :func:`hwa.lib` loads it on first use and raises
if it has not been built.
"""

__all__ = ["inputs", "hwa"]
