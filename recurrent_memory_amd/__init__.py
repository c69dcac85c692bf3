"""MI355X-native chunkwise gated delta-rule forward and single-token decode.

The compute path lives in a C-ABI shared library (``libdeltarule.so``, built
from ``csrc/`` for gfx950); ``ops`` is a thin ctypes binding over it that
marshals torch device tensors and the current HIP stream.
"""
