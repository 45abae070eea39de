"""MI355X-native HGRNBit layer forward (MatMul-free LM): HIP kernels behind a C ABI.

The Python side only marshals arguments to ``libmmf.so`` (see ``binding``);
every step of the computation runs in the HIP kernels. Importing the package
does not touch the GPU; ``load()`` opens the library and raises if it is
missing, so there is no silent fallback.
"""
from .binding import *  # noqa: F401,F403
from .binding import load  # noqa: F401
