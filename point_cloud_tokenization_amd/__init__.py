"""libfpstok: the FPS tokenizer of the Neptune point transformer on AMD
Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libfpstok.so`` (hand-written HIP
kernels); :mod:`.fpstok` is its thin ctypes binding and :mod:`.synth` draws
seeded synthetic batches.  Importing the package does not load the library;
the first call does, and it raises if the library is missing.
"""
from . import synth  # noqa: F401

__all__ = ["synth"]
