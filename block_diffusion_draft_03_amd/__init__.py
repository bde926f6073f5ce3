"""MI355X-native DFlash (block-diffusion) draft head.

The propose path runs in the HIP library ``libdflash.so`` (gfx950 kernels
behind the C ABI declared in ``include/dflash.h``). This package is the thin
Python binding: ``binding`` marshals arguments with ctypes and uses PyTorch
only for device memory and streams. Build the library first with
``python -m block_diffusion_draft_03_amd.build``; loading fails loudly when
it is missing.
"""
from .binding import (  # noqa: F401
    DflashError, Head, State, load_library, library_path, yarn_inv_freq, EXPORTED_SYMBOLS,
)
