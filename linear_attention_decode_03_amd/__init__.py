"""MI355X-native Kimi Delta Attention (KDA) decode / verify step.

The computation lives in hand-written HIP kernels for gfx950 (csrc/),
exported through the C ABI declared in include/kda.h and built into
libkda.so next to this file.  `kda` is the thin ctypes binding; `inputs`
makes seeded synthetic operands.  Importing the package loads nothing.
"""

from .kda import (kda_decode, kda_decode_split, kda_replay, kda_status_string,  # noqa: F401
                  kda_validate, kda_verify, kda_verify_split, kda_verify_split_noalloc,
                  load_library, split_workspace)
