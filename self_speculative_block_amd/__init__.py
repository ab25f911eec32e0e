"""MI355X-native self-speculative block-decoding round engine.

The decoding path (prefill, draft / verify forwards, greedy argmax, accept,
KV overwrite and rollback) runs in the HIP library ``libssb.so`` behind the
C ABI of ``include/ssb.h``; this package only builds and binds it.  Importing
the binding never falls back to another implementation: if the library is
missing, ``load()`` raises.
"""

from ._lib import (SSB_BF16, SSB_EHIP, SSB_EINVAL, SSB_ENOKV, SSB_ENOMEM, SSB_ESTATE, SSB_F32,
                   SSB_MAX_BATCH, SSB_MAX_BLOCK, SSB_OK, SIGNATURES, SsbError, load)
from .build import LIB, build_library

__all__ = ["load", "build_library", "LIB", "SIGNATURES", "SsbError", "SSB_OK", "SSB_EINVAL", "SSB_ENOKV",
           "SSB_EHIP", "SSB_ESTATE", "SSB_ENOMEM", "SSB_F32", "SSB_BF16", "SSB_MAX_BATCH", "SSB_MAX_BLOCK"]
