"""MI355X-native chunked causal Conv3d decode.

The work happens in ``libcc3d.so`` (hand-written HIP for gfx950 behind the C ABI
of ``include/cc3d.h``); this package is its Python binding: ``capi`` declares
the C entry points, ``plan`` wraps them for torch tensors (device memory and
streams only), ``stacks`` builds the op lists of the decoder blocks and
``synth`` makes seeded synthetic inputs.  Nothing here computes a step of the
path on the host, and loading fails if the library is not built.
"""
from .capi import (BF16, EPI_ACT, EPI_NONE, EPI_RESIDUAL, F32, OP_CONV, OP_NORM_ACT, SLOT_AUX,
                   SLOT_NONE, SLOT_X, SLOT_Y, TPAD_REPLICATE, TPAD_ZERO, Cc3dError)

__all__ = ["BF16", "F32", "TPAD_REPLICATE", "TPAD_ZERO", "EPI_NONE", "EPI_RESIDUAL", "EPI_ACT",
           "OP_CONV", "OP_NORM_ACT", "SLOT_NONE", "SLOT_X", "SLOT_Y", "SLOT_AUX", "Cc3dError"]
