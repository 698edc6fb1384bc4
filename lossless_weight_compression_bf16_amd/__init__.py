"""Lossless BF16 / FP32 weight compression on MI355X (gfx950).

Byte-plane split plus chunked 32-lane rANS of the skewed plane, as hand-
written HIP kernels behind a C ABI (include/wc.h).  ``codec`` holds the
tensor-level API; ``_binding`` mirrors the C ABI one to one.  Importing the
package does not load the GPU library; the first codec call does, and fails
if it has not been built.
"""
from ._binding import (  # noqa: F401
    EF_BAD_FINAL_STATE, EF_BAD_SEEK, EF_BAD_TABLE, EF_BAD_TAIL, EF_CAPACITY, EF_WORD_OVERRUN, EXPORTS,
    WC_BF16, WC_FP32, HipEvents, WcError, lib, make_buffers, wc_check_division, wc_decode,
    wc_decode_batch, wc_encode, wc_encode_batch, wc_plan_batch, wc_query_layout, wc_version)


def __getattr__(name):
    # tensor-level API (imports torch lazily)
    if name in ("encode", "decode", "encode_batch", "decode_batch", "Encoded", "EncodedBatch"):
        from . import codec
        return getattr(codec, name)
    raise AttributeError(name)
