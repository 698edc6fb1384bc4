"""The C-ABI library, without a GPU: it loads, exports every function that
include/wc.h declares, and its host-side logic (layout, batch planning,
argument checks, the encoder's reciprocal division) agrees with the oracle
and with arithmetic."""
import ctypes
import os
import re

import numpy as np
import pytest

import lossless_weight_compression_bf16_amd as wc
from lossless_weight_compression_bf16_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from lossless_weight_compression_bf16_amd import build
        build.build()
    return wc.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "wc.h")).read()
    return sorted(set(re.findall(r"^\s*(?:wc_status|int|const char \*|uint64_t)\s*\*?\s*(wc_\w+)\s*\(",
                                 text, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.EXPORTS) == names


def test_version_and_strings(L):
    assert wc.wc_version() >= 10000
    assert L.wc_status_string(1) == b"invalid argument"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n", [0, 1, 7, 65535, 65536, 65537, 3 * 65536 + 5, 8029995008])
def test_layout_matches_oracle(L, oracle_lib, dtype, n):
    a = wc.wc_query_layout(dtype, n).as_dict()
    b = oracle_lib.query_layout(dtype, n)
    for k in ("n", "num_chunks", "raw_bytes", "table_bytes", "seek_bytes", "payload_capacity"):
        assert a[k] == getattr(b, k), k
    c = a["num_chunks"]
    assert a["scratch_bytes"] == (0 if c == 0 else ((8 * c + 255) // 256) * 256 + (c + 1) * 131200)


def test_plan_batch_matches_oracle(L, oracle_lib):
    ns = [65536 * 2 + 5, 1, 0, 70000, 300, 50257 * 768]
    for dtype in ("bf16", "fp32"):
        segs, tot = wc.wc_plan_batch(dtype, ns)
        cb, rb, otot = oracle_lib.plan_batch(dtype, ns)
        assert [segs[i].chunk_base for i in range(len(ns))] == list(cb)
        assert [segs[i].raw_base for i in range(len(ns))] == list(rb)
        assert tot.num_chunks == otot.num_chunks and tot.raw_bytes == otot.raw_bytes
        assert tot.payload_capacity == otot.payload_capacity


FORMATS = [(lay, opts) for lay in ("bf16", "bf16r", "fp16", "fp16r", "fp32", "fp8e4m3", "fp8e5m2")
           for opts in (0, 0x100, 0x200, 0x300, 0x700)]


@pytest.mark.parametrize("lay,opts", FORMATS)
@pytest.mark.parametrize("n", [0, 5, 65536, 3 * 65536 + 5])
def test_variant_layouts_match_oracle(L, oracle_lib, lay, opts, n):
    a = wc.wc_query_layout(B.format_word(lay) | opts, n).as_dict()
    b = oracle_lib.query_layout(lay, n, opts)
    for k in ("n", "num_chunks", "raw_bytes", "table_bytes", "seek_bytes", "payload_capacity"):
        assert a[k] == getattr(b, k), k
    c = a["num_chunks"]
    hist = 2048 if (opts & 0x100) and c else 0
    assert a["scratch_bytes"] == (0 if c == 0 else ((8 * c + 255) // 256) * 256 + (c + 1) * 131200 + hist)
    assert a["crc_bytes"] == (4 * c if opts & 0x400 else 0)


@pytest.mark.parametrize("lay,opts", FORMATS)
def test_variant_plan_batch_matches_oracle(L, oracle_lib, lay, opts):
    ns = [65536 * 2 + 5, 1, 0, 70000, 300]
    segs, tot = wc.wc_plan_batch(B.format_word(lay) | opts, ns)
    cb, rb, otot = oracle_lib.plan_batch(lay, ns, opts)
    assert [segs[i].chunk_base for i in range(len(ns))] == list(cb)
    assert [segs[i].raw_base for i in range(len(ns))] == list(rb)
    for k in ("num_chunks", "raw_bytes", "table_bytes", "payload_capacity"):
        assert getattr(tot, k) == getattr(otot, k), k


def test_bad_format_words_are_rejected(L):
    for f in (7, 0xFF, 0x800, 0x10000, 0x80000000):
        with pytest.raises(B.WcError):
            wc.wc_query_layout(f, 100)
        assert L.wc_query_layout(f, 100, ctypes.byref(B.wc_layout())) == B.WC_ERR_ARG


def test_division_by_reciprocal(L):
    # every divisor 1..4096, boundary and sampled dividends below 2^32
    assert wc.wc_check_division(512) == 0


def test_argument_errors_without_launch(L):
    bufs = B.wc_buffers(0, 0, 0, 0, 0)
    # bad dtype, null buffers, misaligned input: rejected on the host
    assert L.wc_encode(7, None, 10, ctypes.byref(bufs), None, 0, None, None, None) == B.WC_ERR_ARG
    assert L.wc_encode(0, None, 10, ctypes.byref(bufs), None, 0, None, None, None) == B.WC_ERR_ARG
    good = B.wc_buffers(256, 256, 256, 256, 1 << 20)
    assert L.wc_encode(0, 0x1002, 10, ctypes.byref(good), 256, 1 << 30, None, None, None) == B.WC_ERR_ARG
    assert L.wc_encode(0, 0x1000, 10, ctypes.byref(good), 256, 10, None, None, None) == B.WC_ERR_CAPACITY
    assert L.wc_decode(0, ctypes.byref(bufs), 10, 0x1000, None, None) == B.WC_ERR_ARG
    assert L.wc_decode(0, ctypes.byref(good), 1 << 41, 0x1000, None, None) == B.WC_ERR_ARG
    segs, _ = wc.wc_plan_batch("bf16", [100, 200])
    segs[0].ptr, segs[1].ptr = 0x1000, 0x2000
    segs[1].chunk_base = 5  # not what the plan says
    assert L.wc_decode_batch(0, ctypes.cast(segs, ctypes.c_void_p), 0x3000, 2, ctypes.byref(good),
                             None, None) == B.WC_ERR_ARG


def test_tile_order_and_gemm_argument_errors_without_launch(L):
    # ragged shapes, null or misaligned or overlapping buffers: rejected on the host
    assert L.wc_tile_order(0x1000, 0x100000, 24, 16, 0, None) == B.WC_ERR_ARG
    assert L.wc_tile_order(0x1000, 0x100000, 16, 8, 0, None) == B.WC_ERR_ARG
    assert L.wc_tile_order(None, 0x100000, 16, 16, 0, None) == B.WC_ERR_ARG
    assert L.wc_tile_order(0x1008, 0x100000, 16, 16, 0, None) == B.WC_ERR_ARG
    assert L.wc_tile_order(0x1000, 0x1100, 16, 16, 1, None) == B.WC_ERR_ARG  # 512-byte buffers overlap
    assert L.wc_tile_order(0x1000, 0x100000, 1 << 16, 1 << 16, 0, None) == B.WC_ERR_ARG  # 2^32 elements
    assert L.wc_tile_order(0x1000, 0x100000, 0, 16, 0, None) == B.WC_OK  # nothing to do
    segs, tot = wc.wc_plan_batch("bf16", [64 * 2048])
    good = B.wc_buffers(256, 256, 256, 256, 1 << 20)
    g = (B.wc_gemm * 1)()
    g[0].x, g[0].y, g[0].rows, g[0].cols = 0x10000, 0x20000, 64, 2048

    def call(fmt=0, m=16, gemm=g, d_gemm=0x3000):
        return L.wc_decode_gemm_batch(fmt, ctypes.cast(segs, ctypes.c_void_p), 0x4000, 1,
                                      ctypes.cast(gemm, ctypes.c_void_p), d_gemm, m, ctypes.byref(good), None,
                                      None)
    assert call(fmt=B.format_word("fp16")) == B.WC_ERR_ARG      # BF16 layouts only
    assert call(fmt=B.format_word("fp32")) == B.WC_ERR_ARG
    assert call(fmt=B.format_word("bf16", raw_fallback=True)) == B.WC_ERR_ARG
    assert call(m=0) == B.WC_ERR_ARG
    assert call(m=65) == B.WC_ERR_ARG
    assert call(d_gemm=0) == B.WC_ERR_ARG
    assert call(d_gemm=0x3004) == B.WC_ERR_ARG                  # misaligned descriptors
    g[0].rows = 48                                               # rows * cols != segment size
    assert call() == B.WC_ERR_ARG
    g[0].rows, g[0].x = 64, 0x10004                              # X not 8-byte aligned
    assert call() == B.WC_ERR_ARG
    g[0].x, g[0].y = 0x10000, 0x20002                            # Y not 4-byte aligned
    assert call() == B.WC_ERR_ARG
    # 768 columns: a full chunk spans 6 panels of 16 rows, more than m = 64 leaves accumulators for
    segs2, _ = wc.wc_plan_batch("bf16", [256 * 768])
    g2 = (B.wc_gemm * 1)()
    g2[0].x, g2[0].y, g2[0].rows, g2[0].cols = 0x10000, 0x20000, 256, 768
    assert L.wc_decode_gemm_batch(0, ctypes.cast(segs2, ctypes.c_void_p), 0x4000, 1, ctypes.cast(g2, ctypes.c_void_p),
                                  0x3000, 64, ctypes.byref(good), None, None) == B.WC_ERR_ARG


# The entry points that carry the codec's work: each declaration's comment
# names the passage of the pages that defines what it computes.
CITED = ["wc_query_layout", "wc_plan_batch", "wc_encode", "wc_decode", "wc_encode_batch", "wc_decode_batch",
         "wc_tile_order", "wc_decode_gemm_batch"]


def _comment_before(text, name):
    """The block comment that ends right before the declaration of name (for
    wc_decode_batch, declared right after wc_encode_batch, the shared one)."""
    m = re.search(r"^\s*wc_status\s+" + name + r"\s*\(", text, re.M)
    assert m, name
    head = text[: m.start()]
    if name == "wc_decode_batch":
        head = head[: head.rindex("wc_status wc_encode_batch")]
    end = head.rindex("*/")
    return head[head.rindex("/*", 0, end): end]


@pytest.mark.parametrize("name", CITED)
def test_every_entry_point_cites_its_passage(name):
    text = open(os.path.join(ROOT, "include", "wc.h")).read()
    c = _comment_before(text, name)
    assert re.search(r"(README|docs)", c), f"{name}: no passage cited"


def test_decoder_variant_needs_a_device(L):
    """The decoder variant follows the CU count of the stream's device; with
    no device there is none to query, and the call says so instead of
    guessing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: covered by the GPU tests")
    a, b = ctypes.c_int(7), ctypes.c_int(7)
    assert L.wc_decode_variant(0, 100, 100 * 65536, 1 << 20, None, ctypes.byref(a), ctypes.byref(b)) == B.WC_ERR_HIP
    assert L.wc_decode_variant(0, 100, 100 * 65536, 1 << 20, None, None, ctypes.byref(b)) == B.WC_ERR_ARG
    assert L.wc_decode_variant(0x800, 100, 100 * 65536, 1 << 20, None, ctypes.byref(a), ctypes.byref(b)) == B.WC_ERR_ARG


def test_encoder_words_setting(L):
    """wc_set_encoder_words takes the three forms, returns the previous one
    and refuses anything else without changing the setting; the variant
    query checks its arguments and, with no device, says so."""
    import torch
    prev = L.wc_set_encoder_words(B.ENC_WORDS_STAGED)
    try:
        assert prev == B.ENC_WORDS_AUTO
        assert L.wc_set_encoder_words(3) == -1
        assert L.wc_set_encoder_words(-1) == -1
        assert L.wc_set_encoder_words(B.ENC_WORDS_DIRECT) == B.ENC_WORDS_STAGED
        assert L.wc_set_encoder_words(B.ENC_WORDS_AUTO) == B.ENC_WORDS_DIRECT
        with pytest.raises(B.WcError):
            B.wc_set_encoder_words(7)
        assert L.wc_set_encoder_words(B.ENC_WORDS_AUTO) == B.ENC_WORDS_AUTO
    finally:
        L.wc_set_encoder_words(B.ENC_WORDS_AUTO)
    a = ctypes.c_int(7)
    assert L.wc_encode_variant(0, 100, None, None) == B.WC_ERR_ARG
    assert L.wc_encode_variant(0x800, 100, None, ctypes.byref(a)) == B.WC_ERR_ARG
    if not torch.cuda.is_available():
        assert L.wc_encode_variant(0, 100, None, ctypes.byref(a)) == B.WC_ERR_HIP
