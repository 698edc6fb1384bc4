"""Both encoder word-store forms against the oracle, byte for byte.

WC_ENC_WORDS_DIRECT writes each step's renormalisation words straight to the
chunk's scratch slot; WC_ENC_WORDS_STAGED collects them in a 256-word LDS
ring per chunk and, once per 256 symbols, writes the whole 128-byte lines of
the slot they complete (up to 63 words wait below a line).  Both must give
the oracle's tables, seek table, payload and raw planes on: sizes with
partial groups and ragged last chunks, odd chunk counts (a wavefront whose
second half only shadows the first), every layout with and without options,
ragged batches, uniform coded bytes (about 128 words per group and half:
two flush rounds) and chunks at the most words a group can take (192 per
half: every lane renormalising at 6 of its 8 steps, the three-in-a-row
bound's maximum), where a flush moves the most words, and dense groups among
groups of weights, where up to 255 words are live in the ring.  The automatic
choice follows the CU count of the stream's device.
All calls go through the C ABI.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import _binding as B, codec, synthetic as S  # noqa: E402

TT, RF, CRC = 0x100, 0x200, 0x400
TORCH_OF = {"bf16": torch.bfloat16, "bf16r": torch.bfloat16, "fp16": torch.float16, "fp16r": torch.float16,
            "fp32": torch.float32}
FP8 = {"fp8e4m3": torch.float8_e4m3fn, "fp8e5m2": torch.float8_e5m2}
FORMS = {"direct": B.ENC_WORDS_DIRECT, "staged": B.ENC_WORDS_STAGED}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


@pytest.fixture(params=sorted(FORMS))
def form(request, dev):
    B.wc_set_encoder_words(FORMS[request.param])
    yield request.param
    B.wc_set_encoder_words(B.ENC_WORDS_AUTO)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits16(layout, n, seed, sigma=0.02):
    f = (np.random.default_rng(seed).standard_normal(n) * sigma).astype(np.float32)
    if layout.startswith("fp16"):
        return f.astype(np.float16).view(np.uint16)
    return S.f32_to_bf16_bits(f)


def _bits(layout, n, seed):
    if layout == "fp32":
        return (np.random.default_rng(seed).standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
    if layout in FP8:
        if n == 0:
            return np.zeros(0, np.uint8)
        x = torch.from_numpy(np.random.default_rng(seed).standard_normal(n).astype(np.float32))
        dt = FP8[layout]
        return (x * (torch.finfo(dt).max / max(float(x.abs().max()), 1e-30))).to(dt).view(torch.uint8).numpy()
    return _bits16(layout, n, seed)


def _tensor(layout, x, dev):
    if layout in FP8:
        return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(dev)
    a = np.ascontiguousarray(x)
    t = torch.from_numpy(a.view(np.int32 if layout == "fp32" else np.int16)).to(dev)
    return t.view(TORCH_OF[layout])


def _int_view(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def _one(layout, opts, x, dev, oracle_lib, what):
    _say(f"[words] {what}: layout={layout} opts={opts:#x} n={x.size}")
    xt = _tensor(layout, x, dev)
    kw = dict(tensor_table=bool(opts & TT), raw_fallback=bool(opts & RF), crc=bool(opts & CRC))
    if layout in FP8:
        e = codec.encode(xt, layout=layout, **kw)
    else:
        e = codec.encode(xt, reorder=layout.endswith("r"), **kw)
    o = oracle_lib.encode(x, layout, threads=16, opts=opts & (TT | RF))
    h = e.to_host()
    assert np.array_equal(h["tables"].reshape(-1), o.tables.reshape(-1)), f"{what}: tables"
    assert np.array_equal(h["seek"], o.seek), f"{what}: seek"
    assert np.array_equal(h["payload"], o.payload), f"{what}: payload"
    assert np.array_equal(h["raw"], o.raw), f"{what}: raw planes"
    y = codec.decode(e)
    assert torch.equal(_int_view(y).cpu(), _int_view(xt).cpu()), f"{what}: decode"


@pytest.mark.parametrize("n", [1, 31, 255, 256, 257, 65535, 65536, 65537, 2 * 65536 + 3, 3 * 65536,
                               5 * 65536 + 40001])
def test_bf16_sizes(dev, oracle_lib, form, n):
    _one("bf16", 0, _bits("bf16", n, n), dev, oracle_lib, f"{form} bf16 n={n}")


@pytest.mark.parametrize("layout", ["bf16r", "fp16", "fp16r", "fp32", "fp8e4m3", "fp8e5m2"])
@pytest.mark.parametrize("opts", [0, TT | RF])
def test_layouts_and_options(dev, oracle_lib, form, layout, opts):
    n = 3 * 65536 + 12345
    _one(layout, opts, _bits(layout, n, 11), dev, oracle_lib, f"{form} {layout}")


def test_crc_option(dev, oracle_lib, form):
    _one("bf16", CRC, _bits("bf16", 2 * 65536 + 77, 12), dev, oracle_lib, f"{form} bf16 crc")


def _dense_groups(g, n, groups, a=0x3C):
    """n BF16 patterns whose coded (high) bytes are symbol a except in the
    listed 256-element groups, which hold the 255 other symbols once each
    plus one a, shuffled.  With at most 15 such groups in a chunk every other
    symbol occurs fewer than 16 times: its scaled count 4096 c / 65536 is
    below 1, so the normaliser gives it f = 1 and no share of a shortfall,
    and each costs 12 bits: a lane with 8 of them takes 6 words."""
    hi = np.full(n, a, np.uint16)
    rest = np.array([s for s in range(256) if s != a] + [a], np.uint16)
    for q in groups:
        m = min(256, n - 256 * q)
        hi[256 * q:256 * q + m] = g.permutation(rest)[:m]
    return (hi << 8) | g.integers(0, 256, n).astype(np.uint16)


def test_most_words_per_group(dev, oracle_lib, form):
    """Chunks at up to 192 words per group and half: dense groups at a
    chunk's end (encoded first), start, middle, spread out, and in a ragged
    last chunk up to its partial group; 5 chunks, so the last wavefront has
    a shadow half."""
    g = np.random.default_rng(41)
    parts = [_dense_groups(g, 65536, range(241, 256)), _dense_groups(g, 65536, range(0, 15)),
             _dense_groups(g, 65536, list(range(100, 108)) + list(range(140, 147))),
             _dense_groups(g, 65536, range(0, 256, 18)), _dense_groups(g, 40001, range(142, 157))]
    x = np.concatenate(parts)
    _one("bf16", 0, x, dev, oracle_lib, f"{form} dense groups")
    # the same chunks with the tensor's table, raw storage allowed
    _one("bf16", TT | RF, x, dev, oracle_lib, f"{form} dense groups, tensor table + raw fallback")


def test_dense_groups_among_weights(dev, oracle_lib, form):
    """Groups of one of each coded byte (about 160 words per group and half
    with their chunk's table) at random places among groups of weights (about
    45 words), so the words left below a 128-byte line before a dense group
    take many values and the staged ring holds up to 255 live words."""
    g = np.random.default_rng(47)
    parts = []
    for c in range(6):
        w = _bits16("bf16", 65536, 50 + c)
        for q in g.choice(256, 24, replace=False):
            lo = w[256 * q:256 * q + 256] & 0xFF
            w[256 * q:256 * q + 256] = (g.permutation(np.arange(256, dtype=np.uint16)) << 8) | lo
        parts.append(w)
    x = np.concatenate(parts + [_bits16("bf16", 30001, 57)])
    _one("bf16", 0, x, dev, oracle_lib, f"{form} dense groups among weights")


def test_uniform_coded_bytes(dev, oracle_lib, form):
    """Uniform coded bytes (f = 16: 8 bits a symbol, about 128 words per
    group and half) next to weight chunks."""
    g = np.random.default_rng(43)
    u = (g.permutation(np.repeat(np.arange(256, dtype=np.uint16), 256)) << 8) | g.integers(0, 256, 65536).astype(
        np.uint16)
    x = np.concatenate([u, _bits16("bf16", 65536, 44), u[::-1].copy(), _bits16("bf16", 1000, 45)])
    _one("bf16", 0, x, dev, oracle_lib, f"{form} uniform chunks")


def test_ragged_batch(dev, oracle_lib, form):
    xs = [_bits16("bf16", 70000, 51), np.zeros(0, np.uint16), _bits16("bf16", 3, 52),
          _bits16("bf16", 2 * 65536, 53), _bits16("bf16", 65536 + 1, 54)]
    _say(f"[words] {form} ragged batch")
    ts = [_tensor("bf16", x, dev) for x in xs]
    e = codec.encode_batch(ts)
    o = oracle_lib.encode_batch(xs, "bf16", threads=8)
    assert np.array_equal(e.tables.cpu().numpy().view(np.uint16).reshape(-1), o.tables.reshape(-1))
    assert np.array_equal(e.seek.cpu().numpy().view(np.uint64), o.seek)
    assert np.array_equal(e.payload.cpu().numpy(), o.payload)
    assert np.array_equal(e.raw.cpu().numpy(), o.raw)
    for x, y in zip(xs, codec.decode_batch(e)):
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_forms_agree_on_a_large_set(dev):
    """1,111 chunks of weights: the two forms write the same bytes (the
    oracle check of this size is in the other tests' forms)."""
    x = _tensor("bf16", _bits16("bf16", 1111 * 65536 - 5, 61), dev)
    out = {}
    for name, mode in sorted(FORMS.items()):
        B.wc_set_encoder_words(mode)
        try:
            e = codec.encode(x)
        finally:
            B.wc_set_encoder_words(B.ENC_WORDS_AUTO)
        out[name] = e.to_host()
        assert torch.equal(_int_view(codec.decode(e)), _int_view(x)), name
    for k in ("tables", "seek", "payload", "raw"):
        assert np.array_equal(out["direct"][k], out["staged"][k]), k


def test_encoder_variant_follows_the_streams_device(dev):
    """Automatic choice: for the 16-bit layouts staged from 16 wavefronts
    (two chunks each) per CU of the stream's device, direct below; FP32 and
    FP8 always direct; a forced form is reported as such."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    side = torch.cuda.Stream(device=dev)
    c = 2 * 16 * cus
    for stream in (None, side):
        for dtype in ("bf16", "bf16r", "fp16", "fp16r", "fp32", "fp8e4m3", "fp8e5m2"):
            sixteen = dtype in ("bf16", "bf16r", "fp16", "fp16r")
            for chunks, staged in ((c - 2, False), (c - 1, True), (c, True), (1 << 20, True), (1, False)):
                assert B.wc_encode_variant(dtype, chunks, stream) == (staged and sixteen), (dtype, chunks)
        for mode, staged in ((B.ENC_WORDS_STAGED, True), (B.ENC_WORDS_DIRECT, False)):
            B.wc_set_encoder_words(mode)
            try:
                assert B.wc_encode_variant("bf16", 1, stream) == staged
                assert B.wc_encode_variant("bf16", 1 << 20, stream) == staged
            finally:
                B.wc_set_encoder_words(B.ENC_WORDS_AUTO)
