"""Full-size weight sets on the GPU: the whole set is encoded and decoded
as one batch (the launch configuration the benchmark times), every tensor
must round-trip bit for bit, and every chunk's table, every seek entry,
every payload byte and the raw planes are checked byte for byte against the
oracle, which encodes the same bits tensor by tensor on the host cores.
"""
import sys
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import codec, synthetic as S  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _upload_set(w, dev):
    t0 = time.time()
    ts = []
    ity = np.int16 if w.dtype == "bf16" else np.int32
    for i in range(len(w.shapes)):
        x = S.tensor_bits(w, i, threads=16)
        ts.append(torch.from_numpy(x.view(ity)).to(dev))
        if i % 64 == 63:
            _say(f"[full] {w.name}: generated {i + 1}/{len(w.shapes)} tensors ({time.time() - t0:.0f} s)")
    _say(f"[full] {w.name}: {w.n} elements resident ({time.time() - t0:.0f} s)")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return [t.view(tdt) for t in ts]


def _check_set(name, oracle_lib, dev):
    """The set encoded as one batch on the GPU; then, tensor by tensor, the
    oracle encodes the same bits (downloaded from the device) and every
    table, every seek entry (global offsets), every payload byte and the raw
    plane must be equal; the zero gaps between raw planes too."""
    w = S.workload(name)
    ts = _upload_set(w, dev)
    e = codec.encode_batch(ts)
    torch.cuda.synchronize()
    _say(f"[full] {name}: encoded, ratio {e.ratio:.4f}, payload {e.payload.numel()} B")
    outs = codec.decode_batch(e)
    torch.cuda.synchronize()
    ity = torch.int16 if w.dtype == "bf16" else torch.int32
    for t, y in zip(ts, outs):
        assert torch.equal(t.view(ity), y.view(ity))
    del outs
    _say(f"[full] {name}: every tensor round-trips")
    seek = e.seek.cpu().numpy().view("<u8")
    cb, rb, tot = oracle_lib.plan_batch(w.dtype, w.numels)
    assert seek.size == tot.num_chunks + 1 and seek[0] == 0
    assert int(seek[-1]) == e.payload.numel()
    raw_end = 0
    t0 = time.time()
    for i, t in enumerate(ts):
        x = t.view(ity).cpu().numpy().view(np.uint16 if w.dtype == "bf16" else np.uint32)
        o = oracle_lib.encode(x, w.dtype, threads=16)
        c0, c1 = int(cb[i]), int(cb[i]) + o.seek.size - 1
        assert np.array_equal(e.tables[c0:c1].cpu().numpy().view("<u2"), o.tables), (name, i, "tables")
        assert np.array_equal(seek[c0:c1 + 1] - seek[c0], o.seek), (name, i, "seek")
        got_p = e.payload[int(seek[c0]): int(seek[c1])].cpu().numpy()
        assert np.array_equal(got_p, o.payload), (name, i, "payload")
        r0 = int(rb[i])
        assert not e.raw[raw_end:r0].cpu().numpy().any(), (name, i, "raw gap")
        assert np.array_equal(e.raw[r0: r0 + o.raw.size].cpu().numpy(), o.raw), (name, i, "raw plane")
        raw_end = r0 + o.raw.size
        if i % 64 == 63:
            _say(f"[full] {name}: {i + 1}/{len(ts)} tensors equal to the oracle ({time.time() - t0:.0f} s)")
    assert raw_end == e.raw.numel()
    _say(f"[full] {name}: all {tot.num_chunks} chunks (tables, seek, payload) and raw planes equal to the oracle")
    return e


def test_llama3_8b_set(dev, oracle_lib):
    e = _check_set("llama3-8b-bf16", oracle_lib, dev)
    assert 0.66 < e.ratio < 0.69


def test_moe_experts_set(dev, oracle_lib):
    e = _check_set("moe-experts-bf16", oracle_lib, dev)
    assert 0.66 < e.ratio < 0.70


def test_moe_w2_fused_gemm_set(dev, oracle_lib):
    """The fused decode + GEMM over all 256 expert down projections in one
    launch (m = 16, as the benchmark times it): sampled matrices against the
    oracle's double-precision X W^T within the fp32 rounding bound, all of
    them against torch's GEMM of the uncompressed weights in fp32."""
    from lossless_weight_compression_bf16_amd import gemm as G
    w = S.workload("moe-w2-bf16")
    ws = [t.view(r, c) for t, (r, c) in zip(_upload_set(w, dev), w.shapes)]
    m = 16
    g = np.random.default_rng(12345)
    xb = [S.f32_to_bf16_bits(g.standard_normal(m * c).astype(np.float32)).reshape(m, c) for _, c in w.shapes]
    xs = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in xb]
    e = G.encode_weights(ws)
    _say(f"[full] moe-w2-bf16: encoded in tile order, ratio {e.ratio:.4f}")
    ys = G.decode_gemm(e, xs)
    torch.cuda.synchronize()
    for i in sorted({0, 1, 127, 254, 255}):
        wi = ws[i].view(torch.int16).cpu().numpy().view(np.uint16)
        ref, mag = oracle_lib.gemm_bf16(xb[i], wi, magnitude=True)
        bound = (w.shapes[i][1] + 16) * 2.0 ** -24 * mag + 1e-30
        assert np.all(np.abs(ys[i].cpu().numpy().astype(np.float64) - ref) <= bound), i
    for i in range(len(ws)):
        ref = xs[i].float() @ ws[i].float().t()
        tol = (w.shapes[i][1] + 16) * 2.0 ** -23 * (xs[i].float().abs() @ ws[i].float().abs().t()) + 1e-30
        assert bool(((ys[i] - ref).abs() <= tol).all()), i
    _say("[full] moe-w2-bf16: fused Y checked")
