"""The .wcpk container: manifest, per-tensor SHA-256, random access (CPU;
encodings come from the oracle, so no GPU is needed)."""
import os

import numpy as np
import pytest

import oracle
from lossless_weight_compression_bf16_amd import container as C


def _entry(name, x, layout, opts=0):
    e = oracle.encode(x, layout, threads=4, opts=opts)
    sections = {"raw": e.raw, "tables": e.tables.reshape(-1), "seek": e.seek, "payload": e.payload}
    if opts & oracle.OPT_CRC32:
        sections["crc"] = oracle.chunk_crc(e.seek, e.payload)
    meta = {"dtype": "bfloat16", "shape": [x.size], "layout": layout, "format": oracle.DTYPES[layout] | opts,
            "n": int(x.size)}
    return name, meta, sections


def _weights(n, seed):
    x = (np.random.default_rng(seed).standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
    return ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.fixture
def pack(tmp_path):
    xs = {"a": _weights(3 * 65536 + 17, 1), "b": _weights(1000, 2), "empty": np.zeros(0, np.uint16)}
    path = str(tmp_path / "t.wcpk")
    C.write(path, [_entry(k, v, "bf16", oracle.OPT_CRC32) for k, v in xs.items()])
    return path, xs


def test_round_trip_through_the_file(pack):
    path, xs = pack
    idx = C.TensorIndex.open(path)
    assert idx.keys() == ["a", "b", "empty"]
    for name, x in xs.items():
        sec = idx.read_sections(name)
        rec = idx.meta(name)
        e = oracle.Encoded("bf16", rec["n"], sec["raw"], sec["tables"].reshape(-1, 256), sec["seek"],
                           sec["payload"], rec["format"] & 0x300)
        y, err = oracle.decode(e)
        assert err == 0 and np.array_equal(y, x)
        assert np.array_equal(sec["crc"], oracle.chunk_crc(sec["seek"], sec["payload"]))


def test_sections_are_aligned_and_disjoint(pack):
    path, _ = pack
    idx = C.TensorIndex.open(path)
    spans = []
    for name in idx.keys():
        for off, length in idx.meta(name)["sections"].values():
            assert off % C.ALIGN == 0
            spans.append((off, off + length))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))


def test_random_access_reads_only_its_tensor(pack):
    """Damage tensor a's payload: a fails its hash, b still reads and
    verifies (its byte ranges were all that was read)."""
    path, xs = pack
    idx = C.TensorIndex.open(path)
    off, length = idx.meta("a")["sections"]["payload"]
    with open(path, "r+b") as f:
        f.seek(off + length // 2)
        byte = f.read(1)
        f.seek(off + length // 2)
        f.write(bytes([byte[0] ^ 0xFF]))
    with pytest.raises(C.ContainerError, match="SHA-256"):
        idx.read_sections("a")
    sec = idx.read_sections("b")
    assert sec["seek"][-1] == sec["payload"].size
    # without the hash check the damage reaches the CRC table's comparison
    raw = idx.read_sections("a", verify=False)
    crc = oracle.chunk_crc(raw["seek"], raw["payload"])
    assert not np.array_equal(crc, raw["crc"])


def test_malformed_files_and_names(tmp_path, pack):
    path, _ = pack
    bad = str(tmp_path / "bad.wcpk")
    with open(path, "rb") as f:
        data = bytearray(f.read())
    with open(bad, "wb") as f:
        f.write(data[:-3])
    with pytest.raises(C.ContainerError):
        C.TensorIndex.open(bad)
    data[0:4] = b"XXXX"
    with open(bad, "wb") as f:
        f.write(data)
    with pytest.raises(C.ContainerError, match="not a .wcpk"):
        C.TensorIndex.open(bad)
    with pytest.raises(C.ContainerError, match="no tensor"):
        C.TensorIndex.open(path).meta("nope")
    x = _weights(10, 3)
    with pytest.raises(C.ContainerError, match="duplicate"):
        C.write(str(tmp_path / "dup.wcpk"), [_entry("x", x, "bf16"), _entry("x", x, "bf16")])
    assert not os.path.exists(str(tmp_path / "dup.wcpk"))
    assert not os.path.exists(str(tmp_path / "dup.wcpk.tmp"))
