"""Random-access container for encoded tensors (a ``.wcpk`` file).

What the pages describe, and how it is read here:
  - the "PTWM" README ("Random access"; landing page, "Random-access
    container"): tensors bundled with a name-indexed manifest of offset
    records and hash-verified payloads, so that fetching one tensor touches
    only that tensor's bytes;
  - the "SeedPack" README: chunks plus an index at the end; files verified
    with BLAKE3 (SHA-256 where that package is missing: it is not installed
    here), every chunk with a CRC32.

File layout (little-endian):
  bytes 0-7    magic ``WCPK`` + format version (u16) + 2 zero bytes
  sections     each tensor's encoded buffers (raw planes, tables, seek
               table, payload and, with the CRC option, the per-chunk CRC-32
               table), every section starting on a 64-byte boundary
  manifest     UTF-8 JSON: per tensor its torch dtype, shape, plane layout,
               format word, element count, the [offset, length] of every
               section, and the SHA-256 of its sections concatenated in the
               order raw, tables, seek, payload, crc
  trailer      u64 manifest offset, u64 manifest length, ``WCPKEND`` + 0

``write`` / ``TensorIndex.read_sections`` are host-only (numpy and the file);
``save`` encodes device tensors with the GPU codec and ``get_tensor`` decodes
on the GPU (the CRC-32 of every chunk is checked there when the tensor was
saved with ``crc=True``).
"""
from __future__ import annotations

import hashlib
import json
import os
import struct
from typing import Iterable, Mapping

import numpy as np

MAGIC = b"WCPK"
VERSION = 1
TRAILER_MAGIC = b"WCPKEND\x00"
ALIGN = 64
SECTIONS = ("raw", "tables", "seek", "payload", "crc")
_NP = {"raw": np.uint8, "tables": np.uint16, "seek": np.uint64, "payload": np.uint8, "crc": np.uint32}


class ContainerError(ValueError):
    """A malformed container, an unknown tensor, or a failed hash check."""


def _digest(sections: Mapping[str, np.ndarray]) -> str:
    h = hashlib.sha256()
    for s in SECTIONS:
        if s in sections:
            h.update(np.ascontiguousarray(sections[s]).view(np.uint8).tobytes())
    return h.hexdigest()


def write(path: str, entries: Iterable[tuple[str, dict, Mapping[str, np.ndarray]]]) -> None:
    """Writes (name, meta, sections) entries.  meta holds dtype, shape,
    layout, format and n; sections maps section names to host arrays."""
    manifest = {"format": "wcpk", "version": VERSION, "tensors": {}}
    tmp = path + ".tmp"
    try:
        _write_to(tmp, manifest, entries)
    except BaseException:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise
    os.replace(tmp, path)


def _write_to(tmp, manifest, entries):
    with open(tmp, "wb") as f:
        f.write(MAGIC + struct.pack("<HH", VERSION, 0))
        for name, meta, sections in entries:
            if name in manifest["tensors"]:
                raise ContainerError(f"duplicate tensor name {name!r}")
            rec = dict(meta)
            rec["sections"] = {}
            for s in SECTIONS:
                if s not in sections:
                    continue
                a = np.ascontiguousarray(sections[s], _NP[s])
                pad = (-f.tell()) % ALIGN
                f.write(b"\0" * pad)
                rec["sections"][s] = [f.tell(), int(a.nbytes)]
                f.write(a.tobytes())
            rec["sha256"] = _digest(sections)
            manifest["tensors"][name] = rec
        blob = json.dumps(manifest, sort_keys=True).encode()
        off = f.tell()
        f.write(blob)
        f.write(struct.pack("<QQ", off, len(blob)) + TRAILER_MAGIC)


class TensorIndex:
    """The manifest of a container; reads one tensor's byte ranges on demand."""

    def __init__(self, path: str, manifest: dict):
        self.path = path
        self.manifest = manifest

    @classmethod
    def open(cls, path: str) -> "TensorIndex":
        with open(path, "rb") as f:
            head = f.read(8)
            if head[:4] != MAGIC:
                raise ContainerError(f"{path}: not a .wcpk container")
            version = struct.unpack("<H", head[4:6])[0]
            if version != VERSION:
                raise ContainerError(f"{path}: container version {version} is not supported")
            f.seek(0, os.SEEK_END)
            size = f.tell()
            if size < 8 + 24:
                raise ContainerError(f"{path}: truncated")
            f.seek(size - 24)
            off, length = struct.unpack("<QQ", f.read(16))
            if f.read(8) != TRAILER_MAGIC or off + length > size - 24:
                raise ContainerError(f"{path}: bad trailer")
            f.seek(off)
            manifest = json.loads(f.read(length).decode())
        return cls(path, manifest)

    def keys(self):
        return list(self.manifest["tensors"].keys())

    def meta(self, name: str) -> dict:
        try:
            return self.manifest["tensors"][name]
        except KeyError:
            raise ContainerError(f"no tensor {name!r} in {self.path}") from None

    def read_sections(self, name: str, verify: bool = True) -> dict:
        """The tensor's sections as host arrays, read from their byte ranges
        only; with verify, their SHA-256 must match the manifest's."""
        rec = self.meta(name)
        out = {}
        with open(self.path, "rb") as f:
            for s, (off, length) in rec["sections"].items():
                f.seek(off)
                buf = f.read(length)
                if len(buf) != length:
                    raise ContainerError(f"{name}: section {s} is truncated")
                out[s] = np.frombuffer(buf, _NP[s]).copy()
        if verify and _digest(out) != rec["sha256"]:
            raise ContainerError(f"{name}: SHA-256 mismatch (the container is damaged)")
        return out

    def get_tensor(self, name: str, device=None, verify: bool = True):
        """Decodes one tensor on the GPU (its CRC-32 per chunk is checked
        there when present)."""
        import torch
        from . import codec
        rec = self.meta(name)
        sec = self.read_sections(name, verify)
        dev = torch.device(device or "cuda:0")

        def up(a, dt):
            a = np.ascontiguousarray(a)
            t = torch.from_numpy(a.view(dt) if a.size else np.zeros(16 // np.dtype(dt).itemsize, dt)).to(dev)
            return t[: a.size]

        torch_dtype = getattr(torch, rec["dtype"])
        crc = up(sec["crc"], np.int32) if "crc" in sec else None
        e = codec.Encoded(rec["layout"], int(rec["n"]), tuple(rec["shape"]), torch_dtype,
                          up(sec["raw"], np.uint8), up(sec["tables"], np.int16).view(-1, 256),
                          up(sec["seek"], np.int64), up(sec["payload"], np.uint8), int(rec["format"]), crc)
        return codec.decode(e)

    def stream_tensors(self, names=None, device=None, verify: bool = True):
        for name in names or self.keys():
            yield name, self.get_tensor(name, device, verify)


def save(path: str, tensors: Mapping, reorder: bool = False, tensor_table: bool = False,
         raw_fallback: bool = False, crc: bool = True, stream=None) -> dict:
    """Encodes every device tensor with the GPU codec and writes the
    container; returns the manifest."""
    from . import codec

    def entries():
        for name, t in tensors.items():
            e = codec.encode(t, stream, reorder=reorder, tensor_table=tensor_table, raw_fallback=raw_fallback,
                             crc=crc)
            h = e.to_host()
            meta = {"dtype": str(t.dtype).replace("torch.", ""), "shape": list(t.shape), "layout": e.dtype,
                    "format": int(e.fmt), "n": int(e.n)}
            yield name, meta, h

    write(path, entries())
    return TensorIndex.open(path).manifest


def load(path: str, names=None, device=None, verify: bool = True) -> dict:
    idx = TensorIndex.open(path)
    return dict(idx.stream_tensors(names, device, verify))
