"""A small GGUF writer for the reader's tests, written from the container's
published layout (little-endian): magic "GGUF", uint32 version, uint64 tensor
count, uint64 metadata count; metadata entries (string key, uint32 value type,
value); tensor entries (string name, uint32 n_dims, uint64 dims innermost
first, uint32 element type, uint64 offset into the data section); zero padding
to the alignment; the data section, each tensor at an aligned offset.
Strings are a uint64 byte length and the bytes.  Arrays are a uint32 element
type, a uint64 count and the elements.

It can also write malformed files on purpose (wrong offsets, duplicate names,
missing padding) so the tests can check that the reader refuses them."""

from __future__ import annotations

import struct

import numpy as np

# metadata value types
U8, I8, U16, I16, U32, I32, F32, BOOL, STRING, ARRAY, U64, I64, F64 = range(13)
_FMT = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f",
        BOOL: "<B", U64: "<Q", I64: "<q", F64: "<d"}

# tensor element types
T_F32, T_F16, T_Q4_0, T_Q8_0, T_BF16 = 0, 1, 2, 8, 30


def _string(s) -> bytes:
    b = s.encode() if isinstance(s, str) else bytes(s)
    return struct.pack("<Q", len(b)) + b


def _value(t: int, v) -> bytes:
    if t == STRING:
        return _string(v)
    if t == ARRAY:
        et, items = v
        out = struct.pack("<IQ", et, len(items))
        return out + b"".join(_value(et, it) for it in items)
    return struct.pack(_FMT[t], v)


def tensor_nbytes(ttype: int, dims) -> int:
    n = int(np.prod(dims))
    return {T_F32: 4 * n, T_F16: 2 * n, T_BF16: 2 * n, T_Q4_0: n // 32 * 18,
            T_Q8_0: n // 32 * 34}.get(ttype, 0)


def build(metadata, tensors, alignment: int = 32, version: int = 3,
          offsets=None, pad_header: bool = True):
    """Return (file bytes, data section start, [tensor offsets]).

    metadata: list of (key, value type, value); tensors: list of
    (name, dims innermost first, element type, raw bytes).  Offsets default to
    the packed aligned layout; `offsets` overrides them (for malformed files)."""
    head = b"GGUF" + struct.pack("<IQQ", version, len(tensors), len(metadata))
    for key, t, v in metadata:
        head += _string(key) + struct.pack("<I", t) + _value(t, v)
    if offsets is None:
        offsets, pos = [], 0
        for _, _, _, data in tensors:
            pos = -(-pos // alignment) * alignment
            offsets.append(pos)
            pos += len(data)
    for (name, dims, ttype, _), off in zip(tensors, offsets):
        head += _string(name) + struct.pack("<I", len(dims))
        head += b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", ttype, off)
    start = -(-len(head) // alignment) * alignment if pad_header else len(head)
    out = bytearray(head + b"\0" * (start - len(head)))
    for (_, _, _, data), off in zip(tensors, offsets):
        end = start + off + len(data)
        if len(out) < end:
            out.extend(b"\0" * (end - len(out)))
        out[start + off:end] = data
    return bytes(out), start, list(offsets)


def write_shards(blob: bytes, base: str, cuts) -> list[str]:
    """Split `blob` at the byte positions `cuts` into files base.0, base.1..."""
    edges = [0] + sorted(cuts) + [len(blob)]
    paths = []
    for i in range(len(edges) - 1):
        p = f"{base}.{i}"
        with open(p, "wb") as f:
            f.write(blob[edges[i]:edges[i + 1]])
        paths.append(p)
    return paths
