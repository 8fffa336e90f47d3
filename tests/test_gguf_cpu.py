"""GGUF reader (host code in the C library): header, typed metadata, tensor
table and tensor bytes, over one file or its byte-split pieces.  The pages'
model ships as one GGUF Q4_0 file cut into pieces of at most 512 MB that the
loader reads back as one stream ("Implémentation en Rust du modèle Voxtral
Mini 4B Realtime de Mistral pour l'exécuter dans le navigateur", sections
"Architecture" and "Préparation du modèle et sharding").  No GPU needed."""

import ctypes
import os
import struct

import numpy as np
import pytest

import gguf_writer as W
import q4_quantized_speech_amd as q4
from oracle import q4_oracle as O

pytestmark = pytest.mark.skipif(not os.path.exists(q4.LIB_PATH), reason="libq4mi.so not built")

# A one-tensor file assembled by hand from the layout, byte by byte: version 3,
# 1 tensor, 1 metadata entry ("a": uint32 7), tensor "t" (1 dim of 2, F32,
# offset 0), zero padding to 96, then the floats 1.0 and -2.0.
HAND = bytes.fromhex(
    "47475546" "03000000" "0100000000000000" "0100000000000000"
    "0100000000000000" "61" "04000000" "07000000"
    "0100000000000000" "74" "01000000" "0200000000000000" "00000000" "0000000000000000"
    + "00" * 22 + "0000803f" "000000c0")


def _open_status(paths):
    enc = [os.fsencode(p) for p in paths]
    arr = (ctypes.c_char_p * len(enc))(*enc)
    h = ctypes.c_void_p()
    s = q4.lib().q4_gguf_open(ctypes.cast(arr, ctypes.c_void_p), len(enc), ctypes.byref(h))
    if s == q4.Q4_OK:
        q4.lib().q4_gguf_close(h)
    return s


def _write(tmp_path, blob, name="m.gguf"):
    p = str(tmp_path / name)
    with open(p, "wb") as f:
        f.write(blob)
    return p


def _model(alignment=32, version=3):
    """A small file with every metadata value type and the tensor types the
    reader sizes, including a Q4_0 weight encoded by the oracle."""
    rng = np.random.default_rng(11)
    wq = O.quantize_q4_0((rng.standard_normal((37, 96)) * 0.02).astype(np.float32))
    f32 = rng.standard_normal(5).astype(np.float32)
    f16 = rng.standard_normal((3, 4, 2)).astype(np.float16)
    bf = rng.integers(0, 1 << 16, size=64, dtype=np.uint16)
    q8 = rng.integers(0, 256, size=2 * 34 * 3, dtype=np.uint8)
    meta = [("general.architecture", W.STRING, "voxtral"),
            ("v.u8", W.U8, 200), ("v.i8", W.I8, -100), ("v.u16", W.U16, 60000),
            ("v.i16", W.I16, -30000), ("v.u32", W.U32, 4000000000), ("v.i32", W.I32, -2000000000),
            ("v.f32", W.F32, 0.375), ("v.bool", W.BOOL, 1), ("v.u64", W.U64, 1 << 60),
            ("v.i64", W.I64, -(1 << 60)), ("v.f64", W.F64, -1.0e-300),
            ("v.arr_i32", W.ARRAY, (W.I32, [1, -2, 3])),
            ("v.arr_str", W.ARRAY, (W.STRING, ["tok", "", "longer token"])),
            ("v.arr_empty", W.ARRAY, (W.F32, []))]
    if alignment != 32:
        meta.append(("general.alignment", W.U32, alignment))
    tensors = [("blk.0.attn_q.weight", (96, 37), W.T_Q4_0, wq.tobytes()),
               ("output_norm.weight", (5,), W.T_F32, f32.tobytes()),
               ("conv.weight", (2, 4, 3), W.T_F16, f16.tobytes()),
               ("bf.weight", (64,), W.T_BF16, bf.tobytes()),
               ("q8.weight", (64, 3), W.T_Q8_0, q8.tobytes()),
               ("strange.weight", (7,), 99, b"\1" * 7)]
    blob, start, offs = W.build(meta, tensors, alignment=alignment, version=version)
    return blob, start, offs, meta, tensors, wq


def test_writer_matches_hand_assembled_file():
    blob, start, offs = W.build([("a", W.U32, 7)],
                                [("t", (2,), W.T_F32, np.array([1.0, -2.0], "<f4").tobytes())])
    assert blob == HAND and start == 96 and offs == [0]


def test_hand_assembled_file(tmp_path):
    with q4.Gguf(_write(tmp_path, HAND)) as g:
        assert (g.version, g.alignment, g.data_offset) == (3, 32, 96)
        assert g.tensors == {"t": (W.T_F32, (2,), 0, 8)}
        assert g.metadata == [("a", W.U32)]
        assert g.meta_int("a") == 7
        assert np.array_equal(g.read("t").view("<f4"), [1.0, -2.0])


@pytest.mark.parametrize("alignment,version", [(32, 3), (64, 3), (256, 2), (1, 3)])
def test_round_trip(tmp_path, alignment, version):
    blob, start, offs, meta, tensors, wq = _model(alignment, version)
    with q4.Gguf(_write(tmp_path, blob)) as g:
        assert g.version == version and g.alignment == alignment and g.data_offset == start
        assert [k for k, _ in g.metadata] == [m[0] for m in meta]
        assert [t for _, t in g.metadata] == [m[1] for m in meta]
        for (name, dims, ttype, data), off in zip(tensors, offs):
            assert g.tensors[name] == (ttype, dims, off, W.tensor_nbytes(ttype, dims))
            if ttype == 99:
                with pytest.raises(q4.Q4Error):
                    g.read(name)
            else:
                assert g.read(name).tobytes() == data
        got = g.read("blk.0.attn_q.weight")
        assert got.shape == (37, O.row_bytes(96)) and np.array_equal(got, wq)
        assert g.meta_string("general.architecture") == "voxtral"
        for key, t, v in meta:
            if t in (W.U8, W.I8, W.U16, W.I16, W.U32, W.I32, W.U64, W.I64, W.BOOL):
                assert g.meta_int(key) == v, key
        assert g.meta_float("v.f32") == 0.375 and g.meta_float("v.f64") == -1.0e-300
        assert g.meta_array("v.arr_i32") == (W.I32, 3)
        assert g.meta_array("v.arr_str") == (W.STRING, 3)
        assert g.meta_array("v.arr_empty") == (W.F32, 0)


def test_metadata_type_and_lookup_errors(tmp_path):
    blob = _model()[0]
    with q4.Gguf(_write(tmp_path, blob)) as g:
        for fn, key in [(g.meta_int, "v.f32"), (g.meta_float, "v.i32"), (g.meta_string, "v.u8"),
                        (g.meta_array, "v.f64"), (g.meta_int, "general.architecture")]:
            with pytest.raises(q4.Q4Error, match="malformed"):
                fn(key)
        for fn in (g.meta_int, g.meta_float, g.meta_string, g.meta_array):
            with pytest.raises(q4.Q4Error, match="no such"):
                fn("absent.key")
        with pytest.raises(KeyError):
            g.read("absent.weight")
        L = q4.lib()
        assert L.q4_gguf_find_tensor(g._h, b"absent.weight") == -1
        assert L.q4_gguf_find_tensor(g._h, b"conv.weight") == 2
        assert L.q4_gguf_tensor_info(g._h, 6, None, None, None, None, None, None) == q4.Q4_ERR_NOT_FOUND
        assert L.q4_gguf_tensor_info(g._h, -1, None, None, None, None, None, None) == q4.Q4_ERR_NOT_FOUND
        assert L.q4_gguf_metadata_key(g._h, len(g.metadata), None, None) == q4.Q4_ERR_NOT_FOUND
        buf = np.empty(64, np.uint8)
        ptr = buf.ctypes.data_as(ctypes.c_void_p)
        assert L.q4_gguf_read_tensor(g._h, 1, ptr, 19) == q4.Q4_ERR_WORKSPACE
        assert L.q4_gguf_read_tensor(g._h, 1, ptr, 20) == q4.Q4_OK
        assert L.q4_gguf_read_tensor(g._h, 1, None, 20) == q4.Q4_ERR_NULL
    # NULL handles are refused, not dereferenced
    L = q4.lib()
    assert L.q4_gguf_version(None) == 0 and L.q4_gguf_tensor_count(None) == -1
    assert L.q4_gguf_metadata_count(None) == -1 and L.q4_gguf_find_tensor(None, b"x") == -1
    assert L.q4_gguf_tensor_info(None, 0, None, None, None, None, None, None) == q4.Q4_ERR_NULL
    L.q4_gguf_close(None)


@pytest.mark.parametrize("cuts", [[1], [5, 40], [100, 101, 1500], [24, 24, 700]])
def test_byte_split_shards(tmp_path, cuts):
    """Pieces cut anywhere (inside the magic, a string, a tensor, or empty
    pieces) read back exactly as the whole file."""
    blob, _, _, _, tensors, _ = _model()
    paths = W.write_shards(blob, str(tmp_path / "m.gguf"), cuts)
    with q4.Gguf(_write(tmp_path, blob, "whole.gguf")) as whole, q4.Gguf(paths) as split:
        assert split.tensors == whole.tensors and split.metadata == whole.metadata
        for name, _, ttype, _ in tensors:
            if ttype != 99:
                assert np.array_equal(split.read(name), whole.read(name))


def test_shards_of_at_most_512_mb_rule_in_miniature(tmp_path):
    """Equal-size pieces (the pages cut at a fixed size) with a last short one."""
    blob = _model()[0]
    size = 97
    cuts = list(range(size, len(blob), size))
    paths = W.write_shards(blob, str(tmp_path / "p.gguf"), cuts)
    assert all(os.path.getsize(p) <= size for p in paths) and len(paths) > 3
    with q4.Gguf(paths) as g:
        assert np.array_equal(g.read("blk.0.attn_q.weight"), _model()[5])


def test_open_errors(tmp_path):
    blob = _model()[0]
    good = _write(tmp_path, blob)
    assert _open_status([good]) == q4.Q4_OK
    assert _open_status([str(tmp_path / "missing.gguf")]) == q4.Q4_ERR_IO
    assert _open_status([good, str(tmp_path / "missing.gguf")]) == q4.Q4_ERR_IO
    h = ctypes.c_void_p()
    assert q4.lib().q4_gguf_open(None, 1, ctypes.byref(h)) == q4.Q4_ERR_NULL
    arr = (ctypes.c_char_p * 1)(os.fsencode(good))
    assert q4.lib().q4_gguf_open(ctypes.cast(arr, ctypes.c_void_p), 0, ctypes.byref(h)) == q4.Q4_ERR_NULL
    assert q4.lib().q4_gguf_open(ctypes.cast(arr, ctypes.c_void_p), 1, None) == q4.Q4_ERR_NULL
    with pytest.raises(q4.Q4Error, match="could not be opened"):
        q4.Gguf(str(tmp_path / "missing.gguf"))


def _bad(tmp_path, blob):
    return _open_status([_write(tmp_path, blob, "bad.gguf")])


def malformed_cases():
    """(name, bytes) of files the reader must refuse with Q4_ERR_FORMAT."""
    blob, start, offs, meta, tensors, _ = _model()
    out = [("magic", b"GGUX" + blob[4:]),
           ("version 1", blob[:4] + struct.pack("<I", 1) + blob[8:]),
           ("version 4", blob[:4] + struct.pack("<I", 4) + blob[8:]),
           ("empty", b"")]
    # every truncation inside the header or the data is refused
    for cut in sorted({3, 4, 8, 23, 24, 30, 100, start - 1, start, start + offs[-2] + 1}):
        out.append((f"cut {cut}", blob[:cut]))
    # absurd counts are refused before anything is allocated for them
    out.append(("tensor count 2^62", blob[:8] + struct.pack("<QQ", 1 << 62, 1) + blob[24:]))
    out.append(("metadata count 2^62", blob[:8] + struct.pack("<QQ", 1, 1 << 62) + blob[24:]))
    out.append(("misaligned offset",
                W.build(meta, tensors, offsets=[0, 2048, 4096, 6144, 8192, 10001])[0]))
    dup = [tensors[1], ("output_norm.weight",) + tensors[1][1:]]
    out.append(("duplicate names", W.build([], dup)[0]))
    out.append(("tensor past the end", W.build([], [tensors[1]], offsets=[64])[0][:-8]))
    # alignment that is not a power of two, or not an integer
    for a in (0, 24):
        out.append((f"alignment {a}", W.build([("general.alignment", W.U32, a)], [])[0]))
    out.append(("float alignment", W.build([("general.alignment", W.F32, 32.0)], [])[0]))
    # rank 0 and rank 5 tensors, a zero dimension
    for dims in [(), (1, 1, 1, 1, 32), (0, 32)]:
        out.append((f"dims {dims}", W.build([], [("x", dims, W.T_F32, b"")])[0]))
    # unknown metadata value type, bool outside {0, 1}, nested array
    raw = W.build([("k", W.U8, 1)], [])[0]
    out.append(("value type 13", raw[:24 + 8 + 1] + struct.pack("<I", 13) + raw[24 + 8 + 1 + 4:]))
    out.append(("bool 2", W.build([("k", W.U8, 2)], [])[0].replace(
        struct.pack("<IB", W.U8, 2), struct.pack("<IB", W.BOOL, 2))))
    out.append(("nested array", W.build([("k", W.ARRAY, (W.ARRAY, []))], [])[0]))
    return out


def test_malformed_headers(tmp_path):
    for name, blob in malformed_cases():
        assert _bad(tmp_path, blob) == q4.Q4_ERR_FORMAT, name


def test_empty_and_unpadded_files(tmp_path):
    """No tensors and no metadata; a file with no tensors may end unpadded."""
    blob = W.build([], [])[0]
    with q4.Gguf(_write(tmp_path, blob)) as g:
        assert g.tensors == {} and g.metadata == []
    blob = W.build([("general.name", W.STRING, "x")], [], pad_header=False)[0]
    with q4.Gguf(_write(tmp_path, blob, "u.gguf")) as g:
        assert g.meta_string("general.name") == "x" and g.data_offset == len(blob)


def test_q4_0_row_not_multiple_of_block(tmp_path):
    """A Q4_0 tensor whose rows are not whole blocks has no size: listed, not readable."""
    blob = W.build([], [("odd", (48, 2), W.T_Q4_0, b"\0" * 64)])[0]
    with q4.Gguf(_write(tmp_path, blob)) as g:
        assert g.tensors["odd"][3] == 0
        with pytest.raises(q4.Q4Error, match="malformed"):
            g.read("odd")
