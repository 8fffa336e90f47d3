"""q4_quantized_speech_amd -- GGUF Q4_0 hot path for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libq4mi.so`` (declared in
``include/q4.h``).  PyTorch supplies device memory and the current HIP stream;
every computation runs in the library's HIP kernels.  There is no CPU
fallback: if the library is not built, every entry point raises.

Entry points (same names as the C ABI, minus the ``q4_`` prefix):
    matvec(w_q4, x, out=None)                    y = deq(W) x          (M <= 8)
    matmul(w_q4, x, out=None, workspace=True)    Y = X deq(W)^T        (matrix cores)
    matmul_residual(w_q4, x, r, out=None, ...)   Y = R + X deq(W)^T   (fused epilogue)
    embed_rows(table_q4, ids, out=None)          rows of deq(T)
    lmhead_argmax(w_q4, x, workspace=None, ...)  argmax_n (deq(T) x)_n
    quantize(w, out=None, check=True)            float32 -> Q4_0 bytes

Q4_0 tensors are ``torch.uint8`` of shape [N, 18*K/32] (rows of 32-weight
blocks: binary16 scale + 16 bytes of nibbles, as stored in GGUF).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4mi.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "q4.h")

QK = 32
BLOCK_BYTES = 18

(Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_ALIGN, Q4_ERR_WORKSPACE, Q4_ERR_HIP, Q4_ERR_FORMAT,
 Q4_ERR_IO, Q4_ERR_NOT_FOUND) = range(9)


class Q4Error(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        msg = f"{where}: {status_string(status)} (status {status}"
        if status == Q4_ERR_HIP:
            msg += f", hipError {hip_error}"
        super().__init__(msg + ")")
        self.status = status
        self.hip_error = hip_error


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SIGS = {
    "q4_abi_version": ([], ctypes.c_int),
    "q4_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "q4_last_hip_error": ([], ctypes.c_int),
    "q4_row_bytes": ([_I64], _SZ),
    "q4_matvec": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "q4_matmul_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "q4_matmul": ([_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], ctypes.c_int),
    "q4_matmul_residual_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "q4_matmul_residual": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], ctypes.c_int),
    "q4_embed_rows": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "q4_lmhead_argmax_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "q4_lmhead_argmax": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], ctypes.c_int),
    "q4_quantize": ([_P, _P, _I64, _I64, _P, _P], ctypes.c_int),
    "q4_lmhead_argmax_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "q4_decode_chain": ([_P, _I64, _P, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "q4_matmul_route": ([_I64, _I64, _I64, _SZ, _P], ctypes.c_char_p),
    "q4_matvec_route": ([_I64, _I64, ctypes.c_int32], ctypes.c_char_p),
    "q4_gguf_open": ([_P, _I64, _P], ctypes.c_int),
    "q4_gguf_close": ([_P], None),
    "q4_gguf_version": ([_P], ctypes.c_uint32),
    "q4_gguf_alignment": ([_P], ctypes.c_uint64),
    "q4_gguf_data_offset": ([_P], ctypes.c_uint64),
    "q4_gguf_tensor_count": ([_P], _I64),
    "q4_gguf_metadata_count": ([_P], _I64),
    "q4_gguf_tensor_info": ([_P, _I64, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "q4_gguf_find_tensor": ([_P, ctypes.c_char_p], _I64),
    "q4_gguf_read_tensor": ([_P, _I64, _P, ctypes.c_uint64], ctypes.c_int),
    "q4_gguf_metadata_key": ([_P, _I64, _P, _P], ctypes.c_int),
    "q4_gguf_metadata_int": ([_P, ctypes.c_char_p, _P], ctypes.c_int),
    "q4_gguf_metadata_float": ([_P, ctypes.c_char_p, _P], ctypes.c_int),
    "q4_gguf_metadata_string": ([_P, ctypes.c_char_p, _P, _P], ctypes.c_int),
    "q4_gguf_metadata_array": ([_P, ctypes.c_char_p, _P, _P], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """Load libq4mi.so (built in-tree by q4_quantized_speech_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m q4_quantized_speech_amd.build` "
                "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().q4_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != Q4_OK:
        raise Q4Error(status, where, lib().q4_last_hip_error() if status == Q4_ERR_HIP else 0)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which tensors this module allocates (outputs, workspaces,
    flags) come from ``stream``'s pool and their fills run on ``stream``: the
    library's kernel runs there, so nothing else orders them before it, and
    a buffer freed back to another stream's pool could be reused by that
    stream while the kernel still writes it.  The caller orders its own
    inputs with ``stream``."""
    import contextlib
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def q4_shape(w_q4: torch.Tensor):
    """(N, K) of a Q4_0 tensor of shape [N, 18*K/32]."""
    if w_q4.dtype != torch.uint8 or w_q4.dim() != 2 or not w_q4.is_contiguous():
        raise ValueError("Q4_0 weights must be a contiguous uint8 tensor [N, 18*K/32]")
    n, rb = w_q4.shape
    if rb % BLOCK_BYTES:
        raise ValueError(f"row length {rb} is not a multiple of {BLOCK_BYTES}")
    return n, rb // BLOCK_BYTES * QK


def row_bytes(k: int) -> int:
    return int(lib().q4_row_bytes(k))


def _as_2d_f32(x: torch.Tensor, k: int) -> torch.Tensor:
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("activations must be contiguous float32")
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"activations must be [M, {k}]")
    return x


def matvec(w_q4: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """y[m, n] = sum_k deq(W)[n, k] x[m, k] (float32 FMA path); x is [K] or [M, K]."""
    n, k = q4_shape(w_q4)
    squeeze = x.dim() == 1
    x2 = _as_2d_f32(x, k)
    m = x2.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=x.device)
        _need_cuda(w_q4, x2, out)
        _check(lib().q4_matvec(_ptr(w_q4), _ptr(x2), _ptr(out), m, n, k, _stream(stream)),
               "q4_matvec")
    return out.view(n) if squeeze else out


def matmul_workspace(m: int, n: int, k: int, device) -> torch.Tensor | None:
    """A workspace for matmul's K split on the current device (None if no split is planned)."""
    nbytes = int(lib().q4_matmul_workspace_bytes(m, n, k))
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def matmul(w_q4: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None | bool = True, stream=None):
    """Y = X deq(W)^T.  M >= 5: on the matrix cores with binary16 operands and
    float32 accumulation.  M <= 4: q4_matvec's bound, either through the matvec
    kernel (rows of x in pairs) or with exact weights and a two-part x on the
    matrix cores.

    ``workspace``: a uint8 device tensor for the K split, ``True`` to allocate the
    planned size here, or ``None``/``False`` for no split."""
    n, k = q4_shape(w_q4)
    x2 = _as_2d_f32(x, k)
    m = x2.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=x.device)
        if workspace is True:
            workspace = matmul_workspace(m, n, k, x.device)
        elif workspace is False:
            workspace = None
        _need_cuda(w_q4, x2, out, workspace)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().q4_matmul(_ptr(w_q4), _ptr(x2), _ptr(out), m, n, k, _ptr(workspace), ws_bytes,
                               _stream(stream)), "q4_matmul")
    return out


def matmul_residual_workspace(m: int, n: int, k: int, device) -> torch.Tensor | None:
    """A workspace that covers matmul_residual for the shape on the current
    device, in place or not (None if none is needed)."""
    nbytes = int(lib().q4_matmul_residual_workspace_bytes(m, n, k))
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def matmul_residual(w_q4: torch.Tensor, x: torch.Tensor, r: torch.Tensor,
                    out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None | bool = True, stream=None):
    """Y = R + X deq(W)^T, the add fused into the product's epilogue where
    the route allows (bit for bit R + matmul(...) in float32).  ``out`` may be
    ``r`` itself (in place).  ``workspace`` as for matmul; ``True`` allocates
    what the shape needs, in place included."""
    n, k = q4_shape(w_q4)
    x2 = _as_2d_f32(x, k)
    m = x2.shape[0]
    if r.dtype != torch.float32 or tuple(r.shape) != (m, n) or not r.is_contiguous():
        raise ValueError(f"r must be a contiguous float32 [{m}, {n}] tensor")
    with _on(stream):
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=x.device)
        if workspace is True:
            workspace = matmul_residual_workspace(m, n, k, x.device)
        elif workspace is False:
            workspace = None
        _need_cuda(w_q4, x2, r, out, workspace)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().q4_matmul_residual(_ptr(w_q4), _ptr(x2), _ptr(r), _ptr(out), m, n, k,
                                        _ptr(workspace), ws_bytes, _stream(stream)),
               "q4_matmul_residual")
    return out


def matmul_route(m: int, n: int, k: int, ws_bytes: int = 0):
    """(kernel name, K splits) q4_matmul takes for the shape and workspace size."""
    sp = ctypes.c_int32(0)
    r = lib().q4_matmul_route(m, n, k, ws_bytes, ctypes.byref(sp))
    if r is None:
        raise ValueError(f"q4_matmul rejects M={m} N={n} K={k}")
    return r.decode(), int(sp.value)


def matvec_route(n: int, k: int, argmax: bool = False) -> str:
    """Kernel variant q4_matvec (or q4_lmhead_argmax) takes for an N x K matrix."""
    r = lib().q4_matvec_route(n, k, 1 if argmax else 0)
    if r is None:
        raise ValueError(f"rejected shape N={n} K={k}")
    return r.decode()


def embed_rows(table_q4: torch.Tensor, ids: torch.Tensor, out: torch.Tensor | None = None,
               stream=None):
    """out[i, :] = deq(T)[ids[i], :]; ids outside [0, N) give zero rows."""
    n, k = q4_shape(table_q4)
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 vector")
    m = ids.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty((m, k), dtype=torch.float32, device=ids.device)
        _need_cuda(table_q4, ids, out)
        _check(lib().q4_embed_rows(_ptr(table_q4), _ptr(ids), _ptr(out), m, n, k, _stream(stream)),
               "q4_embed_rows")
    return out


def lmhead_workspace(m: int, device) -> torch.Tensor:
    """A zeroed workspace for lmhead_argmax; each call leaves it zeroed, so it
    can be reused by calls ordered on one stream."""
    nbytes = int(lib().q4_lmhead_argmax_workspace_bytes(m, 0, 0))
    if nbytes == 0:
        raise ValueError("M out of range for lmhead_argmax")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def lmhead_argmax(w_q4: torch.Tensor, x: torch.Tensor, workspace: torch.Tensor | None = None,
                  out_idx: torch.Tensor | None = None, out_val: torch.Tensor | None = None,
                  stream=None):
    """(idx, val): per row of x, the lowest n maximising (deq(T) x)_n and that maximum."""
    n, k = q4_shape(w_q4)
    x2 = _as_2d_f32(x, k)
    m = x2.shape[0]
    with _on(stream):
        if workspace is None:
            workspace = lmhead_workspace(m, x.device)   # zero-filled on `stream`
        if out_idx is None:
            out_idx = torch.empty(m, dtype=torch.int32, device=x.device)
        if out_val is None:
            out_val = torch.empty(m, dtype=torch.float32, device=x.device)
        _need_cuda(w_q4, x2, workspace, out_idx, out_val)
        _check(lib().q4_lmhead_argmax(_ptr(w_q4), _ptr(x2), _ptr(out_idx), _ptr(out_val), m, n, k,
                                      _ptr(workspace), workspace.numel(), _stream(stream)),
               "q4_lmhead_argmax")
    return out_idx, out_val


class _Step(ctypes.Structure):
    _fields_ = [("w_q4", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


def decode_chain(steps, table_q4: torch.Tensor | None = None, head_x: torch.Tensor | None = None,
                 out_idx: torch.Tensor | None = None, out_val: torch.Tensor | None = None,
                 out_embed: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None):
    """One decode step's Q4_0 work in order on one stream: ``steps`` is a list
    of (w_q4, x, y) matvecs at M = 1 (x may be a view into an earlier y), then,
    with ``table_q4``, the argmax over deq(T) head_x and, with ``out_embed``,
    the chosen token's decoded row.  Returns (out_idx, out_val, out_embed)."""
    arr = (_Step * max(1, len(steps)))()
    keep = []
    for i, (w, x, y) in enumerate(steps):
        n, k = q4_shape(w)
        if x.dtype != torch.float32 or x.dim() != 1 or x.shape[0] != k or not x.is_contiguous():
            raise ValueError(f"step {i}: x must be a contiguous float32 vector of {k}")
        if y.dtype != torch.float32 or y.dim() != 1 or y.shape[0] != n or not y.is_contiguous():
            raise ValueError(f"step {i}: y must be a contiguous float32 vector of {n}")
        _need_cuda(w, x, y)
        arr[i] = _Step(w.data_ptr(), x.data_ptr(), y.data_ptr(), n, k)
        keep.append((w, x, y))
    vocab = dim = 0
    with _on(stream):
        if table_q4 is not None:
            vocab, dim = q4_shape(table_q4)
            if head_x is None or head_x.dtype != torch.float32 or head_x.numel() != dim \
                    or not head_x.is_contiguous():
                raise ValueError(f"head_x must be a contiguous float32 vector of {dim}")
            if workspace is None:
                workspace = lmhead_workspace(1, head_x.device)
            if out_idx is None:
                out_idx = torch.empty(1, dtype=torch.int32, device=head_x.device)
            _need_cuda(table_q4, head_x, out_idx, out_val, out_embed, workspace)
        ws_bytes = 0 if workspace is None else workspace.numel()
        _check(lib().q4_decode_chain(ctypes.cast(arr, ctypes.c_void_p), len(steps), _ptr(table_q4),
                                     vocab, dim, _ptr(head_x), _ptr(out_idx), _ptr(out_val),
                                     _ptr(out_embed), _ptr(workspace), ws_bytes, _stream(stream)),
               "q4_decode_chain")
    return out_idx, out_val, out_embed


def lmhead_argmax_noalloc(w_q4: torch.Tensor, x: torch.Tensor, out_idx: torch.Tensor,
                          out_val: torch.Tensor | None = None, stream=None):
    """lmhead_argmax with the library's own scratch: the caller passes the
    outputs, nothing is allocated (M <= 64; calls on one GPU must be ordered)."""
    n, k = q4_shape(w_q4)
    x2 = _as_2d_f32(x, k)
    m = x2.shape[0]
    _need_cuda(w_q4, x2, out_idx, out_val)
    if out_idx.dtype != torch.int32 or out_idx.numel() < m or not out_idx.is_contiguous():
        raise ValueError("out_idx must be a contiguous int32 tensor of at least M entries")
    if out_val is not None and (out_val.dtype != torch.float32 or out_val.numel() < m
                                or not out_val.is_contiguous()):
        raise ValueError("out_val must be a contiguous float32 tensor of at least M entries")
    _check(lib().q4_lmhead_argmax_noalloc(_ptr(w_q4), _ptr(x2), _ptr(out_idx), _ptr(out_val), m,
                                          n, k, _stream(stream)), "q4_lmhead_argmax_noalloc")
    return out_idx, out_val


def quantize(w: torch.Tensor, out: torch.Tensor | None = None, check: bool = True, stream=None):
    """GGUF Q4_0 encoding of a float32 [N, K] tensor on the GPU."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 [N, K] tensor")
    n, k = w.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    with _on(stream):
        if out is None:
            out = torch.empty((n, k // QK * BLOCK_BYTES), dtype=torch.uint8, device=w.device)
        flag = torch.zeros(4, dtype=torch.int32, device=w.device) if check else None
        _need_cuda(w, out, flag)
        _check(lib().q4_quantize(_ptr(w), _ptr(out), n, k, _ptr(flag), _stream(stream)),
               "q4_quantize")
        # the copy behind item() runs on `stream`, after the kernel
        bad = check and int(flag[0].item()) != 0
    if bad:
        raise ValueError("q4_quantize: non-finite input or a scale overflowing binary16")
    return out


GGUF_F32, GGUF_F16, GGUF_Q4_0, GGUF_Q8_0, GGUF_BF16 = 0, 1, 2, 8, 30


class Gguf:
    """A GGUF file (or the ordered byte pieces of one) opened with the
    library's reader.  ``tensors`` maps name -> (type, dims, offset, nbytes)
    with dims innermost first; ``read(name)`` returns the tensor's bytes as a
    numpy uint8 array (a Q4_0 weight of N rows of K as [N, 18*K/32])."""

    def __init__(self, paths):
        if isinstance(paths, (str, os.PathLike)):
            paths = [paths]
        enc = [os.fsencode(p) for p in paths]
        arr = (ctypes.c_char_p * len(enc))(*enc)
        h = ctypes.c_void_p()
        _check(lib().q4_gguf_open(ctypes.cast(arr, ctypes.c_void_p), len(enc), ctypes.byref(h)),
               "q4_gguf_open")
        self._h = h
        self.version = int(lib().q4_gguf_version(h))
        self.alignment = int(lib().q4_gguf_alignment(h))
        self.data_offset = int(lib().q4_gguf_data_offset(h))
        self.tensors = {}
        for i in range(int(lib().q4_gguf_tensor_count(h))):
            name, typ, nd = ctypes.c_char_p(), ctypes.c_uint32(), ctypes.c_uint32()
            dims, off, nb = (ctypes.c_int64 * 4)(), ctypes.c_uint64(), ctypes.c_uint64()
            _check(lib().q4_gguf_tensor_info(h, i, ctypes.byref(name), ctypes.byref(typ),
                                             ctypes.byref(nd), dims, ctypes.byref(off),
                                             ctypes.byref(nb)), "q4_gguf_tensor_info")
            self.tensors[name.value.decode()] = (int(typ.value), tuple(dims[: nd.value]),
                                                 int(off.value), int(nb.value))
        self.metadata = []
        for i in range(int(lib().q4_gguf_metadata_count(h))):
            key, vt = ctypes.c_char_p(), ctypes.c_uint32()
            _check(lib().q4_gguf_metadata_key(h, i, ctypes.byref(key), ctypes.byref(vt)),
                   "q4_gguf_metadata_key")
            self.metadata.append((key.value.decode(), int(vt.value)))

    def close(self):
        if self._h:
            lib().q4_gguf_close(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass

    def read(self, name: str):
        import numpy as np
        i = int(lib().q4_gguf_find_tensor(self._h, name.encode()))
        if i < 0:
            raise KeyError(name)
        typ, dims, _, nbytes = self.tensors[name]
        out = np.empty(nbytes, dtype=np.uint8)
        _check(lib().q4_gguf_read_tensor(self._h, i, out.ctypes.data_as(ctypes.c_void_p), nbytes),
               "q4_gguf_read_tensor")
        if typ == GGUF_Q4_0 and len(dims) == 2:
            return out.reshape(dims[1], dims[0] // QK * BLOCK_BYTES)
        return out

    def meta_int(self, key: str) -> int:
        v = ctypes.c_int64()
        _check(lib().q4_gguf_metadata_int(self._h, key.encode(), ctypes.byref(v)), "q4_gguf_metadata_int")
        return int(v.value)

    def meta_float(self, key: str) -> float:
        v = ctypes.c_double()
        _check(lib().q4_gguf_metadata_float(self._h, key.encode(), ctypes.byref(v)), "q4_gguf_metadata_float")
        return float(v.value)

    def meta_string(self, key: str) -> str:
        v, n = ctypes.c_char_p(), ctypes.c_uint64()
        _check(lib().q4_gguf_metadata_string(self._h, key.encode(), ctypes.byref(v), ctypes.byref(n)),
               "q4_gguf_metadata_string")
        return ctypes.string_at(v, n.value).decode()

    def meta_array(self, key: str):
        t, n = ctypes.c_uint32(), ctypes.c_uint64()
        _check(lib().q4_gguf_metadata_array(self._h, key.encode(), ctypes.byref(t), ctypes.byref(n)),
               "q4_gguf_metadata_array")
        return int(t.value), int(n.value)


def declared_symbols(header: str = HEADER):
    """Function names declared in include/q4.h."""
    import re
    with open(header) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text)))
