"""Lossless fixed-codebook entropy coding of e4m3 tensor bytes on MI355X.

Thin ctypes binding of ``libec.so`` (C ABI in ``include/ec.h``).  This module
only marshals arguments: every step of the path runs in the library's HIP
kernels or its host codebook builders.  PyTorch provides device memory and
streams.  There is no CPU fallback: if ``libec.so`` is missing the import of
an entry point raises.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libec binds to the HIP runtime torch already mapped

__all__ = [
    "Codebook", "ECError", "lib", "encode", "encode_noalloc", "decode", "encode_batch", "decode_batch",
    "byte_histogram", "pmf_average", "pmf_kl", "huff_code_lengths", "index_bytes",
    "max_encoded_bytes", "QLC_BASE", "QLC_ADAPTED", "CODEC_QLC", "CODEC_HUFFMAN",
    "CODEC_EXP_GOLOMB", "S_CAPACITY", "S_CORRUPT", "S_BAD_HEADER", "S_CODEBOOK_MISMATCH",
    "S_BAD_CODEBOOK", "EXPORTS", "device_codebook_bytes", "build_huffman_device", "own_max_encoded_bytes",
    "encode_batch_device", "decode_batch_device", "huffman_tables_from_streams", "qlc_optimal_area_layout",
    "bf16_exp_table_from_counts", "bf16_exp_table_from_sigma", "bf16_exp_max_encoded_bytes", "bf16_exp_encode",
    "bf16_exp_decode", "byte_histogram_sized", "encode_sized", "encode_batch_sized",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libec.so")

CODEC_QLC, CODEC_HUFFMAN, CODEC_EXP_GOLOMB = 1, 2, 3
S_CAPACITY, S_CORRUPT, S_BAD_HEADER, S_CODEBOOK_MISMATCH, S_BAD_CODEBOOK = 0x1, 0x2, 0x4, 0x8, 0x10
MAX_BATCH = 128

# QLC area layouts (symbols per area, suffix bits per area)
QLC_BASE = ((8, 8, 8, 8, 8, 16, 32, 168), (3, 3, 3, 3, 3, 4, 5, 8))
QLC_ADAPTED = ((2, 8, 8, 8, 8, 16, 32, 174), (1, 3, 3, 3, 3, 4, 5, 8))

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_int = ctypes.c_int

# name -> (restype, argtypes); every function declared in include/ec.h
EXPORTS = {
    "qlc_build_codebook": (_int, [_u64p, _u16p, _u8p, ctypes.POINTER(_vp)]),
    "qlc_optimal_area_layout": (_int, [_u64p, _u32, _u16p, _u8p]),
    "huff_build_codebook": (_int, [_u64p, ctypes.POINTER(_vp)]),
    "huff_build_codebook_from_lengths": (_int, [_u8p, ctypes.POINTER(_vp)]),
    "eg_build_codebook": (_int, [_u64p, _int, ctypes.POINTER(_vp)]),
    "huff_code_lengths": (_int, [_u64p, _u32, _u8p]),
    "ec_codebook_info": (_int, [_vp, _u32p, _u32p, _u64p, _u8p, _u64p, _u8p, _i32p]),
    "ec_codebook_free": (None, [_vp]),
    "entropy_index_bytes": (_u64, [_u64, _u32, _u32]),
    "entropy_max_encoded_bytes": (_u64, [_vp, _u64, _u32, _u32]),
    "entropy_encode": (_int, [_vp, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _vp]),
    "entropy_encode_noalloc": (_int, [_vp, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _vp]),
    "entropy_decode": (_int, [_vp, _vp, _u64, _vp, _u64, _vp, _vp]),
    "entropy_encode_sized": (_int, [_vp, _vp, _u64, _u32, _vp, _vp, _u64, _vp, _vp, _vp]),
    "entropy_encode_batch_sized": (_int, [ctypes.POINTER(_vp), _u32, _vp, _u64, _u64, _u32, _u32, _vp, _vp, _u64,
                                          _vp, _vp, _vp]),
    "entropy_encode_batch": (_int, [ctypes.POINTER(_vp), _u32, _vp, _u64, _u64, _u32, _u32, _vp, _u64, _vp,
                                    _vp, _vp]),
    "entropy_decode_batch": (_int, [ctypes.POINTER(_vp), _u32, _vp, _u64, _vp, _u64, _u64, _vp, _vp]),
    "ec_device_codebook_bytes": (_u64, []),
    "huff_build_codebooks_device": (_int, [_vp, _u32, _vp, _vp, _vp]),
    "ec_codebook_export": (_int, [_vp, _vp]),
    "huff_tables_from_streams_device": (_int, [_vp, _u64, _u64, _u32, _vp, _vp, _vp]),
    "entropy_own_max_encoded_bytes": (_u64, [_u64, _u32, _u32]),
    "entropy_encode_batch_device": (_int, [_vp, _u32, _vp, _u64, _u64, _u32, _u32, _vp, _u64, _vp, _vp, _vp]),
    "entropy_decode_batch_device": (_int, [_vp, _u32, _u32, _vp, _u64, _vp, _u64, _u64, _vp, _vp]),
    "byte_histogram": (_int, [_vp, _u64, _u32, _u64, _vp, _vp]),
    "byte_histogram_sized": (_int, [_vp, _u64, _u32, _u64, _vp, ctypes.POINTER(_vp), _u32, _u32, _vp, _vp]),
    "pmf_average": (_int, [_vp, _u32, _vp, _vp]),
    "pmf_kl": (_int, [_vp, _u32, _vp, _u32, _vp, _vp]),
    "bf16_exp_table_from_counts": (_int, [_u64p, _u8p]),
    "bf16_exp_table_from_sigma": (_int, [ctypes.c_double, _u8p]),
    "bf16_exp_max_encoded_bytes": (_u64, [_u64, _u32]),
    "bf16_exp_encode": (_int, [_u8p, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _vp]),
    "bf16_exp_decode": (_int, [_vp, _u64, _vp, _u64, _vp, _vp]),
    "ec_error_string": (ctypes.c_char_p, [_int]),
    "ec_status_string": (ctypes.c_char_p, [_u32]),
}

_lib = None


class ECError(RuntimeError):
    pass


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def lib() -> ctypes.CDLL:
    """Load libec.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ECError("libec.so is not built (run __graft_entry__.build() or "
                          "python -m lossless_entropy_coding_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        rts = _hip_runtimes_mapped()
        if len(rts) > 1:
            raise ECError("two HIP runtimes are mapped (%s); import torch before libec" % rts)
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise ECError("%s failed: %s (%d)" % (what, lib().ec_error_string(rc).decode(), rc))


def _arr(ctype, values):
    values = [int(v) for v in values]
    return (ctype * len(values))(*values)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


# The current stream's raw handle straight from torch's C layer: building a
# torch.cuda.Stream object for it costs about 3 us a call, more than a kernel
# launch (public API as the fallback).
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_CUR_DEVICE = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream) -> int | None:
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is not None and _CUR_DEVICE is not None:
        return _RAW_STREAM(_CUR_DEVICE())
    return torch.cuda.current_stream().cuda_stream


def _u8_cuda(t: torch.Tensor, name: str):
    if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
        raise ECError("%s must be a contiguous uint8 CUDA tensor" % name)


class Codebook:
    """A library-owned codebook handle (ec_codebook)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self):
        return self._h

    @classmethod
    def qlc(cls, counts, area_size=QLC_BASE[0], suffix_bits=QLC_BASE[1]) -> "Codebook":
        h = ctypes.c_void_p()
        _check(lib().qlc_build_codebook(_arr(ctypes.c_uint64, counts), _arr(ctypes.c_uint16, area_size),
                                        _arr(ctypes.c_uint8, suffix_bits), ctypes.byref(h)),
               "qlc_build_codebook")
        return cls(h.value)

    @classmethod
    def huffman(cls, counts) -> "Codebook":
        h = ctypes.c_void_p()
        _check(lib().huff_build_codebook(_arr(ctypes.c_uint64, counts), ctypes.byref(h)), "huff_build_codebook")
        return cls(h.value)

    @classmethod
    def huffman_from_lengths(cls, lengths) -> "Codebook":
        h = ctypes.c_void_p()
        _check(lib().huff_build_codebook_from_lengths(_arr(ctypes.c_uint8, lengths), ctypes.byref(h)),
               "huff_build_codebook_from_lengths")
        return cls(h.value)

    @classmethod
    def exp_golomb(cls, counts, k: int = -1) -> "Codebook":
        h = ctypes.c_void_p()
        _check(lib().eg_build_codebook(_arr(ctypes.c_uint64, counts), int(k), ctypes.byref(h)),
               "eg_build_codebook")
        return cls(h.value)

    def info(self) -> dict:
        codec, mx = ctypes.c_uint32(), ctypes.c_uint32()
        cid = ctypes.c_uint64()
        lens = (ctypes.c_uint8 * 256)()
        code = (ctypes.c_uint64 * 256)()
        r2s = (ctypes.c_uint8 * 256)()
        k = ctypes.c_int32()
        _check(lib().ec_codebook_info(self._h, ctypes.byref(codec), ctypes.byref(mx), ctypes.byref(cid), lens,
                                      code, r2s, ctypes.byref(k)), "ec_codebook_info")
        return dict(codec=codec.value, max_len=mx.value, codebook_id=cid.value, code_len=list(lens),
                    code=list(code), rank_to_sym=list(r2s), eg_k=k.value)

    def export(self) -> bytes:
        """The codebook's table in the device table format (ec_codebook_export)."""
        buf = (ctypes.c_uint8 * device_codebook_bytes())()
        _check(lib().ec_codebook_export(self._h, buf), "ec_codebook_export")
        return bytes(buf)

    @property
    def codec(self) -> int:
        return self.info()["codec"]

    @property
    def max_len(self) -> int:
        return self.info()["max_len"]

    @property
    def codebook_id(self) -> int:
        return self.info()["codebook_id"]

    def free(self):
        if self._h and self._h.value:
            lib().ec_codebook_free(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def qlc_optimal_area_layout(counts, max_lengths: int = 4):
    """(area_size, suffix_bits) of the cheapest QLC layout for these counts
    with at most ``max_lengths`` distinct code lengths."""
    n = (ctypes.c_uint16 * 8)()
    b = (ctypes.c_uint8 * 8)()
    _check(lib().qlc_optimal_area_layout(_arr(ctypes.c_uint64, counts), int(max_lengths), n, b),
           "qlc_optimal_area_layout")
    return tuple(int(v) for v in n), tuple(int(v) for v in b)


def huff_code_lengths(weights) -> list:
    n = len(weights)
    out = (ctypes.c_uint8 * n)()
    _check(lib().huff_code_lengths(_arr(ctypes.c_uint64, weights), n, out), "huff_code_lengths")
    return list(out)


# ----------------------------------------------------- BF16 exponent coding

def _bf16_cuda(t: torch.Tensor, name: str):
    if not (t.is_cuda and t.is_contiguous() and t.element_size() == 2):
        raise ECError("%s must be a contiguous CUDA tensor of 2-byte elements (BF16 bit patterns)" % name)


def bf16_exp_table_from_counts(counts) -> tuple:
    """The seven most frequent exponents (counts[e] for exponent e)."""
    t = (ctypes.c_uint8 * 7)()
    _check(lib().bf16_exp_table_from_counts(_arr(ctypes.c_uint64, counts), t), "bf16_exp_table_from_counts")
    return tuple(int(v) for v in t)


def bf16_exp_table_from_sigma(sigma: float) -> tuple:
    """The seven exponents of largest N(0, sigma^2) octave mass."""
    t = (ctypes.c_uint8 * 7)()
    _check(lib().bf16_exp_table_from_sigma(float(sigma), t), "bf16_exp_table_from_sigma")
    return tuple(int(v) for v in t)


def bf16_exp_max_encoded_bytes(n: int, chunk: int = 16384) -> int:
    return int(lib().bf16_exp_max_encoded_bytes(n, chunk))


def bf16_exp_encode(table, x: torch.Tensor, chunk: int = 16384, out: torch.Tensor | None = None,
                    out_len: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """bf16_exp_encode.  Returns (out buffer, out_len int64[1], status int32[1])."""
    _bf16_cuda(x, "x")
    n = x.numel()
    dev = x.device
    if out is None:
        out = torch.empty(bf16_exp_max_encoded_bytes(n, chunk), dtype=torch.uint8, device=dev)
    if out_len is None:
        out_len = torch.zeros(1, dtype=torch.int64, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(lib().bf16_exp_encode(_arr(ctypes.c_uint8, table), _ptr(x), n, chunk, _ptr(out), out.numel(),
                                 _ptr(out_len), _ptr(status), _stream(stream)), "bf16_exp_encode")
    return out, out_len, status


def bf16_exp_decode(data: torch.Tensor, n: int, out: torch.Tensor | None = None,
                    status: torch.Tensor | None = None, in_len: int | None = None, stream=None):
    """bf16_exp_decode.  Returns (out bfloat16[n], status int32[1])."""
    _u8_cuda(data, "data")
    if out is None:
        out = torch.empty(max(n, 8), dtype=torch.bfloat16, device=data.device)[:n]
    _bf16_cuda(out, "out")
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=data.device)
    _check(lib().bf16_exp_decode(_ptr(data), data.numel() if in_len is None else in_len, _ptr(out), n,
                                 _ptr(status), _stream(stream)), "bf16_exp_decode")
    return out, status


def index_bytes(n: int, chunk_symbols: int, embed_lengths: bool = False) -> int:
    return int(lib().entropy_index_bytes(n, chunk_symbols, int(embed_lengths)))


def max_encoded_bytes(cb: Codebook, n: int, chunk_symbols: int, embed_lengths: bool = False) -> int:
    return int(lib().entropy_max_encoded_bytes(cb.handle, n, chunk_symbols, int(embed_lengths)))


def encode(cb: Codebook, x: torch.Tensor, chunk_symbols: int, out: torch.Tensor | None = None,
           out_len: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """entropy_encode.  Returns (out buffer, out_len int64[1], status int32[1]);
    the stream is out[:out_len] once the stream has synchronised."""
    _u8_cuda(x, "x")
    n = x.numel()
    if out is None:
        out = torch.empty(max_encoded_bytes(cb, n, chunk_symbols), dtype=torch.uint8, device=x.device)
    if out_len is None:
        out_len = torch.zeros(1, dtype=torch.int64, device=x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().entropy_encode(cb.handle, _ptr(x), n, chunk_symbols, _ptr(out), out.numel(), _ptr(out_len),
                                _ptr(status), _stream(stream)), "entropy_encode")
    return out, out_len, status


def encode_sized(cb: Codebook, x: torch.Tensor, chunk_symbols: int, sizes: torch.Tensor,
                 out: torch.Tensor | None = None, out_len: torch.Tensor | None = None,
                 status: torch.Tensor | None = None, stream=None):
    """entropy_encode_sized: entropy_encode with the chunk sizes that
    byte_histogram_sized made for cb (its int32 row, ceil(n / chunk_symbols)
    entries).  Returns (out, out_len, status)."""
    _u8_cuda(x, "x")
    n = x.numel()
    if out is None:
        out = torch.empty(max_encoded_bytes(cb, n, chunk_symbols), dtype=torch.uint8, device=x.device)
    if out_len is None:
        out_len = torch.zeros(1, dtype=torch.int64, device=x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _check(lib().entropy_encode_sized(cb.handle, _ptr(x), n, chunk_symbols, _ptr(sizes), _ptr(out), out.numel(),
                                      _ptr(out_len), _ptr(status), _stream(stream)), "entropy_encode_sized")
    return out, out_len, status


def encode_noalloc(cb: Codebook, x: torch.Tensor, chunk_symbols: int, out: torch.Tensor,
                   out_len: torch.Tensor, status: torch.Tensor | None = None, stream=None):
    """entropy_encode_noalloc: entropy_encode into caller buffers, with no
    allocation in the library (the codebook must have been used on this
    device before).  Returns (out, out_len, status)."""
    _u8_cuda(x, "x")
    _check(lib().entropy_encode_noalloc(cb.handle, _ptr(x), x.numel(), chunk_symbols, _ptr(out), out.numel(),
                                        _ptr(out_len), _ptr(status), _stream(stream)), "entropy_encode_noalloc")
    return out, out_len, status


def decode(cb: Codebook, data: torch.Tensor, n: int, out: torch.Tensor | None = None,
           status: torch.Tensor | None = None, in_len: int | None = None, stream=None):
    """entropy_decode.  Returns (out uint8[n], status int32[1])."""
    _u8_cuda(data, "data")
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.uint8, device=data.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=data.device)
    _check(lib().entropy_decode(cb.handle, _ptr(data), data.numel() if in_len is None else in_len, _ptr(out), n,
                                _ptr(status), _stream(stream)), "entropy_decode")
    return (out if out.numel() == n else out[:n]), status


def _handles(cbs):
    if isinstance(cbs, Codebook):
        cbs = [cbs]
    return (ctypes.c_void_p * len(cbs))(*[c.handle.value for c in cbs])


def encode_batch(cbs, x: torch.Tensor, chunk_symbols: int, embed_lengths: bool = False,
                 out: torch.Tensor | None = None, out_len: torch.Tensor | None = None,
                 status: torch.Tensor | None = None, stream=None):
    """entropy_encode_batch over the rows of a 2-D uint8 tensor; cbs is one
    codebook or one per row.  Returns (out [S, stride], out_len int64[S], status int32[S])."""
    _u8_cuda(x, "x")
    S, seg_n = x.shape
    cbl = [cbs] * S if isinstance(cbs, Codebook) else list(cbs)
    if out is None:
        stride = max(max_encoded_bytes(c, seg_n, chunk_symbols, embed_lengths) for c in cbl)
        stride = (stride + 255) // 256 * 256
        out = torch.empty((S, stride), dtype=torch.uint8, device=x.device)
    if out_len is None:
        out_len = torch.zeros(S, dtype=torch.int64, device=x.device)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=x.device)
    _check(lib().entropy_encode_batch(_handles(cbl), S, _ptr(x), seg_n, x.stride(0), chunk_symbols,
                                      int(embed_lengths), _ptr(out), out.stride(0), _ptr(out_len), _ptr(status),
                                      _stream(stream)), "entropy_encode_batch")
    return out, out_len, status


def encode_batch_sized(cbs, x: torch.Tensor, chunk_symbols: int, sizes: torch.Tensor, embed_lengths: bool = False,
                       out: torch.Tensor | None = None, out_len: torch.Tensor | None = None,
                       status: torch.Tensor | None = None, stream=None):
    """entropy_encode_batch_sized: entropy_encode_batch with chunk sizes
    [S, chunks] (int32) from byte_histogram_sized."""
    _u8_cuda(x, "x")
    S, seg_n = x.shape
    cbl = [cbs] * S if isinstance(cbs, Codebook) else list(cbs)
    if out is None:
        stride = max(max_encoded_bytes(c, seg_n, chunk_symbols, embed_lengths) for c in cbl)
        stride = (stride + 255) // 256 * 256
        out = torch.empty((S, stride), dtype=torch.uint8, device=x.device)
    if out_len is None:
        out_len = torch.zeros(S, dtype=torch.int64, device=x.device)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=x.device)
    _check(lib().entropy_encode_batch_sized(_handles(cbl), S, _ptr(x), seg_n, x.stride(0), chunk_symbols,
                                            int(embed_lengths), _ptr(sizes), _ptr(out), out.stride(0),
                                            _ptr(out_len), _ptr(status), _stream(stream)),
           "entropy_encode_batch_sized")
    return out, out_len, status


def decode_batch(cbs, data: torch.Tensor, seg_n: int, out: torch.Tensor | None = None,
                 status: torch.Tensor | None = None, stream=None):
    """entropy_decode_batch of the rows of a 2-D uint8 tensor of streams."""
    _u8_cuda(data, "data")
    S = data.shape[0]
    cbl = [cbs] * S if isinstance(cbs, Codebook) else list(cbs)
    if out is None:
        out = torch.empty((S, (max(seg_n, 1) + 15) // 16 * 16), dtype=torch.uint8, device=data.device)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=data.device)
    _check(lib().entropy_decode_batch(_handles(cbl), S, _ptr(data), data.stride(0), _ptr(out), seg_n,
                                      out.stride(0), _ptr(status), _stream(stream)), "entropy_decode_batch")
    return out[:, :seg_n], status


def device_codebook_bytes() -> int:
    return int(lib().ec_device_codebook_bytes())


def own_max_encoded_bytes(n: int, chunk_symbols: int, embed_lengths: bool = False) -> int:
    return int(lib().entropy_own_max_encoded_bytes(n, chunk_symbols, int(embed_lengths)))


def _tables_cuda(tables: torch.Tensor, S: int):
    _u8_cuda(tables, "tables")
    if tables.numel() < S * device_codebook_bytes():
        raise ECError("tables must hold %d device codebooks" % S)


def build_huffman_device(counts: torch.Tensor, out: torch.Tensor | None = None,
                         status: torch.Tensor | None = None, stream=None):
    """huff_build_codebooks_device over the rows of an int64 [S, 256] count
    tensor.  Returns (tables uint8 [S, device_codebook_bytes()], status int32[S])."""
    c = counts.view(-1, 256)
    if c.dtype != torch.int64 or not c.is_cuda or not c.is_contiguous():
        raise ECError("counts must be a contiguous int64 CUDA tensor of rows of 256")
    S = c.shape[0]
    if out is None:
        out = torch.empty((S, device_codebook_bytes()), dtype=torch.uint8, device=c.device)
    _tables_cuda(out, S)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=c.device)
    _check(lib().huff_build_codebooks_device(_ptr(c), S, _ptr(out), _ptr(status), _stream(stream)),
           "huff_build_codebooks_device")
    return out, status


def huffman_tables_from_streams(data: torch.Tensor, in_len: int | None = None, out: torch.Tensor | None = None,
                                status: torch.Tensor | None = None, stream=None):
    """huff_tables_from_streams_device over the rows of a 2-D uint8 tensor of
    streams with embedded code lengths.  Returns (tables, status int32[S])."""
    _u8_cuda(data, "data")
    S = data.shape[0]
    if out is None:
        out = torch.empty((S, device_codebook_bytes()), dtype=torch.uint8, device=data.device)
    _tables_cuda(out, S)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=data.device)
    _check(lib().huff_tables_from_streams_device(_ptr(data), data.stride(0),
                                                 data.shape[1] if in_len is None else in_len, S, _ptr(out),
                                                 _ptr(status), _stream(stream)), "huff_tables_from_streams_device")
    return out, status


def encode_batch_device(tables: torch.Tensor, x: torch.Tensor, chunk_symbols: int, embed_lengths: bool = False,
                        out: torch.Tensor | None = None, out_len: torch.Tensor | None = None,
                        status: torch.Tensor | None = None, stream=None):
    """entropy_encode_batch_device over the rows of a 2-D uint8 tensor with
    row s's codebook table at tables[s].  Without `out`, streams get the
    own-histogram capacity (entropy_own_max_encoded_bytes)."""
    _u8_cuda(x, "x")
    S, seg_n = x.shape
    _tables_cuda(tables, S)
    if out is None:
        stride = (own_max_encoded_bytes(seg_n, chunk_symbols, embed_lengths) + 255) // 256 * 256
        out = torch.empty((S, stride), dtype=torch.uint8, device=x.device)
    if out_len is None:
        out_len = torch.zeros(S, dtype=torch.int64, device=x.device)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=x.device)
    _check(lib().entropy_encode_batch_device(_ptr(tables), S, _ptr(x), seg_n, x.stride(0), chunk_symbols,
                                             int(embed_lengths), _ptr(out), out.stride(0), _ptr(out_len),
                                             _ptr(status), _stream(stream)), "entropy_encode_batch_device")
    return out, out_len, status


def decode_batch_device(tables: torch.Tensor, data: torch.Tensor, seg_n: int, codec: int = CODEC_HUFFMAN,
                        out: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """entropy_decode_batch_device of the rows of a 2-D uint8 tensor of streams."""
    _u8_cuda(data, "data")
    S = data.shape[0]
    _tables_cuda(tables, S)
    if out is None:
        out = torch.empty((S, (max(seg_n, 1) + 15) // 16 * 16), dtype=torch.uint8, device=data.device)
    if status is None:
        status = torch.zeros(S, dtype=torch.int32, device=data.device)
    _check(lib().entropy_decode_batch_device(_ptr(tables), int(codec), S, _ptr(data), data.stride(0), _ptr(out),
                                             seg_n, out.stride(0), _ptr(status), _stream(stream)),
           "entropy_decode_batch_device")
    return out[:, :seg_n], status


def byte_histogram(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Histogram of each row (2-D) or of the whole tensor (1-D): int64 [S, 256]
    holding the uint64 counts."""
    _u8_cuda(x, "x")
    if x.dim() == 1:
        S, seg_n, stride = 1, x.numel(), x.numel()
    else:
        S, seg_n = x.shape
        stride = x.stride(0)
    if out is None:
        out = torch.empty((S, 256), dtype=torch.int64, device=x.device)
    _check(lib().byte_histogram(_ptr(x), seg_n, S, stride, _ptr(out), _stream(stream)), "byte_histogram")
    return out


def byte_histogram_sized(x: torch.Tensor, cbs, chunk_symbols: int, out: torch.Tensor | None = None,
                         sizes: torch.Tensor | None = None, stream=None):
    """byte_histogram of each row (2-D) or of the whole tensor (1-D) that also
    makes, for each codebook of cbs (1..4), the chunk sizes an encode with
    chunk_symbols makes.  Returns (counts int64 [S, 256], sizes int32
    [n_cb, S, chunks])."""
    _u8_cuda(x, "x")
    if x.dim() == 1:
        S, seg_n, stride = 1, x.numel(), x.numel()
    else:
        S, seg_n = x.shape
        stride = x.stride(0)
    cbl = [cbs] if isinstance(cbs, Codebook) else list(cbs)
    chunks = (seg_n + chunk_symbols - 1) // chunk_symbols
    if out is None:
        out = torch.empty((S, 256), dtype=torch.int64, device=x.device)
    if sizes is None:
        sizes = torch.empty((len(cbl), S, max(chunks, 1)), dtype=torch.int32, device=x.device)
    _check(lib().byte_histogram_sized(_ptr(x), seg_n, S, stride, _ptr(out), _handles(cbl), len(cbl), chunk_symbols,
                                      _ptr(sizes), _stream(stream)), "byte_histogram_sized")
    return out, sizes


def pmf_average(counts: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    c = counts.view(-1, 256)
    if out is None:
        out = torch.empty(256, dtype=torch.float32, device=counts.device)
    _check(lib().pmf_average(_ptr(c), c.shape[0], _ptr(out), _stream(stream)), "pmf_average")
    return out


def pmf_kl(p_counts: torch.Tensor, q_counts: torch.Tensor, q_add: int = 0, out: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    p = p_counts if p_counts.dim() == 2 and p_counts.shape[1] == 256 else p_counts.view(-1, 256)
    if out is None:
        out = torch.empty(p.shape[0], dtype=torch.float32, device=p_counts.device)
    _check(lib().pmf_kl(_ptr(p), p.shape[0], _ptr(q_counts), int(q_add), _ptr(out), _stream(stream)), "pmf_kl")
    return out
