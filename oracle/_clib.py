"""Build and load the oracle's plain C core (``csrc/oracle_codec.c``) with gcc.

Test infrastructure: see the package docstring for who may use it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "csrc", "oracle_codec.c")
LIB = os.path.join(_HERE, "_oracle_codec.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (plain -O2, no vector intrinsics)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, SRC]
        )
        os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        L = ctypes.CDLL(LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        u64 = ctypes.c_uint64
        u32 = ctypes.c_uint32
        L.orc_histogram.argtypes = [u8p, u64, u64p]
        L.orc_histogram.restype = None
        L.orc_encode.argtypes = [u8p, u64, u32, u64p, u8p, u8p, u64, u64p, u32p]
        L.orc_encode.restype = u64
        common = [u8p, u64, u64p, u32p, u64, u32]
        L.orc_decode_qlc.argtypes = common + [u16p, u8p, u8p, u8p]
        L.orc_decode_qlc.restype = ctypes.c_int
        L.orc_decode_huffman.argtypes = common + [i32p, u8p]
        L.orc_decode_huffman.restype = ctypes.c_int
        L.orc_decode_eg.argtypes = common + [u32, u8p, u8p]
        L.orc_decode_eg.restype = ctypes.c_int
        _lib = L
    return _lib


def ptr(a, ctype):
    """ctypes pointer to the data of a C-contiguous numpy array."""
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))
