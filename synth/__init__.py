"""Seeded synthetic inputs shared by the HIP library and the CPU oracle.

The C source (bw_synth.c) is compiled once, with gcc, into ``bw_synth.o``. The library and
the oracle both link that object, so they see the same bytes. This Python module only builds
the object and exposes a ctypes view of the generator for tests; it holds none of the decode
step's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bw_synth.c")
OBJ = os.path.join(HERE, "bw_synth.o")
LIB = os.path.join(HERE, "libbwsynth.so")

# tensor kinds (mirrors bw_synth.h)
EMBED, FINAL_NORM, LM_HEAD = 1, 2, 3
ATTN_NORM, QKV, O, FFN_NORM, GATE, UP, DOWN, ROUTER = 10, 11, 12, 13, 14, 15, 16, 17
KV = 20
SHARED_EXPERT = 0x100000
KV_F16, KV_BF16, KV_FP8 = 1, 2, 3

CFLAGS = ["-O2", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall"]


def build() -> str:
    """Compile bw_synth.c to bw_synth.o and libbwsynth.so (gcc). Returns the object path."""
    subprocess.check_call(["gcc", *CFLAGS, "-c", SRC, "-o", OBJ])
    subprocess.check_call(["gcc", "-shared", "-o", LIB, OBJ, "-lm"])
    return OBJ


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        u64, u32, i64, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        L.bws_key.restype = u64
        L.bws_key.argtypes = [u64, u32, u32, u32, u32]
        L.bws_gauss.restype = ctypes.c_double
        L.bws_gauss.argtypes = [u64, u64]
        L.bws_f16_bits.restype = ctypes.c_uint16
        L.bws_f16_bits.argtypes = [ctypes.c_double]
        L.bws_fill_bytes.argtypes = [u64, u64, vp, ctypes.c_size_t]
        L.bws_fill_f16.argtypes = [u64, u64, vp, ctypes.c_size_t, ctypes.c_double, ctypes.c_double, i32]
        L.bws_int4_matrix.argtypes = [u64, u32, u32, u32, i64, i64, i64, i64, vp, vp]
        L.bws_norm_gain.argtypes = [u64, u32, u32, i64, vp]
        L.bws_embed_rows.argtypes = [u64, i64, i64, i64, vp]
        L.bws_router.argtypes = [u64, u32, i64, i64, vp]
        L.bws_mx_matrix.argtypes = [u64, u32, u32, u32, i64, i64, i64, i32, i32, vp, vp]
        L.bws_kv_value.restype = ctypes.c_double
        L.bws_kv_value.argtypes = [u64, u32, u32, i64, i32, i32, i32, i32, i32]
        L.bws_kv_value_dt.restype = ctypes.c_double
        L.bws_kv_value_dt.argtypes = [u64, u32, u32, i64, i32, i32, i32, i32, i32, i32]
        L.bws_kv_bits.restype = ctypes.c_uint16
        L.bws_kv_bits.argtypes = [u64, u32, u32, i64, i32, i32, i32, i32, i32, i32]
        L.bws_kv_fill.argtypes = [u64, u32, u32, i64, i64, i32, i32, i32, vp]
        _lib = L
    return _lib


def int4_matrix(seed: int, kind: int, layer: int, expert: int, N: int, K: int):
    """Canonical (codes uint8 [N][K/2], scales uint16 fp16-bits [N][K/32])."""
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 32), dtype=np.uint16)
    lib().bws_int4_matrix(seed, kind, layer, expert, N, K, 0, N, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def mx_matrix(seed: int, kind: int, layer: int, expert: int, N: int, K: int, e_lo: int = 117, e_hi: int = 121):
    """MXFP4 (codes uint8 [N][K/2], E8M0 scales uint8 [N][K/32]); scales uniform on [e_lo, e_hi]."""
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 32), dtype=np.uint8)
    lib().bws_mx_matrix(seed, kind, layer, expert, K, 0, N, e_lo, e_hi, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def f16_bits(v: float) -> int:
    return int(lib().bws_f16_bits(float(v)))


def gauss(key: int, i: int) -> float:
    return float(lib().bws_gauss(key, i))


def key(seed: int, kind: int, layer: int, expert: int, sub: int) -> int:
    return int(lib().bws_key(seed, kind, layer, expert, sub))


def fill_f16(key_: int, off: int, n: int, mean: float, sd: float, absolute: bool) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().bws_fill_f16(key_, off, out.ctypes.data, n, mean, sd, int(absolute))
    return out


def norm_gain(seed: int, kind: int, layer: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().bws_norm_gain(seed, kind, layer, n, out.ctypes.data)
    return out


def embed_rows(seed: int, d: int, row0: int, nrows: int) -> np.ndarray:
    out = np.empty((nrows, d), dtype=np.uint16)
    lib().bws_embed_rows(seed, d, row0, nrows, out.ctypes.data)
    return out


def router(seed: int, layer: int, n_experts: int, d: int) -> np.ndarray:
    out = np.empty((n_experts, d), dtype=np.uint16)
    lib().bws_router(seed, layer, n_experts, d, out.ctypes.data)
    return out


def kv_value(seed: int, layer: int, seq: int, pos: int, kv: int, g: int, d: int, G: int, D: int) -> float:
    return float(lib().bws_kv_value(seed, layer, seq, pos, kv, g, d, G, D))


def kv_value_dt(seed: int, layer: int, seq: int, pos: int, kv: int, g: int, d: int, G: int, D: int,
                dtype: int) -> float:
    return float(lib().bws_kv_value_dt(seed, layer, seq, pos, kv, g, d, G, D, dtype))


def kv_fill(seed: int, layer: int, seq: int, pos0: int, ntok: int, G: int, D: int, dtype: int) -> np.ndarray:
    """Synthetic K/V bits [ntok][2][G][D] (uint16; uint8 for an fp8 cache)."""
    out = np.empty((ntok, 2, G, D), dtype=np.uint8 if dtype == KV_FP8 else np.uint16)
    lib().bws_kv_fill(seed, layer, seq, pos0, ntok, G, D, dtype, out.ctypes.data)
    return out
