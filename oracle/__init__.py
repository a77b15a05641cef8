"""Plain CPU reference (the oracle) of the paged KV-record codec.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library (``quantized_paged_kv_rope_amd``) never imports it, and the two share
no code: the arithmetic lives in ``kvrec_oracle.c`` (see its header for the
pages it follows); this module only compiles it with gcc and marshals numpy
arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvrec_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

HEAD_DIM = 512
RECORD_MXFP8 = 528
RECORD_LEGACY = 584
RECORD_BF16 = 1024
RECORD_FP8 = 512

_lib = None

ROPE = {"neox": 0, "interleaved": 1, "none": 2}


class InsertOptions(ctypes.Structure):
    """orc_insert_options: see kvrec_oracle.h."""

    _fields_ = [("rope", ctypes.c_int32), ("compress_ratio", ctypes.c_int32),
                ("amax_floor", ctypes.c_float), ("sanitize_nans", ctypes.c_int32)]


def options(rope="neox", compress_ratio=1, amax_floor=0.0, sanitize_nans=False) -> InsertOptions:
    return InsertOptions(ROPE[rope], int(compress_ratio), float(amax_floor), int(bool(sanitize_nans)))


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with strict IEEE float semantics."""
    cmd = [
        "gcc", "-O2", "-std=c99", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-Wall", "-Wextra", "-Werror",
        _SRC, "-o", _LIB_PATH + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _stale() -> bool:
    if not os.path.exists(_LIB_PATH):
        return True
    return os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "kvrec_oracle.h")))


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it first if nothing is built."""
    global _lib
    if _lib is None:
        if _stale():
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


def _declare(L: ctypes.CDLL) -> None:
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_encode.argtypes = [ctypes.c_double]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_bf16_round.argtypes = [ctypes.c_double]
    L.orc_bf16_round.restype = ctypes.c_uint16
    L.orc_scale_exponent.argtypes = [ctypes.c_float]
    L.orc_scale_exponent.restype = ctypes.c_int
    L.orc_insert.argtypes = [p, i64, p, i64, i64, i32, i32, p, p, p, i64]
    L.orc_insert.restype = ctypes.c_int
    L.orc_insert_ex.argtypes = [p, i64, p, i64, i64, i32, i32, p, p, p, i64,
                                ctypes.POINTER(InsertOptions)]
    L.orc_insert_ex.restype = ctypes.c_int
    L.orc_rope_rows_ex.argtypes = [p, i64, p, p, ctypes.POINTER(InsertOptions), p]
    L.orc_rope_rows_ex.restype = None
    L.orc_insert_full.argtypes = [p, i64, p, i64, i64, i32, i32, p, p, p, i64, ctypes.c_float]
    L.orc_insert_full.restype = ctypes.c_int
    L.orc_qnorm_rope.argtypes = [p, i64, i32, p, p, i64, ctypes.c_double, i32, p]
    L.orc_qnorm_rope.restype = None
    L.orc_expand_candidates.argtypes = [p, i64, p, i64, p, i64, i64, i32, i32, i32, p, i64, p,
                                        i64]
    L.orc_expand_candidates.restype = ctypes.c_int
    L.orc_gather.argtypes = [p, i64, i64, i32, i32, p, i64, p]
    L.orc_gather.restype = ctypes.c_int
    L.orc_e4m3_encode_f32.argtypes = [p, i64, p]
    L.orc_e4m3_encode_bits.argtypes = [ctypes.c_uint32, i64, p]
    L.orc_e4m3_value_all.argtypes = [p]
    L.orc_bf16_round_f32.argtypes = [p, i64, p]
    L.orc_scale_exponent_f32.argtypes = [p, i64, p]
    L.orc_rope_rows.argtypes = [p, i64, p, p, p]
    for f in ("orc_e4m3_encode_f32", "orc_e4m3_encode_bits", "orc_e4m3_value_all",
              "orc_bf16_round_f32", "orc_scale_exponent_f32", "orc_rope_rows"):
        getattr(L, f).restype = None


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


# ---- element codecs ------------------------------------------------------

def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_values() -> np.ndarray:
    out = np.empty(256, np.float64)
    lib().orc_e4m3_value_all(_ptr(out))
    return out


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(float(y))


def e4m3_encode_f32(y: np.ndarray) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e4m3_encode_f32(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_encode_bits(first_bits: int, count: int) -> np.ndarray:
    out = np.empty(count, np.uint8)
    lib().orc_e4m3_encode_bits(first_bits, count, _ptr(out))
    return out


def bf16_round(x: float) -> int:
    return lib().orc_bf16_round(float(x))


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_round_f32(_ptr(x), x.size, _ptr(out))
    return out


def scale_exponent(amax: float) -> int:
    return lib().orc_scale_exponent(amax)


def scale_exponent_f32(amax: np.ndarray) -> np.ndarray:
    amax = _c(amax, np.float32)
    out = np.empty(amax.shape, np.int32)
    lib().orc_scale_exponent_f32(_ptr(amax), amax.size, _ptr(out))
    return out


def rope_rows(kv_bits: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """Rotated fp32 rows [n, 512] (dims < 448 are the widened input)."""
    kv_bits = _c(kv_bits, np.uint16)
    positions = _c(positions, np.int64)
    cos_sin = _c(cos_sin, np.float32)
    n = kv_bits.shape[0]
    assert kv_bits.shape == (n, HEAD_DIM) and positions.shape[0] >= n
    assert cos_sin.ndim == 2 and cos_sin.shape[1] == 64
    assert n == 0 or (positions[:n].min() >= 0 and positions[:n].max() < cos_sin.shape[0])
    out = np.empty((n, HEAD_DIM), np.float32)
    lib().orc_rope_rows(_ptr(kv_bits), n, _ptr(positions), _ptr(cos_sin), _ptr(out))
    return out


def rope_rows_ex(kv_bits: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray,
                 **opts) -> np.ndarray:
    """Rotated (and, if asked, NaN-sanitised) fp32 rows under the insert options."""
    kv_bits = _c(kv_bits, np.uint16)
    positions = _c(positions, np.int64)
    cos_sin = _c(cos_sin, np.float32)
    n = kv_bits.shape[0]
    o = options(**opts)
    out = np.empty((n, HEAD_DIM), np.float32)
    lib().orc_rope_rows_ex(_ptr(kv_bits), n, _ptr(positions), _ptr(cos_sin), ctypes.byref(o),
                           _ptr(out))
    return out


# ---- the two operations --------------------------------------------------

def insert(kv_bits: np.ndarray, backing: np.ndarray, num_blocks: int, page_stride: int,
           block_size: int, record: int, slot_mapping: np.ndarray, positions,
           cos_sin, **opts) -> None:
    """Insert into ``backing`` (uint8, in place; byte 0 = page 0).

    Token count = ``slot_mapping.shape[0]``; kv and positions must cover it.
    Keyword options (rope, compress_ratio, amax_floor, sanitize_nans) select
    the compressed-KV variant; positions and cos_sin may be None only with
    rope="none" and compress_ratio 1.
    """
    kv_bits = _c(kv_bits, np.uint16)
    slot_mapping = _c(slot_mapping, np.int64)
    if positions is None or cos_sin is None:
        o = options(**opts)
        if backing.dtype != np.uint8 or not backing.flags.c_contiguous:
            raise TypeError("backing must be a contiguous uint8 array")
        n = slot_mapping.shape[0]
        if kv_bits.ndim != 2 or kv_bits.shape[1] != HEAD_DIM or kv_bits.shape[0] < n:
            raise ValueError("kv must be [>=n, 512]")
        pos_p = None if positions is None else _ptr(_c(positions, np.int64))
        rc = lib().orc_insert_ex(_ptr(kv_bits), n, _ptr(backing), num_blocks, page_stride,
                                 block_size, record, _ptr(slot_mapping), pos_p, None,
                                 0 if positions is None else _c(positions, np.int64).shape[0],
                                 ctypes.byref(o))
        if rc != 0:
            raise ValueError("oracle insert rejected the options")
        return
    positions = _c(positions, np.int64)
    cos_sin = _c(cos_sin, np.float32)
    if backing.dtype != np.uint8 or not backing.flags.c_contiguous:
        raise TypeError("backing must be a contiguous uint8 array")
    n = slot_mapping.shape[0]
    if kv_bits.ndim != 2 or kv_bits.shape[1] != HEAD_DIM or kv_bits.shape[0] < n:
        raise ValueError("kv must be [>=n, 512]")
    if positions.shape[0] < n:
        raise ValueError("positions must cover every token")
    if cos_sin.ndim != 2 or cos_sin.shape[1] != 64:
        raise ValueError("cos_sin_cache must be [max_pos, 64]")
    if backing.size < (num_blocks - 1) * page_stride + block_size * record and num_blocks > 0:
        raise ValueError("backing too small for the cache geometry")
    if opts:
        o = options(**opts)
        rc = lib().orc_insert_ex(_ptr(kv_bits), n, _ptr(backing), num_blocks, page_stride,
                                 block_size, record, _ptr(slot_mapping), _ptr(positions),
                                 _ptr(cos_sin), cos_sin.shape[0], ctypes.byref(o))
    else:
        rc = lib().orc_insert(_ptr(kv_bits), n, _ptr(backing), num_blocks, page_stride,
                              block_size, record, _ptr(slot_mapping), _ptr(positions),
                              _ptr(cos_sin), cos_sin.shape[0])
    if rc != 0:
        raise ValueError(f"oracle insert rejected record={record} options={opts}")


def insert_full(kv_bits: np.ndarray, backing: np.ndarray, num_blocks: int, page_stride: int,
                block_size: int, record: int, slot_mapping: np.ndarray, positions: np.ndarray,
                cos_sin: np.ndarray, fp8_scale: float = 1.0) -> None:
    """Insert into a non-packed cache (record 1024 = bf16, 512 = fp8 e4m3fn
    with the per-tensor ``fp8_scale``), in place in ``backing``."""
    kv_bits = _c(kv_bits, np.uint16)
    slot_mapping = _c(slot_mapping, np.int64)
    positions = _c(positions, np.int64)
    cos_sin = _c(cos_sin, np.float32)
    if backing.dtype != np.uint8 or not backing.flags.c_contiguous:
        raise TypeError("backing must be a contiguous uint8 array")
    n = slot_mapping.shape[0]
    if kv_bits.ndim != 2 or kv_bits.shape[1] != HEAD_DIM or kv_bits.shape[0] < n:
        raise ValueError("kv must be [>=n, 512]")
    if positions.shape[0] < n:
        raise ValueError("positions must cover every token")
    if cos_sin.ndim != 2 or cos_sin.shape[1] != 64:
        raise ValueError("cos_sin_cache must be [max_pos, 64]")
    if backing.size < (num_blocks - 1) * page_stride + block_size * record and num_blocks > 0:
        raise ValueError("backing too small for the cache geometry")
    rc = lib().orc_insert_full(_ptr(kv_bits), n, _ptr(backing), num_blocks, page_stride,
                               block_size, record, _ptr(slot_mapping), _ptr(positions),
                               _ptr(cos_sin), cos_sin.shape[0], float(fp8_scale))
    if rc != 0:
        raise ValueError(f"oracle full-cache insert rejected record={record}")


def qnorm_rope(q_bits: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, eps: float,
               apply_norm: bool = True, out: np.ndarray = None) -> np.ndarray:
    """q side of the attention write: bf16 bits [n, heads, 512] -> bf16 bits.
    Rows of tokens whose position is out of range keep ``out``'s contents
    (a copy of the input when ``out`` is None)."""
    q_bits = _c(q_bits, np.uint16)
    positions = _c(positions, np.int64)
    cos_sin = _c(cos_sin, np.float32)
    if q_bits.ndim != 3 or q_bits.shape[2] != HEAD_DIM:
        raise ValueError("q must be [n, heads, 512]")
    n, heads = q_bits.shape[:2]
    if positions.shape[0] < n or cos_sin.ndim != 2 or cos_sin.shape[1] != 64:
        raise ValueError("positions must cover every token; cos_sin is [max_pos, 64]")
    if out is None:
        out = q_bits.copy()
    out = _c(out, np.uint16)
    lib().orc_qnorm_rope(_ptr(q_bits), n, heads, _ptr(positions), _ptr(cos_sin),
                         cos_sin.shape[0], float(eps), int(bool(apply_norm)), _ptr(out))
    return out


def expand_candidates(cand: np.ndarray, row_ks: np.ndarray, row_ke: np.ndarray, ratio: int,
                      sparse_block: int):
    """Candidate-block expansion: int32 cand [rows, K], ks/ke [rows] ->
    (sparse_indices int32 [rows, K * ratio], end int32 [rows])."""
    cand = _c(cand, np.int32)
    row_ks = _c(row_ks, np.int32)
    row_ke = _c(row_ke, np.int32)
    rows, k = cand.shape
    if row_ks.shape[0] < rows or row_ke.shape[0] < rows:
        raise ValueError("ks and ke must cover every row")
    sparse = np.empty((rows, k * ratio), np.int32)
    end = np.empty(rows, np.int32)
    rc = lib().orc_expand_candidates(_ptr(cand), k, _ptr(row_ks), 1, _ptr(row_ke), 1, rows, k,
                                     int(ratio), int(sparse_block), _ptr(sparse), k * ratio,
                                     _ptr(end), 1)
    if rc != 0:
        raise ValueError(f"oracle expansion rejected K={k} ratio={ratio} SBK={sparse_block}")
    return sparse, end


def gather(backing: np.ndarray, num_blocks: int, page_stride: int, block_size: int,
           record: int, token_indices: np.ndarray) -> np.ndarray:
    """bf16 bits [*token_indices.shape, 512]."""
    idx = _c(token_indices, np.int32)
    if backing.dtype != np.uint8 or not backing.flags.c_contiguous:
        raise TypeError("backing must be a contiguous uint8 array")
    if backing.size < (num_blocks - 1) * page_stride + block_size * record and num_blocks > 0:
        raise ValueError("backing too small for the cache geometry")
    out = np.empty(idx.shape + (HEAD_DIM,), np.uint16)
    rc = lib().orc_gather(_ptr(backing), num_blocks, page_stride, block_size, record,
                          _ptr(idx), idx.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle gather rejected record={record}")
    return out
