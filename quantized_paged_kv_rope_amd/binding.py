"""Thin Python binding over ``libkvrec.so`` (the C ABI in include/kvrec.h).

Argument marshalling only: every step of insert and gather runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory and the current
stream. There is no CPU or PyTorch fallback: if the library is not built, or
no GPU is present, every compute call raises.

Shapes follow the page's KV-only op ([KV-only op] 实现拆解 1; page title
"[Perf][DSpark] Add KV-only context insertion across V4.1 cache formats"):

* ``kv``             bf16 ``[tokens, 512]`` contiguous (not modified)
* ``k_cache``        uint8 ``[num_blocks, block_size, record]`` with
                     ``stride(2) == 1`` and ``stride(1) == record``; the
                     record (528 or 584; 1024 or 512 for the non-packed
                     caches) is read from the last dimension and the page
                     stride from ``stride(0)`` (a padded stride is expressed
                     with ``as_strided``; see :func:`alloc_cache`). The
                     non-packed caches may also be given as a bf16 or
                     float8_e4m3fn ``[num_blocks, block_size, 512]`` view,
                     as the page's op takes them.
* ``slot_mapping``   int64 ``[tokens]`` (token count = its length)
* ``positions``      int64 covering every token
* ``cos_sin_cache``  fp32 ``[max_pos, 64]`` (32 cos then 32 sin)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvrec.so")

HEAD_DIM = 512
ROPE_DIM = 64
RECORD_MXFP8 = 528
RECORD_LEGACY = 584
RECORD_BF16 = 1024  # non-packed bf16 cache (512 elements per token)
RECORD_FP8 = 512    # non-packed e4m3fn cache with a per-tensor fp32 scale
MAX_POS = 1 << 30  # the C ABI's limit on table rows

KVREC_OK = 0
STATUS_NAMES = {
    0: "KVREC_OK", -1: "KVREC_ERR_NULL", -2: "KVREC_ERR_RECORD", -3: "KVREC_ERR_BLOCK_SIZE",
    -4: "KVREC_ERR_PAGE_STRIDE", -5: "KVREC_ERR_ALIGNMENT", -6: "KVREC_ERR_SIZE",
    -7: "KVREC_ERR_HIP", -8: "KVREC_ERR_OPTION", -9: "KVREC_ERR_OVERLAP",
}
EXPORTED_SYMBOLS = ("kvrec_page_stride", "kvrec_insert", "kvrec_insert_ex", "kvrec_insert_full",
                    "kvrec_qnorm_rope_insert", "kvrec_expand_candidates", "kvrec_gather",
                    "kvrec_status_str")
ROPE = {"neox": 0, "interleaved": 1, "none": 2}


class KvrecError(RuntimeError):
    """A non-zero kvrec_status returned by the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class kvrec_cache(ctypes.Structure):
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("record", ctypes.c_int32),
    ]


class kvrec_insert_options(ctypes.Structure):
    _fields_ = [
        ("rope", ctypes.c_int32),
        ("compress_ratio", ctypes.c_int32),
        ("amax_floor", ctypes.c_float),
        ("sanitize_nans", ctypes.c_int32),
    ]


def insert_options(rope: str = "neox", compress_ratio: int = 1, amax_floor: float = 0.0,
                   sanitize_nans: bool = False) -> kvrec_insert_options:
    """Options of kvrec_insert_ex. The non-default settings follow the
    compressed-KV insert of [MXFP8 record] 关键源码片段: rope="interleaved",
    compress_ratio=R, amax_floor=1e-4, sanitize_nans=True; rope="none" is the
    K insert without RoPE."""
    if rope not in ROPE:
        raise ValueError(f"rope must be one of {sorted(ROPE)}")
    return kvrec_insert_options(ROPE[rope], int(compress_ratio), float(amax_floor),
                                int(bool(sanitize_nans)))


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libkvrec.so`` (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m quantized_paged_kv_rope_amd.build` "
            "(or __graft_entry__.build()). There is no fallback path.")
    L = ctypes.CDLL(path)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.kvrec_page_stride.argtypes = [i32, i32, ctypes.POINTER(i64)]
    L.kvrec_page_stride.restype = ctypes.c_int
    L.kvrec_insert.argtypes = [p, i64, ctypes.POINTER(kvrec_cache), p, p, p, i64, i32, i32, p]
    L.kvrec_insert.restype = ctypes.c_int
    L.kvrec_insert_ex.argtypes = [p, i64, ctypes.POINTER(kvrec_cache), p, p, p, i64, i32, i32,
                                  ctypes.POINTER(kvrec_insert_options), p]
    L.kvrec_insert_ex.restype = ctypes.c_int
    L.kvrec_insert_full.argtypes = [p, i64, ctypes.POINTER(kvrec_cache), p, p, p, i64, i32, i32,
                                    p, p]
    L.kvrec_insert_full.restype = ctypes.c_int
    L.kvrec_qnorm_rope_insert.argtypes = [p, p, i32, ctypes.c_float, i32, p, i64,
                                          ctypes.POINTER(kvrec_cache), p, p, p, i64, i32, i32, p]
    L.kvrec_qnorm_rope_insert.restype = ctypes.c_int
    L.kvrec_expand_candidates.argtypes = [p, i64, p, i64, p, i64, i64, i32, i32, i32, p, i64, p,
                                          i64, p]
    L.kvrec_expand_candidates.restype = ctypes.c_int
    L.kvrec_gather.argtypes = [ctypes.POINTER(kvrec_cache), p, i64, p, p]
    L.kvrec_gather.restype = ctypes.c_int
    L.kvrec_status_str.argtypes = [ctypes.c_int]
    L.kvrec_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def kvrec_status_str(status: int) -> str:
    return load_library().kvrec_status_str(status).decode()


def _check(status: int) -> None:
    if status != KVREC_OK:
        raise KvrecError(status, kvrec_status_str(status))


def kvrec_page_stride(record: int, block_size: int) -> int:
    out = ctypes.c_int64(0)
    _check(load_library().kvrec_page_stride(record, block_size, ctypes.byref(out)))
    return out.value


def _require_gpu(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")


_ELEMENT_CACHES = {torch.bfloat16: RECORD_BF16, torch.float8_e4m3fn: RECORD_FP8}


def cache_descriptor(k_cache: torch.Tensor) -> kvrec_cache:
    """The C descriptor of a ``[num_blocks, block_size, record]`` uint8 view,
    or of a bf16 / float8_e4m3fn ``[num_blocks, block_size, 512]`` view of a
    non-packed cache (record 1024 / 512 bytes)."""
    _require_gpu(k_cache, "k_cache")
    if k_cache.dim() != 3 or (k_cache.dtype != torch.uint8 and
                              k_cache.dtype not in _ELEMENT_CACHES):
        raise TypeError("k_cache must be a 3-D uint8 tensor [num_blocks, block_size, record], "
                        "or a bf16 / float8_e4m3fn [num_blocks, block_size, 512] view")
    nb, bs, width = k_cache.shape
    if k_cache.stride(2) != 1 or (bs > 1 and k_cache.stride(1) != width):
        raise ValueError("k_cache must have stride(2) == 1 and stride(1) == its last dimension")
    item = k_cache.element_size()
    if k_cache.dtype == torch.uint8:
        rec = width
    elif width != HEAD_DIM:
        raise ValueError("a bf16 / fp8 k_cache view must be [num_blocks, block_size, 512]")
    else:
        rec = _ELEMENT_CACHES[k_cache.dtype]
    stride0 = k_cache.stride(0) * item if nb > 1 else kvrec_page_stride(rec, bs)
    return kvrec_cache(k_cache.data_ptr(), nb, stride0, bs, rec)


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def kvrec_insert(kv: torch.Tensor, k_cache: torch.Tensor, slot_mapping: torch.Tensor,
                 positions: Optional[torch.Tensor], cos_sin_cache: Optional[torch.Tensor],
                 block_size: int, record: Optional[int] = None, *, rope: str = "neox",
                 compress_ratio: int = 1, amax_floor: float = 0.0,
                 sanitize_nans: bool = False) -> None:
    """Fused RoPE + quantise + paged insert, in place on ``k_cache``.

    Runs asynchronously on the current stream of ``kv``'s device. The keyword
    options select the compressed-KV variant (see :func:`insert_options`);
    with the defaults this is the C ``kvrec_insert``."""
    opts = insert_options(rope, compress_ratio, amax_floor, sanitize_nans)
    default = (rope == "neox" and compress_ratio == 1 and amax_floor == 0.0
               and not sanitize_nans)
    kvrec_insert_ex(kv, k_cache, slot_mapping, positions, cos_sin_cache, block_size, record,
                    None if default else opts)


def _check_insert_inputs(kv, k_cache, slot_mapping, positions, cos_sin_cache) -> list:
    tensors = [("kv", kv), ("slot_mapping", slot_mapping)]
    if positions is not None:
        tensors.append(("positions", positions))
    if cos_sin_cache is not None:
        tensors.append(("cos_sin_cache", cos_sin_cache))
    for name, t in tensors:
        _require_gpu(t, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if kv.dtype != torch.bfloat16 or kv.dim() != 2 or kv.shape[1] != HEAD_DIM:
        raise TypeError("kv must be bf16 [tokens, 512]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1:
        raise TypeError("slot_mapping must be a 1-D int64 tensor")
    if positions is not None and (positions.dtype != torch.int64 or positions.dim() != 1):
        raise TypeError("positions must be a 1-D int64 tensor")
    if cos_sin_cache is not None and (cos_sin_cache.dtype != torch.float32 or
                                      cos_sin_cache.dim() != 2 or
                                      cos_sin_cache.shape[1] != ROPE_DIM):
        raise TypeError("cos_sin_cache must be fp32 [max_pos, 64]")
    n = slot_mapping.shape[0]
    if kv.shape[0] < n or (positions is not None and positions.shape[0] < n):
        raise ValueError("kv and positions must cover every token of slot_mapping")
    devs = {t.device for _, t in tensors} | {k_cache.device}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    return tensors


def kvrec_insert_ex(kv: torch.Tensor, k_cache: torch.Tensor, slot_mapping: torch.Tensor,
                    positions: Optional[torch.Tensor], cos_sin_cache: Optional[torch.Tensor],
                    block_size: int, record: Optional[int] = None,
                    options: Optional[kvrec_insert_options] = None) -> None:
    """The C ``kvrec_insert_ex``: :func:`kvrec_insert` with an options struct
    (``None`` = the defaults, which calls the C ``kvrec_insert``)."""
    _check_insert_inputs(kv, k_cache, slot_mapping, positions, cos_sin_cache)
    n = slot_mapping.shape[0]
    desc = cache_descriptor(k_cache)
    rec = desc.record if record is None else int(record)
    pos_p = positions.data_ptr() if positions is not None else None
    cs_p = cos_sin_cache.data_ptr() if cos_sin_cache is not None else None
    # Without a table (rotation-free insert) positions only feed the ratio
    # gate, so they are bounded by the ABI's limit alone.
    max_pos = cos_sin_cache.shape[0] if cos_sin_cache is not None else MAX_POS
    with torch.cuda.device(kv.device):
        if options is None:
            _check(load_library().kvrec_insert(
                kv.data_ptr(), n, ctypes.byref(desc), slot_mapping.data_ptr(), pos_p, cs_p,
                max_pos, int(block_size), rec, _stream_handle(kv.device)))
        else:
            _check(load_library().kvrec_insert_ex(
                kv.data_ptr(), n, ctypes.byref(desc), slot_mapping.data_ptr(), pos_p, cs_p,
                max_pos, int(block_size), rec, ctypes.byref(options), _stream_handle(kv.device)))


def kvrec_insert_full(kv: torch.Tensor, k_cache: torch.Tensor, slot_mapping: torch.Tensor,
                      positions: torch.Tensor, cos_sin_cache: torch.Tensor, block_size: int,
                      fp8_scale: Optional[torch.Tensor] = None,
                      record: Optional[int] = None) -> None:
    """The C ``kvrec_insert_full``: RoPE + insert into a non-packed cache
    ([KV-only op] 实现拆解 1): bf16 rows (record 1024) or e4m3fn rows of
    ``r / fp8_scale`` (record 512; ``fp8_scale`` a one-element fp32 GPU
    tensor, required there and refused for bf16)."""
    if positions is None or cos_sin_cache is None:
        raise ValueError("the non-packed insert rotates: positions and cos_sin_cache are needed")
    _check_insert_inputs(kv, k_cache, slot_mapping, positions, cos_sin_cache)
    n = slot_mapping.shape[0]
    desc = cache_descriptor(k_cache)
    rec = desc.record if record is None else int(record)
    scale_p = None
    if fp8_scale is not None:
        _require_gpu(fp8_scale, "fp8_scale")
        if fp8_scale.dtype != torch.float32 or fp8_scale.numel() != 1:
            raise TypeError("fp8_scale must be a one-element fp32 tensor")
        if fp8_scale.device != kv.device:
            raise ValueError("fp8_scale must be on kv's device")
        scale_p = fp8_scale.data_ptr()
    with torch.cuda.device(kv.device):
        _check(load_library().kvrec_insert_full(
            kv.data_ptr(), n, ctypes.byref(desc), slot_mapping.data_ptr(), positions.data_ptr(),
            cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], int(block_size), rec, scale_p,
            _stream_handle(kv.device)))


def kvrec_qnorm_rope_insert(q: torch.Tensor, kv: torch.Tensor, k_cache: torch.Tensor,
                            slot_mapping: torch.Tensor, positions: torch.Tensor,
                            cos_sin_cache: torch.Tensor, block_size: int, eps: float = 1e-6,
                            apply_q_norm: bool = True, q_out: Optional[torch.Tensor] = None,
                            record: Optional[int] = None) -> torch.Tensor:
    """The attention write (the C ``kvrec_qnorm_rope_insert``): for every
    token and head of ``q`` (bf16 ``[tokens, heads, 512]``), RMSNorm over the
    head (if ``apply_q_norm``) and the NeoX rotation of its tail, written to
    ``q_out`` (default: ``q`` itself, in place); and the KV insert of ``kv``
    into the packed ``k_cache``, in one launch. Returns the q output."""
    _check_insert_inputs(kv, k_cache, slot_mapping, positions, cos_sin_cache)
    _require_gpu(q, "q")
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != HEAD_DIM or \
            not q.is_contiguous():
        raise TypeError("q must be contiguous bf16 [tokens, heads, 512]")
    n = slot_mapping.shape[0]
    if q.shape[0] < n:
        raise ValueError("q must cover every token of slot_mapping")
    if q.device != kv.device:
        raise ValueError("q must be on kv's device")
    if q_out is None:
        q_out = q
    else:
        _require_gpu(q_out, "q_out")
        if q_out.dtype != torch.bfloat16 or q_out.shape != q.shape or not q_out.is_contiguous():
            raise ValueError(f"q_out must be contiguous bf16 {tuple(q.shape)}")
        if q_out.device != q.device:
            raise ValueError("q_out must be on q's device")
    desc = cache_descriptor(k_cache)
    rec = desc.record if record is None else int(record)
    with torch.cuda.device(kv.device):
        _check(load_library().kvrec_qnorm_rope_insert(
            q.data_ptr(), q_out.data_ptr(), int(q.shape[1]), float(eps), int(bool(apply_q_norm)),
            kv.data_ptr(), n, ctypes.byref(desc), slot_mapping.data_ptr(), positions.data_ptr(),
            cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], int(block_size), rec,
            _stream_handle(kv.device)))
    return q_out


def kvrec_expand_candidates(candidate_blocks: torch.Tensor, row_ks: torch.Tensor,
                            row_ke: torch.Tensor, ratio: int, sparse_block: int,
                            out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
                            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The sparse indexer's candidate-block expansion (the C
    ``kvrec_expand_candidates``; the page's candidate_blocks_to_sparse_indices):
    int32 ``candidate_blocks [rows, K]`` (any row stride, unit column stride),
    ``row_ks`` / ``row_ke`` int32 ``[rows]`` (any stride) -> ``(sparse_indices
    [rows, K * ratio], end [rows])``, written into ``out`` when given."""
    for name, t in (("candidate_blocks", candidate_blocks), ("row_ks", row_ks),
                    ("row_ke", row_ke)):
        _require_gpu(t, name)
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if candidate_blocks.dim() != 2 or candidate_blocks.stride(1) != 1:
        raise ValueError("candidate_blocks must be [rows, K] with unit column stride")
    rows, k = candidate_blocks.shape
    if row_ks.dim() != 1 or row_ke.dim() != 1 or row_ks.shape[0] < rows or \
            row_ke.shape[0] < rows:
        raise ValueError("row_ks and row_ke must be 1-D and cover every row")
    dev = candidate_blocks.device
    if row_ks.device != dev or row_ke.device != dev:
        raise ValueError("all tensors must be on one device")
    width = k * int(ratio)
    if out is None:
        sparse = torch.empty((rows, width), dtype=torch.int32, device=dev)
        end = torch.empty(rows, dtype=torch.int32, device=dev)
    else:
        sparse, end = out
        _require_gpu(sparse, "sparse_indices")
        _require_gpu(end, "end")
        if sparse.dtype != torch.int32 or sparse.dim() != 2 or tuple(sparse.shape) != (rows, width) \
                or sparse.stride(1) != 1 or end.dtype != torch.int32 or end.dim() != 1 or \
                end.shape[0] < rows:
            raise ValueError(f"out must be int32 ([{rows}, {width}] unit column stride, [{rows}])")
        if sparse.device != dev or end.device != dev:
            raise ValueError("out must be on the inputs' device")
    with torch.cuda.device(dev):
        _check(load_library().kvrec_expand_candidates(
            candidate_blocks.data_ptr(), candidate_blocks.stride(0) if rows > 1 else k,
            row_ks.data_ptr(), row_ks.stride(0), row_ke.data_ptr(), row_ke.stride(0), rows, k,
            int(ratio), int(sparse_block), sparse.data_ptr(),
            sparse.stride(0) if rows > 1 else width, end.data_ptr(), end.stride(0),
            _stream_handle(dev)))
    return sparse, end


def kvrec_gather(k_cache: torch.Tensor, token_indices: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged dequantise-and-gather: bf16 ``[*token_indices.shape, 512]``."""
    _require_gpu(token_indices, "token_indices")
    if token_indices.dtype != torch.int32 or not token_indices.is_contiguous():
        raise TypeError("token_indices must be a contiguous int32 tensor")
    desc = cache_descriptor(k_cache)
    if token_indices.device != k_cache.device:
        raise ValueError("token_indices and k_cache must be on one device")
    shape = tuple(token_indices.shape) + (HEAD_DIM,)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=k_cache.device)
    else:
        _require_gpu(out, "out")
        if out.dtype != torch.bfloat16 or tuple(out.shape) != shape or not out.is_contiguous():
            raise ValueError(f"out must be contiguous bf16 {shape}")
        if out.device != k_cache.device:
            raise ValueError("out and k_cache must be on one device")
    with torch.cuda.device(k_cache.device):
        _check(load_library().kvrec_gather(
            ctypes.byref(desc), token_indices.data_ptr(), token_indices.numel(), out.data_ptr(),
            _stream_handle(k_cache.device)))
    return out


def alloc_cache(num_blocks: int, block_size: int, record: int,
                page_stride: Optional[int] = None, device="cuda",
                backing: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocate (or wrap) a flat uint8 backing and return ``(backing,
    k_cache)`` where ``k_cache`` is the ``[num_blocks, block_size, record]``
    view whose ``stride(0)`` is the page stride (default: block_size * record
    rounded up to the record's alignment)."""
    if page_stride is None:
        page_stride = kvrec_page_stride(record, block_size)
    nbytes = num_blocks * page_stride
    if backing is None:
        backing = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif backing.dtype != torch.uint8 or backing.dim() != 1 or backing.numel() < nbytes:
        raise ValueError("backing must be a flat uint8 tensor of at least num_blocks*page_stride")
    view = backing.as_strided((num_blocks, block_size, record), (page_stride, record, 1))
    return backing, view
