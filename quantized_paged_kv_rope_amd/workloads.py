"""Seeded synthetic inputs for the paged KV-record insert and gather.

This module only draws inputs. It holds none of the codec's arithmetic (no
rotation, scaling, encoding or paging), so both the GPU path and the CPU
oracle can be fed from it. Everything is generated on the host with
``numpy.random.default_rng`` (PCG64) so the same seed gives the same bytes on
every machine; fp32 -> bf16 input rounding uses torch's round-to-nearest-even
cast.

Workloads (sizes from the pages' measured and tested token counts: the
KV-only insert was timed at 16384..262144 tokens and tested at 1..1024
tokens, [KV-only op, 实现拆解 4 and 5]):

* ``mixed_1024``     1024 tokens into the MXFP8 record, 20 pages of 64, with
                     outlier channels, zero groups and 5% skipped slots, then
                     a gather of the same slots.
* ``decode_16384``   16384 tokens (one per sequence) at random positions in
                     [0, 131072) into random distinct slots of 4096 pages.
* ``prefill_262144`` 262144 contiguous tokens at positions 0.. into slots
                     0.. (4096 full pages), then gathered back in order.
* ``legacy_65536``   65536 tokens into the 584 B legacy record.
* ``topk_gather``    a 32768-page MXFP8 cache filled in slot order; 64 queries
                     gather 2048 sorted indices each with 3% set to -1.
* ``attention_write`` 4096 tokens x 128 q heads normalised and rotated, with
                     the KV insert of the same tokens.
* ``sparse_expand``  16384 query rows (4 causal sequences of 4096) expanding
                     up to 128 candidate blocks each into sparse block indices.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

HEAD_DIM = 512
ROPE_DIM = 64
RECORD_MXFP8 = 528
RECORD_LEGACY = 584
RECORD_BF16 = 1024  # non-packed bf16 cache: 512 elements per slot
RECORD_FP8 = 512    # non-packed e4m3fn cache with a per-tensor scale
ROPE_THETA = 10000.0


def page_stride_for(record: int, block_size: int) -> int:
    """Smallest multiple of the record's page alignment (512 B for the MXFP8
    record, 576 B for the legacy one, 16 B for the non-packed rows) that
    holds ``block_size`` records."""
    align = {RECORD_MXFP8: 512, RECORD_LEGACY: 576}.get(record, 16)
    raw = block_size * record
    return (raw + align - 1) // align * align


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rope_table(max_pos: int, theta: float = ROPE_THETA) -> np.ndarray:
    """fp32 [max_pos, 64]: row p = cos(p*f_i) for i < 32, then sin(p*f_i),
    with f_i = theta^(-i/32), evaluated in float64 and rounded once."""
    i = np.arange(ROPE_DIM // 2, dtype=np.float64)
    inv_freq = theta ** (-i / (ROPE_DIM // 2))
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    out = np.empty((max_pos, ROPE_DIM), np.float32)
    out[:, : ROPE_DIM // 2] = np.cos(ang)
    out[:, ROPE_DIM // 2:] = np.sin(ang)
    return out


@dataclasses.dataclass
class InsertCase:
    """One insert (and optional gather) over a paged cache."""

    name: str
    record: int
    block_size: int
    num_blocks: int
    page_stride: int
    kv_bits: np.ndarray        # uint16 [n, 512] (bf16 bits)
    slot_mapping: np.ndarray   # int64 [n]
    positions: np.ndarray      # int64 [n]
    cos_sin: np.ndarray        # float32 [max_pos, 64]
    backing_seed: Optional[int]  # seed of the random pre-fill, None = zeros
    gather_indices: Optional[np.ndarray] = None  # int32, any shape

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def backing_bytes(self) -> int:
        return self.num_blocks * self.page_stride

    def initial_backing(self) -> np.ndarray:
        if self.backing_seed is None:
            return np.zeros(self.backing_bytes, np.uint8)
        rng = np.random.default_rng(self.backing_seed)
        return rng.integers(0, 256, self.backing_bytes, dtype=np.uint8)


def _drop(rng: np.random.Generator, slots: np.ndarray, count: int) -> np.ndarray:
    slots = slots.copy()
    if count:
        slots[rng.choice(slots.shape[0], count, replace=False)] = -1
    return slots


def mixed_1024(seed: int = 1001, n: int = 1024, block_size: int = 64, num_blocks: int = 20,
               record: int = RECORD_MXFP8, max_pos: int = 4096) -> InsertCase:
    """N(0,1) rows; 1% of the 512 channels x100; 2% of the (token, 32-dim
    group) pairs all +0; positions uniform in [0, max_pos); slots a seeded
    permutation of the cache's slots (first n) with 5% set to -1. The gather
    reads the same slots back (-1 gives a zero row)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    chans = rng.choice(HEAD_DIM, int(round(0.01 * HEAD_DIM)), replace=False)
    x[:, chans] *= 100.0
    pairs = n * (HEAD_DIM // 32)
    zero = rng.choice(pairs, int(round(0.02 * pairs)), replace=False)
    xg = x.reshape(n, HEAD_DIM // 32, 32)
    xg[zero // (HEAD_DIM // 32), zero % (HEAD_DIM // 32), :] = 0.0
    positions = rng.integers(0, max_pos, n, dtype=np.int64)
    total = num_blocks * block_size
    if n > total:
        raise ValueError("more tokens than cache slots")
    slots = rng.permutation(total)[:n].astype(np.int64)
    slots = _drop(rng, slots, int(round(0.05 * n)))
    return InsertCase(
        name=f"mixed_{n}", record=record, block_size=block_size, num_blocks=num_blocks,
        page_stride=page_stride_for(record, block_size), kv_bits=to_bf16_bits(x),
        slot_mapping=slots, positions=positions, cos_sin=rope_table(max_pos),
        backing_seed=seed + 100, gather_indices=slots.astype(np.int32))


def decode_16384(seed: int = 1002, n: int = 16384, block_size: int = 64,
                 num_blocks: int = 4096, max_pos: int = 131072) -> InsertCase:
    """N(0,1) * U(0.1, 10) per row; positions uniform in [0, max_pos);
    distinct random slots with 1% set to -1."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    x *= rng.uniform(0.1, 10.0, (n, 1)).astype(np.float32)
    positions = rng.integers(0, max_pos, n, dtype=np.int64)
    slots = rng.permutation(num_blocks * block_size)[:n].astype(np.int64)
    slots = _drop(rng, slots, int(round(0.01 * n)))
    return InsertCase(
        name=f"decode_{n}", record=RECORD_MXFP8, block_size=block_size, num_blocks=num_blocks,
        page_stride=page_stride_for(RECORD_MXFP8, block_size), kv_bits=to_bf16_bits(x),
        slot_mapping=slots, positions=positions, cos_sin=rope_table(max_pos),
        backing_seed=seed + 100, gather_indices=slots.astype(np.int32))


def prefill_262144(seed: int = 1003, n: int = 262144, block_size: int = 64) -> InsertCase:
    """N(0,1) with 0.5% of channels x300; positions 0..n-1; slots 0..n-1
    (whole pages from page 0); gather 0..n-1 in order."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    chans = rng.choice(HEAD_DIM, int(round(0.005 * HEAD_DIM)), replace=False)
    x[:, chans] *= 300.0
    num_blocks = (n + block_size - 1) // block_size
    slots = np.arange(n, dtype=np.int64)
    return InsertCase(
        name=f"prefill_{n}", record=RECORD_MXFP8, block_size=block_size, num_blocks=num_blocks,
        page_stride=page_stride_for(RECORD_MXFP8, block_size), kv_bits=to_bf16_bits(x),
        slot_mapping=slots, positions=np.arange(n, dtype=np.int64), cos_sin=rope_table(n),
        backing_seed=seed + 100, gather_indices=np.arange(n, dtype=np.int32))


def legacy_65536(seed: int = 1004, n: int = 65536, block_size: int = 64,
                 num_blocks: int = 1280, max_pos: int = 65536) -> InsertCase:
    """N(0,1) rows into the 584 B legacy record (page stride padded to a
    multiple of 576 B); positions uniform in [0, max_pos); distinct random
    slots of a 1280-page cache with 5% set to -1."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    positions = rng.integers(0, max_pos, n, dtype=np.int64)
    slots = rng.permutation(num_blocks * block_size)[:n].astype(np.int64)
    slots = _drop(rng, slots, int(round(0.05 * n)))
    return InsertCase(
        name=f"legacy_{n}", record=RECORD_LEGACY, block_size=block_size, num_blocks=num_blocks,
        page_stride=page_stride_for(RECORD_LEGACY, block_size), kv_bits=to_bf16_bits(x),
        slot_mapping=slots, positions=positions, cos_sin=rope_table(max_pos),
        backing_seed=seed + 100, gather_indices=slots.astype(np.int32))


@dataclasses.dataclass
class TopkGather:
    """A cache filled in slot order in chunks, then gathered by sparse
    sorted per-query index lists."""

    name: str
    block_size: int
    num_blocks: int
    page_stride: int
    chunk: int
    max_pos: int
    seed: int
    indices: np.ndarray  # int32 [queries, topk]

    record: int = RECORD_MXFP8

    @property
    def total_slots(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def num_chunks(self) -> int:
        return (self.total_slots + self.chunk - 1) // self.chunk

    def cos_sin(self) -> np.ndarray:
        return rope_table(self.max_pos)

    def fill_chunk(self, k: int):
        """(kv_bits, slot_mapping, positions) of fill chunk k: N(0,1) rows for
        slots [k*chunk, (k+1)*chunk), position = slot % max_pos."""
        first = k * self.chunk
        n = min(self.chunk, self.total_slots - first)
        rng = np.random.default_rng((self.seed, 1, k))
        x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
        slots = np.arange(first, first + n, dtype=np.int64)
        return to_bf16_bits(x), slots, slots % self.max_pos


def topk_gather(seed: int = 1005, num_blocks: int = 32768, block_size: int = 64,
                queries: int = 64, topk: int = 2048, chunk: int = 262144,
                max_pos: int = 4096) -> TopkGather:
    """64 queries x 2048 indices, each list sorted ascending without repeats
    over all slots; 3% of each list set to -1 in place (order kept)."""
    rng = np.random.default_rng(seed)
    total = num_blocks * block_size
    idx = np.empty((queries, topk), np.int32)
    drop = int(round(0.03 * topk))
    for q in range(queries):
        row = np.sort(rng.choice(total, topk, replace=False)).astype(np.int32)
        row[rng.choice(topk, drop, replace=False)] = -1
        idx[q] = row
    return TopkGather(name=f"topk_{queries}x{topk}", block_size=block_size,
                      num_blocks=num_blocks, page_stride=page_stride_for(RECORD_MXFP8, block_size),
                      chunk=min(chunk, total), max_pos=max_pos, seed=seed, indices=idx)


def custom_insert(seed: int, n: int, record: int, block_size: int, num_blocks: int,
                  max_pos: int = 4096, drop_frac: float = 0.05, page_stride: Optional[int] = None,
                  scale_rows: bool = False) -> InsertCase:
    """Generic case for edge-size tests: N(0,1) rows (optionally times a
    per-row U(0.1, 10)), random positions, distinct random slots with a
    fraction set to -1, random pre-fill, and a padded page stride if given."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    if scale_rows:
        x *= rng.uniform(0.1, 10.0, (n, 1)).astype(np.float32)
    positions = rng.integers(0, max_pos, n, dtype=np.int64)
    total = num_blocks * block_size
    if n > total:
        raise ValueError("more tokens than cache slots")
    slots = rng.permutation(total)[:n].astype(np.int64)
    slots = _drop(rng, slots, int(round(drop_frac * n)))
    stride = page_stride if page_stride is not None else page_stride_for(record, block_size)
    return InsertCase(
        name=f"custom_{record}_{n}_bs{block_size}", record=record, block_size=block_size,
        num_blocks=num_blocks, page_stride=stride, kv_bits=to_bf16_bits(x), slot_mapping=slots,
        positions=positions, cos_sin=rope_table(max_pos), backing_seed=seed + 100,
        gather_indices=slots.astype(np.int32))


@dataclasses.dataclass
class AttentionWrite:
    """The attention write: q rows of every head plus the KV insert."""

    name: str
    q_bits: np.ndarray  # uint16 [n, heads, 512] (bf16 bits)
    eps: float
    insert: InsertCase


def attention_write(seed: int = 1006, n: int = 4096, heads: int = 128,
                    block_size: int = 64, eps: float = 1e-6) -> AttentionWrite:
    """A prefill chunk of n tokens through the attention write: q is N(0,1)
    times a per-(token, head) U(0.1, 10) with 1% of the heads all +0; the KV
    part is ``prefill``-like (positions 0.., slots 0.., N(0,1) rows with 0.5%
    of channels x300). The pages give no q shapes: 128 heads stands for a
    padded head count."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, heads, HEAD_DIM), dtype=np.float32)
    q *= rng.uniform(0.1, 10.0, (n, heads, 1)).astype(np.float32)
    zero = rng.random((n, heads)) < 0.01
    q[zero] = 0.0
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    chans = rng.choice(HEAD_DIM, int(round(0.005 * HEAD_DIM)), replace=False)
    x[:, chans] *= 300.0
    num_blocks = (n + block_size - 1) // block_size
    case = InsertCase(
        name=f"attention_write_{n}x{heads}", record=RECORD_MXFP8, block_size=block_size,
        num_blocks=num_blocks, page_stride=page_stride_for(RECORD_MXFP8, block_size),
        kv_bits=to_bf16_bits(x), slot_mapping=np.arange(n, dtype=np.int64),
        positions=np.arange(n, dtype=np.int64), cos_sin=rope_table(n), backing_seed=seed + 100)
    return AttentionWrite(case.name, to_bf16_bits(q), eps, case)


@dataclasses.dataclass
class SparseExpand:
    """Inputs of the sparse indexer's candidate-block expansion."""

    name: str
    cand: np.ndarray    # int32 [rows, K]
    row_ks: np.ndarray  # int32 [rows]
    row_ke: np.ndarray  # int32 [rows]
    ratio: int
    sparse_block: int


def sparse_expand(seed: int = 1007, seqs: int = 4, seq_len: int = 4096, k: int = 128,
                  ratio: int = 2, sparse_block: int = 8) -> SparseExpand:
    """A prefill chunk through the sparse indexer's expansion: `seqs`
    sequences of `seq_len` query tokens laid end to end in the chunk's KV, so
    row i of sequence s sees [s*seq_len, s*seq_len + i + 1) (causal). Its
    candidates are up to K distinct candidate blocks of ratio*sparse_block
    tokens drawn from those it can see, in random (score) order, padded with
    -1 when fewer exist: 2048 top-k tokens as 128 blocks of 16, split into
    sparse blocks of 8."""
    rng = np.random.default_rng(seed)
    rows = seqs * seq_len
    cand = np.full((rows, k), -1, np.int32)
    ks = np.repeat(np.arange(seqs, dtype=np.int64) * seq_len, seq_len).astype(np.int32)
    ke = (ks + np.tile(np.arange(1, seq_len + 1), seqs)).astype(np.int32)
    width = ratio * sparse_block
    for r in range(rows):
        avail = (int(ke[r] - ks[r]) + width - 1) // width
        take = min(k, avail)
        cand[r, :take] = rng.choice(avail, take, replace=False)
    return SparseExpand(f"sparse_expand_{rows}x{k}", cand, ks, ke, ratio, sparse_block)


def retarget(case: InsertCase, record: int, page_stride: Optional[int] = None) -> InsertCase:
    """The same tokens, slots and positions written to another cache format
    (e.g. the non-packed bf16 / fp8 caches), with that format's page stride
    unless one is given."""
    stride = page_stride if page_stride is not None else page_stride_for(record, case.block_size)
    return dataclasses.replace(case, name=f"{case.name}_as_{record}", record=record,
                               page_stride=stride)


CONFIGS = {
    "mixed_1024": mixed_1024,
    "decode_16384": decode_16384,
    "prefill_262144": prefill_262144,
    "legacy_65536": legacy_65536,
}
