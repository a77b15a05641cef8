"""Helpers shared by the GPU parity tests and the smoke check.

The oracle is run over token (or row) chunks in parallel threads. Tokens are
independent and a cache's slots are distinct, so the chunked result is the
same byte for byte as one serial call; ctypes releases the GIL while the C
code runs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
from quantized_paged_kv_rope_amd import binding as B
from quantized_paged_kv_rope_amd import workloads as W


def workers() -> int:
    # at most 16 worker threads: the host CPU share of a one-GPU machine
    return max(1, min(16, os.cpu_count() or 1))


def oracle_insert(case: W.InsertCase, backing: np.ndarray, kv_bits=None, slots=None,
                  positions=None, chunk: int = 8192, **opts) -> np.ndarray:
    kv = case.kv_bits if kv_bits is None else kv_bits
    sl = case.slot_mapping if slots is None else slots
    ps = case.positions if positions is None else positions
    n = sl.shape[0]
    jobs = [(a, min(n, a + chunk)) for a in range(0, n, chunk)]

    def run(ab):
        a, b = ab
        oracle.insert(kv[a:b], backing, case.num_blocks, case.page_stride, case.block_size,
                      case.record, sl[a:b], ps[a:b], case.cos_sin, **opts)

    if len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        with cf.ThreadPoolExecutor(workers()) as ex:
            list(ex.map(run, jobs))
    return backing


def oracle_insert_full(case: W.InsertCase, backing: np.ndarray, fp8_scale: float = 1.0,
                       chunk: int = 8192) -> np.ndarray:
    """The oracle's non-packed insert (record 1024 or 512), over token chunks."""
    n = case.slot_mapping.shape[0]
    jobs = [(a, min(n, a + chunk)) for a in range(0, n, chunk)]

    def run(ab):
        a, b = ab
        oracle.insert_full(case.kv_bits[a:b], backing, case.num_blocks, case.page_stride,
                           case.block_size, case.record, case.slot_mapping[a:b],
                           case.positions[a:b], case.cos_sin, fp8_scale)

    with cf.ThreadPoolExecutor(workers()) as ex:
        list(ex.map(run, jobs))
    return backing


def oracle_gather(case_like, backing: np.ndarray, indices: np.ndarray,
                  chunk: int = 16384) -> np.ndarray:
    flat = np.ascontiguousarray(indices, np.int32).reshape(-1)
    out = np.empty((flat.size, 512), np.uint16)
    jobs = [(a, min(flat.size, a + chunk)) for a in range(0, flat.size, chunk)]

    def run(ab):
        a, b = ab
        out[a:b] = oracle.gather(backing, case_like.num_blocks, case_like.page_stride,
                                 case_like.block_size, case_like.record, flat[a:b])

    with cf.ThreadPoolExecutor(workers()) as ex:
        list(ex.map(run, jobs))
    return out.reshape(indices.shape + (512,))


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceCase:
    """A case's inputs on the GPU plus its cache backing."""

    def __init__(self, case: W.InsertCase, device="cuda", backing: np.ndarray = None):
        self.case = case
        self.kv = dev_bf16(case.kv_bits, device)
        self.slots = dev(case.slot_mapping, device)
        self.positions = dev(case.positions, device)
        self.cos_sin = dev(case.cos_sin, device)
        init = case.initial_backing() if backing is None else backing
        self.backing, self.k_cache = B.alloc_cache(case.num_blocks, case.block_size, case.record,
                                                   case.page_stride, backing=dev(init, device))

    def insert(self, kv=None, slots=None, positions=None, **opts):
        B.kvrec_insert(self.kv if kv is None else kv, self.k_cache,
                       self.slots if slots is None else slots,
                       self.positions if positions is None else positions,
                       self.cos_sin, self.case.block_size, **opts)

    def insert_full(self, fp8_scale=None):
        """Non-packed insert; ``fp8_scale`` a float (uploaded) or None."""
        sc = None
        if fp8_scale is not None:
            sc = torch.tensor([fp8_scale], dtype=torch.float32, device=self.kv.device)
        B.kvrec_insert_full(self.kv, self.k_cache, self.slots, self.positions, self.cos_sin,
                            self.case.block_size, sc)

    def gather(self, indices: np.ndarray) -> np.ndarray:
        out = B.kvrec_gather(self.k_cache, dev(np.ascontiguousarray(indices, np.int32)))
        return host_bits(out)

    def backing_host(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.backing.cpu().numpy()


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    if bad.size == 0:
        return "identical"
    i = int(bad[0])
    return f"{bad.size} differing elements; first at flat index {i}: got {a.reshape(-1)[i]!r}, " \
           f"want {b.reshape(-1)[i]!r}"
