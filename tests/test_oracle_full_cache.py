"""Pins of the oracle's non-packed cache insert (bf16 rows, and e4m3fn rows
with one fp32 per-tensor scale), [KV-only op] 实现拆解 1.

Nothing here calls the HIP path. The expected bytes come from a hand-worked
token (tests/golden/worked_tokens.json, "full_cache"), from library
primitives (torch's fp32 ops and its bf16 / float8_e4m3fn casts, numpy's
IEEE fp32 division) and from a brute-force search that tells the two
readings of the fp8 step apart.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_rope_amd import workloads as W

RNG = np.random.default_rng(1024512)


def _bf16_bits(x) -> np.ndarray:
    return W.to_bf16_bits(np.asarray(x, np.float32))


def _torch_e4m3_sat(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_rope(kv_bits: np.ndarray, positions: np.ndarray, table: np.ndarray) -> np.ndarray:
    """NeoX rotation of the tail as separate fp32 torch ops (no FMA)."""
    x = torch.from_numpy(kv_bits.view(np.int16)).view(torch.bfloat16).float()
    cs = torch.from_numpy(table[positions])
    c, s = cs[:, :32], cs[:, 32:]
    r = x.clone()
    x1, x2 = x[:, 448:480].clone(), x[:, 480:].clone()
    r[:, 448:480] = (x1 * c) - (x2 * s)
    r[:, 480:] = (x2 * c) + (x1 * s)
    return r.numpy()


def _library_full_insert(case: W.InsertCase, fp8_scale: float) -> np.ndarray:
    """Library restatement: torch rotation, torch casts, numpy placement."""
    b = case.initial_backing()
    ok = case.slot_mapping >= 0
    t = np.nonzero(ok)[0]
    r = _torch_rope(case.kv_bits[t], case.positions[t], case.cos_sin)
    if case.record == W.RECORD_BF16:
        rows = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
    else:
        with np.errstate(over="ignore"):  # tiny scales overflow to +-inf: saturated
            rows = _torch_e4m3_sat(r / np.float32(fp8_scale))
    for k, tok in enumerate(t):
        pg, off = divmod(int(case.slot_mapping[tok]), case.block_size)
        at = pg * case.page_stride + off * case.record
        b[at: at + case.record] = rows[k].reshape(-1)
    return b


def _oracle_full(case: W.InsertCase, fp8_scale: float = 1.0, kv=None) -> np.ndarray:
    b = case.initial_backing()
    oracle.insert_full(case.kv_bits if kv is None else kv, b, case.num_blocks, case.page_stride,
                       case.block_size, case.record, case.slot_mapping, case.positions,
                       case.cos_sin, fp8_scale)
    return b


def _golden_case(g, record: int) -> tuple:
    fc = g["full_cache"]
    inp = fc["inputs"]
    x = np.zeros((2, 512), np.float32)
    for d, v in inp["kv_nonzero_token0"]:
        x[0, d] = float(v)
    x[1, :] = 1.0
    table = np.zeros((inp["max_pos"], 64), np.float32)
    table[:, :32] = 1.0
    table[3, 0], table[3, 32] = 0.5, 0.75
    exp = fc["bf16_cache" if record == W.RECORD_BF16 else "fp8_cache"]
    case = W.InsertCase("full_worked", record, inp["block_size"], inp["num_blocks"],
                        exp["page_stride"], _bf16_bits(x),
                        np.array([t["slot"] for t in inp["tokens"]], np.int64),
                        np.array([t["position"] for t in inp["tokens"]], np.int64), table,
                        backing_seed=33)
    return case, exp, inp["fp8_scale"]


@pytest.mark.parametrize("record", [W.RECORD_BF16, W.RECORD_FP8])
def test_worked_token(golden, record):
    case, exp, scale = _golden_case(golden, record)
    got = _oracle_full(case, scale)
    before = case.initial_backing()
    at = exp["row_offset"]
    row = got[at: at + record]
    if record == W.RECORD_BF16:
        want = np.zeros(512, np.uint16)
        for d, v in exp["elements_nonzero"]:
            want[d] = v
        assert row.view(np.uint16).tolist() == want.tolist()
    else:
        want = np.zeros(512, np.uint8)
        for d, v in exp["codes_nonzero"]:
            want[d] = v
        assert row.tolist() == want.tolist()
    # nothing else changed: the skipped token, the padding, the other slots
    mask = np.ones(got.size, bool)
    mask[at: at + record] = False
    assert np.array_equal(got[mask], before[mask])


def test_worked_fp8_scale_three(golden):
    ex = golden["full_cache"]["fp8_cache"]["scale_3_example"]
    case = W.custom_insert(5, 1, W.RECORD_FP8, 1, 1, max_pos=1, drop_frac=0.0)
    kv = np.zeros((1, 512), np.uint16)
    kv[0, 0] = _bf16_bits([ex["value"]])[0]
    got = _oracle_full(case, ex["fp8_scale"], kv=kv)
    assert got[0] == ex["code"]


def test_full_page_geometry():
    for bs in (1, 3, 32, 64, 256):
        assert W.page_stride_for(W.RECORD_BF16, bs) == bs * 1024
        assert W.page_stride_for(W.RECORD_FP8, bs) == bs * 512


@pytest.mark.parametrize("record", [W.RECORD_BF16, W.RECORD_FP8])
@pytest.mark.parametrize("bs,nb,n,pad", [(1, 7, 7, 0), (3, 4, 10, 16), (64, 3, 150, 48)])
def test_full_insert_vs_library(record, bs, nb, n, pad):
    """Every byte of a pre-filled backing, padded page strides included."""
    stride = W.page_stride_for(record, bs) + pad
    case = W.custom_insert(77 + bs + n + record, n, record, bs, nb, max_pos=300,
                           page_stride=stride, drop_frac=0.2, scale_rows=True)
    scales = [1.0] if record == W.RECORD_BF16 else [1.0, 0.0123, 3.7, 2.0 ** -10, 1e3]
    for s in scales:
        got = _oracle_full(case, s)
        want = _library_full_insert(case, s)
        assert np.array_equal(got, want), (record, bs, s)


def test_fp8_saturation_and_tiny_quotients():
    """A tiny scale drives quotients past 448 (and to +-inf in fp32): they
    saturate to 0x7E / 0xFE. A huge scale drives them into the e4m3
    subnormals and to zero, keeping the sign."""
    case = W.custom_insert(91, 40, W.RECORD_FP8, 8, 6, max_pos=64, drop_frac=0.0)
    for s in (1e-3, 1e-38, 2.0 ** 20, 3e38):
        got = _oracle_full(case, s)
        want = _library_full_insert(case, s)
        assert np.array_equal(got, want), s
    r = _torch_rope(case.kv_bits, case.positions, case.cos_sin)
    codes = _oracle_full(case, 1e-38)
    pg, off = divmod(int(case.slot_mapping[0]), case.block_size)
    at = pg * case.page_stride + off * 512
    sat = np.where(r[0] > 0, 0x7E, np.where(r[0] < 0, 0xFE, codes[at: at + 512]))
    assert np.array_equal(codes[at: at + 512], sat)


def test_bf16_nope_dims_are_the_input_bits():
    case = W.custom_insert(17, 64, W.RECORD_BF16, 16, 5, max_pos=1000, drop_frac=0.1)
    kv = case.kv_bits.copy()
    kv[:, :4] = [0x8000, 0x0001, 0x807F, 0x7F7F]  # -0, subnormals, the largest finite
    got = _oracle_full(case, kv=kv)
    for t in np.nonzero(case.slot_mapping >= 0)[0]:
        pg, off = divmod(int(case.slot_mapping[t]), case.block_size)
        at = pg * case.page_stride + off * 1024
        assert np.array_equal(got[at: at + 896].view(np.uint16), kv[t, :448])


def test_fp8_quotient_is_rounded_to_fp32_first():
    """The fp8 element is the e4m3 code of the binary32 quotient, not of the
    exact one. Scales s = fl32(x / T) for e4m3 midpoints T make the fp32
    quotient fl(x / s) land exactly on T while the exact quotient x / s lies
    just above or below it: there the two readings differ, and the oracle
    must follow the fp32 one (ties to the even code)."""
    # midpoints between neighbouring normal e4m3 values: 1.mmm1 * 2^k
    ties = [(1.0 + (2 * m + 1) / 16.0) * 2.0 ** k for m in range(8) for k in (-3, 0, 1, 5)]
    mags = np.arange(0x3C00, 0x4400, 37, dtype=np.uint16)  # bf16 in [2^-7, 2^9)
    xs = (mags.astype(np.uint32) << 16).view(np.float32)
    hits = []
    for T in ties:
        sc = (xs.astype(np.float64) / T).astype(np.float32)
        q = xs / sc  # IEEE binary32 division
        for i in np.nonzero(q == np.float32(T))[0]:
            if Fraction(float(xs[i])) != Fraction(T) * Fraction(float(sc[i])):
                hits.append((int(mags[i]), float(xs[i]), float(sc[i]), T))
    assert len(hits) >= 50, "the search should find fp32-rounded ties"
    differ = 0
    for bits, xv, sv, T in hits[:400]:
        case = W.custom_insert(3, 1, W.RECORD_FP8, 1, 1, max_pos=1, drop_frac=0.0)
        kv = np.zeros((1, 512), np.uint16)
        kv[0, 5] = bits
        got = int(_oracle_full(case, sv, kv=kv)[5])
        # fp32 reading: the tie T goes to the even code
        assert got == int(_torch_e4m3_sat(np.array([T], np.float32))[0]), (xv, sv, T)
        # exact reading: the side of T the exact quotient lies on
        exact = Fraction(xv) / Fraction(sv)
        if (exact > Fraction(T)) != (Fraction(oracle.e4m3_value(got)) > Fraction(T)):
            differ += 1
    assert differ >= 10, "some of the ties must separate the two readings"
