"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's own formulas: each compares it with
a value worked by hand (tests/golden), a library routine that implements the
same format (torch's float8_e4m3fn and bfloat16 casts), an independent
float64 evaluation of the pages' closed form, or an invariant that a dropped
term, a wrong sign or index, or a transposed operand would break.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_rope_amd import workloads as W

RNG = np.random.default_rng(20261202)


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Record sizes and page geometry ([MXFP8 record] 功能与动机; [Sparse indexer]
# 实现拆解 4 for the block-stride rule).
# --------------------------------------------------------------------------

def test_record_byte_counts():
    assert 512 + 16 == oracle.RECORD_MXFP8 == 528
    assert 448 + 128 + 7 + 1 == oracle.RECORD_LEGACY == 584
    assert round((584 - 528) / 584 * 100, 1) == 9.6  # the pages' "-9.6%"
    assert 512 // 32 == 16 and 512 // 64 == 8       # scale bytes per record


@pytest.mark.parametrize("bs,v41,v4", [(32, 16896, 19008), (64, 33792, 37440),
                                        (128, 67584, 74880), (256, 135168, 149760)])
def test_page_stride_closed_form(bs, v41, v4):
    # block_size a multiple of 32 -> the MXFP8 page is an exact multiple of 512
    assert bs * 528 == v41 and v41 % 512 == 0
    assert W.page_stride_for(528, bs) == v41
    assert W.page_stride_for(584, bs) == v4 and v4 % 576 == 0 and v4 >= bs * 584
    assert v4 - bs * 584 == {32: 320, 64: 64, 128: 128, 256: 256}[bs]


def test_mixed_block_stride_rule():
    # The failure the pages describe: a block stride of 212160 B divides by
    # neither TMA stride; rounding block bytes up to lcm(512, 576) = 4608 fixes it.
    assert 212160 % 512 == 192 and 212160 % 576 == 192
    assert math.lcm(512, 576) == 4608


# --------------------------------------------------------------------------
# Hand-worked tokens.
# --------------------------------------------------------------------------

def _golden_inputs(g):
    inp = g["inputs"]
    x = np.zeros(512, np.float32)
    for d, v in inp["kv_nonzero"]:
        x[d] = float(v)
    kv = _torch_bf16(x[None, :])
    assert np.array_equal(_bf16_to_f32(kv[0]).view(np.uint32), x.view(np.uint32)), \
        "worked inputs must be exact bf16 values"
    table = np.zeros((inp["max_pos"], 64), np.float32)
    table[:, :32] = 1.0
    table[3, 0], table[3, 32] = 0.5, 0.75
    table[3, 1], table[3, 33] = 0.0, 1.0
    return kv, table


@pytest.mark.parametrize("record", [528, 584])
def test_worked_token_insert(golden, record):
    inp = golden["inputs"]
    kv, table = _golden_inputs(golden)
    key = "mxfp8_record" if record == 528 else "legacy_record"
    exp = golden[key]
    bs, nb = inp["block_size"], inp["num_blocks"]
    assert W.page_stride_for(record, bs) == exp["page_stride"]
    for fill in (0x00, 0xA5):
        backing = np.full(nb * exp["page_stride"], fill, np.uint8)
        oracle.insert(kv, backing, nb, exp["page_stride"], bs, record,
                      np.array([inp["slot"]], np.int64), np.array([inp["position"]], np.int64), table)
        d0, s0 = exp["data_offset"], exp["scale_offset"]
        if record == 528:
            codes = np.zeros(512, np.uint8)
            for d, c in exp["codes_nonzero"]:
                codes[d] = c
            assert backing[d0:d0 + 512].tolist() == codes.tolist()
            assert backing[s0:s0 + 16].tolist() == exp["scales"]
            written = np.zeros(backing.size, bool)
            written[d0:d0 + 512] = True
            written[s0:s0 + 16] = True
        else:
            codes = np.zeros(448, np.uint8)
            for d, c in exp["codes_nonzero"]:
                codes[d] = c
            assert backing[d0:d0 + 448].tolist() == codes.tolist()
            tail = backing[d0 + 448:d0 + 576].view(np.uint16)  # little-endian host
            want = np.zeros(64, np.uint16)
            for i, h in exp["rope_bf16"]:
                want[i] = h
            assert tail.tolist() == want.tolist()
            assert backing[s0:s0 + 8].tolist() == exp["scale_row"]
            written = np.zeros(backing.size, bool)
            written[d0:d0 + 576] = True
            written[s0:s0 + 8] = True
        assert written.sum() == record
        assert (backing[~written] == fill).all(), "bytes outside the record were touched"


def test_worked_token_gather(golden):
    inp = golden["inputs"]
    kv, table = _golden_inputs(golden)
    exp = golden["mxfp8_record"]
    backing = np.zeros(inp["num_blocks"] * exp["page_stride"], np.uint8)
    oracle.insert(kv, backing, inp["num_blocks"], exp["page_stride"], inp["block_size"], 528,
                  np.array([inp["slot"]], np.int64), np.array([inp["position"]], np.int64), table)
    out = oracle.gather(backing, inp["num_blocks"], exp["page_stride"], inp["block_size"], 528,
                        np.array([inp["slot"], -1], np.int32))
    for d, h in exp["gather_bf16"]:
        assert out[0, d] == h, d
    assert (out[1] == 0).all()


# --------------------------------------------------------------------------
# e4m3fn: library routine (torch's float8_e4m3fn) and an independent
# nearest-value search.
# --------------------------------------------------------------------------

def test_e4m3_decode_all_codes_vs_torch():
    ours = oracle.e4m3_values()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def _sweep_chunk(first, count):
    codes = oracle.e4m3_encode_bits(first, count)
    bits = np.arange(first, first + count, dtype=np.uint64).astype(np.uint32)
    ref = _torch_e4m3(bits.view(np.float32))
    bad = np.nonzero(codes != ref)[0]
    return (first, bad[:5].tolist(), int(bad.size))


def test_e4m3_encode_exhaustive_nonnegative_vs_torch():
    """Every non-negative fp32 up to 448 (1.14e9 values): oracle == torch."""
    last = int(np.float32(448.0).view(np.uint32))
    chunk = 1 << 24
    starts = list(range(0, last + 1, chunk))
    jobs = [(s, min(chunk, last + 1 - s)) for s in starts]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        results = list(ex.map(lambda a: _sweep_chunk(*a), jobs))
    bad = [r for r in results if r[2]]
    assert not bad, bad[:3]


def test_e4m3_encode_negative_and_saturation():
    y = RNG.standard_normal(2_000_000).astype(np.float32) * np.float32(60.0)
    y = y[np.abs(y) <= 448]
    assert np.array_equal(oracle.e4m3_encode_f32(y), _torch_e4m3(y))
    assert np.array_equal(oracle.e4m3_encode_f32(-np.abs(y)), oracle.e4m3_encode_f32(np.abs(y)) | 0x80)
    assert oracle.e4m3_encode(-0.0) == 0x80 and oracle.e4m3_encode(0.0) == 0x00
    for v in (448.0, 460.0, 500.0, 1e30):
        assert oracle.e4m3_encode(v) == 0x7E and oracle.e4m3_encode(-v) == 0xFE


def test_e4m3_encode_nearest_value_search():
    """Independent nearest-representable search with ties to the even code."""
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    y = np.concatenate([
        RNG.uniform(0, 448, 60_000), np.exp2(RNG.uniform(-12, 8.8, 60_000)),
        (vals[:-1] + vals[1:]) / 2,  # every midpoint (ties)
        vals,
    ]).astype(np.float32)
    y = y[(y >= 0) & (y <= 448)]
    d = np.abs(y.astype(np.float64)[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    pick = np.where(cand.sum(1) == 1, cand.argmax(1),
                    np.where(cand & (np.arange(127)[None, :] % 2 == 0), 1, 0).argmax(1))
    assert np.array_equal(oracle.e4m3_encode_f32(y), pick.astype(np.uint8))


# --------------------------------------------------------------------------
# bf16 rounding: torch's round-to-nearest-even cast.
# --------------------------------------------------------------------------

def test_bf16_round_vs_torch():
    hi = RNG.integers(0, 1 << 16, 1_000_000, dtype=np.uint32) << 16
    lo = RNG.integers(0, 1 << 16, hi.size, dtype=np.uint32)
    special = np.array([0x8000, 0x7FFF, 0x8001, 0x18000, 0x17FFF], np.uint32)  # ties and neighbours
    bits = np.concatenate([hi | lo, (hi & 0xFFFE0000) | special[RNG.integers(0, 5, hi.size)]])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.bf16_round_f32(x), _torch_bf16(x))
    # the largest finite bf16 is (2 - 2^-7) * 2^127; the midpoint to 2^128 is a
    # tie with an odd mantissa, so it rounds up to infinity, just below it does not
    edge = np.array([(2 - 2.0 ** -8) * 2.0 ** 127, np.nextafter(np.float32((2 - 2.0 ** -8) * 2.0 ** 127),
                                                                 np.float32(0))], np.float32)
    assert oracle.bf16_round_f32(edge).tolist() == [0x7F80, 0x7F7F] == _torch_bf16(edge).tolist()
    assert oracle.bf16_round(-0.0) == 0x8000


# --------------------------------------------------------------------------
# UE8M0 exponent: the pages' closed form ceil(log2(amax / 448)) evaluated in
# float64 (exact enough to separate every fp32 amax from the 448 * 2^k
# boundaries), plus hand values, clamp and monotonicity.
# --------------------------------------------------------------------------

def test_scale_exponent_worked_values():
    cases = {1.0: -8, 448.0: 0, 449.0: 1, 0.3: -10, 1500.0: 2, 2.0 ** -140: -127, 0.0: 0,
             3.5: -7, 1.75: -8, 1.7500001: -7, 3.4028235e38: 120}
    for a, e in cases.items():
        assert oracle.scale_exponent(a) == e, a


def test_scale_exponent_vs_float64_closed_form():
    mant = np.concatenate([np.arange(0x5FFFF0, 0x600010), RNG.integers(0, 1 << 23, 64)]).astype(np.uint32)
    expo = np.arange(1, 255, dtype=np.uint32)
    bits = (expo[:, None] << 23 | mant[None, :]).ravel()
    bits = np.concatenate([bits, RNG.integers(1, 0x7F800000, 300_000, dtype=np.uint32),
                           np.arange(1, 2000, dtype=np.uint32)])  # subnormals
    amax = bits.view(np.float32)
    got = oracle.scale_exponent_f32(amax)
    want = np.clip(np.ceil(np.log2(amax.astype(np.float64) / 448.0)), -127, 127).astype(np.int32)
    assert np.array_equal(got, want)
    order = np.argsort(amax)
    assert (np.diff(got[order]) >= 0).all(), "exponent must be non-decreasing in amax"
    # every group max lands in (224, 448] after scaling, unless clamped
    scaled = amax.astype(np.float64) * np.exp2(-got.astype(np.float64))
    free = got > -127
    assert (scaled[free] > 224).all() and (scaled[free] <= 448).all()


# --------------------------------------------------------------------------
# RoPE: position 0 is the identity; exact-arithmetic tables; a general bound.
# --------------------------------------------------------------------------

def test_rope_table_values():
    t = W.rope_table(4096)
    assert t[0, :32].tolist() == [1.0] * 32 and t[0, 32:].tolist() == [0.0] * 32
    assert np.float32(t[1, 0]) == np.float32(0.5403023) and np.float32(t[1, 32]) == np.float32(0.84147096)
    assert np.float32(t[1, 31]) == np.float32(1.0) and np.float32(t[1, 63]) == np.float32(1.3335214e-4)
    assert np.float32(t[4095, 0]) == np.float32(-0.065975994)
    assert np.float32(t[4095, 32]) == np.float32(-0.9978212)


def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((64, 512)).astype(np.float32)
    kv = _torch_bf16(x)
    kv[kv == 0x8000] = 0  # -0 under the rotation is +0 in x1*1 - x2*0 when x2 >= 0
    r = oracle.rope_rows(kv, np.zeros(64, np.int64), W.rope_table(8))
    assert np.array_equal(r.view(np.uint32), _bf16_to_f32(kv).view(np.uint32))


def test_rope_exact_tables_pin_pairing_and_signs():
    """Tables whose entries have few significant bits make every product and
    sum exact in fp32, so the rotation must equal the float64 value exactly.
    Distinct c and s per column detect a swapped cos/sin half, a wrong pair
    partner, or a wrong sign."""
    n, P = 256, 5
    # k / 64 with |k| <= 255: at most 8 significant bits (exact in bf16) and
    # a bounded exponent range, so x * c (c = j / 8) is an integer multiple of
    # 2^-9 below 2^12 and so is the sum of two such products: all exact in fp32.
    x = (RNG.integers(-255, 256, (n, 512)) / 64.0).astype(np.float32)
    kv = _torch_bf16(x)
    xf = _bf16_to_f32(kv).astype(np.float64)
    table = np.zeros((P, 64), np.float32)
    table[:, :32] = RNG.integers(-8, 9, (P, 32)) / 8.0
    table[:, 32:] = RNG.integers(-8, 9, (P, 32)) / 8.0
    pos = RNG.integers(0, P, n)
    r = oracle.rope_rows(kv, pos, table).astype(np.float64)
    c, s = table[pos, :32].astype(np.float64), table[pos, 32:].astype(np.float64)
    x1, x2 = xf[:, 448:480], xf[:, 480:512]
    assert np.array_equal(r[:, :448], xf[:, :448])
    assert np.array_equal(r[:, 448:480], x1 * c - x2 * s)
    assert np.array_equal(r[:, 480:512], x2 * c + x1 * s)
    # quarter-turn: (c, s) = (0, 1) maps (x1, x2) -> (-x2, x1)
    q = np.zeros((1, 64), np.float32)
    q[0, 32:] = 1.0
    rq = oracle.rope_rows(kv, np.zeros(n, np.int64), q)
    assert np.array_equal(rq[:, 448:480] + 0.0, -xf[:, 480:512].astype(np.float32) + 0.0)
    assert np.array_equal(rq[:, 480:512] + 0.0, xf[:, 448:480].astype(np.float32) + 0.0)


def test_rope_general_error_bound():
    n = 512
    kv = _torch_bf16(RNG.standard_normal((n, 512)).astype(np.float32) * 3)
    table = W.rope_table(70000)
    pos = RNG.integers(0, 70000, n)
    r = oracle.rope_rows(kv, pos, table).astype(np.float64)
    xf = _bf16_to_f32(kv).astype(np.float64)
    c, s = table[pos, :32].astype(np.float64), table[pos, 32:].astype(np.float64)
    x1, x2 = xf[:, 448:480], xf[:, 480:512]
    for got, a, b in ((r[:, 448:480], x1 * c, -x2 * s), (r[:, 480:512], x2 * c, x1 * s)):
        # two rounded products and one rounded sum: |err| <= u(|a| + |b|) + u|a + b|
        u = 2.0 ** -24
        bound = u * (np.abs(a) + np.abs(b)) * 1.0000001 + u * np.abs(a + b) + 1e-45
        assert (np.abs(got - (a + b)) <= bound).all()
    # the rotation preserves the pair norm up to rounding
    n0 = x1 ** 2 + x2 ** 2
    n1 = r[:, 448:480] ** 2 + r[:, 480:512] ** 2
    assert np.allclose(n1, n0, rtol=1e-5, atol=1e-30)


# --------------------------------------------------------------------------
# Whole-op invariants on the real workload shapes (small sizes).
# --------------------------------------------------------------------------

def _run_insert(case, backing=None, kv=None):
    b = case.initial_backing() if backing is None else backing
    oracle.insert(case.kv_bits if kv is None else kv, b, case.num_blocks, case.page_stride,
                  case.block_size, case.record, case.slot_mapping, case.positions, case.cos_sin)
    return b


def _record_mask(case, slots):
    m = np.zeros(case.backing_bytes, bool)
    for s in slots:
        if s < 0:
            continue
        pg, off = divmod(int(s), case.block_size)
        base = pg * case.page_stride
        if case.record == 528:
            m[base + off * 512: base + off * 512 + 512] = True
            m[base + case.block_size * 512 + off * 16: base + case.block_size * 512 + off * 16 + 16] = True
        else:
            m[base + off * 576: base + off * 576 + 576] = True
            m[base + case.block_size * 576 + off * 8: base + case.block_size * 576 + off * 8 + 8] = True
    return m


@pytest.mark.parametrize("record", [528, 584])
def test_only_record_bytes_change_and_idempotent(record):
    case = W.custom_insert(7, 300, record, 32, 12)
    before = case.initial_backing()
    kv0 = case.kv_bits.copy()
    after = _run_insert(case, before.copy())
    mask = _record_mask(case, case.slot_mapping)
    assert (after[~mask] == before[~mask]).all()
    assert mask.sum() == record * int((case.slot_mapping >= 0).sum())
    again = _run_insert(case, after.copy())
    assert np.array_equal(again, after)
    assert np.array_equal(case.kv_bits, kv0)
    # every slot -1: nothing changes
    case.slot_mapping[:] = -1
    assert np.array_equal(_run_insert(case, before.copy()), before)


def test_out_of_range_guard_skips_token():
    case = W.custom_insert(8, 10, 528, 16, 2)
    case.slot_mapping[:] = np.arange(10)
    case.slot_mapping[3] = 32          # == num_blocks * block_size
    case.positions[5] = case.cos_sin.shape[0]
    before = case.initial_backing()
    after = _run_insert(case, before.copy())
    mask = _record_mask(case, [s for i, s in enumerate(case.slot_mapping) if i not in (3, 5)])
    assert (after[~mask] == before[~mask]).all()
    out = oracle.gather(after, case.num_blocks, case.page_stride, case.block_size, 528,
                        np.array([32, 10 ** 6, -5], np.int32))
    assert (out == 0).all()


def test_scale_equivariance_and_sign_symmetry():
    """Doubling a row's NoPE dims (exact in bf16) must add 1 to every NoPE
    scale byte and leave the codes unchanged; negating them flips only the
    code sign bits."""
    case = W.custom_insert(9, 64, 528, 64, 1, drop_frac=0.0)
    case.positions[:] = 0  # identity rotation
    case.slot_mapping[:] = np.arange(64)
    x = _bf16_to_f32(case.kv_bits)
    base = _run_insert(case, np.zeros(case.backing_bytes, np.uint8))
    dbl = _run_insert(case, np.zeros(case.backing_bytes, np.uint8), kv=_torch_bf16(x * 2))
    neg = _run_insert(case, np.zeros(case.backing_bytes, np.uint8), kv=_torch_bf16(-x))
    data = lambda b: b[:64 * 512].reshape(64, 512)
    scl = lambda b: b[64 * 512:64 * 528].reshape(64, 16)
    assert np.array_equal(data(dbl), data(base))
    assert np.array_equal(scl(dbl).astype(int), scl(base).astype(int) + 1)
    nz = data(base) & 0x7F != 0
    assert np.array_equal(data(neg)[nz], data(base)[nz] ^ 0x80)
    assert np.array_equal(scl(neg), scl(base))


@pytest.mark.parametrize("record", [528, 584])
def test_round_trip_error_bound(record):
    """insert -> gather: |out - r| <= half an e4m3 ulp of the scaled value
    times the group scale; legacy RoPE dims come back as bf16(r) exactly."""
    case = W.mixed_1024(n=512, num_blocks=10, record=record)
    b = _run_insert(case)
    out = oracle.gather(b, case.num_blocks, case.page_stride, case.block_size, record,
                        case.gather_indices)
    valid = case.slot_mapping >= 0
    r = oracle.rope_rows(case.kv_bits, case.positions, case.cos_sin).astype(np.float64)
    got = _bf16_to_f32(out).astype(np.float64)
    assert (out[~valid] == 0).all()
    r, got = r[valid], got[valid]
    fp8 = 512 if record == 528 else 448
    gsz = 32 if record == 528 else 64
    g = r[:, :fp8].reshape(r.shape[0], -1, gsz)
    amax = np.abs(g).max(axis=2)
    e = np.where(amax == 0, 0, np.clip(np.ceil(np.log2(np.maximum(amax, 1e-300) / 448)), -127, 127))
    y = np.abs(g) * np.exp2(-e)[:, :, None]
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.maximum(y, 1e-300))), -6) - 3)
    bound = 0.5 * ulp * np.exp2(e)[:, :, None]
    err = np.abs(got[:, :fp8].reshape(g.shape) - g)
    assert (err <= bound).all()
    # max-code invariant: the largest code magnitude of a non-zero group is 0x76..0x7E
    nz = amax > 0
    assert (y.max(axis=2)[nz] > 224).all() and (y.max(axis=2)[nz] <= 448).all()
    if record == 528:
        recs = np.stack([b[(s // 64) * case.page_stride + (s % 64) * 512:][:512]
                         for s in case.slot_mapping[valid]]).reshape(-1, 16, 32)
        top = (recs & 0x7F).max(axis=2)
        assert ((top[nz] >= 0x76) & (top[nz] <= 0x7E)).all()
    if record == 584:
        tail = _torch_bf16(r[:, 448:].astype(np.float32))
        assert np.array_equal(out[valid][:, 448:], tail)


def test_independent_vectorised_reference_small_caches():
    """A second, vectorised implementation built only from library primitives
    (torch casts, numpy float64 log2) agrees with the oracle on every byte of
    small caches, including padded page strides and tiny block sizes."""
    for record in (528, 584):
        for bs, nb, n in ((1, 5, 5), (2, 3, 6), (3, 4, 9), (32, 3, 90), (64, 2, 100)):
            align = 512 if record == 528 else 576
            stride = W.page_stride_for(record, bs) + align  # one extra aligned unit of padding
            case = W.custom_insert(1000 + bs * 7 + n, n, record, bs, nb, page_stride=stride,
                                   drop_frac=0.2, scale_rows=True)
            got = _run_insert(case)
            want = _vectorised_insert(case)
            assert np.array_equal(got, want), (record, bs)


def _vectorised_insert(case, kv=None, rope="neox", compress_ratio=1, amax_floor=0.0,
                       sanitize_nans=False):
    """Library-primitive restatement (torch casts and elementwise ops, numpy
    indexing) of the insert and its compressed-KV options."""
    kv = case.kv_bits if kv is None else kv
    b = case.initial_backing()
    R = compress_ratio
    ok = (case.slot_mapping >= 0) & ((case.positions + 1) % R == 0)
    t = np.nonzero(ok)[0]
    x = torch.from_numpy(kv[t].view(np.int16)).view(torch.bfloat16).float()
    rows = case.positions[t] // R * R
    cs = torch.from_numpy(case.cos_sin[rows])
    c, s = cs[:, :32], cs[:, 32:]
    r = x.clone()
    if rope == "neox":
        x1, x2 = x[:, 448:480].clone(), x[:, 480:].clone()
        r[:, 448:480] = (x1 * c) - (x2 * s)
        r[:, 480:] = (x2 * c) + (x1 * s)
    elif rope == "interleaved":
        cc = torch.cat([torch.ones(len(t), 224), c], dim=1)
        ss = torch.cat([torch.zeros(len(t), 224), s], dim=1)
        xe, xo = x[:, 0::2].clone(), x[:, 1::2].clone()
        r[:, 0::2] = (xe * cc) - (xo * ss)
        r[:, 1::2] = (xo * cc) + (xe * ss)
    if sanitize_nans:
        r = torch.where(r == r, r, torch.zeros_like(r))
    fp8 = 512 if case.record == 528 else 448
    gsz = 32 if case.record == 528 else 64
    g = r[:, :fp8].reshape(len(t), -1, gsz).double()
    amax = torch.clamp(g.abs().amax(dim=2), min=float(np.float32(amax_floor)))
    e = torch.where(amax == 0, torch.zeros_like(amax),
                    torch.clamp(torch.ceil(torch.log2(amax.clamp_min(1e-300) / 448)), -127, 127))
    y = (g * torch.exp2(-e)[:, :, None]).float().clamp(-448, 448)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(len(t), fp8).numpy()
    sbytes = (e + 127).to(torch.uint8).numpy()
    for k, tok in enumerate(t):
        pg, off = divmod(int(case.slot_mapping[tok]), case.block_size)
        base = pg * case.page_stride
        if case.record == 528:
            b[base + off * 512: base + off * 512 + 512] = codes[k]
            so = base + case.block_size * 512 + off * 16
            b[so: so + 16] = sbytes[k]
        else:
            row = base + off * 576
            b[row: row + 448] = codes[k]
            b[row + 448: row + 576] = r[k, 448:].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
            so = base + case.block_size * 576 + off * 8
            b[so: so + 7] = sbytes[k]
            b[so + 7] = 0
    return b


def test_gather_all_code_scale_pairs_vs_library():
    """Every e4m3 code (NaN codes excluded) under every scale byte 0..254,
    decoded by torch and rounded by torch's bf16 cast."""
    bs = 16
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)  # 254 codes
    scales = np.arange(255, dtype=np.uint8)
    # one record per (scale, chunk of 32 codes): all groups of a record share the scale
    chunks = [codes[i:i + 32] for i in range(0, codes.size, 32)]
    chunks[-1] = np.concatenate([chunks[-1], np.zeros(32 - chunks[-1].size, np.uint8)])
    recs = [(s, ch) for s in scales for ch in chunks]
    nb = (len(recs) + bs - 1) // bs
    stride = W.page_stride_for(528, bs)
    b = np.zeros(nb * stride, np.uint8)
    for j, (s, ch) in enumerate(recs):
        pg, off = divmod(j, bs)
        b[pg * stride + off * 512: pg * stride + off * 512 + 512] = np.tile(ch, 16)
        b[pg * stride + bs * 512 + off * 16: pg * stride + bs * 512 + off * 16 + 16] = s
    out = oracle.gather(b, nb, stride, bs, 528, np.arange(len(recs), dtype=np.int32))
    dec = torch.from_numpy(np.stack([np.tile(ch, 16) for _, ch in recs])).view(
        torch.float8_e4m3fn).to(torch.float64)
    sc = torch.exp2(torch.tensor([float(s) - 127 for s, _ in recs], dtype=torch.float64))
    want = (dec * sc[:, None]).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, want)


# --------------------------------------------------------------------------
# The compressed-KV insert variant ([MXFP8 record] 关键源码片段): interleaved
# pairing, compress-ratio gating, the 1e-4 amax floor, NaN sanitising, and
# the rotation-free K insert.
# --------------------------------------------------------------------------

def _compressed_golden_inputs(g):
    inp = g["compressed_variant"]["inputs"]
    x = np.zeros((2, 512), np.float32)
    for d, v in inp["kv_nonzero_token0"]:
        x[0, d] = float(v)
    x[1, :] = 1.0
    kv = _torch_bf16(x)
    table = np.zeros((inp["max_pos"], 64), np.float32)
    table[:, :32] = 1.0
    table[4, 0], table[4, 32], table[4, 1], table[4, 33] = 0.5, 0.75, 0.0, 1.0
    slots = np.array([t["slot"] for t in inp["tokens"]], np.int64)
    pos = np.array([t["position"] for t in inp["tokens"]], np.int64)
    return kv, table, slots, pos


@pytest.mark.parametrize("record", [528, 584])
def test_compressed_variant_worked_token(golden, record):
    cv = golden["compressed_variant"]
    kv, table, slots, pos = _compressed_golden_inputs(golden)
    exp = cv["mxfp8_record" if record == 528 else "legacy_record"]
    bs, nb = cv["inputs"]["block_size"], cv["inputs"]["num_blocks"]
    for fill in (0x00, 0x5A):
        b = np.full(nb * exp["page_stride"], fill, np.uint8)
        oracle.insert(kv, b, nb, exp["page_stride"], bs, record, slots, pos, table, **cv["options"])
        d0, s0 = exp["data_offset"], exp["scale_offset"]
        written = np.zeros(b.size, bool)
        if record == 528:
            codes = np.zeros(512, np.uint8)
            for d, c in exp["codes_nonzero"]:
                codes[d] = c
            assert b[d0:d0 + 512].tolist() == codes.tolist()
            assert b[s0:s0 + 16].tolist() == exp["scales"]
            written[d0:d0 + 512] = written[s0:s0 + 16] = True
        else:
            codes = np.zeros(448, np.uint8)
            for d, c in exp["codes_nonzero"]:
                codes[d] = c
            assert b[d0:d0 + 448].tolist() == codes.tolist()
            tail = np.zeros(64, np.uint16)
            for i, h in exp["rope_bf16"]:
                tail[i] = h
            assert b[d0 + 448:d0 + 576].view(np.uint16).tolist() == tail.tolist()
            assert b[s0:s0 + 8].tolist() == exp["scale_row"]
            written[d0:d0 + 576] = written[s0:s0 + 8] = True
        # the gated-out token (slot 1) and everything else keep the pre-fill
        assert (b[~written] == fill).all()


def test_interleaved_exact_tables():
    n, P = 128, 6
    x = np.clip(RNG.standard_normal((n, 512)), -4, 4).astype(np.float32)
    kv = _torch_bf16(x)
    xf = _bf16_to_f32(kv).astype(np.float64)
    table = np.zeros((P, 64), np.float32)
    table[:, :32] = RNG.integers(-8, 9, (P, 32)) / 8.0
    table[:, 32:] = RNG.integers(-8, 9, (P, 32)) / 8.0
    pos = RNG.integers(0, P, n)
    r = oracle.rope_rows_ex(kv, pos, table, rope="interleaved").astype(np.float64)
    c, s = table[pos, :32].astype(np.float64), table[pos, 32:].astype(np.float64)
    xe, xo = xf[:, 448::2], xf[:, 449::2]
    assert np.array_equal(r[:, 448::2], xe * c - xo * s)
    assert np.array_equal(r[:, 449::2], xo * c + xe * s)
    nz = xf[:, :448] != 0
    assert np.array_equal(r[:, :448][nz], xf[:, :448][nz])  # NoPE pairs: (1, 0)
    assert np.array_equal(oracle.rope_rows_ex(kv, pos, table, rope="none"), _bf16_to_f32(kv))


def test_compress_ratio_gates_tokens_and_picks_the_row():
    """Exactly the tokens with (pos + 1) % R == 0 are written, and each is
    rotated with row pos // R * R: a table whose rows all differ (few-bit
    values, so products are exact) identifies the row from the result."""
    R, n, bs, nb = 4, 96, 8, 16
    case = W.custom_insert(77, n, 528, bs, nb, max_pos=64, drop_frac=0.1)
    table = np.zeros((64, 64), np.float32)
    table[:, :32] = RNG.integers(-8, 9, (64, 32)) / 8.0
    table[:, 32:] = RNG.integers(-8, 9, (64, 32)) / 8.0
    case.cos_sin = table
    kv = _torch_bf16(np.clip(_bf16_to_f32(case.kv_bits), -4, 4))
    b0 = case.initial_backing()
    b = b0.copy()
    oracle.insert(kv, b, nb, case.page_stride, bs, 528, case.slot_mapping, case.positions, table,
                  compress_ratio=R)
    gate = ((case.positions + 1) % R == 0) & (case.slot_mapping >= 0)
    written = _record_mask(case, case.slot_mapping[gate])
    assert (b[~written] == b0[~written]).all()
    # compare each written record with a ratio-1 insert of the same token at row pos // R * R
    for t in np.nonzero(gate)[0]:
        one = b0.copy()
        oracle.insert(kv[t:t + 1], one, nb, case.page_stride, bs, 528, case.slot_mapping[t:t + 1],
                      np.array([case.positions[t] // R * R]), table)
        m = _record_mask(case, case.slot_mapping[t:t + 1])
        assert np.array_equal(b[m], one[m]), t
    assert gate.sum() > 10


def test_amax_floor_closed_form():
    assert oracle.scale_exponent(np.float32(1e-4)) == -22  # ceil(log2(1e-4 / 448)) = -22
    x = np.zeros((1, 512), np.float32)
    x[0, 0] = 5e-5  # below the floor
    kv = _torch_bf16(x)
    v = float(_bf16_to_f32(kv)[0, 0])
    b = np.zeros(2048, np.uint8)
    oracle.insert(kv, b, 1, 2048, 2, 528, np.array([0]), np.array([0]), W.rope_table(1),
                  amax_floor=1e-4)
    assert b[1024:1040].tolist() == [105] * 16
    assert b[0] == oracle.e4m3_encode(v * 2.0 ** 22) and (b[1:512] == 0).all()
    b2 = np.zeros(2048, np.uint8)
    oracle.insert(kv, b2, 1, 2048, 2, 528, np.array([0]), np.array([0]), W.rope_table(1))
    assert b2[1024] == oracle.scale_exponent(np.float32(v)) + 127 and b2[1025] == 127


VARIANTS = [dict(rope="interleaved", compress_ratio=1, amax_floor=1e-4, sanitize_nans=True),
            dict(rope="interleaved", compress_ratio=4, amax_floor=1e-4, sanitize_nans=False),
            dict(rope="neox", compress_ratio=2, amax_floor=0.0, sanitize_nans=True),
            dict(rope="none", compress_ratio=1, amax_floor=1e-4, sanitize_nans=True),
            dict(rope="none", compress_ratio=3, amax_floor=0.0, sanitize_nans=False)]


@pytest.mark.parametrize("opts", VARIANTS, ids=lambda o: "-".join(str(v) for v in o.values()))
@pytest.mark.parametrize("record", [528, 584])
def test_variant_matches_independent_vectorised_reference(opts, record):
    for bs, nb, n in ((3, 4, 9), (32, 3, 90), (64, 3, 150)):
        case = W.custom_insert(3000 + bs + n, n, record, bs, nb, max_pos=64, drop_frac=0.2,
                               scale_rows=True)
        kv = case.kv_bits.copy()
        if opts["sanitize_nans"]:
            kv[RNG.random(kv.shape) < 0.01] = 0x7FC0  # NaN inputs
        got = case.initial_backing()
        oracle.insert(kv, got, nb, case.page_stride, bs, record, case.slot_mapping, case.positions,
                      case.cos_sin, **opts)
        want = _vectorised_insert(case, kv=kv, **opts)
        assert np.array_equal(got, want), (record, bs, opts)


def test_rotation_free_insert_without_positions():
    case = W.custom_insert(91, 50, 528, 16, 4)
    a = case.initial_backing()
    oracle.insert(case.kv_bits, a, 4, case.page_stride, 16, 528, case.slot_mapping, None, None,
                  rope="none")
    b = case.initial_backing()
    oracle.insert(case.kv_bits, b, 4, case.page_stride, 16, 528, case.slot_mapping,
                  np.zeros(50, np.int64), W.rope_table(1), rope="none")
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.insert(case.kv_bits, b, 4, case.page_stride, 16, 528, case.slot_mapping, None, None,
                      rope="interleaved")


@pytest.mark.parametrize("record", [528, 584])
def test_rotation_free_ratio1_does_not_read_positions(record):
    """With no rotation and ratio 1 the positions take no part (no table row,
    no gate), so out-of-range ones skip nothing: the result equals the
    insert without positions. With ratio 2 they are read again, and an
    out-of-range position skips its token."""
    case = W.custom_insert(93 + record, 60, record, 16, 5)
    none = case.initial_backing()
    oracle.insert(case.kv_bits, none, 5, case.page_stride, 16, record, case.slot_mapping, None,
                  None, rope="none")
    bad = np.array([-5, 10 ** 6, 3] * 20, np.int64)
    got = case.initial_backing()
    oracle.insert(case.kv_bits, got, 5, case.page_stride, 16, record, case.slot_mapping, bad,
                  W.rope_table(4), rope="none")
    assert np.array_equal(got, none)
    gated = case.initial_backing()
    oracle.insert(case.kv_bits, gated, 5, case.page_stride, 16, record, case.slot_mapping, bad,
                  W.rope_table(4), rope="none", compress_ratio=2)
    kept = case.slot_mapping[(bad == 3) & (case.slot_mapping >= 0)]
    want = case.initial_backing()
    sel = np.isin(case.slot_mapping, kept)
    oracle.insert(case.kv_bits[sel], want, 5, case.page_stride, 16, record,
                  case.slot_mapping[sel], None, None, rope="none")
    assert np.array_equal(gated, want)


@pytest.mark.parametrize("rope", ["neox", "interleaved", "none"])
@pytest.mark.parametrize("record", [528, 584])
@pytest.mark.parametrize("floor", [0.0, 1e-4])
def test_sanitised_nan_rows_store_zero_records(rope, record, floor):
    """Rows made only of NaNs (both signs, quiet and signalling payloads),
    sanitised: every rotated value is NaN and becomes +0, so each group's
    amax is 0 (or the floor): scale byte 127 (105 with the 1e-4 floor, the
    smallest e with 1e-4 <= 448 * 2^e being -22), every code 0x00, the legacy
    tail bf16 +0 and its pad byte 0. At position 0 (cos 1, sin 0) the +0 row
    rotates to +0 as well and stores the same bytes."""
    bs, n = 4, 4
    stride = W.page_stride_for(record, bs)
    kv = np.array([[[0x7FC0, 0xFFC0, 0x7F81, 0xFFFF][(d + t) % 4] for d in range(512)]
                   for t in range(n)], np.uint16)
    slots, pos = np.arange(n), np.zeros(n, np.int64)
    table = W.rope_table(1)
    got = np.full(stride, 0xA5, np.uint8)
    oracle.insert(kv, got, 1, stride, bs, record, slots, pos, table, rope=rope,
                  amax_floor=floor, sanitize_nans=True)
    sbyte = 105 if floor else 127
    if record == 528:
        assert (got[:n * 512] == 0).all()
        assert (got[bs * 512:bs * 512 + n * 16] == sbyte).all()
    else:
        assert (got[:n * 576] == 0).all()  # 448 codes and the 64 bf16 of each row
        rows = got[bs * 576:bs * 576 + n * 8].reshape(n, 8)
        assert (rows[:, :7] == sbyte).all() and (rows[:, 7] == 0).all()
    zero = np.full(stride, 0xA5, np.uint8)
    oracle.insert(np.zeros_like(kv), zero, 1, stride, bs, record, slots, pos, table, rope=rope,
                  amax_floor=floor, sanitize_nans=True)
    assert np.array_equal(got, zero)
    assert (got[bs * (512 if record == 528 else 576) + n * (16 if record == 528 else 8):]
            == 0xA5).all()
