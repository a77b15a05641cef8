"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Insert: every byte of the cache backing (pre-filled with seeded random bytes,
so untouched slots and page padding are checked too) must equal the oracle's.
Gather: every bf16 output bit must equal the oracle's dequantisation of the
oracle's own cache. Sizes span several launch blocks and ragged tails, and
the full workloads run at their real sizes in the same launch configuration
the benchmark times.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_rope_amd import binding as B
from quantized_paged_kv_rope_amd import workloads as W
from tests import parity_util as P

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(777)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    B.load_library()
    yield
    torch.cuda.synchronize()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return W.to_bf16_bits(x)


def check_insert(case: W.InsertCase) -> P.DeviceCase:
    d = P.DeviceCase(case)
    want = case.initial_backing()
    kv0 = case.kv_bits.copy()
    P.oracle_insert(case, want)
    d.insert()
    got = d.backing_host()
    assert np.array_equal(got, want), P.first_diff(got, want)
    assert np.array_equal(P.host_bits(d.kv), kv0), "kv was modified"
    return d


# ---------------------------------------------------------------------------
# Hand-worked token (golden values, independent of the oracle).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("record", [528, 584])
def test_worked_token(golden, record):
    inp = golden["inputs"]
    x = np.zeros((1, 512), np.float32)
    for dim, v in inp["kv_nonzero"]:
        x[0, dim] = float(v)
    table = np.zeros((inp["max_pos"], 64), np.float32)
    table[:, :32] = 1.0
    table[3, 0], table[3, 32], table[3, 1], table[3, 33] = 0.5, 0.75, 0.0, 1.0
    exp = golden["mxfp8_record" if record == 528 else "legacy_record"]
    bs, nb = inp["block_size"], inp["num_blocks"]
    case = W.InsertCase("worked", record, bs, nb, exp["page_stride"], _bf16_bits(x),
                        np.array([inp["slot"]], np.int64), np.array([inp["position"]], np.int64),
                        table, backing_seed=5)
    d = P.DeviceCase(case)
    d.insert()
    got = d.backing_host()
    d0, s0 = exp["data_offset"], exp["scale_offset"]
    if record == 528:
        codes = np.zeros(512, np.uint8)
        for dim, c in exp["codes_nonzero"]:
            codes[dim] = c
        assert got[d0:d0 + 512].tolist() == codes.tolist()
        assert got[s0:s0 + 16].tolist() == exp["scales"]
        out = d.gather(np.array([inp["slot"], -1], np.int32))
        for dim, h in exp["gather_bf16"]:
            assert out[0, dim] == h, dim
        assert (out[1] == 0).all()
    else:
        codes = np.zeros(448, np.uint8)
        for dim, c in exp["codes_nonzero"]:
            codes[dim] = c
        assert got[d0:d0 + 448].tolist() == codes.tolist()
        want_tail = np.zeros(64, np.uint16)
        for i, h in exp["rope_bf16"]:
            want_tail[i] = h
        assert got[d0 + 448:d0 + 576].view(np.uint16).tolist() == want_tail.tolist()
        assert got[s0:s0 + 8].tolist() == exp["scale_row"]
    want = case.initial_backing()
    P.oracle_insert(case, want)
    assert np.array_equal(got, want), P.first_diff(got, want)


# ---------------------------------------------------------------------------
# Edge sizes, block sizes, padded strides, three rounds on one backing
# (new kv/positions/slots each round; the third round all -1).
# ---------------------------------------------------------------------------

EDGE = [(528, n, 64, None) for n in (1, 17, 1023, 1024, 4099)] + \
       [(584, n, 64, None) for n in (1, 17, 1023, 4099)] + \
       [(528, 300, bs, None) for bs in (1, 3, 16, 32, 128)] + \
       [(584, 300, bs, None) for bs in (1, 3, 16, 32, 128)] + \
       [(528, 777, 64, 33792 + 1024), (584, 777, 64, 37440 + 576 * 2), (584, 513, 32, 19008)]


@pytest.mark.parametrize("record,n,bs,stride", EDGE)
def test_insert_rounds_whole_backing(record, n, bs, stride):
    nb = (n * 5 // 4) // bs + 2
    case = W.custom_insert(31 * n + bs + record, n, record, bs, nb, page_stride=stride,
                           scale_rows=True)
    d = P.DeviceCase(case)
    want = case.initial_backing()
    written = np.zeros(nb * bs, bool)
    for rnd in range(3):
        if rnd > 0:
            nxt = W.custom_insert(31 * n + bs + record + 1000 * rnd, n, record, bs, nb,
                                  page_stride=stride, scale_rows=True)
            slots = nxt.slot_mapping.copy()
            if rnd == 2:
                slots[:] = -1
            kv, pos = nxt.kv_bits, nxt.positions
        else:
            kv, slots, pos = case.kv_bits, case.slot_mapping, case.positions
        kv_dev = P.dev_bf16(kv)
        d.insert(kv=kv_dev, slots=P.dev(slots), positions=P.dev(pos))
        P.oracle_insert(case, want, kv_bits=kv, slots=slots, positions=pos)
        written[slots[slots >= 0]] = True
        got = d.backing_host()
        assert np.array_equal(got, want), f"round {rnd}: " + P.first_diff(got, want)
        assert np.array_equal(P.host_bits(kv_dev), kv), "kv was modified"
    # gather every written slot plus invalid entries, against the oracle's cache
    idx = np.where(written, np.arange(nb * bs), -1).astype(np.int32)
    idx = np.concatenate([idx, np.array([-1, -7], np.int32)])
    got = d.gather(idx)
    want_g = P.oracle_gather(case, want, idx)
    assert np.array_equal(got, want_g), P.first_diff(got, want_g)


def test_zero_tokens_and_all_skipped():
    case = W.custom_insert(5, 64, 528, 64, 2)
    d = P.DeviceCase(case)
    empty = torch.empty(0, dtype=torch.int64, device="cuda")
    B.kvrec_insert(d.kv[:0], d.k_cache, empty, empty, d.cos_sin, 64)
    out = B.kvrec_gather(d.k_cache, torch.empty(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 512)
    d.insert(slots=torch.full((64,), -1, dtype=torch.int64, device="cuda"))
    assert np.array_equal(d.backing_host(), case.initial_backing())


def test_out_of_range_guard():
    case = W.custom_insert(6, 32, 528, 16, 2)
    case.slot_mapping[:] = np.arange(32)
    case.slot_mapping[3] = 32                       # == num_blocks * block_size
    case.slot_mapping[4] = 2 ** 40
    case.positions[5] = case.cos_sin.shape[0]       # == max_pos
    case.positions[6] = -2
    d = check_insert(case)
    idx = np.array([0, 32, 2 ** 31 - 1, -1, -2 ** 31], np.int32)
    got = d.gather(idx)
    assert (got[1:] == 0).all()


# ---------------------------------------------------------------------------
# Hardware conversions, checked through the real kernels.
# ---------------------------------------------------------------------------

def _fp32_class_sweep() -> np.ndarray:
    """Every fp32 exponent field up to 448, every top-8 mantissa pattern, and
    low 15 bits in {0, 1, 0x3FFF, 0x4000, 0x7FFF}: all rounding classes of
    fp32 -> e4m3 (round bit, sticky bits, carries into the exponent,
    subnormal e4m3 outputs), both signs; plus random values."""
    expo = np.arange(0, 136, dtype=np.uint32)
    top = np.arange(256, dtype=np.uint32) << 15
    low = np.array([0, 1, 0x3FFF, 0x4000, 0x7FFF], np.uint32)
    bits = (expo[:, None, None] << 23 | top[None, :, None] | low[None, None, :]).ravel()
    y = bits.view(np.float32)
    y = y[(y <= 448) & (y > 0)]
    rnd = RNG.uniform(-448, 448, 400_000).astype(np.float32)
    tiny = (np.exp2(RNG.uniform(-150, -5, 100_000)) * RNG.choice([-1, 1], 100_000)).astype(np.float32)
    return np.concatenate([y, -y, rnd, tiny, np.float32([448.0, -448.0, 2.0 ** -10, 2.0 ** -9])])


def _tail_case(values: np.ndarray, anchor_exp: int, record: int) -> W.InsertCase:
    """Tokens whose rotated tail is exactly the given fp32 values: x1 = 1 and
    x2 = 0 make r[448+i] = cos_i and r[480+i] = sin_i, so the table carries
    the values; column 0 of each half is the group anchor 448 * 2^e so that
    the group exponent is e and every other value v*2^e is encoded as v."""
    per = 62
    n = (values.size + per - 1) // per
    v = np.zeros(n * per, np.float32)
    v[:values.size] = values
    v = v.reshape(n, 2, 31)
    scale = np.float32(2.0 ** anchor_exp)
    table = np.zeros((n, 64), np.float32)
    table[:, 0] = table[:, 32] = np.float32(448.0) * scale
    table[:, 1:32] = v[:, 0] * scale
    table[:, 33:64] = v[:, 1] * scale
    table[table == 0] = 0.0  # no -0 in the table
    x = np.zeros((n, 512), np.float32)
    x[:, 448:480] = 1.0
    x[:, 0] = 1.0
    bs = 64
    nb = (n + bs - 1) // bs
    return W.InsertCase("tail_sweep", record, bs, nb, W.page_stride_for(record, bs), _bf16_bits(x),
                        np.arange(n, dtype=np.int64), np.arange(n, dtype=np.int64), table,
                        backing_seed=11)


@pytest.mark.parametrize("anchor_exp", [0, -8, 7, -120])
def test_e4m3_conversion_sweep_mxfp8(anchor_exp):
    y = _fp32_class_sweep()
    if anchor_exp != 0:
        y = y[::7]
    case = _tail_case(y, anchor_exp, 528)
    d = check_insert(case)
    # round trip through the gather as well
    idx = np.arange(case.num_tokens, dtype=np.int32)
    want = P.oracle_gather(case, P.oracle_insert(case, case.initial_backing()), idx)
    got = d.gather(idx)
    assert np.array_equal(got, want), P.first_diff(got, want)


def test_bf16_tail_rounding_legacy():
    """Legacy record: the rotated tail is stored as bf16 (nearest even); the
    fp32 sweep exercises every rounding class of that conversion."""
    y = _fp32_class_sweep()[::3]
    check_insert(_tail_case(y, 0, 584))


@pytest.mark.parametrize("record", [528, 584])
def test_every_bf16_input_at_many_scales(record):
    """Every finite bf16 value whose magnitude does not exceed the group's
    anchor 448 * 2^E, in the NoPE groups, for a range of E (including the
    clamp at -127 and subnormal inputs)."""
    allv = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allv = allv[np.isfinite(allv)]
    gsz = 32 if record == 528 else 64
    groups = 14 if record == 528 else 7
    rows = []
    for E in (-127, -126, -100, -20, -8, -1, 0, 1, 8, 100, 119):
        anchor = np.float32(448.0 * 2.0 ** E)
        vals = allv[np.abs(allv) <= anchor]
        per = gsz - 1
        k = (vals.size + per - 1) // per
        g = np.zeros(k * per, np.float32)
        g[:vals.size] = vals
        g = np.concatenate([np.full((k, 1), anchor, np.float32), g.reshape(k, per)], axis=1)
        rows.append(g)
    grp = np.concatenate(rows)
    n = (grp.shape[0] + groups - 1) // groups
    pad = np.zeros((n * groups - grp.shape[0], gsz), np.float32)
    x = np.zeros((n, 512), np.float32)
    x[:, :groups * gsz] = np.concatenate([grp, pad]).reshape(n, groups * gsz)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: values are bf16
    bs = 64
    nb = (n + bs - 1) // bs
    case = W.InsertCase("bf16_sweep", record, bs, nb, W.page_stride_for(record, bs), bits,
                        np.arange(n, dtype=np.int64), np.zeros(n, np.int64), W.rope_table(4),
                        backing_seed=12)
    d = check_insert(case)
    idx = np.arange(n, dtype=np.int32)
    want = P.oracle_gather(case, P.oracle_insert(case, case.initial_backing()), idx)
    got = d.gather(idx)
    assert np.array_equal(got, want), P.first_diff(got, want)


@pytest.mark.parametrize("record", [528, 584])
def test_gather_every_code_and_scale(record):
    """All 254 non-NaN e4m3 codes under every scale byte 0..254 (64770 pairs),
    written straight into the cache bytes, gathered on the GPU."""
    bs = 16
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = np.concatenate([codes, np.zeros(2, np.uint8)])  # 256 = whole groups
    fp8 = 512 if record == 528 else 448
    gsz = 32 if record == 528 else 64
    gpr = fp8 // gsz                                        # groups per record
    grp_codes = np.tile(codes.reshape(-1, gsz), (255, 1))   # [255 * 256/gsz, gsz]
    grp_scale = np.repeat(np.arange(255, dtype=np.uint8), 256 // gsz)
    n = (grp_codes.shape[0] + gpr - 1) // gpr
    padg = n * gpr - grp_codes.shape[0]
    grp_codes = np.concatenate([grp_codes, np.zeros((padg, gsz), np.uint8)])
    grp_scale = np.concatenate([grp_scale, np.full(padg, 127, np.uint8)])
    nb = (n + bs - 1) // bs
    stride = W.page_stride_for(record, bs)
    b = RNG.integers(0, 256, nb * stride, dtype=np.uint8)
    for j in range(n):
        pg, off = divmod(j, bs)
        base = pg * stride
        data = grp_codes[j * gpr:(j + 1) * gpr].reshape(-1)
        sc = grp_scale[j * gpr:(j + 1) * gpr]
        if record == 528:
            b[base + off * 512: base + off * 512 + 512] = data
            b[base + bs * 512 + off * 16: base + bs * 512 + off * 16 + 16] = sc
        else:
            b[base + off * 576: base + off * 576 + 448] = data
            b[base + bs * 576 + off * 8: base + bs * 576 + off * 8 + 7] = sc
    like = W.InsertCase("codes", record, bs, nb, stride, np.zeros((0, 512), np.uint16),
                        np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros((1, 64), np.float32),
                        backing_seed=None)
    d = P.DeviceCase(like, backing=b)
    idx = np.concatenate([np.arange(n, dtype=np.int32), [-1]]).astype(np.int32)
    got = d.gather(idx)
    want = P.oracle_gather(like, b, idx)
    assert np.array_equal(got, want), P.first_diff(got, want)
    assert (got[-1] == 0).all()


# ---------------------------------------------------------------------------
# The workloads at their full sizes.
# ---------------------------------------------------------------------------

def test_config_mixed_1024():
    case = W.mixed_1024()
    d = check_insert(case)
    want = P.oracle_insert(case, case.initial_backing())
    got = d.gather(case.gather_indices)
    want_g = P.oracle_gather(case, want, case.gather_indices)
    assert np.array_equal(got, want_g), P.first_diff(got, want_g)
    assert (got[case.gather_indices < 0] == 0).all()


def test_config_decode_16384():
    check_insert(W.decode_16384())


def test_config_legacy_65536():
    """Every byte of the backing, then the gather of all 65536 slots (the
    skipped ones as -1, giving zero rows)."""
    case = W.legacy_65536()
    d = check_insert(case)
    idx = case.gather_indices
    want = P.oracle_gather(case, P.oracle_insert(case, case.initial_backing()), idx)
    got = d.gather(idx)
    assert np.array_equal(got, want), P.first_diff(got, want)
    assert (got[idx < 0] == 0).all()


def test_config_prefill_262144_with_round_trip():
    case = W.prefill_262144()
    d = check_insert(case)
    want = P.oracle_insert(case, case.initial_backing())
    got = d.gather(case.gather_indices)
    want_g = P.oracle_gather(case, want, case.gather_indices)
    assert np.array_equal(got, want_g), P.first_diff(got, want_g)


def test_config_topk_gather():
    """The 32768-page cache (2,097,152 slots, 1.1 GB) is filled by the GPU
    insert in 262144-token chunks, and by the oracle from the same seeded
    chunks into a host backing: every byte of the two backings must agree.
    Then all 64 x 2048 gathered rows (the -1 entries as zero rows) must equal
    the oracle's gather of its own cache."""
    tk = W.topk_gather()
    idx = tk.indices
    backing, k_cache = B.alloc_cache(tk.num_blocks, tk.block_size, tk.record, tk.page_stride)
    want = np.zeros(tk.num_blocks * tk.page_stride, np.uint8)
    table = tk.cos_sin()
    cos_sin = P.dev(table)
    fill = W.InsertCase("topk_fill", tk.record, tk.block_size, tk.num_blocks, tk.page_stride,
                        np.zeros((0, 512), np.uint16), np.zeros(0, np.int64),
                        np.zeros(0, np.int64), table, backing_seed=None)
    for k in range(tk.num_chunks):
        kv_bits, slots, pos = tk.fill_chunk(k)
        B.kvrec_insert(P.dev_bf16(kv_bits), k_cache, P.dev(slots), P.dev(pos), cos_sin,
                       tk.block_size)
        P.oracle_insert(fill, want, kv_bits=kv_bits, slots=slots, positions=pos)
    out = B.kvrec_gather(k_cache, P.dev(idx))
    got = backing.cpu().numpy()
    assert np.array_equal(got, want), P.first_diff(got, want)
    del got
    got_rows = P.host_bits(out).reshape(idx.shape + (512,))
    want_rows = P.oracle_gather(fill, want, idx)
    assert np.array_equal(got_rows, want_rows), P.first_diff(got_rows, want_rows)
    assert (got_rows[idx < 0] == 0).all() and (idx < 0).sum() == 64 * 61
    del backing, k_cache, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("record", [528, 584])
def test_largest_page(record):
    """One page just under 2^31 bytes (the ABI's limit: in-page offsets are
    32-bit on the device), written at its last 64 slots and gathered back:
    the rows and scale bytes near the end of the page equal the oracle's."""
    limit = 2 ** 31
    bs = limit // record - 1
    stride = W.page_stride_for(record, bs)
    assert stride < limit and bs * record < limit
    n = 64
    rng = np.random.default_rng(2 ** 20 + record)
    x = rng.standard_normal((n, 512), dtype=np.float32) * rng.uniform(0.1, 10, (n, 1)).astype(np.float32)
    slots = (bs - n + rng.permutation(n)).astype(np.int64)
    slots[5] = -1
    case = W.InsertCase("largest_page", record, bs, 1, stride, W.to_bf16_bits(x), slots,
                        rng.integers(0, 4096, n).astype(np.int64), W.rope_table(4096), None)
    backing = torch.zeros(stride, dtype=torch.uint8, device="cuda")
    _, kc = B.alloc_cache(1, bs, record, stride, backing=backing)
    B.kvrec_insert(P.dev_bf16(case.kv_bits), kc, P.dev(slots), P.dev(case.positions),
                   P.dev(case.cos_sin), bs)
    idx = np.where(slots >= 0, slots, -1).astype(np.int32)
    out = P.host_bits(B.kvrec_gather(kc, P.dev(idx)))
    torch.cuda.synchronize()
    want = np.zeros(stride, np.uint8)
    oracle.insert(case.kv_bits, want, 1, stride, bs, record, slots, case.positions, case.cos_sin)
    row_bytes, scale_bytes = (512, 16) if record == 528 else (576, 8)
    lo_data, lo_scale = (bs - n) * row_bytes, bs * row_bytes + (bs - n) * scale_bytes
    got_data = backing[lo_data: bs * row_bytes].cpu().numpy()
    got_scale = backing[lo_scale: bs * row_bytes + bs * scale_bytes].cpu().numpy()
    assert np.array_equal(got_data, want[lo_data: bs * row_bytes])
    assert np.array_equal(got_scale, want[lo_scale: bs * row_bytes + bs * scale_bytes])
    want_out = oracle.gather(want, 1, stride, bs, record, idx)
    assert np.array_equal(out, want_out), P.first_diff(out, want_out)
    del backing, kc
    torch.cuda.empty_cache()


def test_concurrent_calls_on_two_streams():
    """The library keeps no state: two host threads, each with its own
    stream (default priority) and cache, insert and gather at the same time
    (ctypes releases the interpreter lock around each call); both caches
    and both gathers equal the oracle's."""
    import threading

    cases = [W.custom_insert(3100 + i, 3000, rec, 64, 60, max_pos=4096)
             for i, rec in enumerate((528, 584))]
    devs = [P.DeviceCase(c) for c in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [None, None]
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(20):
                    devs[i].insert()
                    outs[i] = B.kvrec_gather(devs[i].k_cache, P.dev(cases[i].gather_indices))
            streams[i].synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for c, d, o in zip(cases, devs, outs):
        want = P.oracle_insert(c, c.initial_backing())
        got = d.backing_host()
        assert np.array_equal(got, want), (c.record, P.first_diff(got, want))
        want_g = P.oracle_gather(c, want, c.gather_indices)
        assert np.array_equal(P.host_bits(o), want_g), c.record
