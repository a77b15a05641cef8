"""GPU: calls larger than one kernel launch takes.

A call over more than 2^21 waves of work runs as several launches, one per
consecutive slice of its rows. Each test makes such a call and checks it
(a) against the same work issued as smaller calls that each fit one launch
(every byte of the backing, every output element), and (b) against the
oracle on the rows around the first launch boundary (or on every row where
the oracle is fast enough). Inputs are drawn on the GPU from seeded
generators; only the rows the oracle recomputes come back to the host.
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

LAUNCH_WAVES = 2 ** 21  # waves per launch
INSERT_TOKENS_PER_WAVE = 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _records_equal_oracle(backing: torch.Tensor, record: int, bs: int, stride: int,
                          kv: torch.Tensor, slots: torch.Tensor, positions: torch.Tensor,
                          table: np.ndarray, rows: slice, **opts) -> int:
    """Inserts kv[rows] with the oracle into a zeroed copy of the cache and
    compares every record those tokens own. Returns the records compared."""
    sl = slots[rows].cpu().numpy()
    ps = positions[rows].cpu().numpy()
    kvb = P.host_bits(kv[rows].contiguous())
    nb = backing.numel() // stride
    want = np.zeros(backing.numel(), np.uint8)
    oracle.insert(kvb, want, nb, stride, bs, record, sl, ps, table, **opts)
    got = backing.cpu().numpy()
    row_b, scale_b = (512, 16) if record == 528 else (576, 8)
    checked = 0
    for s in sl[sl >= 0].tolist():
        page, off = divmod(s, bs)
        d0 = page * stride + off * row_b
        s0 = page * stride + bs * row_b + off * scale_b
        assert np.array_equal(got[d0:d0 + row_b], want[d0:d0 + row_b]), f"data row of slot {s}"
        assert np.array_equal(got[s0:s0 + scale_b], want[s0:s0 + scale_b]), f"scales of slot {s}"
        checked += 1
    return checked


@pytest.mark.parametrize("record", [528, 584])
def test_insert_over_one_launch(record):
    per_launch = LAUNCH_WAVES * INSERT_TOKENS_PER_WAVE
    n, bs = per_launch + 37, 64
    stride = W.page_stride_for(record, bs)
    nb = (n + n // 50) // bs + 1
    g = _gen(71 + record)
    kv = torch.randn((n, 512), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.randperm(nb * bs, generator=g, device="cuda")[:n]
    slots[torch.rand(n, generator=g, device="cuda") < 0.01] = -1
    positions = torch.randint(0, 4096, (n,), generator=g, device="cuda")
    table = W.rope_table(4096)
    cs = P.dev(table)
    one, k_one = B.alloc_cache(nb, bs, record, stride)
    two, k_two = B.alloc_cache(nb, bs, record, stride)
    one.zero_()
    two.zero_()
    B.kvrec_insert(kv, k_one, slots, positions, cs, bs)
    m = per_launch // 2 + 11
    B.kvrec_insert(kv[:m], k_two, slots[:m], positions[:m], cs, bs)
    B.kvrec_insert(kv[m:], k_two, slots[m:], positions[m:], cs, bs)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    edge = slice(per_launch - 40, per_launch + 37)
    assert _records_equal_oracle(one, record, bs, stride, kv, slots, positions, table, edge) > 60


def test_gated_insert_over_one_launch():
    """Compressed-KV insert with ratio 2: groups of 4 tokens per wave, so a
    launch takes 2^23 tokens."""
    ratio, group = 2, 4
    n, bs, record = LAUNCH_WAVES * group + 21, 64, 528
    stride = W.page_stride_for(record, bs)
    nb = n // bs + 1
    g = _gen(73)
    kv = torch.randn((n, 512), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.arange(n, device="cuda", dtype=torch.int64)
    positions = torch.arange(n, device="cuda", dtype=torch.int64) % 4096
    table = W.rope_table(4096)
    cs = P.dev(table)
    opts = dict(rope="interleaved", compress_ratio=ratio, amax_floor=1e-4, sanitize_nans=True)
    one, k_one = B.alloc_cache(nb, bs, record, stride)
    two, k_two = B.alloc_cache(nb, bs, record, stride)
    one.zero_()
    two.zero_()
    B.kvrec_insert(kv, k_one, slots, positions, cs, bs, **opts)
    m = LAUNCH_WAVES * group // 2 + 6
    B.kvrec_insert(kv[:m], k_two, slots[:m], positions[:m], cs, bs, **opts)
    B.kvrec_insert(kv[m:], k_two, slots[m:], positions[m:], cs, bs, **opts)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    del two, k_two
    edge = slice(LAUNCH_WAVES * group - 40, LAUNCH_WAVES * group + 21)
    kept = _records_equal_oracle(one, record, bs, stride, kv, slots, positions, table, edge,
                                 **opts)
    assert kept == 61  # every slot of the range is compared; gated ones hold zeros


def test_gather_over_one_launch():
    """2^22 + 3 rows (two rows per wave) from a 256-slot cache: each output
    row is the oracle's row for its index (zeros for -1)."""
    case = W.custom_insert(75, 256, 528, 64, 4)
    case.slot_mapping[:] = np.arange(256)
    d = P.DeviceCase(case)
    d.insert()
    want_backing = case.initial_backing()
    P.oracle_insert(case, want_backing)
    assert np.array_equal(d.backing_host(), want_backing)
    rows = oracle.gather(want_backing, case.num_blocks, case.page_stride, case.block_size,
                         case.record, np.arange(-1, 256, dtype=np.int32))
    table = P.dev(rows.view(np.int16)).view(torch.bfloat16)
    n = 2 * LAUNCH_WAVES + 3
    idx = torch.randint(-1, 256, (n,), generator=_gen(76), device="cuda", dtype=torch.int32)
    out = B.kvrec_gather(d.k_cache, idx)
    want = table[(idx + 1).long()]
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def test_expand_over_one_launch():
    rows, k, ratio, sbk = LAUNCH_WAVES + 5, 8, 2, 8
    rng = np.random.default_rng(77)
    cand = rng.integers(-1, 64, (rows, k)).astype(np.int32)
    ks = rng.integers(0, 100, rows).astype(np.int32)
    ke = (ks + rng.integers(0, 1000, rows)).astype(np.int32)
    sparse, end = B.kvrec_expand_candidates(P.dev(cand), P.dev(ks), P.dev(ke), ratio, sbk)
    want_sparse, want_end = oracle.expand_candidates(cand, ks, ke, ratio, sbk)
    assert np.array_equal(sparse.cpu().numpy(), want_sparse)
    assert np.array_equal(end.cpu().numpy(), want_end)


@pytest.mark.parametrize("heads", [1, 3])
def test_attention_write_over_one_launch(heads):
    """ceil(heads / 2) + 1 waves per token: a launch takes 2^21 / that many
    tokens. The cache records of the tokens at the first boundary are
    checked against the oracle as well."""
    per_launch = LAUNCH_WAVES // ((heads + 1) // 2 + 1)
    n, bs, record = per_launch + 9, 64, 528
    stride = W.page_stride_for(record, bs)
    nb = n // bs + 1
    g = _gen(78 + heads)
    q = torch.randn((n, heads, 512), generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn((n, 512), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.arange(n, device="cuda", dtype=torch.int64)
    positions = torch.randint(0, 4096, (n,), generator=g, device="cuda")
    table = W.rope_table(4096)
    cs = P.dev(table)
    one, k_one = B.alloc_cache(nb, bs, record, stride)
    two, k_two = B.alloc_cache(nb, bs, record, stride)
    one.zero_()
    two.zero_()
    q1, q2 = torch.empty_like(q), torch.empty_like(q)
    B.kvrec_qnorm_rope_insert(q, kv, k_one, slots, positions, cs, bs, eps=1e-6, q_out=q1)
    m = per_launch // 2 + 3
    B.kvrec_qnorm_rope_insert(q[:m], kv[:m], k_two, slots[:m], positions[:m], cs, bs,
                              eps=1e-6, q_out=q2[:m])
    B.kvrec_qnorm_rope_insert(q[m:], kv[m:], k_two, slots[m:], positions[m:], cs, bs,
                              eps=1e-6, q_out=q2[m:])
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))
    edge = slice(per_launch - 20, per_launch + 9)
    assert _records_equal_oracle(one, record, bs, stride, kv, slots, positions, table, edge) == 29
