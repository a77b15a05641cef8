"""GPU parity over seeded random combinations of the insert's and gather's
parameters, so that interactions the per-feature tests do not pair up are
covered too: record (528, 584, and the non-packed 1024 / 512), block size
(1 .. 257), padded page stride, token count (0 .. 3000), skipped slots,
out-of-range slots and positions (which the kernels skip, like the oracle),
the compressed-KV options (rotation, ratio gate, amax floor, NaN sanitising)
and the fp8 cache's scale. Every byte of the pre-filled cache backing and
every gathered row is compared with the oracle.

The case counts default to 48 and 24; KVREC_RANDOM_CASES and
KVREC_RANDOM_QKV_CASES raise them for a longer campaign.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

from quantized_paged_kv_rope_amd import workloads as W
from tests import parity_util as P

pytestmark = pytest.mark.gpu

CASES = int(os.environ.get("KVREC_RANDOM_CASES", "48"))
ALIGN = {W.RECORD_MXFP8: 512, W.RECORD_LEGACY: 576, W.RECORD_BF16: 16, W.RECORD_FP8: 16}


def _case(seed: int):
    rng = np.random.default_rng(71000 + seed)
    record = int(rng.choice([W.RECORD_MXFP8, W.RECORD_LEGACY, W.RECORD_BF16, W.RECORD_FP8]))
    bs = int(rng.choice([1, 2, 3, 7, 16, 31, 64, 100, 128, 257]))
    nb = int(rng.integers(1, 40))
    n = int(rng.integers(0, min(nb * bs, 3000) + 1))
    stride = W.page_stride_for(record, bs) + int(rng.integers(0, 3)) * ALIGN[record]
    max_pos = int(rng.integers(1, 5000))
    case = W.custom_insert(seed, n, record, bs, nb, max_pos=max_pos,
                           drop_frac=float(rng.uniform(0.0, 0.3)), page_stride=stride,
                           scale_rows=bool(rng.integers(2)))
    if n and rng.integers(2):
        # a few slots past the cache and positions outside the table: skipped
        bad = rng.random(n) < 0.02
        case.slot_mapping[bad] = nb * bs + rng.integers(0, 50, int(bad.sum()))
        bad = rng.random(n) < 0.02
        case.positions[bad] = rng.choice([-1, max_pos, max_pos + 7], int(bad.sum()))
    return rng, case


@pytest.mark.parametrize("seed", range(CASES))
def test_random_configuration(seed):
    rng, case = _case(seed)
    packed = case.record in (W.RECORD_MXFP8, W.RECORD_LEGACY)
    opts = {}
    if packed and rng.integers(2):
        opts = dict(rope=str(rng.choice(["neox", "interleaved", "none"])),
                    compress_ratio=int(rng.choice([1, 2, 4, 7])),
                    amax_floor=float(rng.choice([0.0, 1e-4])),
                    sanitize_nans=bool(rng.integers(2)))
        if opts["sanitize_nans"] and case.num_tokens:
            kv = case.kv_bits.copy()
            kv[rng.random(kv.shape) < 0.003] = 0x7FC0
            case.kv_bits = kv
    d = P.DeviceCase(case)
    if packed:
        d.insert(**opts)
        want = P.oracle_insert(case, case.initial_backing(), **opts)
    else:
        scale = None
        if case.record == W.RECORD_FP8:
            scale = float(rng.choice([1.0, 0.0123, 3.7, 2.0 ** -20]))
        d.insert_full(scale)
        want = P.oracle_insert_full(case, case.initial_backing(), 1.0 if scale is None else scale)
    got = d.backing_host()
    assert np.array_equal(got, want), (case.name, opts, P.first_diff(got, want))
    if packed and case.num_tokens:
        # The gather reads slots this insert wrote (a precondition: other
        # slots hold the random pre-fill), negative indices and indices past
        # the cache (both give +0 rows).
        total = case.num_blocks * case.block_size
        sl, ps = case.slot_mapping, case.positions
        ratio = opts.get("compress_ratio", 1)
        written = sl[(sl >= 0) & (sl < total) & (ps >= 0) & (ps < case.cos_sin.shape[0])
                     & ((ps + 1) % ratio == 0)]
        m = int(rng.integers(1, 2000))
        pool = np.concatenate([written, [-1, -3, total, total + 4]]).astype(np.int32)
        idx = rng.choice(pool, m)
        out = d.gather(idx)
        want_g = P.oracle_gather(case, want, idx)
        assert np.array_equal(out, want_g), (case.name, P.first_diff(out, want_g))


QKV_CASES = int(os.environ.get("KVREC_RANDOM_QKV_CASES", "24"))


@pytest.mark.parametrize("seed", range(QKV_CASES))
def test_random_attention_write(seed):
    """The attention write over random head counts, eps, norm on or off,
    both packed records, odd block sizes, skipped and out-of-range slots and
    positions, and in-place or separate q output: cache bytes exact, q rows
    within the fp32 error bound (tests/test_gpu_qside.py derives it), rows
    of out-of-range positions left as they were."""
    import oracle
    from tests import test_gpu_qside as Q

    rng = np.random.default_rng(72000 + seed)
    record = int(rng.choice([W.RECORD_MXFP8, W.RECORD_LEGACY]))
    bs = int(rng.choice([1, 5, 16, 64, 130]))
    n = int(rng.integers(1, 400))
    heads = int(rng.choice([1, 2, 3, 7, 16, 33, 128]))
    nb = n // bs + 2
    max_pos = int(rng.integers(2, 3000))
    case = W.custom_insert(5000 + seed, n, record, bs, nb, max_pos=max_pos,
                           drop_frac=float(rng.uniform(0.0, 0.3)), scale_rows=True)
    bad = rng.random(n) < 0.05
    case.positions[bad] = rng.choice([-2, max_pos, max_pos + 100], int(bad.sum()))
    x = rng.standard_normal((n, heads, 512)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-3, 3, (n, heads, 1))).astype(np.float32)
    x[rng.random((n, heads)) < 0.02] = 0.0  # all-zero heads
    eps = float(rng.choice([1e-6, 1e-5, 1e-2]))
    norm = bool(rng.integers(2))
    in_place = bool(rng.integers(2))
    aw = W.AttentionWrite(f"rand_qkv_{seed}", W.to_bf16_bits(x), eps, case)
    sentinel = np.full_like(aw.q_bits, 0x1234)
    got_q, got_cache = Q._run(aw, apply_norm=norm, in_place=in_place, q_out_init=sentinel)
    want_cache = P.oracle_insert(case, case.initial_backing())
    assert np.array_equal(got_cache, want_cache), P.first_diff(got_cache, want_cache)
    init = aw.q_bits.copy() if in_place else sentinel.copy()
    want_q = oracle.qnorm_rope(aw.q_bits, case.positions, case.cos_sin, eps, norm, out=init)
    ok = (case.positions >= 0) & (case.positions < max_pos)
    assert np.array_equal(got_q[~ok], want_q[~ok])
    if ok.any():
        Q._check_q(got_q[ok], want_q[ok], Q._magnitude(aw.q_bits[ok], case.positions[ok],
                                                          case.cos_sin, eps, norm))
