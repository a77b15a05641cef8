"""GPU parity of the compressed-KV insert variant (kvrec_insert_ex).

The options follow the compressed-KV insert printed in [MXFP8 record]
关键源码片段 (interleaved neighbour pairs, compress-ratio gating, the 1e-4
amax floor, NaN sanitising) and the rotation-free K insert. Every byte of the
pre-filled cache backing is compared with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from quantized_paged_kv_rope_amd import binding as B
from quantized_paged_kv_rope_amd import workloads as W
from tests import parity_util as P

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(4242)

VARIANTS = [dict(rope="interleaved", compress_ratio=4, amax_floor=1e-4, sanitize_nans=True),
            dict(rope="interleaved", compress_ratio=1, amax_floor=1e-4, sanitize_nans=False),
            dict(rope="neox", compress_ratio=3, amax_floor=0.0, sanitize_nans=True),
            dict(rope="none", compress_ratio=1, amax_floor=1e-4, sanitize_nans=True),
            dict(rope="none", compress_ratio=128, amax_floor=0.0, sanitize_nans=False)]


def _ids(o):
    return "-".join(str(v) for v in o.values())


@pytest.mark.parametrize("record", [528, 584])
def test_compressed_worked_token(golden, record):
    cv = golden["compressed_variant"]
    inp = cv["inputs"]
    x = np.zeros((2, 512), np.float32)
    for d, v in inp["kv_nonzero_token0"]:
        x[0, d] = float(v)
    x[1, :] = 1.0
    table = np.zeros((inp["max_pos"], 64), np.float32)
    table[:, :32] = 1.0
    table[4, 0], table[4, 32], table[4, 1], table[4, 33] = 0.5, 0.75, 0.0, 1.0
    exp = cv["mxfp8_record" if record == 528 else "legacy_record"]
    case = W.InsertCase("compressed_worked", record, inp["block_size"], inp["num_blocks"],
                        exp["page_stride"], W.to_bf16_bits(x),
                        np.array([t["slot"] for t in inp["tokens"]], np.int64),
                        np.array([t["position"] for t in inp["tokens"]], np.int64), table,
                        backing_seed=21)
    d = P.DeviceCase(case)
    d.insert(**cv["options"])
    got = d.backing_host()
    d0, s0 = exp["data_offset"], exp["scale_offset"]
    if record == 528:
        codes = np.zeros(512, np.uint8)
        for dim, c in exp["codes_nonzero"]:
            codes[dim] = c
        assert got[d0:d0 + 512].tolist() == codes.tolist()
        assert got[s0:s0 + 16].tolist() == exp["scales"]
    else:
        assert got[s0:s0 + 8].tolist() == exp["scale_row"]
    want = P.oracle_insert(case, case.initial_backing(), **cv["options"])
    assert np.array_equal(got, want), P.first_diff(got, want)


@pytest.mark.parametrize("opts", VARIANTS, ids=_ids)
@pytest.mark.parametrize("record", [528, 584])
@pytest.mark.parametrize("n,bs", [(1, 64), (17, 16), (1023, 64), (4099, 32)])
def test_variant_whole_backing(opts, record, n, bs):
    nb = (n * 5 // 4) // bs + 2
    case = W.custom_insert(9000 + n + bs + record, n, record, bs, nb, max_pos=512, scale_rows=True)
    kv = case.kv_bits.copy()
    if opts["sanitize_nans"]:
        kv[RNG.random(kv.shape) < 0.005] = 0x7FC0
        kv[RNG.random(kv.shape) < 0.002] = 0xFFC1  # negative-signed NaN payloads too
    case.kv_bits = kv
    d = P.DeviceCase(case)
    d.insert(**opts)
    got = d.backing_host()
    want = P.oracle_insert(case, case.initial_backing(), **opts)
    assert np.array_equal(got, want), P.first_diff(got, want)
    assert np.array_equal(P.host_bits(d.kv), kv), "kv was modified"
    # the gather reads the variant's records like any other
    idx = case.gather_indices.copy()
    gated = (case.positions + 1) % opts["compress_ratio"] == 0
    idx[~gated] = -1
    out = d.gather(idx)
    want_g = P.oracle_gather(case, want, idx)
    assert np.array_equal(out, want_g), P.first_diff(out, want_g)


@pytest.mark.parametrize("record", [528, 584])
def test_rotation_free_without_positions(record):
    case = W.custom_insert(77 + record, 3000, record, 64, 60)
    d = P.DeviceCase(case)
    B.kvrec_insert(d.kv, d.k_cache, d.slots, None, None, 64, rope="none")
    got = d.backing_host()
    want = case.initial_backing()
    import oracle
    oracle.insert(case.kv_bits, want, case.num_blocks, case.page_stride, 64, record,
                  case.slot_mapping, None, None, rope="none")
    assert np.array_equal(got, want), P.first_diff(got, want)


def test_compressed_prefill_262144():
    """The prefill workload's shape through the compressed variant (ratio 4:
    one token in four written), every byte of the backing compared."""
    case = W.prefill_262144()
    opts = dict(rope="interleaved", compress_ratio=4, amax_floor=1e-4, sanitize_nans=True)
    d = P.DeviceCase(case)
    d.insert(**opts)
    got = d.backing_host()
    want = P.oracle_insert(case, case.initial_backing(), **opts)
    assert np.array_equal(got, want), P.first_diff(got, want)
    del d
    torch.cuda.empty_cache()
