"""HIP-graph capture of the insert and the gather.

The library allocates nothing and never synchronises, so both calls can be
captured into a graph (the page's KV-only op is tested under CUDA-graph
capture as well: [KV-only op] 实现拆解 4). The graph is replayed several
times with fresh inputs written in place between replays, eager work and
synchronisations in between, and every replay is compared with the eager
result of the same inputs (itself compared with the oracle).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from quantized_paged_kv_rope_amd import binding as B
from quantized_paged_kv_rope_amd import workloads as W
from tests import parity_util as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("record", [528, 584])
def test_graph_replays_match_eager(record):
    n, bs, nb = 3000, 64, 60
    base = W.custom_insert(500 + record, n, record, bs, nb, scale_rows=True)
    cap = P.DeviceCase(base)
    idx = P.dev(base.gather_indices)
    out = torch.empty((n, 512), dtype=torch.bfloat16, device="cuda")
    init = P.dev(base.initial_backing())

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.kvrec_insert(cap.kv, cap.k_cache, cap.slots, cap.positions, cap.cos_sin, bs)
        B.kvrec_gather(cap.k_cache, idx, out=out)

    for rnd in range(3):
        nxt = W.custom_insert(600 + record + rnd, n, record, bs, nb, scale_rows=True)
        # the graph's slots, indices and cache pre-fill stay fixed; kv and positions change
        nxt.slot_mapping = base.slot_mapping.copy()
        nxt.gather_indices = base.gather_indices.copy()
        nxt.backing_seed = base.backing_seed
        # fresh inputs in place, cache reset, eager torch work in between
        cap.kv.copy_(P.dev_bf16(nxt.kv_bits))
        cap.positions.copy_(P.dev(nxt.positions))
        cap.backing.copy_(init)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_backing = cap.backing.cpu().numpy()
        got_out = P.host_bits(out)
        # eager result of the same inputs on a separate cache
        eager = P.DeviceCase(nxt)
        eager.insert()
        want_backing = eager.backing_host()
        want_out = eager.gather(nxt.gather_indices)
        assert np.array_equal(got_backing, want_backing), f"replay {rnd}: " + P.first_diff(
            got_backing, want_backing)
        assert np.array_equal(got_out, want_out), f"replay {rnd}: " + P.first_diff(got_out, want_out)
        # and the eager result is the oracle's
        oracle_backing = P.oracle_insert(nxt, nxt.initial_backing())
        assert np.array_equal(want_backing, oracle_backing)
        del junk


def _replay_rounds(capture, refill, eager, rounds=3):
    """Capture `capture` once; per round write new inputs in place
    (`refill(rnd)`), run eager torch work, replay, and compare every output
    of the replay with `eager(rnd)` (the uncaptured call on the same inputs)."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outputs = capture()
    for rnd in range(rounds):
        refill(rnd)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy().copy() for o in outputs]
        want = eager(rnd)
        for k, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"replay {rnd}, output {k}: " + P.first_diff(a, b)
        del junk


def test_graph_compressed_and_full_inserts():
    """kvrec_insert_ex (gated ratio 4 and rotation-free) and kvrec_insert_full
    (bf16, fp8 with the scale changed between replays) under graph capture."""
    n, bs, nb = 2000, 16, 160
    base = W.custom_insert(710, n, 528, bs, nb, max_pos=800, scale_rows=True)
    d = P.DeviceCase(base)
    init = P.dev(base.initial_backing())
    full = {rec: W.retarget(base, rec) for rec in (W.RECORD_BF16, W.RECORD_FP8)}
    fdev = {rec: P.DeviceCase(c) for rec, c in full.items()}
    finit = {rec: P.dev(c.initial_backing()) for rec, c in full.items()}
    scale = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    cmp_opts = B.insert_options("interleaved", 4, 1e-4, True)

    def capture():
        B.kvrec_insert_ex(d.kv, d.k_cache, d.slots, d.positions, d.cos_sin, bs, options=cmp_opts)
        B.kvrec_insert_full(d.kv, fdev[W.RECORD_BF16].k_cache, d.slots, d.positions, d.cos_sin, bs)
        B.kvrec_insert_full(d.kv, fdev[W.RECORD_FP8].k_cache, d.slots, d.positions, d.cos_sin, bs,
                            scale)
        return [d.backing, fdev[W.RECORD_BF16].backing, fdev[W.RECORD_FP8].backing]

    kvs = [W.custom_insert(720 + r, n, 528, bs, nb, max_pos=800, scale_rows=True) for r in range(3)]

    def refill(rnd):
        d.kv.copy_(P.dev_bf16(kvs[rnd].kv_bits))
        d.positions.copy_(P.dev(kvs[rnd].positions))
        d.backing.copy_(init)
        for rec in full:
            fdev[rec].backing.copy_(finit[rec])
        scale.fill_(0.5 + rnd)

    def eager(rnd):
        e = W.InsertCase("g", 528, bs, nb, base.page_stride, kvs[rnd].kv_bits, base.slot_mapping,
                         kvs[rnd].positions, base.cos_sin, base.backing_seed)
        de = P.DeviceCase(e)
        de.insert(rope="interleaved", compress_ratio=4, amax_floor=1e-4, sanitize_nans=True)
        outs = [de.backing_host()]
        for rec in (W.RECORD_BF16, W.RECORD_FP8):
            fe = P.DeviceCase(W.retarget(e, rec))
            fe.insert_full(None if rec == W.RECORD_BF16 else 0.5 + rnd)
            outs.append(fe.backing_host())
        return outs

    _replay_rounds(capture, refill, eager)


def test_graph_attention_write_and_expansion():
    """kvrec_qnorm_rope_insert (in place) and kvrec_expand_candidates under
    graph capture."""
    n, heads, bs, nb = 300, 8, 16, 30
    base = W.custom_insert(730, n, 528, bs, nb, max_pos=600, scale_rows=True)
    d = P.DeviceCase(base)
    init = P.dev(base.initial_backing())
    rng = np.random.default_rng(731)
    qs = [W.to_bf16_bits(rng.standard_normal((n, heads, 512)).astype(np.float32)) for _ in range(3)]
    q = P.dev_bf16(qs[0].reshape(-1, 512)).view(n, heads, 512)
    rows, k = 200, 64
    cands = [rng.integers(-1, 200, (rows, k)).astype(np.int32) for _ in range(3)]
    ks = P.dev(rng.integers(0, 500, rows).astype(np.int32))
    ke = P.dev((ks.cpu().numpy() + rng.integers(0, 2000, rows)).astype(np.int32))
    cand = P.dev(cands[0])
    sp = torch.empty((rows, 2 * k), dtype=torch.int32, device="cuda")
    end = torch.empty(rows, dtype=torch.int32, device="cuda")

    def capture():
        B.kvrec_qnorm_rope_insert(q, d.kv, d.k_cache, d.slots, d.positions, d.cos_sin, bs,
                                  eps=1e-6)
        B.kvrec_expand_candidates(cand, ks, ke, 2, 8, out=(sp, end))
        return [q.view(torch.int16), d.backing, sp, end]

    def refill(rnd):
        q.copy_(P.dev_bf16(qs[rnd].reshape(-1, 512)).view(n, heads, 512))
        d.backing.copy_(init)
        cand.copy_(P.dev(cands[rnd]))

    def eager(rnd):
        qe = P.dev_bf16(qs[rnd].reshape(-1, 512)).view(n, heads, 512)
        de = P.DeviceCase(base)
        B.kvrec_qnorm_rope_insert(qe, de.kv, de.k_cache, de.slots, de.positions, de.cos_sin, bs,
                                  eps=1e-6)
        spe, ende = B.kvrec_expand_candidates(P.dev(cands[rnd]), ks, ke, 2, 8)
        torch.cuda.synchronize()
        return [qe.view(torch.int16).cpu().numpy(), de.backing_host(), spe.cpu().numpy(),
                ende.cpu().numpy()]

    _replay_rounds(capture, refill, eager)
