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
