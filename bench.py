"""Benchmark of the paged KV-record codec on one MI355X.

One step = the whole path over one batch: kvrec_insert of 262144 contiguous
prefill tokens into the 528 B MXFP8 record (RoPE + quantise + paged store),
then kvrec_gather of all 262144 slots back to bf16 (the round trip). Inputs
are seeded synthetic data, resident in HBM before the timed region.

Prints ONE JSON line: tokens/s through the path, per-kernel durations from
HIP events recorded on the stream the kernels run on, the dominant kernel's
achieved bandwidth against the 8 TB/s HBM peak, every kernel the 70% target
covers ("target_rows": the 262144-token insert and gather, the 65536-token
584 B insert and the 64 x 2048 top-k gather, each timed cold, back to back
over copies of its buffers, and back to back), and the CPU oracle timed on
a bounded sample of the same workload (single-threaded, median of 3, and on
all the host threads it is given, the two results asserted identical).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-target-rows]
    python bench.py --all-configs     # adds a per-workload table on stderr

The JSON line on stdout is the only headline. --all-configs also times each
kernel on the other workloads (single launches after a 1 GiB read that
leaves the caches clean, and back-to-back launches replayed from a HIP graph),
prints them as a table on stderr and adds them to the JSON line as
"all_configs".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
TOKENS = 262144
# Algorithmic bytes per token (what the method must move):
#   insert: kv 1024 + slot 8 + position 8 + cos/sin row 256 + record 528
#   gather: index 4 + record 528 + bf16 row 1024
INSERT_BYTES_PER_TOKEN = 1024 + 8 + 8 + 256 + 528
GATHER_BYTES_PER_ROW = 4 + 528 + 1024
PROFILE_PMC = os.path.join(ROOT, "profiles", "insert_mxfp8_prefill_262144_pmc.txt")
KERNEL_SRC = os.path.join(ROOT, "quantized_paged_kv_rope_amd", "csrc", "kvrec_kernels.hip")


def kernel_code_hash(path: str = KERNEL_SRC) -> str:
    """sha256[:16] of a kernel source's code: comments removed and every run
    of whitespace made one space, so that an edit of comments or layout keeps
    the hash and any change to the code changes it."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def counter_traffic():
    """HBM bytes per insert launch from the committed rocprofv3 counter
    summary, or None if there is none or the kernel code changed since."""
    if not os.path.exists(PROFILE_PMC):
        return None
    text = open(PROFILE_PMC).read()
    m = re.search(r"kernel_code_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_code_hash():
        return None
    return float(t.group(1))


def host_threads() -> int:
    """Threads for the threaded oracle run: the CPUs this process may use,
    at most 16 (the host share of a one-GPU machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_round_trip(case, n: int, sub_blocks: int, threads: int, chunk: int = 4096):
    """The oracle's insert of the first n tokens into a zeroed cache of
    sub_blocks pages, then its gather of their slots: one call each, or
    `threads` threads over token chunks (tokens are independent and the
    slots distinct, so the bytes cannot depend on the split)."""
    import concurrent.futures as cf

    import oracle

    backing = np.zeros(sub_blocks * case.page_stride, np.uint8)
    out = np.empty((n, 512), np.uint16)

    def ins(a, b):
        oracle.insert(case.kv_bits[a:b], backing, sub_blocks, case.page_stride, case.block_size,
                      case.record, case.slot_mapping[a:b], case.positions[a:b], case.cos_sin)

    def gat(a, b):
        out[a:b] = oracle.gather(backing, sub_blocks, case.page_stride, case.block_size,
                                 case.record, case.gather_indices[a:b])

    t0 = time.perf_counter()
    if threads == 1:
        ins(0, n)
        gat(0, n)
    else:
        spans = [(a, min(n, a + chunk)) for a in range(0, n, chunk)]
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda ab: ins(*ab), spans))
            list(ex.map(lambda ab: gat(*ab), spans))
    return time.perf_counter() - t0, backing, out


def cpu_baseline(case, d_backing, d_out, sample: int):
    """The oracle, as it stands, on the host: insert and gather of the first
    `sample` tokens of the workload, (i) single-threaded, median of 3 runs,
    and (ii) over token chunks on every host thread it is given; the two
    results must be identical byte for byte, and equal to the GPU's records
    and rows for those tokens. `value` is run (ii)."""
    import oracle

    oracle.lib()
    n = sample
    sub_blocks = (n + case.block_size - 1) // case.block_size
    singles = []
    for _ in range(3):
        dt, backing, out = _oracle_round_trip(case, n, sub_blocks, 1)
        singles.append(dt)
    threads = host_threads()
    dt_mt, backing_mt, out_mt = _oracle_round_trip(case, n, sub_blocks, threads)
    same = bool(np.array_equal(backing_mt, backing) and np.array_equal(out_mt, out))
    if not same:
        raise AssertionError("threaded oracle run differs from the single-threaded run")
    gpu_rec = d_backing[: sub_blocks * case.page_stride].cpu().numpy()
    gpu_out = d_out[:n].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    exact = bool(np.array_equal(gpu_rec, backing) and np.array_equal(gpu_out, out))
    single = float(np.median(singles))
    return {"value": n / dt_mt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"insert + gather of the first {n} of the {case.num_tokens} tokens "
                      f"(whole pages {sub_blocks}) on {threads} threads over 4096-token "
                      f"chunks, {dt_mt:.2f} s; single-threaded median of 3 {single:.2f} s",
            "seconds": round(dt_mt, 3),
            "single_thread": {"value": n / single, "unit": "tokens/s", "cores": 1,
                              "seconds_runs": [round(x, 3) for x in singles],
                              "seconds_median": round(single, 3)},
            "threaded_equals_single_thread": same,
            "gpu_matches_oracle_on_sample": exact,
            "host_cpu": _cpu_model(), "host_threads_available": os.cpu_count()}


def _time_cold(fn, flush, reps=50):
    """Single launches on clean caches: before each one (untimed) a 1 GiB
    read replaces the L2 and Infinity Cache contents. HIP events on the
    current stream around the launch; they also bracket its dispatch."""
    import torch

    for _ in range(5):
        fn()
    ts = []
    for _ in range(reps):
        flush.sum(dtype=torch.int64)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return np.array(ts)


def _time_back_to_back(fn, batches=10, per_batch=20):
    """Launches issued back to back on the current stream: `batches` runs of
    `per_batch` launches, one pair of HIP events around each run; the time
    per launch of each run (its kernels and the gaps between them, without
    an event between every two launches)."""
    import torch

    for _ in range(5):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(batches)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record()
        for _ in range(per_batch):
            fn()
        e1.record()
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) * 1e3 / per_batch for e0, e1 in ev])


def _time_rotating(fns, batches=10, per_batch=20):
    """Launches back to back on the current stream, rotating over copies of
    the workload's buffers (fns[i] runs on copy i): with enough copies every
    launch finds its inputs and outputs evicted from the L2 and the Infinity
    Cache by the launches in between, as on clean caches, but without a flush
    and an event pair around each launch. Median over `batches` runs of
    `per_batch` launches, one event pair per run."""
    import torch

    for f in fns:
        f()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(batches)]
    torch.cuda.synchronize()
    i = 0
    for e0, e1 in ev:
        e0.record()
        for _ in range(per_batch):
            fns[i % len(fns)]()
            i += 1
        e1.record()
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) * 1e3 / per_batch for e0, e1 in ev])


TARGET_FRAC = 0.70


def _target_row(workload, op, rows, valid, nbytes, cold, b2b, rotating=None, copies=0):
    def stats(ts):
        med = float(np.median(ts))
        return {"median_us": med, "mean_us": float(ts.mean()),
                "p10_us": float(np.percentile(ts, 10)), "p90_us": float(np.percentile(ts, 90)),
                "GBps": nbytes / med / 1e3, "frac": nbytes / med / 1e3 / HBM_PEAK_GBPS,
                "reps": int(ts.size)}

    c, b = stats(cold), stats(b2b)
    target_us = nbytes / (TARGET_FRAC * HBM_PEAK_GBPS * 1e3)
    row = {"workload": workload, "op": op, "rows": rows, "valid_rows": valid,
           "algorithmic_bytes": nbytes, "target_us": target_us, "cold": c, "back_to_back": b,
           "meets_target": {"cold": c["median_us"] <= target_us,
                            "back_to_back": b["median_us"] <= target_us}}
    if rotating is not None:
        r = stats(rotating)
        r["copies"] = copies
        row["cold_rotating"] = r
        row["meets_target"]["cold_rotating"] = r["median_us"] <= target_us
    return row


def target_rows(dev, prefill) -> list:
    """Every kernel the >= 70% target covers, timed cold (median of 50
    single launches, each after a 1 GiB read), cold by rotation (back to back
    over copies of the buffers, each launch's data evicted by the others) and
    back to back on one copy (median over 10 runs of 20 launches):
    the 262144-token insert and gather (the headline's tensors), the
    65536-token 584 B insert (random slots, 5% -1) and the 64 x 2048 top-k
    gather from the 32768-page cache."""
    import torch

    from quantized_paged_kv_rope_amd import binding as B
    from quantized_paged_kv_rope_amd import workloads as W

    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    rows = []

    def add(workload, op, n, valid, nbytes, fns):
        """fns: one launch per copy of the buffers; fns[0] is also timed
        cold and back to back."""
        rows.append(_target_row(workload, op, n, valid, nbytes, _time_cold(fns[0], flush),
                                _time_back_to_back(fns[0]), _time_rotating(fns), len(fns)))

    def copies(tensors, k):
        """k sets of the tensors: the originals, then k - 1 clones."""
        return [tuple(tensors)] + [tuple(t.clone() for t in tensors) for _ in range(k - 1)]

    def cache_view(backing, nb, bs, rec, stride):
        return B.alloc_cache(nb, bs, rec, stride, backing=backing)[1]

    # 262144 tokens: one launch moves more than the 256 MB Infinity Cache
    # holds, so three copies leave nothing of a launch's data in cache by its
    # next turn.
    case, kv, slots, pos, cos_sin, idx, k_cache, out = prefill
    n = case.num_tokens
    geo = (case.num_blocks, case.block_size, case.record, case.page_stride)
    backing = k_cache.as_strided((case.num_blocks * case.page_stride,), (1,))
    sets = [s + (cache_view(s[4], *geo),) for s in copies((kv, slots, pos, cos_sin, backing), 3)]
    add(case.name, "insert 528 B", n, n, n * INSERT_BYTES_PER_TOKEN,
        [lambda s=s: B.kvrec_insert(s[0], s[5], s[1], s[2], s[3], case.block_size)
         for s in sets])
    gsets = [(s[5], gi, go) for s, (gi, go) in zip(sets, copies((idx, out), 3))]
    add(case.name, "gather 528 B", n, n, n * GATHER_BYTES_PER_ROW,
        [lambda s=s: B.kvrec_gather(s[0], s[1], out=s[2]) for s in gsets])
    del sets, gsets

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # 65536 legacy tokens move 117 MB: five copies put 468 MB of other
    # launches between two turns of one copy.
    lg = W.legacy_65536()
    lkv = up(lg.kv_bits.view(np.int16)).view(torch.bfloat16)
    lsl, lps, lcs = up(lg.slot_mapping), up(lg.positions), up(lg.cos_sin)
    lback, _ = B.alloc_cache(lg.num_blocks, lg.block_size, lg.record, lg.page_stride, device=dev)
    lback.zero_()
    lgeo = (lg.num_blocks, lg.block_size, lg.record, lg.page_stride)
    lsets = [s + (cache_view(s[4], *lgeo),) for s in copies((lkv, lsl, lps, lcs, lback), 5)]
    valid = int((lg.slot_mapping >= 0).sum())
    lbytes = valid * (1024 + 8 + 8 + 256 + lg.record) + (lg.num_tokens - valid) * 8
    add(lg.name, "insert 584 B", lg.num_tokens, valid, lbytes,
        [lambda s=s: B.kvrec_insert(s[0], s[5], s[1], s[2], s[3], lg.block_size)
         for s in lsets])
    del lkv, lsl, lps, lcs, lback, lsets

    # the top-k gather reads 84 MB of records and writes 134 MB per launch:
    # six copies of the 1.1 GB cache put over 1 GB between two turns.
    tk = W.topk_gather()
    tback, tkc = B.alloc_cache(tk.num_blocks, tk.block_size, tk.record, tk.page_stride, device=dev)
    tcs = up(tk.cos_sin())
    for k in range(tk.num_chunks):
        kvb, sl, ps = tk.fill_chunk(k)
        B.kvrec_insert(up(kvb.view(np.int16)).view(torch.bfloat16), tkc, up(sl), up(ps), tcs,
                       tk.block_size)
    tidx = up(tk.indices)
    tout = torch.empty(tuple(tidx.shape) + (512,), dtype=torch.bfloat16, device=dev)
    tgeo = (tk.num_blocks, tk.block_size, tk.record, tk.page_stride)
    tsets = [(cache_view(s[0], *tgeo),) + s[1:] for s in copies((tback, tidx, tout), 6)]
    gv = int((tk.indices >= 0).sum())
    gb = gv * GATHER_BYTES_PER_ROW + (tidx.numel() - gv) * (4 + 1024)
    add(tk.name, "gather 528 B (32768 pages)", tidx.numel(), gv, gb,
        [lambda s=s: B.kvrec_gather(s[0], s[1], out=s[2]) for s in tsets])
    del tback, tkc, tidx, tout, tsets, flush
    torch.cuda.empty_cache()
    return rows


def all_configs_report(dev, out=sys.stderr) -> list:
    """Per-kernel timings of every workload (cold and back-to-back)."""
    import torch

    from quantized_paged_kv_rope_amd import binding as B
    from quantized_paged_kv_rope_amd import workloads as W

    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)

    def cold(fn, reps=50):
        for _ in range(5):
            fn()
        ts = []
        for _ in range(reps):
            flush.sum(dtype=torch.int64)  # reads 1 GiB: caches left holding clean lines
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return np.percentile(ts, [50, 10, 90])

    def replayed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (5 * reps)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    rows = []

    def add(workload, op, n, valid, nbytes, fn):
        (c, c10, c90), r = cold(fn), replayed(fn)
        rows.append({"workload": workload, "op": op, "rows": n, "valid": valid,
                     "algorithmic_bytes": nbytes, "cold_us": c, "cold_p10_us": c10,
                     "cold_p90_us": c90, "replayed_us": r,
                     "cold_GBps": nbytes / c / 1e3, "replayed_GBps": nbytes / r / 1e3,
                     "tokens_per_s_replayed": n / r * 1e6,
                     "valid_tokens_per_s_replayed": valid / r * 1e6})

    cases = [W.mixed_1024(), W.decode_16384(), W.prefill_262144(), W.legacy_65536()]
    for case in cases:
        kv = up(case.kv_bits.view(np.int16)).view(torch.bfloat16)
        sl, ps, cs = up(case.slot_mapping), up(case.positions), up(case.cos_sin)
        backing, kc = B.alloc_cache(case.num_blocks, case.block_size, case.record,
                                    case.page_stride, device=dev)
        backing.zero_()
        valid = int((case.slot_mapping >= 0).sum())
        n = case.num_tokens
        ib = valid * (1024 + 8 + 8 + 256 + case.record) + (n - valid) * 8
        add(case.name, f"insert {case.record} B", n, valid, ib,
            lambda: B.kvrec_insert(kv, kc, sl, ps, cs, case.block_size))
        if case.name.startswith("prefill"):
            # the compressed-KV insert: gated tokens read slot + position only
            p1 = case.positions[:n] + 1
            for ratio in (1, 4):
                keep = (case.slot_mapping >= 0) & (p1 % ratio == 0) & (p1 >= ratio)
                kept = int(keep.sum())
                vb = kept * (1024 + 8 + 8 + 256 + case.record) + (valid - kept) * 16 + \
                    (n - valid) * 8
                add(case.name, f"cmp r{ratio} {case.record}", n, kept, vb,
                    lambda r=ratio: B.kvrec_insert(kv, kc, sl, ps, cs, case.block_size,
                                                   rope="interleaved", compress_ratio=r,
                                                   amax_floor=1e-4, sanitize_nans=True))
            nb = valid * (1024 + 8 + case.record) + (n - valid) * 8
            add(case.name, f"norope {case.record}", n, valid, nb,
                lambda: B.kvrec_insert_ex(kv, kc, sl, None, None, case.block_size,
                                          options=B.insert_options(rope="none")))
            # the non-packed caches: bf16 rows and per-tensor-scaled fp8 rows
            for rec in (B.RECORD_BF16, B.RECORD_FP8):
                fb, fc = B.alloc_cache(case.num_blocks, case.block_size, rec, device=dev)
                sc = torch.tensor([0.0625], dtype=torch.float32, device=dev) \
                    if rec == B.RECORD_FP8 else None
                fbytes = valid * (1024 + 8 + 8 + 256 + rec) + (n - valid) * 8
                add(case.name, f"full {rec} B", n, valid, fbytes,
                    lambda fc=fc, sc=sc: B.kvrec_insert_full(kv, fc, sl, ps, cs,
                                                             case.block_size, sc))
                del fb, fc
        if case.name.startswith("decode"):
            continue
        idx = up(case.gather_indices)
        o = torch.empty((idx.numel(), 512), dtype=torch.bfloat16, device=dev)
        gv = int((case.gather_indices >= 0).sum())
        gb = gv * (4 + case.record + 1024) + (idx.numel() - gv) * (4 + 1024)
        add(case.name, f"gather {case.record} B", idx.numel(), gv, gb,
            lambda: B.kvrec_gather(kc, idx, out=o))
        del backing, kc, kv, o
        torch.cuda.empty_cache()
    # the attention write: q RMSNorm + RoPE over 128 heads fused with the insert
    aw = W.attention_write()
    ac = aw.insert
    q = up(aw.q_bits.view(np.int16)).view(torch.bfloat16)
    qo = torch.empty_like(q)
    kv = up(ac.kv_bits.view(np.int16)).view(torch.bfloat16)
    sl, ps, cs = up(ac.slot_mapping), up(ac.positions), up(ac.cos_sin)
    backing, kc = B.alloc_cache(ac.num_blocks, ac.block_size, ac.record, ac.page_stride,
                                device=dev)
    heads = aw.q_bits.shape[1]
    ab = ac.num_tokens * (1824 + 2048 * heads)
    add(aw.name, f"qkv {heads}h 528", ac.num_tokens, ac.num_tokens, ab,
        lambda: B.kvrec_qnorm_rope_insert(q, kv, kc, sl, ps, cs, ac.block_size, eps=aw.eps,
                                          q_out=qo))
    del q, qo, kv, backing, kc
    torch.cuda.empty_cache()
    # the sparse indexer's candidate-block expansion (integer; per row: the
    # candidates, ks and ke in, the sparse indices and end out)
    sx = W.sparse_expand()
    xc, xks, xke = up(sx.cand), up(sx.row_ks), up(sx.row_ke)
    xrows, k = sx.cand.shape
    xout = (torch.empty((xrows, k * sx.ratio), dtype=torch.int32, device=dev),
            torch.empty(xrows, dtype=torch.int32, device=dev))
    xb = xrows * (4 * k + 8 + 4 * k * sx.ratio + 4)
    add(sx.name, f"expand r{sx.ratio} sbk{sx.sparse_block}", xrows, xrows, xb,
        lambda: B.kvrec_expand_candidates(xc, xks, xke, sx.ratio, sx.sparse_block, out=xout))
    del xc, xks, xke, xout
    tk = W.topk_gather()
    backing, kc = B.alloc_cache(tk.num_blocks, tk.block_size, tk.record, tk.page_stride, device=dev)
    cs = up(tk.cos_sin())
    for k in range(tk.num_chunks):
        kvb, sl, ps = tk.fill_chunk(k)
        B.kvrec_insert(up(kvb.view(np.int16)).view(torch.bfloat16), kc, up(sl), up(ps), cs,
                       tk.block_size)
    idx = up(tk.indices)
    o = torch.empty(tuple(idx.shape) + (512,), dtype=torch.bfloat16, device=dev)
    gv = int((tk.indices >= 0).sum())
    gb = gv * (4 + tk.record + 1024) + (idx.numel() - gv) * (4 + 1024)
    add(tk.name + " (32768 pages)", "gather 528 B", idx.numel(), gv, gb,
        lambda: B.kvrec_gather(kc, idx, out=o))
    del backing, kc, o, flush
    torch.cuda.empty_cache()
    print(f"{'workload':28s} {'op':14s} {'rows':>7s} {'cold us':>8s} {'p10-p90':>11s} "
          f"{'GB/s':>6s} {'%peak':>6s} {'replay us':>9s} {'GB/s':>6s} {'%peak':>6s}", file=out)
    for r in rows:
        print(f"{r['workload']:28s} {r['op']:14s} {r['rows']:7d} {r['cold_us']:8.1f} "
              f"{r['cold_p10_us']:5.1f}-{r['cold_p90_us']:<5.1f} "
              f"{r['cold_GBps']:6.0f} {100 * r['cold_GBps'] / HBM_PEAK_GBPS:5.1f}% "
              f"{r['replayed_us']:9.1f} {r['replayed_GBps']:6.0f} "
              f"{100 * r['replayed_GBps'] / HBM_PEAK_GBPS:5.1f}%", file=out, flush=True)
    return rows


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# hipDeviceAttribute_t values (hip_runtime_api.h, ROCm 7).
_HIP_ATTR = {"shader_clock_khz": 5, "memory_bus_width_bits": 59, "memory_clock_khz": 60,
             "compute_units": 63}


def device_info() -> dict:
    """What the device reports about itself (name, arch, CU count, clocks,
    memory bus width), read through the HIP runtime torch loaded. The HBM
    peak used for `frac` stays the published 8 TB/s: the reported memory
    clock is not the HBM3E data rate."""
    import ctypes

    import torch

    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    info = {"name": props.name, "arch": props.gcnArchName,
            "total_memory_GiB": round(props.total_memory / 2 ** 30, 1)}
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
    except OSError:
        return info
    for key, attr in _HIP_ATTR.items():
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, torch.cuda.current_device()) == 0:
            info[key] = v.value
    return info


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=TOKENS // 2)
    ap.add_argument("--no-target-rows", action="store_true",
                    help="skip the cold / back-to-back timing of every targeted kernel")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also print per-kernel timings of every workload on stderr")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the insert and gather "
              "have no cross-GPU step; each GPU would run the same kernels on its own cache.",
              file=sys.stderr)
        return 2

    import torch

    from quantized_paged_kv_rope_amd import binding as B
    from quantized_paged_kv_rope_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load_library()

    case = W.prefill_262144(n=TOKENS)
    kv = torch.from_numpy(case.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    pos = torch.from_numpy(case.positions).to(dev)
    cos_sin = torch.from_numpy(case.cos_sin).to(dev)
    idx = torch.from_numpy(case.gather_indices).to(dev)
    backing, k_cache = B.alloc_cache(case.num_blocks, case.block_size, case.record,
                                     case.page_stride, device=dev)
    backing.zero_()
    out = torch.empty((TOKENS, 512), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        B.kvrec_insert(kv, k_cache, slots, pos, cos_sin, case.block_size)
        if ev is not None:
            ev[1].record()
        B.kvrec_gather(k_cache, idx, out=out)
        if ev is not None:
            ev[2].record()

    # One untimed step gives the records and rows the CPU baseline compares
    # with; the baseline and the per-kernel rows run before the headline's
    # warm-up, so the timed steps follow GPU work rather than host work.
    step()
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, backing, out, min(args.cpu_sample, TOKENS))
    rows = None
    if not args.no_target_rows:
        rows = target_rows(dev, (case, kv, slots, pos, cos_sin, idx, k_cache, out))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ins_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    gat_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    ins_s, gat_s = ins_ms.mean() / 1e3, gat_ms.mean() / 1e3
    ins_bytes = TOKENS * INSERT_BYTES_PER_TOKEN
    gat_bytes = TOKENS * GATHER_BYTES_PER_ROW
    ins_gbps = ins_bytes / ins_s / 1e9
    gat_gbps = gat_bytes / gat_s / 1e9

    copy_gbps = None
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * src.numel() * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9
        del src, dst

    traffic = counter_traffic()
    result = {
        "metric": "insert & gather tokens/s + achieved HBM GB/s vs MI355X peak (528B MXFP8)",
        "value": TOKENS * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill_262144: insert 262144 contiguous tokens (positions 0.., slots "
                        "0.., 4096 pages of 64) into the 528 B MXFP8 record, then gather all "
                        "262144 slots back to bf16",
            "tokens": TOKENS, "record_bytes": case.record, "block_size": case.block_size,
            "page_stride": case.page_stride, "io": "bf16 in; e4m3 + UE8M0 record; bf16 out",
        },
        "roofline": {
            "bound": "hbm", "kernel": "insert_kernel (528 B MXFP8 record)",
            "achieved": ins_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": ins_gbps / HBM_PEAK_GBPS, "traffic": traffic,
            "algorithmic_bytes_per_launch": ins_bytes,
        },
        "kernels": {
            "insert": {"avg_us": ins_s * 1e6, "p50_us": float(np.median(ins_ms)) * 1e3,
                                    "p10_us": float(np.percentile(ins_ms, 10)) * 1e3,
                                    "p90_us": float(np.percentile(ins_ms, 90)) * 1e3,
                                    "GBps": ins_gbps, "frac_of_peak": ins_gbps / HBM_PEAK_GBPS,
                                    "tokens_per_s": TOKENS / ins_s},
            "gather": {"avg_us": gat_s * 1e6, "p50_us": float(np.median(gat_ms)) * 1e3,
                                    "p10_us": float(np.percentile(gat_ms, 10)) * 1e3,
                                    "p90_us": float(np.percentile(gat_ms, 90)) * 1e3,
                                    "GBps": gat_gbps, "frac_of_peak": gat_gbps / HBM_PEAK_GBPS,
                                    "tokens_per_s": TOKENS / gat_s,
                                    "algorithmic_bytes_per_launch": gat_bytes},
        },
        "kernel_code_sha256_16": kernel_code_hash(),
        "device": device_info(),
    }
    if copy_gbps is not None:
        result["device_copy_GBps"] = copy_gbps
    if cpu is not None:
        result["cpu_baseline"] = cpu
    if rows is not None:
        result["target_rows"] = rows
    if args.all_configs:
        del kv, slots, pos, cos_sin, idx, backing, k_cache, out
        torch.cuda.empty_cache()
        result["all_configs"] = [
            {k: (v.item() if isinstance(v, np.generic) else v) for k, v in row.items()}
            for row in all_configs_report(dev)]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
