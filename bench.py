#!/usr/bin/env python3
"""Benchmark of one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: the cache write of each
sequence's newest token (reshape_and_cache), then paged-attention decode over
contexts that include it.  Inputs are synthetic, drawn by the seeded workload
generator, and resident in HBM before the timed region starts.

    python bench.py [--steps K] [--warmup W] [--config 3] [--partition 0]

prints ONE JSON line (``--swap`` measures preemption instead: swapping KV
blocks to pinned host memory and back, and batched copy-on-write copies;
``--block-size-sweep`` the decode of the configuration at block sizes 8, 16
and 32 with the internal fragmentation of each).  ``value`` is context tokens attended per second over the
timed steps (tokens attended per step, i.e. the context lengths or, with a
sliding window, min(length, window), x steps / wall time between two device
synchronisations).  ``roofline`` reports the decode call (the dominant
kernel) against HBM bandwidth: algorithmic bytes per call (K and V of every
context token read once, each shared block counted once, plus Q, the output,
the block-table entries, the lengths and int8 scales) over its average
duration from HIP events on the launch stream.  The timed steps rotate
through identical copies of the K/V caches (``cache_copies``, enough that at
least 768 MiB of other cache data passes between two uses of one copy), so a
step reads its K/V from HBM, not from the MALL the previous step filled; the
event-timed sweeps fill a 512 MiB buffer before each timed call for the same
reason.  ``read_probe_gbps`` is the library's read-only streaming probe
(the decode's loads over 2 GiB, one contiguous stretch per workgroup), the
read bandwidth of a plain stream on this GPU.  ``cpu_baseline`` times the CPU
oracle (test infrastructure, fp64 NumPy) on a bounded sample of the same
workload on this host.

After the timed steps the decode call alone is timed ``--sweep-calls`` times
(100) from cold caches (a 512 MiB fill before each call, outside the HIP
events): its median, p10 and p90 go into ``roofline``; ``parity`` compares
every sequence of the batch with the oracle.  ``configs`` then holds the same
statistics, algorithmic bytes, fraction of the HBM peak, context tokens/s,
token x heads/s and whole-batch parity for every configuration in
``--sweep-configs`` (default all eight; the headline's entry reuses its own
numbers).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention: context tokens attended/s and achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "fp8": 1}
SCALED = ("i8", "fp8")
TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-3, "i8": 2e-2, "fp8": 2e-3}
KERNEL_SOURCES = ["decode_kernel.h", "decode_gqa_kernel.h", "decode_prefix_kernel.h",
                  "decode_dispatch.h", "decode.hip", "decode_f32.hip", "decode_f16.hip",
                  "decode_bf16.hip", "decode_i8.hip", "decode_fp8.hip"]


# Caches between timed calls: each XCD's L2 (4 MiB) and the 256 MiB MALL in
# front of HBM.  A call reads its K/V cold when at least COLD_BYTES of other
# data went through them since its last use.
COLD_BYTES = 768 << 20
FLUSH_BYTES = 512 << 20


def cache_copies(kv_bytes):
    """Copies of the K/V caches that the timed steps rotate through, so that
    every step reads its K/V from HBM rather than from the MALL that the
    previous steps filled: the other copies' K/V, at least COLD_BYTES, pass
    between two uses of one copy (at most 16 copies).  K/V of COLD_BYTES or
    more evicts itself within one call: one copy."""
    if kv_bytes >= COLD_BYTES:
        return 1
    return int(min(16, 1 + math.ceil(COLD_BYTES / max(kv_bytes, 1))))


def kernel_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_379_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl):
    """Bytes the decode must move: every (block, kv head) row slice of a valid
    token once (shared blocks once), int8 scales per used block, the table
    entries and lengths it reads, Q in and the output out."""
    bs = wl.block_size
    row = wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_fmt]   # one token, all kv heads
    slots = {}   # physical block -> set of attended offsets
    table_entries = 0
    logical_tokens = 0
    for s in range(wl.num_seqs):
        n = int(wl.context_lens[s])
        first = max(0, n - wl.window) if wl.window else 0
        logical_tokens += n - first
        for j in range(first // bs, (n + bs - 1) // bs):
            table_entries += 1
            b = int(wl.block_tables[s, j])
            lo, hi = max(first - j * bs, 0), min(bs, n - j * bs)
            slots.setdefault(b, set()).update(range(lo, hi))
    valid = {b: len(o) for b, o in slots.items()}
    unique_tokens = sum(valid.values())
    kv = 2 * unique_tokens * row
    scales = 2 * 4 * wl.num_kv_heads * len(valid) if wl.kv_fmt in SCALED else 0
    qo = 2 * wl.num_seqs * wl.num_heads * wl.head_dim * ELEM_BYTES[wl.q_fmt]
    meta = 4 * table_entries + 4 * wl.num_seqs
    return dict(total=kv + scales + qo + meta, kv=kv, unique_tokens=unique_tokens,
                logical_tokens=logical_tokens, logical_kv=2 * logical_tokens * row,
                per_token=2 * row)


def load_traffic(workload, ws):
    """HBM bytes per decode call from committed rocprofv3 counter runs, if they
    were taken on the kernel as it is now; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash() or rec.get("partition_size") != ws:
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(wl, budget_s):
    """The oracle (never tuned) on the sequences of the same workload taken in
    order, cache write + decode per sequence, until ``budget_s`` of CPU time is
    spent."""
    import contextlib
    import oracle.paged_attention as pa
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    limiter = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
    kc, vc = wl.key_cache, wl.value_cache
    done, tokens, spent = 0, 0, 0.0
    with limiter:
        # sequences in order, wrapping around, until the budget is spent
        while spent < budget_s:
            s = done % wl.num_seqs
            t0 = time.perf_counter()
            kc, vc = pa.reshape_and_cache(wl.k_new[s:s + 1], wl.v_new[s:s + 1], wl.new_fmt, kc, vc,
                                          wl.kv_fmt, wl.slot_mapping[s:s + 1], wl.block_size,
                                          wl.k_scales, wl.v_scales, in_place=True)
            pa.paged_decode(wl.q[s:s + 1], wl.q_fmt, kc, vc, wl.kv_fmt, wl.block_tables[s:s + 1],
                            wl.context_lens[s:s + 1], wl.block_size, wl.scale, wl.k_scales,
                            wl.v_scales, window=wl.window)
            spent += time.perf_counter() - t0
            n = int(wl.context_lens[s])
            tokens += min(n, wl.window) if wl.window else n
            done += 1
    return {"value": tokens / spent, "unit": "context tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} sequence decodes ({done / wl.num_seqs:.2f} passes over the "
                      f"{wl.num_seqs} sequences, {tokens} context tokens), cache write + decode "
                      f"per sequence, fp64 NumPy, BLAS threads limited to {cores}",
            "seconds": round(spent, 3)}


def parity_all(wl, out):
    """Max abs error of the whole output against the oracle (every sequence and
    head), the oracle's seconds, and the number of sequences."""
    import oracle.paged_attention as pa
    t = time.perf_counter()
    ref = pa.paged_decode(wl.q, wl.q_fmt, wl.key_cache, wl.value_cache, wl.kv_fmt, wl.block_tables,
                          wl.context_lens, wl.block_size, wl.scale, wl.k_scales, wl.v_scales,
                          window=wl.window)
    got = out.float().cpu().numpy().astype(np.float64)
    return float(np.abs(got - ref).max()), time.perf_counter() - t


def cold_call_times(torch, fn, calls, warmup, flush):
    """Durations (us) of `calls` calls of fn from HIP events on the current
    stream, each after filling `flush` (outside the events), so every call
    starts with cold L2 and MALL."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for e0, e1 in ev:
        flush.fill_(1)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])


def time_stats(us, ab, wl, num_heads):
    """Median / p10 / p90 of the call durations with the rates they give."""
    med = float(np.median(us))
    tokens = ab["logical_tokens"]
    return {"calls": int(len(us)), "decode_us_median": med,
            "decode_us_p10": float(np.percentile(us, 10)),
            "decode_us_p90": float(np.percentile(us, 90)), "decode_us_mean": float(np.mean(us)),
            "algorithmic_bytes": ab["total"], "achieved_gbps": ab["total"] / (med * 1e-6) / 1e9,
            "frac_of_hbm_peak": ab["total"] / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "context_tokens_per_s": tokens / (med * 1e-6),
            "token_heads_per_s": tokens * num_heads / (med * 1e-6)}


def config_sweep(args, torch, pkv, W, log, indices, flush, headline=None):
    """Every listed configuration decoded `args.sweep_calls` times from cold
    caches (HIP events; the shared-prompt workload on its shared-prefix path),
    with the whole batch checked against the oracle.  `headline` = (index,
    stats, parity) of the configuration already measured."""
    rows = {}
    for idx in indices:
        if headline and idx == headline[0]:
            rows[W.CONFIG_NAMES[idx]] = headline[1]
            continue
        t0 = time.perf_counter()
        wl = W.make_workload(idx)
        dev = torch.device("cuda:0")

        def up(arr, fmt):
            arr = np.ascontiguousarray(arr)
            if fmt == "bf16":
                return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
            if fmt == "fp8":
                return torch.from_numpy(arr.view(np.uint8)).to(dev).view(torch.float8_e4m3fn)
            return torch.from_numpy(arr).to(dev)

        q = up(wl.q, wl.q_fmt)
        kc, vc = up(wl.key_cache, wl.kv_fmt), up(wl.value_cache, wl.kv_fmt)
        tables, lens = up(wl.block_tables, "i32"), up(wl.context_lens, "i32")
        ks = up(wl.k_scales, "f32") if wl.kv_fmt in SCALED else None
        vs = up(wl.v_scales, "f32") if wl.kv_fmt in SCALED else None
        out = torch.empty_like(q)
        B, H, D = q.shape
        MB = tables.shape[1]
        groups = None
        if wl.shared_prefix_blocks and not wl.window:
            groups = pkv.find_shared_prefixes(wl.block_tables, wl.context_lens, wl.block_size)
            need = pkv.decode_prefix_workspace_size(B, H, wl.num_kv_heads, D, wl.block_size, MB,
                                                    groups)
            plens = torch.full((B,), groups[0][2], dtype=torch.int32, device=dev)
        else:
            need = pkv.decode_workspace_size(B, H, wl.num_kv_heads, D, wl.block_size, MB, 0,
                                             wl.window)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def decode():
            if groups:
                pkv.paged_attention_decode_prefix(out, q, kc, vc, tables, lens, wl.block_size,
                                                  wl.scale, groups, ks, vs, workspace=ws,
                                                  prefix_lens=plens)
            else:
                pkv.paged_attention_decode(out, q, kc, vc, tables, lens, wl.block_size, wl.scale,
                                           ks, vs, workspace=ws, window=wl.window)

        us = cold_call_times(torch, decode, args.sweep_calls, 10, flush)
        ab = algorithmic_bytes(wl)
        row = time_stats(us, ab, wl, H)
        part = pkv.decode_partition_size(B, H, wl.num_kv_heads, D, wl.block_size, MB, 0, wl.window)
        row["kernel"] = decode_kernel_names(wl, part, bool(groups))
        row["decode_path"] = "shared-prefix" if groups else "per-sequence"
        if ab["unique_tokens"] != ab["logical_tokens"]:
            row["logical_bytes"] = ab["total"] - ab["kv"] + ab["logical_kv"]
        err, osec = parity_all(wl, out)
        tol = TOL[wl.kv_fmt]
        row["parity"] = {"max_abs_err": err, "tol": tol, "seqs": "all", "num_seqs": B,
                         "ok": err <= tol, "oracle_s": round(osec, 2)}
        rows[wl.name] = row
        log(f"config {idx} {wl.name}: median {row['decode_us_median']:.1f} us (p10 "
            f"{row['decode_us_p10']:.1f}, p90 {row['decode_us_p90']:.1f}), "
            f"{row['frac_of_hbm_peak']:.1%} of HBM peak, parity {err:.3g} on all {B} sequences "
            f"({time.perf_counter() - t0:.1f}s)")
        del q, kc, vc, tables, lens, ks, vs, out, ws
        torch.cuda.empty_cache()
    return rows


def parity_sample(wl, out, n=4, seed=0):
    import oracle.paged_attention as pa
    rng = np.random.default_rng(seed)
    seqs = np.sort(rng.choice(wl.num_seqs, size=min(n, wl.num_seqs), replace=False))
    ref = pa.paged_decode(wl.q[seqs], wl.q_fmt, wl.key_cache, wl.value_cache, wl.kv_fmt,
                          wl.block_tables[seqs], wl.context_lens[seqs], wl.block_size, wl.scale,
                          wl.k_scales, wl.v_scales, window=wl.window)
    got = out.float().cpu().numpy().astype(np.float64)[seqs]
    return float(np.abs(got - ref).max()), seqs.tolist()


PCIE_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)


def swap_bench(args, torch, pkv, log):
    """Preemption on the 70B-shaped fp16 pool: swap 8 sequences of 2048 tokens
    out to pinned host memory and back in through the allocator's pair lists,
    and copy-on-write one partly filled block for each of 32 forked sequences.
    Prints one JSON line."""
    dev = torch.device("cuda:0")
    bs, hkv, d, n_pre, ctx = 16, 64, 128, 8, 2048
    nb = 4096                         # 2 GiB of K and V
    blocks = n_pre * ctx // bs
    nhb = blocks
    shape = (nb, bs, hkv, d)
    kc = torch.randn(shape, dtype=torch.float16, device=dev)
    vc = torch.randn(shape, dtype=torch.float16, device=dev)
    hk = torch.empty((nhb,) + shape[1:], dtype=torch.float16, pin_memory=True)
    hv = torch.empty((nhb,) + shape[1:], dtype=torch.float16, pin_memory=True)
    block_bytes = bs * hkv * d * 2
    a = pkv.BlockAllocator(nb, bs)
    a.set_free_order(np.random.default_rng(0).permutation(nb))
    a.set_host_pool(nhb)
    seqs = []
    for _ in range(n_pre):
        s = a.seq_create()
        a.seq_append_tokens(s, ctx)
        seqs.append(s)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out_us, in_us, host_us = [], [], []
    for rep in range(args.warmup + args.steps):
        t = time.perf_counter()
        out_pairs = [p for s in seqs for p in a.seq_swap_out(s)]
        t_out = time.perf_counter() - t
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        pkv.swap_blocks(kc, vc, hk, hv, out_pairs, pkv.SWAP_OUT)
        e1.record()
        t = time.perf_counter()
        in_pairs = [p for s in seqs for p in a.seq_swap_in(s)]
        t_in = time.perf_counter() - t
        pkv.swap_blocks(kc, vc, hk, hv, in_pairs, pkv.SWAP_IN)
        e2.record()
        torch.cuda.synchronize()
        if rep >= args.warmup:
            out_us.append(e0.elapsed_time(e1) * 1e3)
            in_us.append(e1.elapsed_time(e2) * 1e3)
            host_us.append((t_out + t_in) * 1e6 / 2)
    moved = 2 * blocks * block_bytes
    out_gbps = moved / (np.mean(out_us) * 1e-6) / 1e9
    in_gbps = moved / (np.mean(in_us) * 1e-6) / 1e9
    # Reference: one contiguous DMA copy of the same size each way.
    flat = kc.view(-1)[: moved // 2]
    pinned = torch.empty(moved // 2, dtype=torch.float16, pin_memory=True)
    dma = {}
    for name, fn in (("d2h", lambda: pinned.copy_(flat, non_blocking=True)),
                     ("h2d", lambda: flat.copy_(pinned, non_blocking=True))):
        fn()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(3):
            fn()
        e1.record()
        torch.cuda.synchronize()
        dma[name] = moved * 3 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # Batched copy-on-write: 32 forks of a 2056-token prompt append one token each.
    cow_a = pkv.BlockAllocator(nb, bs)
    root = cow_a.seq_create()
    cow_a.seq_append_tokens(root, 2056)
    cow_pairs = []
    for _ in range(32):
        c = cow_a.seq_fork(root)
        cow_pairs += cow_a.seq_append_tokens(c, 1)[1]
    pkv.copy_blocks(kc, vc, cow_pairs)
    # The calls are queued behind a 1 GiB copy so that the events time the
    # kernels back to back, not the host's launch rate (the binding's own
    # cost per call is larger than the kernel's).
    filler = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    filler2 = torch.empty_like(filler)
    cow_calls = 16
    e0, e1 = ev(), ev()
    pkv.stream_copy(filler2, filler)
    e0.record()
    for _ in range(cow_calls):
        pkv.copy_blocks(kc, vc, cow_pairs)
    e1.record()
    torch.cuda.synchronize()
    cow_us = e0.elapsed_time(e1) * 1e3 / cow_calls
    del filler, filler2
    log(f"swap out {np.mean(out_us):.0f} us ({out_gbps:.1f} GB/s), in {np.mean(in_us):.0f} us "
        f"({in_gbps:.1f} GB/s); DMA probe d2h {dma['d2h']:.1f} h2d {dma['h2d']:.1f} GB/s; "
        f"CoW of {len(cow_pairs)} blocks {cow_us:.1f} us")
    result = {
        "metric": "preemption swap: KV bytes moved between HBM and pinned host memory per second",
        "value": 2 * moved / ((np.mean(out_us) + np.mean(in_us)) * 1e-6),
        "unit": "B/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": (np.mean(out_us) + np.mean(in_us)) / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "swap_llama2_70b_fp16", "preempted_seqs": n_pre,
                   "tokens_per_seq": ctx, "block_size": bs, "num_kv_heads": hkv, "head_dim": d,
                   "blocks_swapped": blocks, "block_bytes_k_plus_v": 2 * block_bytes},
        "roofline": {"bound": "pcie", "achieved": (out_gbps + in_gbps) / 2, "peak": PCIE_PEAK_GBPS,
                     "unit": "GB/s", "frac": (out_gbps + in_gbps) / 2 / PCIE_PEAK_GBPS,
                     "traffic": None, "kernel": "copy_blocks_kernel"},
        "swap_out_us": float(np.mean(out_us)), "swap_in_us": float(np.mean(in_us)),
        "swap_out_gbps": out_gbps, "swap_in_gbps": in_gbps,
        "dma_probe_gbps": dma, "allocator_us_per_swap_call_set": float(np.mean(host_us)),
        "cow_blocks": len(cow_pairs), "cow_copy_us": cow_us,
        # bytes written (one K and one V block per pair); the shared source
        # block is read from cache after its first reader
        "cow_bytes_written": len(cow_pairs) * 2 * block_bytes,
        "cow_write_gbps": len(cow_pairs) * 2 * block_bytes / (cow_us * 1e-6) / 1e9,
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(result), flush=True)


def block_size_sweep(args, torch, pkv, W, log):
    """The same workload at block sizes 8, 16 and 32 ([P1] deployment section:
    smaller blocks waste less memory, larger ones cost the kernel less): decode
    time and bandwidth from HIP events, table entries read, and the internal
    fragmentation of the allocated blocks.  Prints one JSON line."""
    dev = torch.device("cuda:0")
    mb16 = W.make_structure(args.config)["tables"].shape[1]

    def up(arr, fmt):
        arr = np.ascontiguousarray(arr)
        if fmt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        if fmt == "fp8":
            return torch.from_numpy(arr.view(np.uint8)).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(arr).to(dev)

    rows = {}
    name = None
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for bs in (8, 16, 32):
        wl = W.make_workload(args.config, seed=args.seed, block_size=bs,
                             max_blocks=-(-mb16 * 16 // bs))
        name = wl.name
        q = up(wl.q, wl.q_fmt)
        kc, vc = up(wl.key_cache, wl.kv_fmt), up(wl.value_cache, wl.kv_fmt)
        tables, lens = up(wl.block_tables, "i32"), up(wl.context_lens, "i32")
        ks = up(wl.k_scales, "f32") if wl.kv_fmt in SCALED else None
        vs = up(wl.v_scales, "f32") if wl.kv_fmt in SCALED else None
        out = torch.empty_like(q)
        B, H, D = q.shape
        MB = tables.shape[1]
        part = pkv.decode_partition_size(B, H, wl.num_kv_heads, D, bs, MB, 0, wl.window)
        need = pkv.decode_workspace_size(B, H, wl.num_kv_heads, D, bs, MB, 0, wl.window)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def decode():
            pkv.paged_attention_decode(out, q, kc, vc, tables, lens, bs, wl.scale, ks, vs,
                                       workspace=ws, window=wl.window)

        for _ in range(args.warmup):
            decode()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e0, e1 in ev:
            flush.fill_(1)   # the caches start cold, outside the timed span
            e0.record()
            decode()
            e1.record()
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
        ab = algorithmic_bytes(wl)
        held = tokens = 0
        for s in range(wl.num_seqs):
            n = int(wl.context_lens[s])
            first = max(0, n - wl.window) if wl.window else 0
            held += ((n + bs - 1) // bs - first // bs) * bs
            tokens += n - first
        err, seqs = parity_sample(wl, out, n=2)
        gbps = ab["total"] / (us * 1e-6) / 1e9
        rows[bs] = {"decode_us": us, "achieved_gbps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
                    "context_tokens_per_s": ab["logical_tokens"] / (us * 1e-6),
                    "bytes_per_call": ab["total"], "partition_tokens": part,
                    "slots_allocated": held, "tokens": tokens,
                    "internal_fragmentation": (held - tokens) / held,
                    "parity": {"max_abs_err": err, "seqs": seqs, "tol": TOL[wl.kv_fmt],
                               "ok": err <= TOL[wl.kv_fmt]}}
        log(f"block size {bs}: decode {us:.1f} us ({gbps:.0f} GB/s, {gbps / HBM_PEAK_GBPS:.1%}), "
            f"internal fragmentation {(held - tokens) / held:.2%}, parity err {err:.3g}")
        del q, kc, vc, tables, lens, ks, vs, out, ws
    result = {
        "metric": "decode attention at block sizes 8/16/32: achieved HBM GB/s and internal "
                  "fragmentation of the allocated blocks",
        "value": rows[16]["achieved_gbps"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": rows[16]["decode_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "block_sizes": [8, 16, 32]},
        "sweep": {str(k): v for k, v in rows.items()},
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(result), flush=True)


def decode_kernel_names(wl, part, shared_prefix):
    """The kernels one decode call launches, joined by '+'."""
    vector = wl.kv_fmt == "f32" or wl.num_heads == wl.num_kv_heads
    if shared_prefix and wl.kv_fmt != "f32":
        if vector:
            return "paged_prefix_kernel+paged_decode_kernel+paged_decode_reduce_kernel"
        return "paged_prefix_fused_kernel+paged_decode_reduce_kernel"
    return ("paged_decode_kernel" if vector else "paged_decode_gqa_kernel") + \
        ("+paged_decode_reduce_kernel" if part else "")


def shared_prefix_sweep(args, torch, pkv, W, log):
    """The shared-prompt workload (64 sequences of 8 kv heads x 8 query heads,
    bf16, a shared prefix plus 1..512 tokens each) at prefix lengths 2000,
    8000, 16000 and 32000: decode sequence by sequence against the shared
    prefix attended once for all sequences ([P2] Prefix Cache section).
    HIP events around each call; both outputs checked against each other and
    sampled sequences against the oracle.  Prints one JSON line."""
    dev = torch.device("cuda:0")

    def up(arr, fmt):
        arr = np.ascontiguousarray(arr)
        if fmt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(arr).to(dev)

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in ev:
            flush.fill_(1)   # the caches start cold, outside the timed span
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

    rows = {}
    for prefix in (2000, 8000, 16000, 32000):
        mb = (prefix + 512) // 16 + 2
        wl = W.make_workload(4, seed=args.seed, prefix=prefix,
                             ctx=("prefix_plus_uniform", prefix, 1, 512), max_blocks=mb)
        q, kc, vc = up(wl.q, wl.q_fmt), up(wl.key_cache, wl.kv_fmt), up(wl.value_cache, wl.kv_fmt)
        tables, lens = up(wl.block_tables, "i32"), up(wl.context_lens, "i32")
        B, H, D = q.shape
        bs = wl.block_size
        groups = pkv.find_shared_prefixes(wl.block_tables, wl.context_lens, bs)
        assert groups == [(0, B, wl.shared_prefix_blocks * bs)], groups
        ws = torch.empty(max(pkv.decode_workspace_size(B, H, wl.num_kv_heads, D, bs, mb), 1),
                         dtype=torch.uint8, device=dev)
        wsp = torch.empty(pkv.decode_prefix_workspace_size(B, H, wl.num_kv_heads, D, bs, mb, groups),
                          dtype=torch.uint8, device=dev)
        plens = torch.full((B,), groups[0][2], dtype=torch.int32, device=dev)
        out, out2 = torch.empty_like(q), torch.empty_like(q)
        per_seq = timed(lambda: pkv.paged_attention_decode(out, q, kc, vc, tables, lens, bs, wl.scale,
                                                           workspace=ws))
        shared = timed(lambda: pkv.paged_attention_decode_prefix(
            out2, q, kc, vc, tables, lens, bs, wl.scale, groups, workspace=wsp, prefix_lens=plens))
        err, seqs = parity_sample(wl, out2, n=2)
        diff = float((out.float() - out2.float()).abs().max())
        ab = algorithmic_bytes(wl)
        rows[prefix] = {"per_sequence_us": per_seq, "shared_prefix_us": shared,
                        "speedup": per_seq / shared, "unique_bytes": ab["total"],
                        "logical_kv_bytes": ab["logical_kv"],
                        "shared_prefix_unique_gbps": ab["total"] / (shared * 1e-6) / 1e9,
                        "max_abs_diff_paths": diff, "parity_max_abs_err": err,
                        "parity_seqs": seqs, "tol": TOL[wl.kv_fmt]}
        log(f"prefix {prefix}: per-sequence {per_seq:.1f} us, shared prefix {shared:.1f} us "
            f"({per_seq / shared:.2f}x), paths differ by {diff:.2g}, oracle err {err:.3g}")
        del q, kc, vc, tables, lens, ws, wsp, out, out2
    result = {
        "metric": "decode of 64 sequences sharing a prompt: per-sequence against shared-prefix path",
        "value": rows[32000]["speedup"], "unit": "x (per-sequence time / shared-prefix time, "
                                                 "32000-token prefix)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": rows[32000]["shared_prefix_us"] / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "shared_prefix_gqa_bf16 at longer prefixes",
                   "prefix_tokens": list(rows)},
        "sweep": {str(k): v for k, v in rows.items()},
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1..8 (default 3: 70B-shaped fp16; 6: sliding window; "
                         "7, 8: configurations 3 and 5 with an FP8 cache)")
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition (0 = library default)")
    ap.add_argument("--per-sequence", action="store_true",
                    help="decode a shared-prefix workload sequence by sequence (default: the shared "
                         "prefix attended once for all sequences)")
    ap.add_argument("--shared-prefix-sweep", action="store_true",
                    help="measure both decode paths of the shared-prompt workload at prefix lengths "
                         "2000 .. 32000 instead")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--sweep-configs", default="1,2,3,4,5,6,7,8",
                    help="configurations measured after the headline (cold-cache median / p10 / "
                         "p90 of --sweep-calls decode calls, whole-batch parity); '' for none")
    ap.add_argument("--sweep-calls", type=int, default=100)
    ap.add_argument("--swap", action="store_true",
                    help="measure preemption instead: swap-out/in over PCIe and batched CoW copies")
    ap.add_argument("--block-size-sweep", action="store_true",
                    help="measure the decode of --config at block sizes 8, 16 and 32 instead")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the decode path runs on one GPU; the multi-GPU layout (sequences or kv "
              "heads per GPU, no collective inside attention) is not built here; use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_379_amd as pkv
    from paged_kv_cache_379_amd import workloads as W

    pkv.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.swap:
        swap_bench(args, torch, pkv, log)
        return
    if args.block_size_sweep:
        block_size_sweep(args, torch, pkv, W, log)
        return
    if args.shared_prefix_sweep:
        shared_prefix_sweep(args, torch, pkv, W, log)
        return

    t = time.perf_counter()
    wl = W.make_workload(args.config, seed=args.seed)
    log(f"workload {wl.name}: {wl.num_seqs} seqs, {wl.num_heads}/{wl.num_kv_heads} heads, "
        f"D={wl.head_dim}, {wl.kv_fmt} KV, sum ctx {int(wl.context_lens.sum())} "
        f"(drawn in {time.perf_counter() - t:.1f}s)")

    def up(arr, fmt):
        arr = np.ascontiguousarray(arr)
        if fmt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        if fmt == "fp8":
            return torch.from_numpy(arr.view(np.uint8)).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(arr).to(dev)

    q = up(wl.q, wl.q_fmt)
    kc, vc = up(wl.key_cache, wl.kv_fmt), up(wl.value_cache, wl.kv_fmt)
    tables, lens = up(wl.block_tables, "i32"), up(wl.context_lens, "i32")
    k_new, v_new = up(wl.k_new, wl.new_fmt), up(wl.v_new, wl.new_fmt)
    slots = up(wl.slot_mapping, "i32")
    ks = up(wl.k_scales, "f32") if wl.kv_fmt in SCALED else None
    vs = up(wl.v_scales, "f32") if wl.kv_fmt in SCALED else None
    out = torch.empty_like(q)
    B, H, D = q.shape
    MB = tables.shape[1]
    part = pkv.decode_partition_size(B, H, wl.num_kv_heads, D, wl.block_size, MB, args.partition,
                                     wl.window)
    need = pkv.decode_workspace_size(B, H, wl.num_kv_heads, D, wl.block_size, MB, args.partition,
                                     wl.window)
    # A workload whose sequences share a prompt's blocks is decoded with the
    # shared prefix attended once for the whole batch (unless --per-sequence);
    # the groups come from the host tables, as a scheduler would find them.
    groups = prefix_lens = None
    if wl.shared_prefix_blocks and not wl.window and not args.per_sequence:
        groups = pkv.find_shared_prefixes(wl.block_tables, wl.context_lens, wl.block_size)
        if len(groups) != 1:
            raise SystemExit(f"expected one shared-prefix group, found {groups}")
        need = pkv.decode_prefix_workspace_size(B, H, wl.num_kv_heads, D, wl.block_size, MB, groups)
        prefix_lens = torch.full((B,), groups[0][2], dtype=torch.int32, device=dev)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ab = algorithmic_bytes(wl)
    # Identical copies of the caches, used in turn: a step then finds none of
    # its K/V in the MALL or L2 that the steps before it filled, as in serving,
    # where the other layers' caches pass through between two decodes of one
    # layer.  Every copy receives every cache write, so all stay identical.
    copies = cache_copies(ab["kv"])
    sets = [(kc, vc, ks, vs)]
    for _ in range(copies - 1):
        sets.append(tuple(None if x is None else x.clone() for x in (kc, vc, ks, vs)))
    torch.cuda.synchronize()

    def write(i=0):
        kci, vci, ksi, vsi = sets[i % copies]
        pkv.reshape_and_cache(k_new, v_new, kci, vci, slots, ksi, vsi)

    def decode(i=0):
        kci, vci, ksi, vsi = sets[i % copies]
        if groups:
            pkv.paged_attention_decode_prefix(out, q, kci, vci, tables, lens, wl.block_size,
                                              wl.scale, groups, ksi, vsi, workspace=ws,
                                              prefix_lens=prefix_lens)
        else:
            pkv.paged_attention_decode(out, q, kci, vci, tables, lens, wl.block_size, wl.scale, ksi,
                                       vsi, partition_size=args.partition, workspace=ws,
                                       window=wl.window)

    for i in range(max(args.warmup, copies)):
        write(i)
        decode(i)
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps over {copies} cache copies")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        write(i)
        ev[i][1].record()
        decode(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    write_us = float(np.mean([a.elapsed_time(b) for a, b, _ in ev])) * 1e3
    decode_us = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) * 1e3
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms; decode {decode_us:.1f} us, "
        f"cache write {write_us:.1f} us")

    # Reference point: the library's own streaming copy of 1 GiB.
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    pkv.stream_copy(dst, src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        pkv.stream_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    # ... and its read-only probe with the decode's loads, over 2 GiB (past
    # the MALL): the read bandwidth a decode can reach on this GPU.
    rbytes = 2 << 30
    rsrc = torch.ones(rbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    pkv.stream_read(rsrc, sink)
    e0.record()
    for _ in range(reps):
        pkv.stream_read(rsrc, sink)
    e1.record()
    torch.cuda.synchronize()
    read_gbps = rbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del rsrc, sink

    ctx_per_step = ab["logical_tokens"]
    value = ctx_per_step * args.steps / elapsed
    achieved = ab["total"] / (decode_us * 1e-6) / 1e9
    traffic = load_traffic(wl.name, part)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "num_seqs": wl.num_seqs, "num_heads": wl.num_heads, "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "block_size": wl.block_size, "kv_dtype": wl.kv_fmt,
            "q_dtype": wl.q_fmt, "sum_context_tokens": ctx_per_step,
            "max_blocks_per_seq": MB, "num_blocks": wl.num_blocks,
            "partition_tokens": part, "seed": wl.seed, "sliding_window": wl.window,
            "shared_prefix_tokens": groups[0][2] if groups else 0,
            "decode_path": "shared-prefix" if groups else "per-sequence",
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "kernel": decode_kernel_names(wl, part, bool(groups)),
            "bytes_per_call": ab["total"], "decode_us": decode_us,
        },
        "decode_tokens_per_s": ctx_per_step / (decode_us * 1e-6),
        "cache_write_us": write_us,
        "cache_copies": copies,
        "copy_probe_gbps": copy_gbps,
        "read_probe_gbps": read_gbps,
        "decode_frac_of_read_probe": achieved / read_gbps,
        "kernel_hash": kernel_hash(),
    }
    if ab["unique_tokens"] != ab["logical_tokens"]:
        result["roofline"]["logical_bytes_per_call"] = ab["total"] - ab["kv"] + ab["logical_kv"]
        result["roofline"]["logical_gbps"] = (ab["total"] - ab["kv"] + ab["logical_kv"]) / (decode_us * 1e-6) / 1e9
    # The decode call alone from cold caches, many times: median and spread.
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    cold = time_stats(cold_call_times(torch, decode, args.sweep_calls, 10, flush), ab, wl, H)
    cold["kernel"] = result["roofline"]["kernel"]
    cold["decode_path"] = result["config"]["decode_path"]
    result["roofline"].update({k: cold[k] for k in ("decode_us_median", "decode_us_p10",
                                                     "decode_us_p90")})
    result["roofline"]["cold_calls"] = cold["calls"]
    result["token_heads_per_s"] = cold["token_heads_per_s"]
    log(f"cold calls: median {cold['decode_us_median']:.1f} us, p10 {cold['decode_us_p10']:.1f}, "
        f"p90 {cold['decode_us_p90']:.1f}")
    if not args.no_parity:
        # one more step, then compare every sequence with the oracle
        write()
        decode()
        torch.cuda.synchronize()
        import oracle.paged_attention as pa
        pa.reshape_and_cache(wl.k_new, wl.v_new, wl.new_fmt, wl.key_cache, wl.value_cache,
                             wl.kv_fmt, wl.slot_mapping, wl.block_size, wl.k_scales, wl.v_scales,
                             in_place=True)
        err, osec = parity_all(wl, out)
        tol = TOL[wl.kv_fmt]
        result["parity"] = {"max_abs_err": err, "tol": tol, "seqs": "all", "num_seqs": B,
                            "ok": err <= tol}
        cold["parity"] = dict(result["parity"], oracle_s=round(osec, 2))
        log(f"parity on all {B} sequences: max abs err {err:.3g} (tol {tol:g}, oracle {osec:.1f}s)")
        # the oracle leg below reads the caches as written (idempotent rewrite)
    sweep = [int(x) for x in args.sweep_configs.split(",") if x.strip()]
    if sweep:
        del sets, kc, vc, ks, vs
        torch.cuda.empty_cache()
        result["configs"] = config_sweep(args, torch, pkv, W, log, sweep, flush,
                                         headline=(args.config, cold) if args.seed is None else None)
    del flush
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for about {args.cpu_budget:.0f}s")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        # the GPU's rate over the oracle's, both in context tokens/s
        result["cpu_baseline"]["gpu_speedup"] = result["value"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
