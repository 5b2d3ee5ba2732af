#!/usr/bin/env python3
"""Benchmark of one INT2 KV-cache decode step on one MI355X.

A step is the whole hot path for one new token per sequence: quantize-append
(rotate, evict the oldest recent token into INT2, write the ring) followed by
fused split-K decode attention over the sink, INT2 and recent segments, as
one kvq_decode_step call (--two-calls: the two separate calls).

Default workload: 28 sequences x 100000-token contexts, 32 query / 8 KV heads,
head_dim 128, sink 4, recent 256, page 16, physical pages a seeded random
permutation; one layer.  Inputs are seeded synthetic tensors drawn on the
device; the cache is built before timing (inputs resident in HBM).

Prints one JSON line: value = algorithmic bytes per step / step time (GB/s),
with the K timed steps run back to back between one pair of HIP events;
ms_per_step; a roofline object for the decode call (algorithmic bytes per
call / its average duration: K calls over the cache after the last step run
back to back as one HIP graph between two events on their stream; the
spread comes from K more calls, each between its own event pair); and the
CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT2 paged decode-attention HBM GB/s (% of peak) + µs/step at 100K ctx"
HBM_PEAK_GBS = 8000.0
HEAD_DIM = 128
INT2_BYTES = 72          # per (token, KV head): 2 x 32 code bytes + 2 x (fp16 s, fp16 z)
BF16_BYTES = 512         # per (token, KV head): 2 x 128 bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def segment_counts(L, ns, W):
    n_s = min(L, ns)
    n_i = max(0, L - W - ns)
    return n_s, n_i, L - n_s - n_i


def int2_bytes(ng=1):
    """Bytes of one INT2 (token, KV head): 2 x 32 code bytes and 2 x ng
    fp16 (scale, zero) pairs (quantization groups of 128 / ng channels)."""
    return 64 + 8 * ng


def decode_bytes(w, lens, n_query=1, ng=1):
    """Algorithmic HBM bytes of one decode launch (what the method must move);
    with n_query queries per sequence the cache is read once for all of them."""
    tot = 0
    for L in lens:
        _, n_i, _ = segment_counts(int(L), w.n_sink, w.n_recent)
        n_b = int(L) - n_i
        tot += w.n_kv_heads * (int2_bytes(ng) * n_i + BF16_BYTES * n_b)
        tot += 4 * math.ceil(int(L) / w.page_size)                  # block-table entries
    tot += w.batch * n_query * w.n_q_heads * HEAD_DIM * (2 + 4)     # q bf16 in, out fp32
    tot += 2 * w.n_kv_heads * HEAD_DIM * HEAD_DIM * 4               # R_K, R_V
    return tot


def shared_prefix_repeat_bytes(w, sharers, ng=1):
    """INT2 bytes of the shared prefix pages that every sharer after the
    first reads again (the unique bytes of a decode are decode_bytes minus
    these)."""
    if not w.shared_prefix or len(sharers) < 2:
        return 0
    return (len(sharers) - 1) * w.n_kv_heads * int2_bytes(ng) * (w.shared_prefix - w.n_sink)


def append_bytes(w, lens_before, n_new=1, ng=1):
    """Algorithmic HBM bytes of one quantize-append launch of n_new tokens
    per sequence."""
    per_vec = 256 + 256                                             # new bf16 in, ring write
    tot = 0
    for L0 in lens_before:
        for j in range(n_new):
            L = int(L0) + j
            evict = L - w.n_recent >= w.n_sink and L >= w.n_sink
            tot += w.n_kv_heads * 2 * (per_vec + ((256 + 32 + 4 * ng) if evict else 0))
    tot += 2 * w.n_kv_heads * HEAD_DIM * HEAD_DIM * 4               # R_K, R_V
    return tot


def build_cache(w, kvq2, W, lens_before, n_steps, device, quant_group=0):
    """Calibrate, allocate and fill the cache to `lens_before` tokens per sequence."""
    import numpy as np
    import torch

    t0 = time.time()
    kd = kvq2.dims(w.n_q_heads, w.n_kv_heads, w.page_size, w.n_sink, w.n_recent,
                   quant_group=quant_group, hadamard_block=quant_group)
    q_c, k_c, v_c = W.calibration_tokens(w)
    R_K, R_V, clip_K, clip_V = kvq2.calibrate(kd, q_c, k_c, v_c, 0.999)
    log(f"[bench] calibrated on {q_c.shape[0]} tokens in {time.time() - t0:.1f}s "
        f"(clip_K={clip_K:.3f}, clip_V={clip_V:.3f})")
    final = lens_before + n_steps
    bt, n_pages, _ = W.page_assignment(w, final)
    dc = kvq2.DeviceCache(kd, w.batch, n_pages, bt, device=device)
    dR_K = torch.from_numpy(R_K).to(device)
    dR_V = torch.from_numpy(R_V).to(device)
    lay = kvq2.layer(dR_K, dR_V, clip_K, clip_V)
    t0 = time.time()
    chunk = 8192
    done = np.zeros(w.batch, np.int64)
    while True:
        todo = np.minimum(lens_before - done, chunk)
        if todo.sum() == 0:
            break
        ks, vs = [], []
        for b in range(w.batch):
            if todo[b]:
                k, v = W.sequence_kv_device(w, b, int(done[b]), int(todo[b]), device)
                ks.append(k)
                vs.append(v)
        cu = np.zeros(w.batch + 1, np.int32)
        cu[1:] = np.cumsum(todo)
        kvq2.quantize_append(kd, lay, dc.handle, w.batch,
                             torch.from_numpy(done.astype(np.int32)).to(device),
                             torch.from_numpy(cu).to(device), int(cu[-1]), int(todo.max()),
                             torch.cat(ks), torch.cat(vs))
        done += todo
    torch.cuda.synchronize()
    log(f"[bench] built cache: {w.batch} x {int(lens_before.max())} tokens, {n_pages} pages "
        f"({dc.pool.numel() / 2**30:.2f} GiB pool) in {time.time() - t0:.1f}s")
    return kd, dc, lay, (dR_K, dR_V, R_K, R_V, clip_K, clip_V)


# HBM traffic of the decode kernel from rocprofv3 counters (see profiles/):
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the bench command, each
# scaled by bytes / counter measured on a plain device copy of known size
# (`bench.py --copy-probe`).  The counters are tied to a hash of the kernel
# sources; after any source change the figure is stale and reported as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_conc_28x100k_traffic.txt")
KERNEL_SOURCES = ("kvq2_decode.hip", "kvq2_decode_mfma.hip", "kvq2_decode_mfma_kernels.h",
                  "kvq2_decode_common.h", "kvq2_device.h", "kvq2_internal.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_decode_kvq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(l.split(":", 1) for l in fh.read().splitlines() if ":" in l and not l.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("workload") != workload or kv.get("source_hash") != kernel_source_hash():
            return None
        fetch = float(kv["decode_fetch_kib"]) * 1024 * float(kv["copy_fetch_bytes_per_kib"]) / 1024
        write = float(kv["decode_write_kib"]) * 1024 * float(kv["copy_write_bytes_per_kib"]) / 1024
        return fetch + write
    except (OSError, KeyError, ValueError):
        return None


def copy_probe(n_bytes=1 << 30, reps=5):
    """A plain device copy of known size, to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[copy-probe] {reps} copies of {n_bytes} bytes")


def cached_pages_probe(w, calls=50, reps=5, cached_target=1200 * 1024):
    """The decode call with its pages in HBM against the same call with every
    block-table entry pointing into the first ~1.2 MB of pages (which the
    caches then serve): the second time is what the kernels take when HBM is
    not the limit.  Each figure is the median over `reps` replays of one HIP
    graph of `calls` back-to-back decode calls.  Prints one JSON line."""
    import numpy as np
    import torch

    from long_context_decode_kvq_amd import kvq2
    from long_context_decode_kvq_amd import workloads as W

    dev = torch.device("cuda:0")
    lens = w.seq_lens()
    kd, dc, lay, keep = build_cache(w, kvq2, W, lens, 1, dev, 0)
    max_len = int(lens.max()) + 1
    ws = torch.zeros(kvq2.decode_workspace_bytes(kd, w.batch, max_len), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.batch, w.n_q_heads, HEAD_DIM), dtype=torch.float32, device=dev)
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    q = W.decode_queries_device(w, 0, dev).contiguous()

    def call(st):
        kvq2.decode_attention(kd, lay, dc.handle, w.batch, seq, max_len, q, out, ws, st)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(calls):
            call(cap)
    torch.cuda.synchronize()

    def timed():
        t = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1000.0 / calls)
        return float(np.median(t))

    t0 = time.time()
    while time.time() - t0 < 0.5:      # out of the idle power state
        graph.replay()
        torch.cuda.synchronize()
    hbm = timed()
    page_bytes = dc.pool.numel() // dc.num_pages
    n_phys = max(1, cached_target // page_bytes)
    bt = dc.block_table.clone()
    # every sequence's logical page j -> sequence 0's physical page j mod n_phys
    cols = torch.arange(bt.shape[1], device=dev) % n_phys
    dc.block_table.copy_(bt[0, :n_phys][cols].unsqueeze(0).expand(bt.shape[0], -1))
    graph.replay()
    torch.cuda.synchronize()
    cached = timed()
    dc.block_table.copy_(bt)
    torch.cuda.synchronize()
    hbm_again = timed()
    nbytes = decode_bytes(w, lens)
    print(json.dumps({
        "probe": "cached_pages", "workload": w.name, "decode_bytes": int(nbytes),
        "decode_us_hbm": round(hbm, 2), "decode_us_cached_pages": round(cached, 2),
        "decode_us_hbm_again": round(hbm_again, 2), "cached_page_bytes": int(n_phys * page_bytes),
        "timing": f"median of {reps} replays of one HIP graph of {calls} decode calls"}),
        flush=True)
    del keep


def _oracle_pair_run(w, b, h, seconds_budget, max_steps, barrier=None):
    """The CPU oracle on one (sequence b, KV head h) pair of workload w: build
    the pair's cache to L - 1 tokens (untimed), then decode steps (append one
    token + decode the G query heads) until about `seconds_budget` of timed
    work.  Single-threaded.  Host-drawn tokens of the workload's distribution
    (the same recipe as the device draw).  Returns (bytes, seconds, steps,
    build seconds)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    from long_context_decode_kvq_amd import workloads as W

    L = int(w.seq_lens()[b])
    with threadpool_limits(limits=1):
        q_c, k_c, v_c = W.calibration_tokens(w, 256)
        cal = O.calibrate(q_c[:, h * w.group:(h + 1) * w.group], k_c[:, h:h + 1], v_c[:, h:h + 1],
                          w.group, 1, 1 / math.sqrt(HEAD_DIM), 0.999)
        k, v = W.sequence_kv(w, b, L + max_steps)
        k, v = k[:, h:h + 1], v[:, h:h + 1]
        od = O.Dims(w.group, 1, w.page_size, w.n_sink, w.n_recent)
        npg = math.ceil((L + max_steps) / w.page_size)
        oc = O.OracleCache(od, 1, npg, np.arange(npg, dtype=np.int32)[None])
        t0 = time.perf_counter()
        oc.append(cal.R_K, cal.R_V, cal.clip_K, cal.clip_V, 0, 0, k[:L - 1], v[:L - 1])
        build_s = time.perf_counter() - t0
        q = W.decode_queries(w)[b:b + 1, h * w.group:(h + 1) * w.group]
        if barrier is not None:
            barrier.wait()
        timed, steps, nbytes = 0.0, 0, 0
        while steps < max_steps and timed < seconds_budget:
            t0 = time.perf_counter()
            p = L - 1 + steps
            oc.append(cal.R_K, cal.R_V, cal.clip_K, cal.clip_V, 0, p, k[p:p + 1], v[p:p + 1])
            oc.decode(cal.R_K, cal.R_V, [p + 1], q)
            timed += time.perf_counter() - t0
            _, n_i, _ = segment_counts(p + 1, w.n_sink, w.n_recent)
            nbytes += (INT2_BYTES * n_i + BF16_BYTES * (p + 1 - n_i) + w.group * HEAD_DIM * 6
                       + 2 * HEAD_DIM * HEAD_DIM * 4)
            steps += 1
    return nbytes, timed, steps, build_s


_POOL_BARRIER = None


def _pool_init(barrier):
    global _POOL_BARRIER
    _POOL_BARRIER = barrier


def _pool_task(args):
    name, b, h, budget, max_steps = args
    from long_context_decode_kvq_amd import workloads as W
    return _oracle_pair_run(W.WORKLOADS[name], b, h, budget, max_steps, _POOL_BARRIER)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class OraclePool:
    """Worker processes for the all-cores oracle leg, forked at start-up,
    before anything in this process touches the GPU (the workers only run
    NumPy).  One worker per host core, at most 16 (the host share of one GPU)."""

    def __init__(self):
        import multiprocessing as mp
        self.n = max(1, min(16, os.cpu_count() or 1))
        ctx = mp.get_context("fork")
        self.barrier = ctx.Barrier(self.n, timeout=600)
        self.pool = ctx.Pool(self.n, initializer=_pool_init, initargs=(self.barrier,))

    def run(self, w, seconds_budget, max_steps):
        # distinct (sequence, KV head) pairs, one per worker
        pairs = [(b % w.batch, (b // w.batch) % w.n_kv_heads) for b in range(self.n)]
        tasks = [(w.name, b, h, seconds_budget, max_steps) for b, h in pairs]
        res = self.pool.map_async(_pool_task, tasks, chunksize=1).get(timeout=900)
        return res

    def close(self):
        self.pool.terminate()
        self.pool.join()


def cpu_baseline(w, pool, single_s=6.0, multi_s=10.0, max_steps=400):
    """The oracle timed on the host cores: (i) one core, (ii) every worker of
    `pool` at once, one (sequence, KV head) pair each; bytes are the
    algorithmic bytes of the steps each ran."""
    nb1, t1, s1, b1 = _oracle_pair_run(w, 0, 0, single_s, max_steps)
    res = pool.run(w, multi_s, max_steps) if pool is not None else []
    single = nb1 / t1 / 1e9
    if res:
        agg = sum(r[0] for r in res) / max(r[1] for r in res) / 1e9
        steps = sum(r[2] for r in res)
        cores = len(res)
    else:
        agg, steps, cores = single, s1, 1
    L = int(w.seq_lens()[0])
    return {
        "value": agg,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{cores} worker processes at once, each one (sequence, KV head) pair of the "
                   f"workload at context ~{L}: decode steps (append 1 token + decode {w.group} "
                   f"query heads), NumPy fp64 oracle, 1 thread per worker, ~{multi_s:.0f}s timed "
                   f"per worker, {steps} steps in all (pair cache builds untimed)"),
        "single_core_value": single,
        "single_core_sample": f"one pair, {s1} steps, {t1:.1f}s timed (cache build {b1:.1f}s untimed)",
        "host_cpu_count": os.cpu_count(),
        "host_cpu_model": cpu_model(),
    }


def int2_chunk_offsets(w, bt, lens):
    """Byte offsets in the pool of every INT2 chunk the decode streams, in
    (sequence, KV head, chunk) order: the access pattern of the read probe."""
    import numpy as np
    P, Hkv = w.page_size, w.n_kv_heads
    cpp = P // 16
    out = []
    for b, L in enumerate(lens):
        int2_end = max(w.n_sink, int(L) - w.n_recent)
        c = np.arange(w.n_sink // 16, (int2_end + 15) // 16, dtype=np.int64)
        if int2_end <= w.n_sink or c.size == 0:
            continue
        pages = bt[b, (c * 16) // P].astype(np.int64)
        cip = (c * 16 % P) // 16
        for h in range(Hkv):
            out.append(((pages * Hkv + h) * cpp + cip) * 1152)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


HQMQ_METRIC = "HQMQ paged decode-attention HBM GB/s (% of peak) + µs/step"
HQMQ_TOKEN_BYTES = 192     # per (token, KV head): K and V records of 96 bytes


def hqmq_decode_bytes(w, lens, n_secondary):
    """Algorithmic HBM bytes of one HQMQ decode launch."""
    tot = sum(w.n_kv_heads * HQMQ_TOKEN_BYTES * int(L) + 4 * math.ceil(int(L) / w.page_size)
              for L in lens)
    tot += w.batch * w.n_q_heads * HEAD_DIM * (2 + 4)               # q bf16 in, out fp32
    tot += 2 * w.n_kv_heads * 24 * n_secondary * 16                 # codebooks
    return tot


def hqmq_append_bytes(w, n_new, n_secondary):
    """Algorithmic HBM bytes of one HQMQ append of n_new tokens per sequence:
    the new bf16 K and V in, their records out, the codebooks."""
    return (w.batch * n_new * w.n_kv_heads * (2 * 256 + HQMQ_TOKEN_BYTES)
            + 2 * w.n_kv_heads * 24 * n_secondary * 16)


def run_hqmq(args):
    """The HQMQ step (kvq_hqmq_append of one token per sequence, then
    kvq_hqmq_decode_attention over every position) on the workload's shape,
    timed like the INT2 step."""
    import numpy as np
    import torch

    from long_context_decode_kvq_amd import kvq2
    from long_context_decode_kvq_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    S = args.hqmq_secondary
    device = torch.device("cuda:0")
    n_steps = args.warmup + args.steps
    lens_before = w.seq_lens() - 1
    kd = kvq2.hqmq_dims(w.n_q_heads, w.n_kv_heads, w.page_size, S)
    sec = W.hqmq_secondary(8000 + w.index, w.n_kv_heads, S)
    cbs = [torch.from_numpy(np.stack([kvq2.hqmq_codebook(sec[r, h])
                                      for h in range(w.n_kv_heads)])).to(device)
           for r in range(2)]
    lay = kvq2.hqmq_layer(cbs[0], cbs[1])
    final = lens_before + n_steps
    bt, n_pages, _ = W.page_assignment(w, final)
    dc = kvq2.HqmqDeviceCache(kd, n_pages, bt, device=device)
    t0 = time.time()
    chunk = 8192
    done = np.zeros(w.batch, np.int64)
    while True:
        todo = np.minimum(lens_before - done, chunk)
        if todo.sum() == 0:
            break
        ks, vs = [], []
        for b in range(w.batch):
            if todo[b]:
                k, v = W.sequence_kv_device(w, b, int(done[b]), int(todo[b]), device)
                ks.append(k)
                vs.append(v)
        cu = np.zeros(w.batch + 1, np.int32)
        cu[1:] = np.cumsum(todo)
        kvq2.hqmq_append(kd, lay, dc.handle, w.batch,
                         torch.from_numpy(done.astype(np.int32)).to(device),
                         torch.from_numpy(cu).to(device), int(cu[-1]), int(todo.max()),
                         torch.cat(ks), torch.cat(vs), dc.append_ws)
        done += todo
    torch.cuda.synchronize()
    log(f"[bench] built HQMQ cache: {w.batch} x {int(lens_before.max())} tokens, {n_pages} pages "
        f"({dc.pool.numel() / 2**30:.2f} GiB pool) in {time.time() - t0:.1f}s")
    pool_bytes = dc.pool.numel()
    copies = 1 if pool_bytes >= 512 * 2**20 else int(math.ceil(512 * 2**20 / pool_bytes))
    pools = [dc.pool] + [dc.pool.clone() for _ in range(copies - 1)]
    handles = [dc.handle] + [kvq2.hqmq_cache(p, n_pages, dc.block_table) for p in pools[1:]]
    max_len = int(final.max())
    ws = torch.empty(kvq2.hqmq_decode_workspace_bytes(kd, w.batch, max_len), dtype=torch.uint8,
                     device=device)
    out = torch.empty((w.batch, w.n_q_heads, HEAD_DIM), dtype=torch.float32, device=device)
    cu1 = torch.arange(w.batch + 1, dtype=torch.int32, device=device)
    starts = [torch.from_numpy((lens_before + k).astype(np.int32)).to(device)
              for k in range(n_steps)]
    seqs = [torch.from_numpy((lens_before + k + 1).astype(np.int32)).to(device)
            for k in range(n_steps)]
    qs = [W.decode_queries_device(w, k, device) for k in range(n_steps)]
    new_kv = [W.sequence_kv_device(w, b, int(lens_before[b]), n_steps, device)
              for b in range(w.batch)]
    k_new = [torch.cat([new_kv[b][0][k:k + 1] for b in range(w.batch)]).contiguous()
             for k in range(n_steps)]
    v_new = [torch.cat([new_kv[b][1][k:k + 1] for b in range(w.batch)]).contiguous()
             for k in range(n_steps)]
    stream = torch.cuda.current_stream()

    def decode_call(h, seq, q, st):
        kvq2.hqmq_decode_attention(kd, lay, h, w.batch, seq, max_len, q, out, ws, st)

    def step(k, st):
        h = handles[k % copies]
        kvq2.hqmq_append(kd, lay, h, w.batch, starts[k], cu1, w.batch, 1, k_new[k], v_new[k],
                         dc.append_ws, st)
        decode_call(h, seqs[k], qs[k], st)

    for k in range(args.warmup):
        step(k, stream)
    torch.cuda.synchronize()
    graph = None
    last = args.warmup + args.steps - 1
    dgraph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(args.warmup + i, cap)
        torch.cuda.synchronize()
        # the decode call alone, K times back to back (see main())
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph, stream=cap):
            for _ in range(args.steps):
                decode_call(handles[last % copies], seqs[last], qs[last], cap)
        torch.cuda.synchronize()
    # untimed pre-warm (decode calls only read the cache)
    t_pre, n_pre = time.perf_counter(), 0
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(8):
            decode_call(handles[n_pre % copies], seqs[0], qs[0], stream)
            n_pre += 1
        torch.cuda.synchronize()
    prewarm_wall = time.perf_counter() - t_pre
    e_begin = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_begin.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i, stream)
    e_end.record(stream)
    d_begin = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    if dgraph is not None:
        d_begin.record(stream)
        dgraph.replay()
        d_end.record(stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a0, a1 in ev:
        a0.record(stream)
        decode_call(handles[last % copies], seqs[last], qs[last], stream)
        a1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e_begin.elapsed_time(e_end) / args.steps
    dec_ms = np.array([a0.elapsed_time(a1) for a0, a1 in ev])
    dec_event_avg_ms = float(np.mean(dec_ms))
    dec_avg_ms = (d_begin.elapsed_time(d_end) / args.steps if dgraph is not None
                  else dec_event_avg_ms)
    pct = {p: float(np.percentile(dec_ms, p)) * 1e3 for p in (10, 50, 90)}
    step_bytes = [hqmq_decode_bytes(w, lens_before + args.warmup + i + 1, S) +
                  hqmq_append_bytes(w, 1, S) for i in range(args.steps)]
    value = float(np.sum(step_bytes)) / (ms_per_step * 1e-3 * args.steps) / 1e9
    dec_bytes = hqmq_decode_bytes(w, lens_before + last + 1, S)
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    log(f"[bench] HQMQ step {ms_per_step * 1e3:.1f} us; decode {dec_avg_ms * 1e3:.1f} us "
        f"(p10 {pct[10]:.1f}, p50 {pct[50]:.1f}, p90 {pct[90]:.1f}); decode {achieved:.0f} GB/s "
        f"= {100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s")
    rec = {
        "metric": HQMQ_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "codec": "hqmq", "n_secondary": S,
            "batch": w.batch, "context": int(lens_before.max()) + 1,
            "context_note": "step k appends 1 token per sequence and decodes at context + k",
            "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": HEAD_DIM,
            "page_size": w.page_size, "layers": 1, "pool_copies": copies,
            "step_call": "kvq_hqmq_append + kvq_hqmq_decode_attention",
            "launch": ("host loop" if graph is None
                       else f"one HIP graph of the {args.steps} steps, replayed once"),
            "us_per_step": round(ms_per_step * 1e3, 2),
            "decode_us": round(dec_avg_ms * 1e3, 2),
            "decode_timing": ("one HIP graph of the K decode calls between two events"
                              if dgraph is not None else "an event pair around each call"),
            "decode_event_us_mean": round(dec_event_avg_ms * 1e3, 2),
            "decode_us_p10": round(pct[10], 2),
            "decode_us_p50": round(pct[50], 2),
            "decode_us_p90": round(pct[90], 2),
            "decode_bytes": int(dec_bytes),
        },
        "prewarm": {"seconds": round(prewarm_wall, 3), "decode_calls": n_pre},
        "roofline": {
            "bound": "hbm",
            "kernel": "hqmq decode",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    # After an idle spell, back-to-back calls go through a power-state
    # transient (calls 6-35 up to 30 % slower; it recurs after every idle or
    # low-duty spell, so it is not a first-touch cost).  A fixed spell of
    # untimed decode calls before the warm-up puts any --warmup/--steps
    # setting in the sustained state; it is reported on its own.
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed back-to-back decode calls before the warm-up")
    ap.add_argument("--workload", default="conc_28x100k")
    ap.add_argument("--n-query", type=int, default=1,
                    help="queries per sequence and step: M > 1 times multi-query attention "
                         "(kvq_quantize_append of M tokens + kvq_decode_multi_attention)")
    ap.add_argument("--quant-group", type=int, default=0, choices=(0, 32, 64, 128),
                    help="channels per (scale, zero) pair (0 = 128); narrower groups also "
                         "use a Hadamard of the same block size and run on the VALU decode")
    ap.add_argument("--codec", default="int2", choices=("int2", "hqmq"),
                    help="int2: the OSCAR-style INT2 cache (default); hqmq: the HQMQ codec "
                         "(quaternion product codebook, Med3x fp16 chunks) on the same shape")
    ap.add_argument("--hqmq-secondary", type=int, default=10,
                    help="secondary quaternions S of the HQMQ codebook (24 S words)")
    ap.add_argument("--prefix-aware", action="store_true",
                    help="decode a workload with a shared prefix through "
                         "kvq_decode_prefix_attention (the sharers as one group)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the read-ceiling probes")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps from the host one by one instead of replaying "
                         "them as one captured HIP graph")
    ap.add_argument("--two-calls", action="store_true",
                    help="run each step as kvq_quantize_append + kvq_decode_attention instead "
                         "of one kvq_decode_step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--cached-pages-probe", action="store_true",
                    help="only time the decode call of --workload with its pages in HBM and "
                         "again with every block-table entry remapped into ~1.2 MB of pages")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the decode kernel source hash and exit")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(one process, one MI355X). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.codec == "hqmq":
        run_hqmq(args)
        return

    # the oracle's worker processes are forked before this process touches the GPU
    # (the oracle leg times the one-query decode step; multi-query lines go without it)
    pool = None
    if (not args.no_cpu_baseline and not args.copy_probe and not args.cached_pages_probe
            and args.n_query == 1
            and args.quant_group in (0, 128)):
        pool = OraclePool()

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe()
        return
    if args.cached_pages_probe:
        from long_context_decode_kvq_amd import workloads as W
        cached_pages_probe(W.WORKLOADS[args.workload])
        return

    from long_context_decode_kvq_amd import kvq2
    from long_context_decode_kvq_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    device = torch.device("cuda:0")
    n_steps = args.warmup + args.steps
    M = args.n_query
    lens_before = w.seq_lens() - M               # the first step appends tokens L-M .. L-1
    qg = args.quant_group
    ng = HEAD_DIM // (qg or HEAD_DIM)
    kd, dc, lay, keep = build_cache(w, kvq2, W, lens_before, n_steps * M, device, qg)

    # Small caches would be served from the 256 MB Infinity Cache: rotate
    # independent pool copies so every step reads its pages from HBM.
    pool_bytes = dc.pool.numel()
    copies = 1 if pool_bytes >= 512 * 2**20 else int(math.ceil(512 * 2**20 / pool_bytes))
    pools = [dc.pool] + [dc.pool.clone() for _ in range(copies - 1)]
    handles = [dc.handle] + [kvq2.cache(p, dc.num_pages, dc.sink if w.n_sink > 0 else None,
                                        dc.recent, dc.block_table) for p in pools[1:]]

    max_len = int(lens_before.max()) + n_steps * M
    # --prefix-aware: the sequences sharing the prefix pages form one group
    _, _, sharers = W.page_assignment(w, lens_before + n_steps * M)
    prefix = args.prefix_aware and bool(w.shared_prefix) and M == 1 and ng == 1
    if args.prefix_aware and not prefix:
        raise SystemExit("--prefix-aware needs a workload with a shared prefix, one query per "
                         "sequence and 128-channel quantization groups")
    groups = group_tensors = None
    if prefix:
        group_tensors = [torch.tensor(x, dtype=torch.int32, device=device)
                         for x in ([0, len(sharers)], sharers, [w.shared_prefix])]
        groups = kvq2.prefix_groups(len(sharers), *group_tensors)
        ws_bytes = kvq2.decode_prefix_workspace_bytes(kd, w.batch, max_len, groups)
    else:
        ws_bytes = kvq2.decode_multi_workspace_bytes(kd, w.batch, max_len, M)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=device)
    out = torch.empty((w.batch, M, w.n_q_heads, HEAD_DIM), dtype=torch.float32, device=device)
    cu1 = torch.arange(w.batch + 1, dtype=torch.int32, device=device) * M
    starts = [torch.from_numpy((lens_before + k * M).astype(np.int32)).to(device)
              for k in range(n_steps)]
    seqs = [torch.from_numpy((lens_before + (k + 1) * M).astype(np.int32)).to(device)
            for k in range(n_steps)]
    seq0 = torch.from_numpy(lens_before.astype(np.int32)).to(device)
    # queries [B][M][Hq][128] of step k (M draws of the step's query generator)
    qs = [torch.stack([W.decode_queries_device(w, k * M + j, device) for j in range(M)], 1)
          .contiguous() for k in range(n_steps)]
    new_kv = [W.sequence_kv_device(w, b, int(lens_before[b]), n_steps * M, device)
              for b in range(w.batch)]
    k_new = [torch.cat([new_kv[b][0][k * M:(k + 1) * M] for b in range(w.batch)]).contiguous()
             for k in range(n_steps)]
    v_new = [torch.cat([new_kv[b][1][k * M:(k + 1) * M] for b in range(w.batch)]).contiguous()
             for k in range(n_steps)]
    stream = torch.cuda.current_stream()

    def decode_call(h, seq, q, st):
        if prefix:
            kvq2.decode_prefix_attention(kd, lay, h, w.batch, seq, max_len, q, out, groups, ws, st)
        elif M == 1:
            kvq2.decode_attention(kd, lay, h, w.batch, seq, max_len, q, out, ws, st)
        else:
            kvq2.decode_multi_attention(kd, lay, h, w.batch, seq, max_len, M, q, out, ws, st)

    def step(k, st):
        h = handles[k % copies]
        if M > 1 or prefix:
            kvq2.quantize_append(kd, lay, h, w.batch, starts[k], cu1, w.batch * M, M, k_new[k],
                                 v_new[k], st)
            decode_call(h, seqs[k], qs[k], st)
        elif args.two_calls:
            kvq2.quantize_append(kd, lay, h, w.batch, starts[k], cu1, w.batch, 1, k_new[k],
                                 v_new[k], st)
            kvq2.decode_attention(kd, lay, h, w.batch, seqs[k], max_len, qs[k], out, ws, st)
        else:
            kvq2.decode_step(kd, lay, h, w.batch, starts[k], cu1, w.batch, 1, k_new[k], v_new[k],
                             seqs[k], max_len, qs[k], out, ws, st)

    for k in range(args.warmup):
        step(k, stream)
    torch.cuda.synchronize()
    # The K timed steps, captured as one HIP graph (replayed once below): a
    # serving loop launches its decode step that way, and at batch 1 the
    # per-call host cost of launching from Python exceeds the GPU time.
    graph = None
    last = args.warmup + args.steps - 1
    dgraph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(args.warmup + i, cap)
        torch.cuda.synchronize()
        # the decode call alone, K times back to back over the cache after
        # the last step: one graph, timed by one event pair (an event pair
        # around each call adds its own GPU time, ~10 us per call)
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph, stream=cap):
            for _ in range(args.steps):
                decode_call(handles[last % copies], seqs[last], qs[last], cap)
        torch.cuda.synchronize()

    # ---- untimed pre-warm: back-to-back decode calls over the cache (whose
    # contents they only read), at most two groups of ~10 ms queued so that
    # the host stays just ahead of the GPU.
    def pre_call(i):
        decode_call(handles[i % copies], seq0, qs[0], stream)

    pre_call(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pre_call(1)
    torch.cuda.synchronize()
    est_s = max(time.perf_counter() - t0, 1e-5)
    group = max(1, int(0.010 / est_s))
    n_pre, marks = 2, []
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(group):
            pre_call(n_pre)
            n_pre += 1
        e = torch.cuda.Event()
        e.record(stream)
        marks.append(e)
        if len(marks) > 2:
            marks.pop(0).synchronize()
    prewarm_wall = time.perf_counter() - t_pre
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back, one event pair around them
    # (an event recorded between kernels costs ~5 us of GPU time per event).
    e_begin = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_begin.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i, stream)
    e_end.record(stream)
    # The decode call on its own, for the roofline, queued behind the timed
    # steps (no idle gap: the GPU stays in its sustained-load state): K calls
    # over the cache after the last step as one graph between two events on
    # the stream they run on (the average), then K calls each bracketed by
    # its own event pair (the spread; those times include the events' cost).
    d_begin = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    if dgraph is not None:
        d_begin.record(stream)
        dgraph.replay()
        d_end.record(stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a0, a1 in ev:
        a0.record(stream)
        decode_call(handles[last % copies], seqs[last], qs[last], stream)
        a1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e_begin.elapsed_time(e_end) / args.steps
    dec_ms = np.array([a0.elapsed_time(a1) for a0, a1 in ev])
    dec_event_avg_ms = float(np.mean(dec_ms))
    dec_avg_ms = (d_begin.elapsed_time(d_end) / args.steps if dgraph is not None
                  else dec_event_avg_ms)
    pct = {p: float(np.percentile(dec_ms, p)) * 1e3 for p in (10, 50, 90)}

    step_bytes = []
    for i in range(args.steps):
        lb = lens_before + (args.warmup + i) * M
        step_bytes.append(decode_bytes(w, lb + M, M, ng) + append_bytes(w, lb, M, ng))
    value = float(np.sum(step_bytes)) / (ms_per_step * 1e-3 * args.steps) / 1e9
    dec_bytes = decode_bytes(w, lens_before + (last + 1) * M, M, ng)
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    # A shared prefix is read by every sharer (its pages are then mostly
    # served from the Infinity Cache) unless the decode is prefix-aware
    # (then once per row set of four sharers): achieved counts the bytes
    # every sequence attends to, unique counts each physical page once.
    dec_unique = dec_bytes - shared_prefix_repeat_bytes(w, sharers, ng)
    log(f"[bench] pre-warm {n_pre} decode calls in {prewarm_wall:.2f}s; step "
        f"{ms_per_step * 1e3:.1f} us; decode {dec_avg_ms * 1e3:.1f} us (each call between "
        f"events: mean {dec_event_avg_ms * 1e3:.1f}, p10 {pct[10]:.1f}, p50 {pct[50]:.1f}, "
        f"p90 {pct[90]:.1f}); decode {achieved:.0f} GB/s = "
        f"{100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s")

    ceiling = None
    if not args.no_probes:
        ceiling = read_ceilings(w, kvq2, dc, pools, lens_before + (last + 1) * M, stream, achieved,
                                chunk_probe=(ng == 1))

    cpu = None
    if pool is not None:
        t0 = time.time()
        cpu = cpu_baseline(w, pool)
        pool.close()
        log(f"[bench] cpu baseline {cpu['value']:.4f} GB/s on {cpu['cores']} cores "
            f"({cpu['single_core_value']:.4f} GB/s on one) in {time.time() - t0:.1f}s")

    # narrower quantization groups always decode on the VALU kernel
    kernel = os.environ.get("KVQ_DECODE_KERNEL", "mfma") if ng == 1 else "valu"
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # products on the f16 matrix cores (INT2 codes exact, q' and the
        # softmax weights as f16 hi + lo pairs), fp32 accumulation, softmax
        # and combine
        "dtype": "f16/f32" if kernel == "mfma" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "context": int(lens_before.max()) + M,
            "context_note": (f"step k appends {M} token(s) per sequence and decodes at context "
                             f"+ {M} k"),
            "n_query": M,
            "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": HEAD_DIM,
            "page_size": w.page_size, "n_sink": w.n_sink, "n_recent": w.n_recent,
            "layers": 1, "decode_kernel": kernel, "pool_copies": copies,
            "quant_group": qg or HEAD_DIM,
            "step_call": ("kvq_quantize_append + kvq_decode_prefix_attention" if prefix else
                          "kvq_quantize_append + kvq_decode_multi_attention" if M > 1 else
                          "kvq_quantize_append + kvq_decode_attention" if args.two_calls
                          else "kvq_decode_step"),
            "launch": ("host loop" if graph is None
                       else f"one HIP graph of the {args.steps} steps, replayed once"),
            "us_per_step": round(ms_per_step * 1e3, 2),
            "decode_us": round(dec_avg_ms * 1e3, 2),
            "decode_timing": ("one HIP graph of the K decode calls between two events"
                              if dgraph is not None else "an event pair around each call"),
            "decode_event_us_mean": round(dec_event_avg_ms * 1e3, 2),
            "decode_us_p10": round(pct[10], 2),
            "decode_us_p50": round(pct[50], 2),
            "decode_us_p90": round(pct[90], 2),
            "decode_us_pct_note": "p10/p50/p90 of the calls bracketed each by its own event pair",
            "step_pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "decode_bytes": int(dec_bytes),
        },
        "prewarm": {
            "seconds": round(prewarm_wall, 3),
            "decode_calls": n_pre,
            "note": "untimed back-to-back decode calls before the warm-up steps (power-state "
                    "transient after an idle spell)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name),
        },
        "read_ceiling": ceiling,
        "shared_prefix": None if not w.shared_prefix else {
            "tokens": w.shared_prefix,
            "sharers": len(sharers),
            "decode_unique_bytes": int(dec_unique),
            "decode_unique_gbs": round(dec_unique / (dec_avg_ms * 1e-3) / 1e9, 1),
            "decode_effective_gbs": round(achieved, 1),
            "prefix_aware": prefix,
            "note": ("the sharers form one group of kvq_decode_prefix_attention: the prefix "
                     "tiles are read once per row set of four sharers" if prefix else
                     "every sharer reads the shared prefix pages") +
                    "; effective counts what every sequence attends to, unique each page once",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def read_ceilings(w, kvq2, dc, pools, lens, stream, achieved, reps=5, chunk_probe=True):
    """What plain reads reach on this GPU (include/kvq2_probe.h): a 2 GiB
    sequential pass, and the decode's own 1152-byte INT2 chunks in the order
    it streams them (pool copies rotated as in the timed steps).  Median of
    `reps` launches each, timed with HIP events on the launch stream.  The
    chunk probe reads 1152-byte chunks (quantization groups of 128 only)."""
    import numpy as np
    import torch

    dev = dc.pool.device
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    t_stream = []
    for _ in range(reps):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        kvq2.probe_stream_read(buf, sink, 8192, stream)
        a1.record(stream)
        t_stream.append((a0, a1))
    offs_np = (int2_chunk_offsets(w, dc.block_table.cpu().numpy(), lens) if chunk_probe
               else np.zeros(0, np.int64))
    t_chunk = []
    if offs_np.size:
        offs = torch.from_numpy(offs_np).to(dev)
        for i in range(reps):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            kvq2.probe_chunk_read(pools[i % len(pools)], offs, sink, 2048, stream)
            a1.record(stream)
            t_chunk.append((a0, a1))
    torch.cuda.synchronize()
    del buf
    ms = lambda ev: float(np.median([a.elapsed_time(b) for a, b in ev]))
    stream_gbs = (2 << 30) / (ms(t_stream) * 1e-3) / 1e9
    rec = {"unit": "GB/s", "stream_read": round(stream_gbs, 1),
           "stream_read_bytes": 2 << 30,
           "decode_frac_of_stream_read": round(achieved / stream_gbs, 4)}
    if t_chunk:
        chunk_gbs = offs_np.size * 1152 / (ms(t_chunk) * 1e-3) / 1e9
        rec.update({"int2_chunk_read": round(chunk_gbs, 1),
                    "int2_chunk_bytes": int(offs_np.size * 1152),
                    "decode_frac_of_int2_chunk_read": round(achieved / chunk_gbs, 4)})
    log(f"[bench] read ceilings: {rec}")
    return rec


if __name__ == "__main__":
    main()
