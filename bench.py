"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the decode batch -- 32 sequences, seq_len ~ U[128, 2048], block
size 16, a 16384-block 32-layer bf16 pool (16 GiB each for K and V), 8 kv
heads, head_dim 128, 32 query heads.  One step is one decode step of the
serving loop, all on the device and in one launch (paged_attn_decode_append):
the slot of every sequence's new token, the write of its K/V row into the
pool, and fused paged decode attention over every cached token, the new one
included.  The same step as two calls (kv_append, then paged_attn_decode) is
timed too.
Step i works on layer i % 32 with the same tables, so consecutive steps read
disjoint memory (4.5 GB per 32-step cycle) and the 256 MB last-level cache
cannot serve repeats.

Printed: one JSON line.  `value` is decode-attention KV bytes per second of
whole-step time.  `roofline` describes the step's one kernel (timed with HIP
events on the launch stream, back to back).
`cpu_baseline` times the CPU oracle on the same decode batch.  `ops` reports
the scatter and gather rates on the prefill shape (8 x 1024 rows, 10%
padding) for reference.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode-attn KV GB/s & % HBM peak; scatter/gather GB/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(w, lens):
    """Algorithmic bytes of one decode call: every cached K and V element
    once, q and out once, the used block-table entries, lengths, offsets."""
    e = w.k_pool.element_size()
    kv = int(lens.sum()) * w.num_kv_heads * w.head_dim * e * 2
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * e
    offs = w.offsets.cpu().numpy().astype("int64")
    tables = int(((offs + lens.astype("int64") + w.block_size - 1) // w.block_size).sum()) * 4
    return kv, kv + qo + tables + 8 * w.num_seqs


def append_bytes(w):
    """Extra algorithmic bytes of the in-kernel append: each sequence's new
    K and V rows read once and written once."""
    row = w.num_kv_heads * w.head_dim * w.k_pool.element_size()
    return 2 * 2 * row * int((w.seq_lens > 0).sum())


def decode_schedule(N, w, split_req):
    """(split tokens or 0 for the balanced schedule, kernel label) of one
    paged_attn_decode call on this batch."""
    sched = N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                         w.max_seq_len, w.block_size, w.dtype, split_req)
    g = w.num_q_heads // w.num_kv_heads
    if sched == 0:
        return sched, f"decode_stream_kernel<D={w.head_dim},G={g}> (balanced schedule)"
    if sched == N.SCHEDULE_PLANNED:
        return sched, (f"decode_mfma_kernel<D={w.head_dim},G={g}> (device-planned split: pieces fit "
                       "2 workgroups per CU, merged in the kernel)")
    name = f"decode_mfma_kernel<D={w.head_dim},G={g}>"
    max_splits = -(-(w.max_seq_len + w.block_size - 1) // sched)
    if max_splits == 1:
        return sched, name + f" (split {sched}: one split per sequence)"
    if max_splits <= 16:
        return sched, name + f" (split {sched}: up to {max_splits} splits/seq, merged in the kernel)"
    return sched, name + f" + reduce_kernel (split {sched})"


def block_manager_host(N, W, steps=2000):
    """The native block manager's bookkeeping for one decode step of the
    decode batch, on the host: one new slot for each of the 32 sequences
    (append_slots) and the export of their tables, lengths and offsets for
    the kernels, called from Python through ctypes."""
    import numpy as np

    w = W.decode_batch(device="cpu", with_pools=False)
    lens = w.seq_lens.numpy()
    m = N.BlockManager(w.num_blocks, w.block_size)
    ids = np.arange(w.num_seqs, dtype=np.int64)
    for i, ln in enumerate(lens):
        assert m.allocate(i, int(ln))
    t0 = time.perf_counter()
    for _ in range(steps):
        n, _slots = m.append_slots(ids)
        if n != w.num_seqs:
            raise RuntimeError("block manager ran out of blocks")
        m.tables(ids)
    dt = time.perf_counter() - t0
    st = m.stats()
    return {"us_per_step": dt / steps * 1e6, "steps": steps, "num_seqs": w.num_seqs,
            "utilization_after": st["utilization"], "peak_used_blocks": st["peak_used"],
            "what": "append_slots for every sequence + table/length/offset export, "
                    "native manager called from Python"}


def other_decode_configs(w, N, W, reps=32):
    """Decode alone on the prefix-sharing and long-context batches, over the
    same pools (same geometry), back to back with the layer rotated."""
    import ctypes

    import torch

    out = {}
    for name in ("prefix_sharing", "long_context"):
        o = W.PRESETS[name](device=w.k_pool.device, with_pools=False)
        o.k_pool, o.v_pool = w.k_pool, w.v_pool
        lens = o.seq_lens.cpu().numpy()
        kv, alg = decode_bytes(o, lens)
        need = N.paged_attn_decode_workspace_size(o.num_seqs, o.num_kv_heads, o.num_q_heads,
                                                  o.head_dim, o.max_seq_len, o.block_size, 0)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=o.q.device)
        res = torch.empty_like(o.q)
        # arguments marshalled once, as in the timed step
        lib = N.load_library()
        pool = N.make_pool(o.k_pool, o.v_pool)
        stream = ctypes.c_void_p(torch.cuda.current_stream(o.q.device).cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        args = [(ctypes.byref(pool), l, P(o.q), o.num_q_heads, P(o.block_tables),
                 o.block_tables.shape[1], P(o.seq_lens), P(o.offsets), o.num_seqs, o.max_seq_len,
                 ctypes.c_float(o.scale), 0, P(res), P(ws), ws.numel(), stream)
                for l in range(o.num_layers)]

        def f(layer):
            if lib.paged_attn_decode(*args[layer]):
                raise RuntimeError(f"paged_attn_decode failed on {name}")

        for i in range(3):
            f(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            f(i % o.num_layers)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        sched, label = decode_schedule(N, o, 0)
        entry = {"us": us, "algorithmic_bytes": alg, "GB/s": alg / us / 1e3,
                 "frac": alg / us / 1e3 / HBM_PEAK_GBS, "kernel": label}
        if name == "prefix_sharing":
            bt = o.block_tables.cpu()
            uniq = int(torch.unique(bt[bt >= 0]).numel())
            entry["unique_kv_bytes"] = uniq * o.block_size * o.num_kv_heads * o.head_dim * 4
        out[name] = entry
        del o, ws, res
    return out


def prefill_attention(w, N, W, reps=6):
    """Prefill / append attention on the prefix-sharing batch (64 sequences
    whose first 32 blocks are shared, from a common first-block offset):
    every suffix token is a query, attending causally to the shared prefix
    and its own earlier tokens, read in place.  Over the decode batch's
    pools (same geometry), layer rotated, back to back.  Algorithmic work:
    4 * head_dim flops per (query, visible key, query head) -- QK^T and P.V
    -- against the dense bf16 matrix-core peak."""
    import ctypes

    import numpy as np
    import torch

    dev = w.q.device
    o = W.prefix_sharing(device=dev, with_pools=False)
    lens = o.seq_lens.cpu().numpy().astype(np.int64)
    prefix = int(o.meta["shared_blocks"]) * o.block_size
    counts = np.array([max(1, int(l) - prefix) for l in lens], np.int64)
    q_start = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
    rows = int(counts.sum())
    q = torch.empty((rows, o.num_q_heads, o.head_dim), dtype=o.dtype, device=dev)
    W.fill_normal_(q, 8201)
    out = torch.empty_like(q)
    # pairs (query, visible key): query i of n sits at position L - n + i
    pairs = int(sum(n * (l - n) + n * (n + 1) // 2 for n, l in zip(counts, lens)))
    flops = pairs * o.num_q_heads * 4 * o.head_dim
    lib = N.load_library()
    pool = N.make_pool(w.k_pool, w.v_pool)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [(ctypes.byref(pool), l, P(q), o.num_q_heads, P(q_start), rows, int(counts.max()),
             P(o.block_tables), o.block_tables.shape[1], P(o.seq_lens), P(o.offsets), o.num_seqs,
             ctypes.c_float(o.scale), P(out), stream) for l in range(w.num_layers)]
    if lib.paged_attn_prefill(*args[0]):
        raise RuntimeError("paged_attn_prefill failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        lib.paged_attn_prefill(*args[(i + 1) % w.num_layers])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    g = o.num_q_heads // o.num_kv_heads
    return {"query_rows": rows, "query_key_pairs": pairs, "flops": flops, "ms": ms,
            "TFLOP/s": flops / ms / 1e9, "frac_of_bf16_mfma_peak": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "kernel": f"prefill_mfma_kernel<D={o.head_dim},G={g}>"}


def int8_decode(w, N, W, reps=32):
    """Decode over an int8 pool of the decode batch's geometry (16384 blocks
    x 32 layers x 16 x 8 x 128 codes, one float32 scale per token and kv
    head), same tables, lengths, offsets and bf16 queries; back to back with
    the layer rotated.  Algorithmic bytes: every cached token's K and V
    codes and scales once, q and out (bf16) once, the used table entries,
    lengths and offsets."""
    import ctypes

    import torch

    dev = w.q.device
    shape = (w.num_blocks, w.num_layers, w.block_size, w.num_kv_heads, w.head_dim)
    k = N.QuantizedPool(*W.int8_pool_tensors(*shape, dev, 8101))
    v = N.QuantizedPool(*W.int8_pool_tensors(*shape, dev, 8102))
    lens = w.seq_lens.cpu().numpy()
    tokens = int(lens.sum())
    kv = tokens * w.num_kv_heads * (w.head_dim + 4) * 2
    _, alg_bf16 = decode_bytes(w, lens)
    kv_bf16 = tokens * w.num_kv_heads * w.head_dim * 2 * 2
    alg = alg_bf16 - kv_bf16 + kv
    split = N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                         w.max_seq_len, w.block_size, torch.int8, 0)
    need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                              w.head_dim, w.max_seq_len, w.block_size, 0)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    res = torch.empty_like(w.q)
    lib = N.load_library()
    pool = N.make_pool(k, v)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(w.block_tables),
             w.block_tables.shape[1], P(w.seq_lens), P(w.offsets), w.num_seqs, w.max_seq_len,
             ctypes.c_float(w.scale), 0, P(res), P(ws), ws.numel(), stream)
            for l in range(w.num_layers)]
    for i in range(3):
        if lib.paged_attn_decode(*args[i]):
            raise RuntimeError("int8 paged_attn_decode failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        lib.paged_attn_decode(*args[i % w.num_layers])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    g = w.num_q_heads // w.num_kv_heads
    out = {"us": us, "algorithmic_bytes": alg, "GB/s": alg / us / 1e3,
           "frac": alg / us / 1e3 / HBM_PEAK_GBS,
           "kernel": f"decode_q8_kernel<D={w.head_dim},G={g}> " + (
               "(device-planned split)" if split == N.SCHEDULE_PLANNED else f"(split {split})"),
           "kv_bytes_vs_bf16": kv / kv_bf16}
    del k, v, ws, res
    torch.cuda.empty_cache()
    return out


def read_ceiling(w, N, reps=32):
    """The measured read rate for the step's bytes: kv_read_blocks over
    every block the decode batch's tables use (the K and V layer slices, the
    bytes paged decode attention reads), back to back with the layer
    rotated.  No compute, one workgroup per block."""
    import ctypes

    import numpy as np
    import torch

    bt = w.block_tables.cpu().numpy()
    lens = w.seq_lens.cpu().numpy().astype(np.int64)
    offs = w.offsets.cpu().numpy().astype(np.int64)
    used = [bt[s, j] for s in range(w.num_seqs) if lens[s] > 0
            for j in range(offs[s] // w.block_size, (offs[s] + lens[s] - 1) // w.block_size + 1)]
    ids_np = np.unique(np.array([b for b in used if b >= 0], np.int32))
    ids = torch.from_numpy(ids_np).to(w.q.device)
    out = torch.empty(ids.numel(), dtype=torch.int32, device=w.q.device)
    lib = N.load_library()
    pool = N.make_pool(w.k_pool, w.v_pool)
    stream = ctypes.c_void_p(torch.cuda.current_stream(w.q.device).cuda_stream)
    args = [(ctypes.byref(pool), l, ctypes.c_void_p(ids.data_ptr()), ids.numel(),
             ctypes.c_void_p(out.data_ptr()), stream) for l in range(w.num_layers)]
    for i in range(3):
        if lib.kv_read_blocks(*args[i]):
            raise RuntimeError("kv_read_blocks failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        lib.kv_read_blocks(*args[i % w.num_layers])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    nbytes = int(ids.numel()) * 2 * w.block_size * w.row_bytes
    return {"blocks": int(ids.numel()), "bytes": nbytes, "us": us, "GB/s": nbytes / us / 1e3,
            "frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "kernel": "read_blocks_kernel (kv_read_blocks)",
            "what": "the K and V layer slices of every block the tables use, read and XOR-folded, "
                    f"{reps} back-to-back calls, layer rotated"}


def time_op(fn, reps, layers, warm=3):
    """Median and mean of per-call HIP-event times (ms) of fn(layer), with
    the layer rotated so repeats touch different memory."""
    import torch

    for i in range(warm):
        fn(layers[i % len(layers)])
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record()
        fn(layers[i % len(layers)])
        ends[i].record()
    torch.cuda.synchronize()
    ts = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return ts[len(ts) // 2], sum(ts) / len(ts)


def cpu_baseline(w, lens, min_seconds=10.0, layers=8):
    """The CPU oracle on the same decode batch: full decode steps over the
    first `layers` layers in rotation (distinct memory, so host caches do
    not serve repeats) until at least `min_seconds` of wall time, on all
    host threads; then one step on one thread.  Host copies of only the
    referenced blocks are made before the clock starts."""
    import numpy as np
    import torch

    import oracle as O

    bt = w.block_tables.cpu()
    ids = torch.unique(bt[bt >= 0]).to(torch.int64)
    dev_ids = ids.to(w.k_pool.device)

    def host(t):
        t = t.contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    pos = torch.searchsorted(ids, bt.clamp(min=0).to(torch.int64)).to(torch.int32)
    bt_c = torch.where(bt >= 0, pos, torch.full_like(pos, -1)).numpy()
    pools = [(host(w.k_pool[:, l].index_select(0, dev_ids).unsqueeze(1)),
              host(w.v_pool[:, l].index_select(0, dev_ids).unsqueeze(1)))
             for l in range(min(layers, w.num_layers))]
    rest = (host(w.q), bt_c, host(w.seq_lens), host(w.offsets), w.scale)
    threads = max(1, min(16, os.cpu_count() or 1))
    kv, _ = decode_bytes(w, lens)
    n = 0
    t0 = time.perf_counter()
    while True:
        k_c, v_c = pools[n % len(pools)]
        O.decode(k_c, v_c, 0, *rest, num_threads=threads)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds and n >= len(pools):
            break
    t1 = time.perf_counter()
    O.decode(pools[0][0], pools[0][1], 0, *rest, num_threads=1)
    dt1 = time.perf_counter() - t1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": kv * n / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} full decode steps of the {w.num_seqs}-sequence batch "
                      f"({int(lens.sum())} cached tokens each), layers 0-{len(pools) - 1} in "
                      f"rotation, float64 gather-then-attention, {dt:.1f} s wall",
            "seconds": dt, "single_thread_GB/s": kv / dt1 / 1e9,
            "host_cpu": model, "host_cpus_visible": os.cpu_count()}


def prefill_ops(w_dec, N, W, reps=64):
    """Scatter and gather rates on the prefill shape, run in the decode
    batch's pool (same shape: 16384 x 32 x 16 x 8 x 128 bf16).  Like the
    step, each op's C-ABI call is marshalled once and issued `reps` times
    back to back (layer rotated), one event pair around all of them; the
    median of per-call event pairs is reported beside it."""
    import ctypes

    import torch

    pf = W.prefill(device=w_dec.k_pool.device, with_pools=False)
    slots = N.kv_slot_mapping(pf.block_tables, pf.offsets, pf.token_seq, pf.token_pos,
                              pf.block_size)
    valid = int((pf.token_seq >= 0).sum())
    rows = pf.k_new.shape[0]
    row = pf.row_bytes
    layers = list(range(w_dec.num_layers))
    scat_bytes = valid * row * 2 * 2 + rows * 8
    total = int(pf.seq_lens.sum())
    k_out = torch.empty((total, pf.num_kv_heads, pf.head_dim), dtype=pf.dtype,
                        device=pf.k_new.device)
    v_out = torch.empty_like(k_out)
    starts = torch.cumsum(pf.seq_lens.to(torch.int64), 0) - pf.seq_lens.to(torch.int64)
    mx = pf.max_seq_len
    gath_bytes = total * row * 2 * 2

    lib = N.load_library()
    pool = N.make_pool(w_dec.k_pool, w_dec.v_pool)
    stream = ctypes.c_void_p(torch.cuda.current_stream(w_dec.k_pool.device).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sc_args = [(ctypes.byref(pool), l, P(pf.k_new), P(pf.v_new), P(slots), rows, stream)
               for l in layers]
    ga_args = [(ctypes.byref(pool), l, P(pf.block_tables), pf.block_tables.shape[1],
                P(pf.seq_lens), P(pf.offsets), P(starts), pf.num_seqs, mx, P(k_out), P(v_out),
                total, stream) for l in layers]

    def back_to_back(f, args):
        for i in range(3):
            if f(*args[i % len(args)]):
                raise RuntimeError("library call failed")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            f(*args[i % len(args)])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_s = back_to_back(lib.kv_scatter, sc_args)
    t_g = back_to_back(lib.kv_gather, ga_args)
    t_s_med, _ = time_op(lambda l: lib.kv_scatter(*sc_args[l]), reps, layers)
    t_g_med, _ = time_op(lambda l: lib.kv_gather(*ga_args[l]), reps, layers)
    return {
        "scatter_prefill": {"rows": rows, "valid_rows": valid, "bytes": scat_bytes,
                            "ms": t_s, "GB/s": scat_bytes / t_s / 1e6,
                            "frac": scat_bytes / t_s / 1e6 / HBM_PEAK_GBS, "bound": "hbm",
                            "per_call_events_median_ms": t_s_med},
        "gather_prefill": {"rows": total, "bytes": gath_bytes, "ms": t_g,
                           "GB/s": gath_bytes / t_g / 1e6, "frac": gath_bytes / t_g / 1e6 / HBM_PEAK_GBS,
                           "bound": "hbm", "per_call_events_median_ms": t_g_med},
        "timing": f"{reps} back-to-back C-ABI calls, layer rotated, one event pair around them",
    }


def block_ops(w_dec, N, pairs=64, sets=4, reps=32, swap_blocks=64, swap_reps=6):
    """Whole-block copies (the copy of copy-on-write) and swaps in the decode
    batch's pool: `sets` disjoint sets of `pairs` (source: a block the
    tables use, destination: one they do not), issued back to back with the
    set rotated; swap out / in of `swap_blocks` blocks to / from pinned host
    memory (runs of consecutive ids, one copy each)."""
    import ctypes

    import numpy as np
    import torch

    dev = w_dec.k_pool.device
    nb = w_dec.k_pool.shape[0]
    bt = w_dec.block_tables.cpu()
    used = torch.unique(bt[bt >= 0]).numpy()
    free = np.setdiff1d(np.arange(nb), used)
    rng = np.random.default_rng(7)
    src = rng.choice(used, size=(sets, pairs), replace=len(used) < sets * pairs)
    dst = rng.choice(free, size=(sets, pairs), replace=False)
    src_d = [torch.from_numpy(src[i].astype(np.int32)).to(dev) for i in range(sets)]
    dst_d = [torch.from_numpy(dst[i].astype(np.int32)).to(dev) for i in range(sets)]
    lib = N.load_library()
    pool = N.make_pool(w_dec.k_pool, w_dec.v_pool)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    block_bytes = w_dec.k_pool[0].numel() * w_dec.k_pool.element_size()
    args = [(ctypes.byref(pool), ctypes.c_void_p(src_d[i].data_ptr()),
             ctypes.c_void_p(dst_d[i].data_ptr()), pairs, stream) for i in range(sets)]
    for i in range(3):
        if lib.kv_copy_blocks(*args[i % sets]):
            raise RuntimeError("kv_copy_blocks failed")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        lib.kv_copy_blocks(*args[i % sets])
    b.record()
    torch.cuda.synchronize()
    t_c = a.elapsed_time(b) / reps
    copy_bytes = pairs * block_bytes * 2 * 2     # K and V, read + write

    ids = free[:swap_blocks].astype(np.int32)
    kh = torch.empty((swap_blocks,) + tuple(w_dec.k_pool.shape[1:]), dtype=w_dec.dtype,
                     pin_memory=True)
    vh = torch.empty_like(kh, pin_memory=True)
    swap_bytes = swap_blocks * block_bytes * 2

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(swap_reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / swap_reps

    t_out = timed(lambda: N.kv_swap_out(w_dec.k_pool, w_dec.v_pool, ids, kh, vh))
    t_in = timed(lambda: N.kv_swap_in(w_dec.k_pool, w_dec.v_pool, ids, kh, vh))
    return {
        "copy_blocks": {"pairs": pairs, "block_bytes_per_tensor": block_bytes,
                        "bytes": copy_bytes, "ms": t_c, "GB/s": copy_bytes / t_c / 1e6,
                        "frac": copy_bytes / t_c / 1e6 / HBM_PEAK_GBS, "bound": "hbm",
                        "timing": f"{reps} back-to-back C-ABI calls over {sets} disjoint pair "
                                  "sets, one event pair around them"},
        "swap_out": {"blocks": swap_blocks, "bytes": swap_bytes, "ms": t_out,
                     "GB/s": swap_bytes / t_out / 1e6, "host": "pinned"},
        "swap_in": {"blocks": swap_blocks, "bytes": swap_bytes, "ms": t_in,
                    "GB/s": swap_bytes / t_in / 1e6, "host": "pinned"},
    }


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_batch_traffic.json")
DECODE_SOURCES = [os.path.join(ROOT, "paged_attention_decode_scatter_amd", "csrc", f)
                  for f in ("kernels_decode.hip", "attn_common.h", "pagedkv_api.hip", "pkv_internal.h")]


def decode_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per step launch (decode with append) from the committed
    counter record, or None when the record is missing or the decode sources
    changed since."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != decode_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def pmc_target(which, reps):
    """Run only what a counter pass should see: the decode call on the
    decode batch (layer rotated), or a plain device copy of 1 GiB (the
    calibration for FETCH_SIZE / WRITE_SIZE)."""
    import torch

    from paged_attention_decode_scatter_amd import native as N
    from paged_attention_decode_scatter_amd import workloads as W

    dev = torch.device("cuda:0")
    if which == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {reps} x 1 GiB")
        return
    N.load_library()
    w = W.decode_tokens(W.decode_batch(device=dev))
    mx = w.max_seq_len
    out = torch.empty_like(w.q)
    split = 0  # the automatic schedule, as in the timed run
    ws = torch.zeros(max(16, N.paged_attn_decode_workspace_size(
        w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim, mx, w.block_size, split)),
        dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for i in range(reps):
        N.paged_attn_decode_append(w.k_pool, w.v_pool, i % w.num_layers, w.q, w.k_new, w.v_new,
                                   w.block_tables, w.seq_lens, w.offsets, mx, w.scale,
                                   split_tokens=split, out=out, workspace=ws)
    torch.cuda.synchronize()
    _, alg = decode_bytes(w, w.seq_lens.cpu().numpy())
    log(f"ran {reps} step launches (decode with append), {alg + append_bytes(w)} algorithmic "
        f"bytes each, split {split}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager calls only (no HIP graph replay)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--pmc-target", choices=["decode", "copy"], default=None,
                    help="run only the decode launches (or a 1 GiB copy) for counter passes")
    ap.add_argument("--pmc-reps", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the hot path "
              "shards by sequence or kv head with no exchange, so there is no multi-GPU "
              "measurement to make here", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    from paged_attention_decode_scatter_amd import native as N
    from paged_attention_decode_scatter_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.pmc_target:
        pmc_target(args.pmc_target, args.pmc_reps)
        return
    dev = torch.device("cuda:0")
    N.load_library()
    log("building the decode-batch workload (2 x 16 GiB pools)")
    w = W.decode_tokens(W.decode_batch(device=dev))
    lens = w.seq_lens.cpu().numpy()
    mx = w.max_seq_len
    kv_bytes, alg_bytes = decode_bytes(w, lens)
    split = args.split_tokens
    sched, kernel_label = decode_schedule(N, w, split)
    ws_bytes = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                                  w.head_dim, mx, w.block_size, split)
    workspace = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty_like(w.q)
    slots = torch.empty(w.token_seq.shape[0], dtype=torch.int64, device=dev)
    dec_start = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    dec_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    # The step issues its C-ABI call with arguments marshalled once up
    # front (the values the binding would pass), so host-side Python does
    # not starve the ~40 us device step.
    import ctypes

    lib = N.load_library()
    pool = N.make_pool(w.k_pool, w.v_pool)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    # one new K/V row per sequence (all 32 have tokens), in sequence order
    assert torch.equal(w.token_seq.cpu(), torch.arange(w.num_seqs, dtype=torch.int32))
    # the step: the new tokens' slots and writes + decode, one launch
    step_args = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(w.k_new), P(w.v_new),
                  P(w.block_tables), w.block_tables.shape[1], P(w.seq_lens), P(w.offsets),
                  w.num_seqs, mx, ctypes.c_float(w.scale), split, P(out), P(workspace),
                  workspace.numel(), stream)
                 for l in range(w.num_layers)]
    # the same step as two calls: slots + scatter (kv_append), then decode
    app_args = [(ctypes.byref(pool), l, P(w.k_new), P(w.v_new), P(w.block_tables),
                 w.block_tables.shape[1], P(w.offsets), w.num_seqs, P(w.token_seq),
                 P(w.token_pos), w.token_seq.shape[0], P(slots), stream)
                for l in range(w.num_layers)]
    dec_args = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(w.block_tables),
                 w.block_tables.shape[1], P(w.seq_lens), P(w.offsets), w.num_seqs, mx,
                 ctypes.c_float(w.scale), split, P(out), P(workspace), workspace.numel(), stream)
                for l in range(w.num_layers)]
    f_step, f_app, f_dec = lib.paged_attn_decode_append, lib.kv_append, lib.paged_attn_decode

    def step(i, timed=False):
        layer = i % w.num_layers
        if timed:
            dec_start[i].record()
        rc = f_step(*step_args[layer])
        if timed:
            dec_end[i].record()
        if rc:
            raise RuntimeError(f"a library call failed in step {i}")

    def two_call_step(i):
        layer = i % w.num_layers
        if f_app(*app_args[layer]) | f_dec(*dec_args[layer]):
            raise RuntimeError(f"a library call failed in step {i}")

    def capture(calls):
        """One HIP graph per layer holding `calls(layer, stream)`."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                cs = ctypes.c_void_p(side.cuda_stream)
                calls(i % w.num_layers, cs)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gs = []
        for layer in range(w.num_layers):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                calls(layer, ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
            gs.append(g)
        torch.cuda.synchronize()
        return gs

    def fused_calls(layer, cs):
        if f_step(*step_args[layer][:-1], cs):
            raise RuntimeError(f"paged_attn_decode_append failed while capturing layer {layer}")

    def two_calls(layer, cs):
        if f_app(*app_args[layer][:-1], cs) | f_dec(*dec_args[layer][:-1], cs):
            raise RuntimeError(f"a library call failed while capturing layer {layer}")

    def time_graphs(gs):
        for i in range(args.warmup):
            gs[i % w.num_layers].replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            gs[i % w.num_layers].replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    def time_eager(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    log(f"warmup {args.warmup} steps (split_tokens={split}, workspace={ws_bytes} B)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed steps: K calls back to back on the stream (layer rotated),
    # one event pair around all of them.
    log(f"timing {args.steps} steps")
    ms_step = time_eager(step)
    alg_step = alg_bytes + append_bytes(w)
    achieved = alg_step / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us ({achieved:.0f} GB/s algorithmic)")
    # the same calls with an event pair around each (adds per-call latency)
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    dec_ms = [s.elapsed_time(e) for s, e in zip(dec_start, dec_end)]
    dec_avg = sum(dec_ms) / len(dec_ms)
    dec_med = sorted(dec_ms)[len(dec_ms) // 2]
    # the step replayed as one HIP graph per layer
    graph_ms = None if args.no_graph else time_graphs(capture(fused_calls))
    us = lambda ms: "n/a" if ms is None else f"{ms * 1e3:.1f}"
    log(f"per-call events avg {dec_avg * 1e3:.1f} us (median {dec_med * 1e3:.1f}); graph replay "
        f"{us(graph_ms)} us")

    # The same step as two calls (append kernel, then decode), for comparison.
    two_eager = time_eager(two_call_step)
    two_graph = None if args.no_graph else time_graphs(capture(two_calls))
    log(f"two-call step: eager {us(two_eager)} us, graph {us(two_graph)} us")
    dec_b2b = ms_step
    d_start = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    # and decode alone (no append), the same way
    for i in range(3):
        f_dec(*dec_args[i % w.num_layers])
    torch.cuda.synchronize()
    d_start.record()
    for i in range(args.steps):
        f_dec(*dec_args[i % w.num_layers])
    d_end.record()
    torch.cuda.synchronize()
    dec_only = d_start.elapsed_time(d_end) / args.steps
    log(f"decode alone back to back {dec_only * 1e3:.1f} us per call")

    result = {
        "metric": METRIC,
        "value": kv_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_batch",
            "num_seqs": w.num_seqs,
            "seq_len": "U[128,2048]",
            "cached_tokens": int(lens.sum()),
            "block_size": w.block_size,
            "pool_blocks": w.num_blocks,
            "num_layers": w.num_layers,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "num_q_heads": w.num_q_heads,
            "split_tokens": sched if sched > 0 else "balanced",
            "kv_bytes_per_step": kv_bytes,
            "step": "paged_attn_decode_append: slot + write of 1 new K/V row per sequence and "
                    "paged decode attention in one launch, layer rotated over 32",
            "step_launch": "one C-ABI call per step, issued back to back",
            "graph_replay_ms_per_step": graph_ms,
            "two_call_step": {"calls": "kv_append + paged_attn_decode",
                              "ms_per_step": two_eager, "graph_replay_ms_per_step": two_graph},
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": kernel_label + ", with the new-token write",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": alg_step,
            "avg_launch_us": dec_b2b * 1e3,
            "timing": f"HIP events around the {args.steps} back-to-back step calls on the launch "
                      "stream (the timed steps themselves)",
            "decode_alone_us": dec_only * 1e3,
            "decode_alone_GBps": alg_bytes / (dec_only * 1e-3) / 1e9,
            "per_call_events_avg_us": dec_avg * 1e3,
            "per_call_events_median_us": dec_med * 1e3,
            "measured_read_ceiling": read_ceiling(w, N),
        },
    }
    if not args.no_ops:
        log("scatter/gather on the prefill shape")
        result["ops"] = prefill_ops(w, N, W)
        log("block copies and swaps")
        result["ops"].update(block_ops(w, N))
        log("decode on the prefix-sharing and long-context batches")
        result["other_decode"] = other_decode_configs(w, N, W)
        log("prefill attention on the prefix-sharing batch")
        result["prefill_attention"] = prefill_attention(w, N, W)
        log("int8 pool decode on the decode batch")
        result["int8_decode"] = int8_decode(w, N, W)
        log("host block manager")
        result["block_manager"] = block_manager_host(N, W)
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, lens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
