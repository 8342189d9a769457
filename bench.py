"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one decode step of the serving loop, all on the device in one
C-ABI call (paged_attn_decode_append): the slot of every sequence's new
token, the write of its K/V row into the pool, and fused paged decode
attention over every cached token, the new one included.  The pool is
16384 blocks x 32 layers x block size 16 x 8 kv heads x head_dim 128, bf16
(16 GiB each for K and V); step i works on layer i % 32 with the same
tables, so consecutive steps read disjoint memory and the 256 MB last-level
cache cannot serve repeats.

Headline workload: the long-context batch, 8 sequences x 32768 tokens (the
whole 262,144-token pool), 64 query heads (8 per kv head), randomly
permuted block tables.  The decode batch (32 sequences, U[128, 2048]
tokens, 32 query heads) and the prefix-sharing batch (64 sequences sharing a
512-token prefix from a nonzero first-block offset, up to 4096 tokens) are
timed the same way, each in its own block of `decode_configs`.

Printed: one JSON line.  `value` is the headline step's KV bytes per second
of step time.  `roofline` describes the headline step (HIP events on the
launch stream around the back-to-back timed steps).  `cpu_baseline` times
the CPU oracle on the headline batch.  `ops` reports the scatter and gather
rates on the prefill shape (8 x 1024 rows, 10% padding), block copies and
swaps; `prefill_attention`, `int8_decode`, `int4_decode` and
`block_manager` the other entry points.
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
    """(split tokens or SCHEDULE_PLANNED, kernel label) of one
    paged_attn_decode call on this batch."""
    sched = N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                         w.max_seq_len, w.block_size, w.dtype, split_req)
    g = w.num_q_heads // w.num_kv_heads
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


def prefill_setup(w, N, W):
    """Arguments of paged_attn_prefill on the prefix-sharing batch over the
    pools of `w`, one tuple per layer, and the workload's size."""
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
    pool = N.make_pool(w.k_pool, w.v_pool)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [(ctypes.byref(pool), l, P(q), o.num_q_heads, P(q_start), rows, int(counts.max()),
             P(o.block_tables), o.block_tables.shape[1], P(o.seq_lens), P(o.offsets), o.num_seqs,
             ctypes.c_float(o.scale), P(out), stream) for l in range(w.num_layers)]
    keep = (o, q, q_start, out, pool)
    g = o.num_q_heads // o.num_kv_heads
    info = {"query_rows": rows, "query_key_pairs": pairs, "flops": flops,
            "kernel": f"prefill_mfma_kernel<D={o.head_dim},G={g}>"}
    return args, info, keep


def prefill_attention(w, N, W, reps=4):
    """Prefill / append attention on the prefix-sharing batch (64 sequences
    whose first 32 blocks are shared, from a common first-block offset):
    every suffix token is a query, attending causally to the shared prefix
    and its own earlier tokens, read in place.  Over the decode batch's
    pools (same geometry), layer rotated, back to back.  Algorithmic work:
    4 * head_dim flops per (query, visible key, query head) -- QK^T and P.V
    -- against the dense bf16 matrix-core peak."""
    import torch

    import numpy as np

    lib = N.load_library()
    args, info, keep = prefill_setup(w, N, W)
    for i in range(3):
        if lib.paged_attn_prefill(*args[i]):
            raise RuntimeError("paged_attn_prefill failed")
    # blocks of `reps` back-to-back calls (layer rotated), one event pair
    # around each block; the median block
    blocks = []
    for blk in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            lib.paged_attn_prefill(*args[(3 + blk * reps + i) % len(args)])
        b.record()
        torch.cuda.synchronize()
        blocks.append(a.elapsed_time(b) / reps)
    ms = float(np.median(blocks))
    flops = info["flops"]
    return dict(info, ms=ms, ms_blocks=blocks,
                timing=f"3 warm-up calls, then 5 blocks of {reps} back-to-back calls (layer rotated), "
                       "one event pair per block, median block",
                **{"TFLOP/s": flops / ms / 1e9, "frac_of_bf16_mfma_peak": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS})


def quant_decode(base, N, W, bits=8, reps=32):
    """Decode over a quantised pool of the decode workloads' geometry (16384
    blocks x 32 layers x 16 x 8 x 128 codes; int8: one byte per element,
    int4: two elements per byte; one float32 scale per token and kv head)
    with each workload's tables, lengths, offsets and bf16 queries: decode
    alone, and the step (paged_attn_decode_append); blocks of `reps` back-to-
    back calls with the layer rotated, the two in turn, the upper median of
    4 blocks each.  Algorithmic bytes: every cached token's K and V codes
    and scales once, q and out (bf16) once, the used table entries, lengths
    and offsets."""
    import copy
    import ctypes

    import torch

    dev = base.q.device
    shape = (base.num_blocks, base.num_layers, base.block_size, base.num_kv_heads, base.head_dim)
    k, v = quant_pools(W, N, shape, dev, bits)
    lib = N.load_library()
    pool = N.make_pool(k, v)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    res = {}
    for name in DECODE_CONFIGS:
        w = base if name == "decode_batch" else W.PRESETS[name](device=dev, with_pools=False)
        w = copy.copy(w)
        w.k_pool, w.v_pool = base.k_pool, base.v_pool   # bf16 geometry for decode_bytes
        lens = w.seq_lens.cpu().numpy()
        tokens = int(lens.sum())
        kv = tokens * w.num_kv_heads * (w.head_dim * bits // 8 + 4) * 2
        kv_bf16, alg_bf16 = decode_bytes(w, lens)
        alg = alg_bf16 - kv_bf16 + kv
        sched = N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                             w.max_seq_len, w.block_size,
                                             torch.int8 if bits == 8 else torch.uint8, 0)
        need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                                  w.head_dim, w.max_seq_len, w.block_size, 0)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
        out = torch.empty_like(w.q)
        args = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(w.block_tables),
                 w.block_tables.shape[1], P(w.seq_lens), P(w.offsets), w.num_seqs, w.max_seq_len,
                 ctypes.c_float(w.scale), 0, P(out), P(ws), ws.numel(), stream)
                for l in range(w.num_layers)]
        # the step: paged_attn_decode_append (the quantising append of each
        # sequence's new row at position len - 1, then decode)
        kn = torch.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        W.fill_normal_(kn, 8103)
        vn = kn.flip(0).contiguous()
        sargs = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(kn), P(vn), P(w.block_tables),
                  w.block_tables.shape[1], P(w.seq_lens), P(w.offsets), w.num_seqs, w.max_seq_len,
                  ctypes.c_float(w.scale), 0, P(out), P(ws), ws.numel(), stream)
                 for l in range(w.num_layers)]
        # three untimed passes over the layers (the quantised pools are
        # freshly filled: the first passes run slower), one of the step,
        # then blocks of decode and of the step in turn; medians of blocks
        for i in range(3 * w.num_layers):
            if lib.paged_attn_decode(*args[i % w.num_layers]):
                raise RuntimeError(f"int{bits} paged_attn_decode failed on {name}")
        for i in range(w.num_layers):
            if lib.paged_attn_decode_append(*sargs[i]):
                raise RuntimeError(f"int{bits} paged_attn_decode_append failed on {name}")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        blocks = {"decode": [], "step": []}
        for _ in range(4):
            for kind, f, fa in (("decode", lib.paged_attn_decode, args),
                                ("step", lib.paged_attn_decode_append, sargs)):
                torch.cuda.synchronize()
                a.record()
                for i in range(reps):
                    f(*fa[i % w.num_layers])
                b.record()
                torch.cuda.synchronize()
                blocks[kind].append(a.elapsed_time(b) / reps * 1e3)
        us = sorted(blocks["decode"])[2]
        step_us = sorted(blocks["step"])[2]
        g = w.num_q_heads // w.num_kv_heads
        max_splits = -(-(w.max_seq_len + w.block_size - 1) // max(sched, 1))
        label = f"decode_q8_kernel<D={w.head_dim},G={g},QB={bits}> " + (
            "(device-planned split)" if sched == N.SCHEDULE_PLANNED else
            f"(split {sched}" + (", + reduce_kernel)" if max_splits > 16 else ")"))
        res[name] = {"us": us, "algorithmic_bytes": alg, "GB/s": alg / us / 1e3,
                     "frac": alg / us / 1e3 / HBM_PEAK_GBS, "kernel": label,
                     "kv_bytes_vs_bf16": kv / kv_bf16,
                     "step_us": step_us,
                     "step": "paged_attn_decode_append: scatter_q8_kernel (decode-step mode) then decode"}
        del ws, out, kn, vn
    del k, v, pool
    torch.cuda.empty_cache()
    return res


def quant_pools(W, N, shape, dev, bits):
    """K and V QuantizedPools of `shape` (random codes and positive scales),
    int8 or packed int4."""
    make = W.int8_pool_tensors if bits == 8 else W.int4_pool_tensors
    return (N.QuantizedPool(*make(*shape, dev, 8101)),
            N.QuantizedPool(*make(*shape, dev, 8102)))


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


def cpu_baseline(w, lens, min_seconds=10.0, layers=2):
    """The CPU oracle on the same batch: full decode steps over the first
    `layers` layers in rotation (each layer's K/V is far larger than the
    host caches) until at least `min_seconds` of wall time, on all host
    threads; then one step on one thread.  Host copies of only the
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
            "sample": f"{n} full decode steps of the {w.name} batch ({w.num_seqs} sequences, "
                      f"{w.num_q_heads} q heads, "
                      f"{int(lens.sum())} cached tokens each), layers 0-{len(pools) - 1} in "
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


# the files that decide the decode kernels' code: their sources and the
# build (which compiles part of them with their own flags)
DECODE_SOURCES = [os.path.join(ROOT, "paged_attention_decode_scatter_amd", "csrc", f)
                  for f in ("kernels_decode.hip", "attn_common.h", "pagedkv_api.hip", "pkv_internal.h")] + [
    os.path.join(ROOT, "paged_attention_decode_scatter_amd", "build.py")]


def torch_context(w, W, reps=3):
    """The pages' own PyTorch forms on the same GPU, for context only (they
    are not the library's path): over the decode batch, P1's per-block
    loop-and-cat gather and its flattened advanced-index gather of every
    sequence's K and V, each followed by standard attention (torch's
    scaled_dot_product_attention per sequence, kv heads repeated for the
    query groups, in float32: bf16 batched products on a transposed operand
    have faulted on these GPUs); and P1's index-put scatter of the prefill
    shape's rows at slots computed with the slot formula.  Medians of `reps`
    runs, each bracketed by device synchronisations; tables, lengths and
    offsets are host lists, as the loop form reads them."""
    import time

    import torch
    import torch.nn.functional as F

    dev = w.k_pool.device
    bs, layer = w.block_size, w.layer
    bt = w.block_tables.cpu().tolist()
    lens = w.seq_lens.cpu().tolist()
    offs = w.offsets.cpu().tolist()
    G = w.num_q_heads // w.num_kv_heads

    def gather_loop_cat(pool, s):
        out, off, left = [], offs[s], lens[s]
        for j, b in enumerate(bt[s]):
            if left <= 0:
                break
            start = off if j == 0 else 0
            take = min(bs - start, left)
            out.append(pool[b, layer, start:start + take])
            left -= take
        return torch.cat(out) if out else pool[0, layer, :0]

    bt_d = w.block_tables.to(torch.int64)

    def gather_index(pool, s):
        p = offs[s] + torch.arange(lens[s], device=dev)
        return pool[bt_d[s, p // bs], layer, p % bs]

    def attend(s, k, v):
        q = w.q[s].float().unsqueeze(0).unsqueeze(2)                       # (1, Hq, 1, D)
        kk = k.float().permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        vv = v.float().permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        return F.scaled_dot_product_attention(q, kk, vv, scale=w.scale)

    def timed(fn):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2] * 1e3

    live = [s for s in range(w.num_seqs) if lens[s] > 0]
    res = {}
    first = {}
    for name, g in (("loop_cat", gather_loop_cat), ("index", gather_index)):
        kv = {}

        def gather_all():
            for s in live:
                kv[s] = (g(w.k_pool, s), g(w.v_pool, s))

        gather_all()
        first[name] = dict(kv)
        res[f"gather_{name}_ms"] = timed(gather_all)
        res[f"gather_{name}_then_attention_ms"] = timed(lambda: [attend(s, *g_kv) for s in live
                                                             for g_kv in [(g(w.k_pool, s), g(w.v_pool, s))]])
    res["attention_only_ms"] = timed(lambda: [attend(s, *kv[s]) for s in live])
    res["gathers_agree"] = all(torch.equal(first["loop_cat"][s][i], first["index"][s][i])
                               for s in live for i in (0, 1))
    del first
    # index-put scatter on the prefill shape (8 x 1024 rows, 10 % padding)
    pf = W.prefill(device=dev, with_pools=False)
    seq = pf.token_seq.to(torch.int64)
    valid = seq >= 0
    p = pf.offsets.to(torch.int64)[seq.clamp(min=0)] + pf.token_pos.to(torch.int64)
    blk = pf.block_tables.to(torch.int64)[seq.clamp(min=0), p // bs]
    slot = torch.where(valid, blk * bs + p % bs, torch.full_like(blk, -1))
    m = slot >= 0
    rows_k, rows_v, sl = pf.k_new[m], pf.v_new[m], slot[m]
    lay = [0]

    def scatter():
        l = lay[0] = (lay[0] + 1) % w.num_layers
        w.k_pool[sl // bs, l, sl % bs] = rows_k
        w.v_pool[sl // bs, l, sl % bs] = rows_v

    scatter()
    res["scatter_index_put_ms"] = timed(scatter)
    res["what"] = ("the pages' PyTorch forms on this GPU, context only: loop-and-cat and flattened-index gather of "
                   f"all {len(live)} decode-batch sequences (K and V), attention by torch SDPA per sequence in "
                   f"float32, and index-put scatter of the prefill shape's rows; medians of {reps} synchronised runs")
    return res


def decode_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(name):
    return os.path.join(ROOT, "profiles", f"{name}_traffic.json")


def measured_traffic(name):
    """HBM bytes per step (decode with append) on workload `name` from the
    committed counter record, or None when the record is missing or the
    decode sources changed since."""
    try:
        with open(traffic_record(name)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != decode_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def pmc_target(which, reps):
    """Run only what a counter pass should see: the step call on one decode
    workload (layer rotated), or a plain device copy of 1 GiB (the
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
    lib = N.load_library()
    if which == "prefill":
        base = W.decode_batch(device=dev)
        args, info, keep = prefill_setup(base, N, W)
        torch.cuda.synchronize()
        for i in range(reps):
            if lib.paged_attn_prefill(*args[i % len(args)]):
                raise RuntimeError("paged_attn_prefill failed")
        torch.cuda.synchronize()
        log(f"ran {reps} prefill launches on the prefix-sharing batch ({info['flops']} flops each)")
        return
    if which.startswith(("int8_", "int4_")):
        import copy
        import ctypes

        bits = int(which[3])
        base = W.decode_batch(device=dev)
        shape = (base.num_blocks, base.num_layers, base.block_size, base.num_kv_heads, base.head_dim)
        k, v = quant_pools(W, N, shape, dev, bits)
        name = which[5:]
        w = base if name == "decode_batch" else W.PRESETS[name](device=dev, with_pools=False)
        w = copy.copy(w)
        ws = torch.zeros(max(16, N.paged_attn_decode_workspace_size(
            w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim, w.max_seq_len, w.block_size, 0)),
            dtype=torch.uint8, device=dev)
        out = torch.empty_like(w.q)
        pool = N.make_pool(k, v)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        torch.cuda.synchronize()
        for i in range(reps):
            if lib.paged_attn_decode(ctypes.byref(pool), i % w.num_layers, P(w.q), w.num_q_heads,
                                     P(w.block_tables), w.block_tables.shape[1], P(w.seq_lens),
                                     P(w.offsets), w.num_seqs, w.max_seq_len,
                                     ctypes.c_float(w.scale), 0, P(out), P(ws), ws.numel(), stream):
                raise RuntimeError(f"int{bits} paged_attn_decode failed")
        torch.cuda.synchronize()
        log(f"ran {reps} int{bits} decode launches on {name}")
        return
    w = config_workload(which, W.decode_batch(device=dev), W)
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
    log(f"ran {reps} step launches (decode with append) on {which}, {alg + append_bytes(w)} "
        f"algorithmic bytes each, split {split}")


DECODE_CONFIGS = ("long_context", "decode_batch", "prefix_sharing")
HEADLINE = "long_context"


def config_workload(name, base, W):
    """The decode workload `name` over the shared pools of `base` (same
    geometry: 16384 blocks x 32 layers x 16 x 8 x 128 bf16), with one new
    K/V row per sequence at position seq_len - 1."""
    if name == "decode_batch":
        w = base
    else:
        w = W.PRESETS[name](device=base.k_pool.device, with_pools=False)
        w.k_pool, w.v_pool = base.k_pool, base.v_pool
    w = W.decode_tokens(w)
    if int(w.token_seq.numel()) != w.num_seqs:
        raise RuntimeError(f"{name}: every sequence needs a token for the decode step")
    return w


def unique_live_bytes(w):
    """K and V bytes of the distinct (block, slot) rows the batch's tables
    hold live at the layer (a shared prefix counted once)."""
    import numpy as np

    bt = w.block_tables.cpu().numpy()
    lens = w.seq_lens.cpu().numpy().astype(np.int64)
    offs = w.offsets.cpu().numpy().astype(np.int64)
    rows = set()
    for s in range(w.num_seqs):
        p = offs[s] + np.arange(lens[s], dtype=np.int64)
        b = bt[s, p // w.block_size].astype(np.int64)
        rows.update((b * w.block_size + p % w.block_size).tolist())
    return len(rows) * w.row_bytes * 2


def schedule_label(N, w, split):
    """(kernel label, split label) of paged_attn_decode on this batch."""
    sched, label = decode_schedule(N, w, split)
    if sched == N.SCHEDULE_PLANNED:
        return label, "planned (device-planned split)"
    return label, sched


def decode_config(name, w, N, args, lib, stream, headline):
    """Times the decode step (paged_attn_decode_append: the new token's slot
    and write, and paged decode attention over every cached token) on one
    workload, back to back with the layer rotated; also decode alone, one
    cold step after a 1 GiB flush read, and the read-rate reference over the
    same blocks.  The headline workload also times the step as HIP graph
    replays and as two calls (kv_append + paged_attn_decode)."""
    import ctypes

    import torch

    dev = w.q.device
    lens = w.seq_lens.cpu().numpy()
    kv_bytes, alg_bytes = decode_bytes(w, lens)
    alg_step = alg_bytes + append_bytes(w)
    split = args.split_tokens
    kernel, split_label = schedule_label(N, w, split)
    ws_bytes = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                                  w.head_dim, w.max_seq_len, w.block_size, split)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty_like(w.q)
    kn, vn = w.k_new, w.v_new   # rows in sequence order (every sequence has its token)
    slots = torch.empty(w.num_seqs, dtype=torch.int64, device=dev)
    pool = N.make_pool(w.k_pool, w.v_pool)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    L = w.num_layers
    step_args = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(kn), P(vn), P(w.block_tables),
                  w.block_tables.shape[1], P(w.seq_lens), P(w.offsets), w.num_seqs, w.max_seq_len,
                  ctypes.c_float(w.scale), split, P(out), P(ws), ws.numel(), stream)
                 for l in range(L)]
    dec_args = [(ctypes.byref(pool), l, P(w.q), w.num_q_heads, P(w.block_tables),
                 w.block_tables.shape[1], P(w.seq_lens), P(w.offsets), w.num_seqs, w.max_seq_len,
                 ctypes.c_float(w.scale), split, P(out), P(ws), ws.numel(), stream)
                for l in range(L)]
    app_args = [(ctypes.byref(pool), l, P(kn), P(vn), P(w.block_tables), w.block_tables.shape[1],
                 P(w.offsets), w.num_seqs, P(w.token_seq), P(w.token_pos), w.num_seqs, P(slots),
                 stream) for l in range(L)]
    f_step, f_dec, f_app = lib.paged_attn_decode_append, lib.paged_attn_decode, lib.kv_append

    def back_to_back(fn):
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

    def step(i):
        if f_step(*step_args[i % L]):
            raise RuntimeError(f"paged_attn_decode_append failed on {name}")

    def decode_only(i):
        if f_dec(*dec_args[i % L]):
            raise RuntimeError(f"paged_attn_decode failed on {name}")

    def two_call(i):
        if f_app(*app_args[i % L]) | f_dec(*dec_args[i % L]):
            raise RuntimeError(f"kv_append / paged_attn_decode failed on {name}")

    # The first passes over the freshly filled 32 GiB pool run slower
    # (long context: ~350 us per step over the first 20 steps, settled at
    # ~170 us from about step 100 on), and a short step settles in time
    # rather than in calls: untimed passes over the 32 layers, at least
    # three and at least 0.2 s of them, precede the warmup steps.
    t0 = time.perf_counter()
    passes = 0
    while passes < 3 or time.perf_counter() - t0 < 0.2:
        for i in range(L):
            step(i)
        torch.cuda.synchronize()
        passes += 1
    log(f"{name}: timing {args.steps} steps ({kernel})")
    ms_step = back_to_back(step)
    # per-call event pairs around the same calls
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    per_call = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    ms_dec = back_to_back(decode_only)
    # cold steps: each after a 1 GiB device copy (reads 1 GiB, so no cache
    # holds the step's bytes), on a layer the previous steps did not touch last
    flush_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    cold = []
    for i in range(5):
        flush_dst.copy_(flush_src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(7 * i + 3)
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush_src, flush_dst
    cold.sort()
    entry = {
        "kernel": kernel + ", with the new-token write",
        "split_tokens": split_label,
        "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim, "cached_tokens": int(lens.sum()),
        "step_us": ms_step * 1e3,
        "kv_bytes": kv_bytes,
        "algorithmic_bytes_per_step": alg_step,
        "achieved_GBps": alg_step / ms_step / 1e6,
        "frac": alg_step / ms_step / 1e6 / HBM_PEAK_GBS,
        "per_call_events_median_us": per_call[len(per_call) // 2] * 1e3,
        "per_call_events_avg_us": sum(per_call) / len(per_call) * 1e3,
        "decode_alone_us": ms_dec * 1e3,
        "decode_alone_GBps": alg_bytes / ms_dec / 1e6,
        "cold_step_us_median_of_5": cold[2] * 1e3,
        "cold_step_GBps": alg_step / cold[2] / 1e6,
        "measured_read_ceiling": read_ceiling(w, N),
        "traffic": measured_traffic(name),
    }
    if name == "prefix_sharing":
        uniq = unique_live_bytes(w)
        alg_unique = alg_step - kv_bytes + uniq
        entry["unique_kv_bytes"] = uniq
        entry["algorithmic_bytes_unique"] = alg_unique
        entry["achieved_GBps_unique"] = alg_unique / ms_step / 1e6
        entry["frac_unique"] = alg_unique / ms_step / 1e6 / HBM_PEAK_GBS
        entry["note"] = ("frac_unique counts the shared prefix once (its 64 readers are served "
                         "from cache after the first); frac counts it once per sequence")
    if headline and not args.no_graph:
        def capture(calls):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for i in range(3):
                    calls(i % L, ctypes.c_void_p(side.cuda_stream))
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            gs = []
            for layer in range(L):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    calls(layer, ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
                gs.append(g)
            torch.cuda.synchronize()
            return gs

        def fused_calls(layer, cs):
            if f_step(*step_args[layer][:-1], cs):
                raise RuntimeError("paged_attn_decode_append failed while capturing")

        def two_calls(layer, cs):
            if f_app(*app_args[layer][:-1], cs) | f_dec(*dec_args[layer][:-1], cs):
                raise RuntimeError("a library call failed while capturing")

        gs = capture(fused_calls)
        entry["graph_replay_us"] = back_to_back(lambda i: gs[i % L].replay()) * 1e3
        del gs
        entry["two_call_step_us"] = back_to_back(two_call) * 1e3
        gs = capture(two_calls)
        entry["two_call_graph_replay_us"] = back_to_back(lambda i: gs[i % L].replay()) * 1e3
        del gs
    log(f"{name}: step {ms_step * 1e3:.1f} us, {entry['frac']:.3f} of peak; decode alone "
        f"{ms_dec * 1e3:.1f} us; cold {cold[2] * 1e3:.1f} us")
    del ws, out
    return entry, ms_step


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager calls only (no HIP graph replay)")
    ap.add_argument("--configs", default=",".join(DECODE_CONFIGS),
                    help="decode workloads to time (the headline, long_context, is always first)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--pmc-target", default=None,
                    choices=list(DECODE_CONFIGS) + ["int8_" + c for c in DECODE_CONFIGS]
                    + ["int4_" + c for c in DECODE_CONFIGS] + ["prefill", "copy"],
                    help="run only the step launches of one workload (or int8 / int4 decode on it, the "
                         "prefill launches, or a 1 GiB copy) for counter passes")
    ap.add_argument("--pmc-reps", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the hot path "
              "shards by sequence or kv head with no exchange, so there is no multi-GPU "
              "measurement to make here", file=sys.stderr)
        sys.exit(2)

    import ctypes

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
    lib = N.load_library()
    log("building the pools (2 x 16 GiB) and the decode workloads")
    base = W.decode_batch(device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    names = [HEADLINE] + [c for c in args.configs.split(",") if c and c != HEADLINE]
    configs, head_ms, head_w = {}, None, None
    for name in names:
        w = config_workload(name, base, W)
        configs[name], ms = decode_config(name, w, N, args, lib, stream, name == HEADLINE)
        if name == HEADLINE:
            head_ms, head_w = ms, w
    h = configs[HEADLINE]
    result = {
        "metric": METRIC,
        "value": h["kv_bytes"] / (head_ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": HEADLINE,
            "num_seqs": head_w.num_seqs,
            "seq_len": head_w.max_seq_len,
            "cached_tokens": h["cached_tokens"],
            "block_size": head_w.block_size,
            "pool_blocks": head_w.num_blocks,
            "num_layers": head_w.num_layers,
            "num_kv_heads": head_w.num_kv_heads,
            "head_dim": head_w.head_dim,
            "num_q_heads": head_w.num_q_heads,
            "split_tokens": h["split_tokens"],
            "kv_bytes_per_step": h["kv_bytes"],
            "step": "paged_attn_decode_append: slot + write of 1 new K/V row per sequence and "
                    "paged decode attention over every cached token, one C-ABI call per step, "
                    "layer rotated over 32",
            "step_launch": "one C-ABI call per step, issued back to back",
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": h["kernel"],
            "bound": "hbm",
            "achieved": h["achieved_GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": h["frac"],
            "traffic": h["traffic"],
            "algorithmic_bytes_per_launch": h["algorithmic_bytes_per_step"],
            "avg_launch_us": h["step_us"],
            "timing": f"HIP events around the {args.steps} back-to-back step calls on the launch "
                      "stream (the timed steps themselves)",
            "measured_read_ceiling": h["measured_read_ceiling"],
        },
        "decode_configs": configs,
    }
    if not args.no_ops:
        log("scatter/gather on the prefill shape")
        result["ops"] = prefill_ops(base, N, W)
        log("block copies and swaps")
        result["ops"].update(block_ops(base, N))
        log("prefill attention on the prefix-sharing batch")
        result["prefill_attention"] = prefill_attention(base, N, W)
        log("int8 pool decode")
        result["int8_decode"] = quant_decode(base, N, W, 8)
        log("int4 pool decode")
        result["int4_decode"] = quant_decode(base, N, W, 4)
        log("the pages' PyTorch forms (context)")
        result["torch_context"] = torch_context(base, W)
        log("host block manager")
        result["block_manager"] = block_manager_host(N, W)
    if not args.no_cpu_baseline:
        log("CPU oracle baseline on the long-context batch")
        result["cpu_baseline"] = cpu_baseline(head_w, head_w.seq_lens.cpu().numpy())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
