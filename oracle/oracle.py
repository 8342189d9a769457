"""ctypes front end of the C oracle, plus small pure-Python/numpy forms.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources cited below:
  [P1] mini-vllm tutorial, "step14_2 - index_select gather"
  [P2] "vLLM PagedAttention source notes" (minivLLM Task 6 background)
  [P3] mini-runtime, chapter 12 "Paged KV Cache"

Array conventions (host numpy):
  pool           (num_blocks, num_layers, block_size, num_kv_heads, head_dim)
                 float32, or uint16 holding bfloat16 bit patterns
  block_tables   int32 (num_seqs, bt_stride); entries past a table's end unused
  seq_lens, offsets  int32 (num_seqs,)
  slot_mapping   int64 (num_tokens,), -1 = padding
"""
import ctypes
import os

import numpy as np

ORC_F32 = 0
ORC_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("PKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) and "PKV_ORACLE_LIB" not in os.environ:
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.orc_slot_mapping.restype = i64
    lib.orc_slot_mapping.argtypes = [p, i64, p, i64, p, p, i64, i64, p]
    lib.orc_scatter.restype = i64
    lib.orc_scatter.argtypes = [p, i64, i64, i64, i64, i64, p, p, i64]
    lib.orc_gather.restype = i64
    lib.orc_gather.argtypes = [p, i64, i64, i64, i64, i64, p, i64, p, p, i64, p]
    lib.orc_prefill.restype = i64
    lib.orc_prefill.argtypes = [p, p, i64, i64, i64, i64, i64, i64, i64, p, p, i64, p, i64,
                                p, p, i64, ctypes.c_double, p, i64]
    lib.orc_decode.restype = i64
    lib.orc_decode.argtypes = [p, p, i64, i64, i64, i64, i64, i64, i64, p, i64,
                               p, i64, p, p, i64, ctypes.c_double, p, i64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return ORC_F32
    if a.dtype == np.uint16:
        return ORC_BF16
    raise TypeError(f"pool dtype must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# C oracle wrappers
# --------------------------------------------------------------------------
def slot_mapping(block_tables, offsets, token_seq, token_pos, block_size):
    """Slot per token: block_tables[seq][(off+pos)//bs]*bs + (off+pos)%bs,
    -1 for padding rows (token_seq < 0).  [P2 sec. 2.2 with P3 sec. 2.2]"""
    bt = _c(block_tables, np.int32)
    off = _c(offsets, np.int32)
    ts = _c(token_seq, np.int32)
    tp = _c(token_pos, np.int32)
    out = np.empty(ts.shape[0], dtype=np.int64)
    rc = _load().orc_slot_mapping(_ptr(bt), bt.shape[1], _ptr(off), off.shape[0],
                                  _ptr(ts), _ptr(tp), ts.shape[0], block_size, _ptr(out))
    if rc != 0:
        raise ValueError("oracle slot_mapping: token outside its table")
    return out


def scatter(pool, layer, src, slots):
    """In-place scatter of src rows into pool at `layer` (slot -1 skipped).
    [P1 "relation to step14_1"; P2 sec. 2.2]"""
    if not pool.flags.c_contiguous:
        raise ValueError("pool must be C-contiguous")
    nb, nl, bs, h, d = pool.shape
    src = _c(src, pool.dtype)
    slots = _c(slots, np.int64)
    row_bytes = h * d * pool.itemsize
    if src.size * src.itemsize != slots.shape[0] * row_bytes:
        raise ValueError("src must hold one row per slot")
    rc = _load().orc_scatter(_ptr(pool), nb, nl, bs, row_bytes, layer, _ptr(src),
                             _ptr(slots), slots.shape[0])
    if rc != 0:
        raise ValueError("oracle scatter: slot outside the pool")
    return pool


def gather(pool, layer, block_tables, seq_lens, offsets):
    """Loop-and-cat gather with the first-block offset; sequences concatenated.
    Returns (sum seq_lens, num_kv_heads, head_dim).  [P1 "Problem"; P3 sec. 2.2]"""
    pool = _c(pool, pool.dtype)
    nb, nl, bs, h, d = pool.shape
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    off = _c(offsets, np.int32)
    total = int(sl.astype(np.int64).sum())
    out = np.empty((total, h, d), dtype=pool.dtype)
    rc = _load().orc_gather(_ptr(pool), nb, nl, bs, h * d * pool.itemsize, layer,
                            _ptr(bt), bt.shape[1], _ptr(sl), _ptr(off), sl.shape[0], _ptr(out))
    if rc != total:
        raise ValueError("oracle gather: table too short or block id outside the pool")
    return out


def decode(k_pool, v_pool, layer, q, block_tables, seq_lens, offsets, scale,
           num_threads=1):
    """Gather-then-attention in double; returns float64 (num_seqs, Hq, D).
    [P2 sec. 2.3; P3 sec. 3.1; P1 "comparison with vLLM"]"""
    k_pool = _c(k_pool, k_pool.dtype)
    v_pool = _c(v_pool, k_pool.dtype)
    dt = _dtype_code(k_pool)
    nb, nl, bs, hkv, d = k_pool.shape
    q = _c(q, k_pool.dtype)
    ns, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim mismatch")
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    off = _c(offsets, np.int32)
    out = np.empty((ns, hq, d), dtype=np.float64)
    rc = _load().orc_decode(_ptr(k_pool), _ptr(v_pool), nb, nl, bs, hkv, d, dt, layer,
                            _ptr(q), hq, _ptr(bt), bt.shape[1], _ptr(sl), _ptr(off), ns,
                            float(scale), _ptr(out), int(num_threads))
    if rc != 0:
        raise ValueError("oracle decode: bad arguments or table")
    return out


def prefill(k_pool, v_pool, layer, q, q_start, block_tables, seq_lens, offsets, scale,
            num_threads=1):
    """Causal attention of each sequence's last n = q_start[s+1]-q_start[s]
    tokens (rows q_start[s].. of q) over its cached tokens, in double;
    returns float64 (rows, Hq, D).  [P2 sec. 2.4 prefill; sec. 2.3]"""
    k_pool = _c(k_pool, k_pool.dtype)
    v_pool = _c(v_pool, k_pool.dtype)
    dt = _dtype_code(k_pool)
    nb, nl, bs, hkv, d = k_pool.shape
    q = _c(q, k_pool.dtype)
    rows, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim mismatch")
    qs = _c(q_start, np.int32)
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    off = _c(offsets, np.int32)
    ns = sl.shape[0]
    if qs.shape[0] != ns + 1 or int(qs[-1]) != rows:
        raise ValueError("q_start must have num_seqs + 1 entries ending at the row count")
    out = np.empty((rows, hq, d), dtype=np.float64)
    rc = _load().orc_prefill(_ptr(k_pool), _ptr(v_pool), nb, nl, bs, hkv, d, dt, layer, _ptr(q),
                             _ptr(qs), hq, _ptr(bt), bt.shape[1], _ptr(sl), _ptr(off), ns,
                             float(scale), _ptr(out), int(num_threads))
    if rc != 0:
        raise ValueError("oracle prefill: bad arguments or table")
    return out


# --------------------------------------------------------------------------
# Whole-block moves: the copy of copy-on-write and the swap of preemption
# --------------------------------------------------------------------------
def copy_blocks(pool, src_blocks, dst_blocks):
    """In place: for each pair in order, every layer of block src[i] is
    copied to block dst[i] (pool: (num_blocks, num_layers, bs, H, D)); a
    pair with an id outside the pool is skipped.  The copy a writer makes
    of a shared block before writing into it ("vLLM PagedAttention" in
    ch. 12, 3.1: sharing by copy-on-write + ref_count)."""
    nb = pool.shape[0]
    for s, d in zip(np.asarray(src_blocks).tolist(), np.asarray(dst_blocks).tolist()):
        if 0 <= s < nb and 0 <= d < nb:
            pool[d] = pool[s].copy()
    return pool


def swap_out(pool, block_ids):
    """The blocks' contents, all layers, in the order given: a host array
    (n, num_layers, bs, H, D).  The GPU -> CPU move of preemption ("vLLM
    PagedAttention source notes", 2.4 scheduler integration)."""
    ids = np.asarray(block_ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= pool.shape[0]):
        raise ValueError("block id outside the pool")
    return np.stack([pool[b].copy() for b in ids.tolist()]) if ids.size else \
        np.empty((0,) + pool.shape[1:], dtype=pool.dtype)


def swap_in(pool, block_ids, host):
    """In place: block ids[i] of the pool takes host[i] (all layers): the
    CPU -> GPU move that brings a swapped-out sequence back."""
    ids = np.asarray(block_ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= pool.shape[0]):
        raise ValueError("block id outside the pool")
    if host.shape != (ids.size,) + pool.shape[1:]:
        raise ValueError("host buffer shape")
    for i, b in enumerate(ids.tolist()):
        pool[b] = host[i]
    return pool


# --------------------------------------------------------------------------
# Pure-Python / numpy forms (tiny inputs; second formulations for the pins)
# --------------------------------------------------------------------------
def gather_loop_cat(pool_layer, block_table, seq_len, block_size, offset=0):
    """[P1 "Problem"] loop over the table's block ids, slice each block,
    concatenate; the first block starts at `offset` [P3 sec. 2.2].
    pool_layer: (num_blocks, block_size, H, D)."""
    pieces = []
    remaining = seq_len
    first = True
    for bid in block_table:
        if remaining <= 0:
            break
        lo = offset if first else 0
        first = False
        n = min(block_size - lo, remaining)
        pieces.append(pool_layer[bid, lo:lo + n])
        remaining -= n
    if remaining > 0:
        raise ValueError("table too short")
    if not pieces:
        return pool_layer[:0, 0]
    return np.concatenate(pieces, axis=0)


def gather_flat_index(pool_layer, block_table, seq_len, block_size, offset=0):
    """[P1 "Solution"] one advanced-indexing gather over flattened positions,
    shifted by the first-block offset [P3 sec. 2.2]."""
    pos = np.arange(seq_len, dtype=np.int64) + offset
    bt = np.asarray(block_table, dtype=np.int64)
    return pool_layer[bt[pos // block_size], pos % block_size]


def scatter_index_put(pool_layer, slots, rows, block_size):
    """[P1 "relation to step14_1"] kv_pool[physical_blocks, slot_indices] = K,
    padding (-1) rows dropped [P2 sec. 2.2].  Mutates pool_layer."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots != -1
    s = slots[keep]
    pool_layer[s // block_size, s % block_size] = rows[keep]
    return pool_layer


def blocks_needed(num_tokens, block_size):
    """ceil(num_tokens / block_size) blocks for a request.
    [P2 sec. 2.1 prefill_allocate; P3 sec. 2.3 allocate]"""
    return -(-num_tokens // block_size)


def capacity(num_table_blocks, block_size, offset):
    """Tokens a BlockTable can hold: num_blocks*block_size - offset, with
    num_blocks the table's own length.  [P3 sec. 2.2 and sec. 4.3]"""
    return num_table_blocks * block_size - offset


def last_block_fill(num_tokens, block_size):
    """Tokens held by the last allocated block of a request (P3 think-question
    arithmetic: 30 tokens at block_size 16 leave 14 in the second block)."""
    if num_tokens == 0:
        return 0
    return num_tokens - (blocks_needed(num_tokens, block_size) - 1) * block_size


def fragmentation_ratio(total_allocated_blocks, block_size, total_used_tokens):
    """(allocated slots - used tokens) / allocated slots.  [P2 sec. 3]"""
    slots = total_allocated_blocks * block_size
    return (slots - total_used_tokens) / slots
