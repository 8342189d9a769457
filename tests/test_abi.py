"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no GPU needed: every call here
fails its argument checks, so nothing is enqueued)."""
import ctypes
import glob
import os
import re

import pytest

from paged_attention_decode_scatter_amd import native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL, DTYPE, SHAPE, LAYER, ALIGN, WORKSPACE, LAUNCH, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    names = []
    for h in HEADERS:
        names += re.findall(r"PKV_API\s+[\w\s\*]+?\b(\w+)\s*\(", open(h).read())
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.LIB_PATH):
        from paged_attention_decode_scatter_amd import build
        build.build()
    return N.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == len(set(names)) == 34
    assert set(names) == set(N.SYMBOLS) | set(N.BM_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_only_declared_symbols_are_exported(lib):
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_status_strings(lib):
    for st in (OK, NULL, DTYPE, SHAPE, LAYER, ALIGN, WORKSPACE, LAUNCH, UNSUP, -9):
        assert N.status_string(st)
    assert N.status_string(12345) == "unknown status"


def pool(k=0x1000, v=0x2000, nb=16, nl=2, bs=16, h=8, d=128, dtype=1, reserved=0, stride=0,
         ks=0x3000, vs=0x4000):
    return N.PkvPool(k, v, nb, nl, bs, h, d, dtype, reserved, stride, ks, vs)


A = 0x10000  # an aligned fake device address; never dereferenced on these paths


def test_scatter_argument_checks(lib):
    f = lib.kv_scatter
    by = ctypes.byref
    assert f(None, 0, A, A, A, 4, None) == NULL
    assert f(by(pool(k=None)), 0, A, A, A, 4, None) == NULL
    assert f(by(pool(dtype=7)), 0, A, A, A, 4, None) == DTYPE
    assert f(by(pool(bs=12)), 0, A, A, A, 4, None) == SHAPE
    assert f(by(pool(nb=0)), 0, A, A, A, 4, None) == SHAPE
    assert f(by(pool(reserved=1)), 0, A, A, A, 4, None) == SHAPE
    assert f(by(pool(h=1, d=3, dtype=0)), 0, A, A, A, 4, None) == ALIGN  # 12-byte rows
    assert f(by(pool(k=0x1004)), 0, A, A, A, 4, None) == ALIGN
    assert f(by(pool()), 2, A, A, A, 4, None) == LAYER
    assert f(by(pool()), -1, A, A, A, 4, None) == LAYER
    assert f(by(pool()), 0, A, A, A, -1, None) == SHAPE
    assert f(by(pool()), 0, A, A, A, 0, None) == OK          # nothing to do, nothing enqueued
    assert f(by(pool()), 0, None, A, A, 4, None) == NULL
    assert f(by(pool()), 0, A, A, None, 4, None) == NULL
    assert f(by(pool()), 0, A + 8, A, A, 4, None) == ALIGN
    assert f(by(pool(v=None)), 0, A, A, A, 4, None) == NULL  # V source given, V pool missing


def test_gather_argument_checks(lib):
    f = lib.kv_gather
    by = ctypes.byref
    args = lambda **kw: dict(dict(layer=0, bt=A, stride=4, sl=A, off=A, rs=A, ns=2, mx=10,
                                  ko=A, vo=A, rows=20), **kw)

    def call(p, **kw):
        a = args(**kw)
        return f(by(p), a["layer"], a["bt"], a["stride"], a["sl"], a["off"], a["rs"], a["ns"],
                 a["mx"], a["ko"], a["vo"], a["rows"], None)

    assert call(pool(), layer=5) == LAYER
    assert call(pool(), ns=-1) == SHAPE
    assert call(pool(), mx=-1) == SHAPE
    assert call(pool(), rows=-1) == SHAPE
    assert call(pool(), ns=0) == OK
    assert call(pool(), mx=0) == OK
    assert call(pool(), bt=None) == NULL
    assert call(pool(), rs=None) == NULL
    assert call(pool(), ko=None) == NULL
    assert call(pool(), ko=A + 4) == ALIGN
    assert call(pool(v=None)) == NULL


def test_slot_mapping_argument_checks(lib):
    f = lib.kv_slot_mapping
    assert f(A, 4, A, 2, A, A, 10, 12, A, None) == SHAPE    # block_size not a power of two
    assert f(A, 4, A, 2, A, A, -1, 16, A, None) == SHAPE
    assert f(A, 4, A, 2, A, A, 0, 16, A, None) == OK
    assert f(A, 4, A, 2, None, A, 10, 16, A, None) == NULL
    assert f(None, 4, A, 2, A, A, 10, 16, A, None) == NULL
    assert f(A, 4, A, 2, A, A, 10, 16, None, None) == NULL


def test_decode_argument_checks(lib):
    f = lib.paged_attn_decode
    by = ctypes.byref

    def call(p=None, hq=32, ns=4, mx=100, split=0, q=A, out=A, ws=A, wsb=1 << 30, layer=0):
        return f(by(p or pool()), layer, q, hq, A, 8, A, A, ns, mx, 0.1, split, out, ws, wsb, None)

    assert call(hq=30) == SHAPE        # not a multiple of num_kv_heads
    assert call(hq=24) == UNSUP        # G = 3
    assert call(p=pool(d=96)) == UNSUP
    assert call(layer=3) == LAYER
    assert call(split=24) == SHAPE     # not a multiple of 16
    assert call(split=-16) == SHAPE
    assert call(split=-1) == SHAPE     # negative: only the planned-schedule request
    assert call(ns=0) == OK
    assert call(q=None) == NULL
    assert call(out=A + 2) == ALIGN
    # needs a workspace when a sequence spans several splits
    need = lib.paged_attn_decode_workspace_size(4, 8, 32, 128, 100, 16, 16)
    assert need > 0
    assert call(split=16, ws=None, wsb=0) == WORKSPACE
    assert call(split=16, wsb=need - 1) == WORKSPACE
    assert call(split=16, ws=A + 4, wsb=need) == ALIGN


def test_decode_noalloc_argument_checks(lib):
    """Rejections that come before the scratch lookup (so no GPU is
    touched): pool and shape checks, and sizes whose workspace would not fit
    the fixed scratch."""
    f = lib.paged_attn_decode_noalloc
    by = ctypes.byref
    SCRATCH = -13

    def call(p=None, hq=32, ns=4, mx=100, split=0, q=A, out=A, layer=0):
        return f(by(p or pool()), layer, q, hq, A, 8, A, A, ns, mx, 0.1, split, out, None)

    assert f(None, 0, A, 32, A, 8, A, A, 4, 100, 0.1, 0, A, None) == NULL
    assert call(hq=30) == SHAPE
    assert call(split=24) == SHAPE
    assert call(ns=-1) == SHAPE
    # 64 sequences of 32768 tokens at 16-token splits: far beyond 32 MiB
    need = lib.paged_attn_decode_workspace_size(64, 8, 64, 128, 32768, 16, 16)
    assert need > N.NOALLOC_SCRATCH_BYTES
    assert call(p=pool(nb=16384), hq=64, ns=64, mx=32768, split=16) == SCRATCH
    assert "scratch" in N.status_string(SCRATCH)


def test_decode_append_argument_checks(lib):
    f = lib.paged_attn_decode_append
    by = ctypes.byref

    def call(p=None, hq=32, ns=4, mx=100, split=0, q=A, kn=A, vn=A, out=A, ws=A, wsb=1 << 30,
             layer=0):
        return f(by(p or pool()), layer, q, hq, kn, vn, A, 8, A, A, ns, mx, 0.1, split, out, ws,
                 wsb, None)

    assert call(kn=None) == NULL
    assert call(vn=None) == NULL
    assert call(kn=A + 8) == ALIGN
    assert call(vn=A + 4) == ALIGN
    assert call(hq=24) == UNSUP
    assert call(layer=3) == LAYER
    assert call(split=24) == SHAPE
    assert call(ns=0, kn=None, vn=None) == OK
    assert call(split=16, ws=None, wsb=0) == WORKSPACE


def test_workspace_size_and_split_choice(lib):
    ws = lib.paged_attn_decode_workspace_size
    # one split covers everything: no workspace
    assert ws(1, 2, 4, 64, 30, 16, 64) == 0
    # automatic choice: room for the schedule any pool dtype takes (the
    # automatic split differs between bf16 and the other pools)
    split = lib.paged_attn_decode_split_tokens
    assert ws(1, 2, 4, 64, 30, 16, 0) == 0    # one split in either schedule
    assert ws(8, 8, 64, 128, 32768, 16, 0) >= ws(8, 8, 64, 128, 32768, 16, split(8, 8, 32768, 16))
    # split counters (seqs x kv heads) and the (m, l) block, each padded to
    # 256 bytes, then the fp32 accumulators.  Splits cover flat table
    # positions, so a first-block offset of up to block_size - 1 can add
    # one: ceil((32768 + 15) / 8192) = 5
    n = 8 * 5 * 64                     # seqs x splits x q heads at split 8192, len 32768
    cnt = (8 * 8 * 4 + 255) // 256 * 256
    assert ws(8, 8, 64, 128, 32768, 16, 8192) == cnt + (n * 8 + 255) // 256 * 256 + n * 128 * 4
    assert ws(8, 8, 64, 128, 32768, 16, 24) == ctypes.c_size_t(-1).value
    for args in ((32, 8, 2048, 16), (64, 8, 4096, 16), (8, 8, 32768, 16), (1, 2, 30, 16),
                 (3, 1, 5000, 1)):
        s = split(*args)
        assert s > 0 and s % 16 == 0
        assert s // args[3] + 2 <= 1024
    assert split(4, 8, 100, 12) == SHAPE
    # the choices on 256 compute units (the count assumed without a device)
    assert split(32, 8, 2048, 16) == 256
    assert split(8, 8, 32768, 16) == 2048
    # many (sequence, kv head) pairs (>= 2 per compute unit): up to 32 work
    # items per compute unit, no long-split rule
    assert split(96, 8, 4096, 16) == 512
    assert split(128, 8, 3072, 16) == 512
    assert split(256, 8, 1536, 16) == 512
    # the split stops growing once it covers max_seq_len
    assert split(2000, 8, 128, 16) == 256
    sched = lib.paged_attn_decode_schedule
    assert sched(8, 8, 64, 128, 32768, 16, 1, 0) == 2048   # bf16: one workgroup per CU
    assert sched(8, 8, 64, 128, 32768, 16, 2, 0) == 1024   # int8: two per CU
    assert sched(8, 8, 64, 128, 32768, 16, 0, 0) == 1024   # fp32
    # the workspace for split_tokens = 0 covers the smaller (int8) split
    assert ws(8, 8, 64, 128, 32768, 16, 0) >= ws(8, 8, 64, 128, 32768, 16, 1024)


def test_append_argument_checks(lib):
    f = lib.kv_append
    by = ctypes.byref

    def call(p=None, layer=0, k=A, v=A, bt=A, stride=8, off=A, ns=2, ts=A, tp=A, n=4, out=None):
        return f(by(p or pool()), layer, k, v, bt, stride, off, ns, ts, tp, n, out, None)

    assert call(layer=2) == LAYER
    assert call(n=-1) == SHAPE
    assert call(ns=-1) == SHAPE
    assert call(stride=-1) == SHAPE
    assert call(n=0) == OK
    assert call(k=None) == NULL
    assert call(ts=None) == NULL
    assert call(tp=None) == NULL
    assert call(bt=None) == NULL
    assert call(off=None) == NULL
    assert call(k=A + 8) == ALIGN
    assert call(p=pool(bs=6)) == SHAPE
    assert call(p=pool(dtype=5)) == DTYPE
    assert call(p=pool(v=0)) == NULL       # V rows given but no V pool


def test_prefill_argument_checks(lib):
    f = lib.paged_attn_prefill
    by = ctypes.byref

    def call(p=None, layer=0, q=A, hq=32, qs=A, rows=64, mq=16, bt=A, stride=8, sl=A, off=A, ns=4,
             out=A):
        return f(by(p or pool()), layer, q, hq, qs, rows, mq, bt, stride, sl, off, ns, 0.1, out, None)

    assert call(layer=2) == LAYER
    assert call(hq=30) == SHAPE
    assert call(rows=-1) == SHAPE
    assert call(mq=-1) == SHAPE
    assert call(p=pool(d=96)) == UNSUP
    assert call(hq=8 * 16) == UNSUP          # G = 16
    assert call(ns=0) == OK
    assert call(rows=0) == OK
    assert call(q=None) == NULL
    assert call(qs=None) == NULL
    assert call(out=A + 2) == ALIGN


def test_decode_schedule_choice(lib):
    """The automatic schedule: the device-planned split for bf16 batches of
    at most 64 sequences with at most (compute units / 2) (sequence, head
    group) pairs and max_seq_len / 2 + 32 within the largest split (also
    int8 pools); the automatic split otherwise; an explicit split is always
    kept.  (No device here: 256 compute units are assumed.)"""
    f = lib.paged_attn_decode_schedule
    F32, BF16 = 0, 1
    PLANNED, SPLIT_PLANNED = 1, -2
    split = lib.paged_attn_decode_split_tokens
    assert f(32, 8, 32, 128, 2048, 16, BF16, 0) == PLANNED                 # decode batch
    assert f(64, 8, 32, 128, 4096, 16, BF16, 0) == PLANNED                 # prefix sharing
    assert f(32, 8, 32, 128, 2048, 16, F32, 0) == split(32, 8, 2048, 16)
    assert f(32, 8, 32, 128, 2048, 16, 2, 0) == PLANNED                    # int8 pool
    assert f(65, 8, 32, 128, 4096, 16, BF16, 0) == split(65, 8, 4096, 16)  # 65 sequences, 1 GiB
    assert f(65, 8, 32, 128, 1024, 16, BF16, 0) == split(65, 8, 1024, 16)  # 65 sequences, 0.27 GiB
    assert f(64, 16, 64, 128, 4096, 16, BF16, 0) == split(64, 16, 4096, 16)  # 4 head groups: 256 pairs
    assert f(8, 8, 64, 128, 32768, 16, BF16, 0) == split(8, 8, 32768, 16)  # past the largest split
    assert f(8, 8, 64, 128, 32768, 16, BF16, SPLIT_PLANNED) == UNSUP
    assert f(2, 2, 8, 128, 100, 16, F32, SPLIT_PLANNED) == UNSUP
    assert f(2, 2, 8, 128, 100, 16, BF16, SPLIT_PLANNED) == PLANNED
    assert f(8, 8, 64, 128, 32768, 16, F32, 0) == 1024                     # fp32: no long-split rule
    assert f(8, 8, 64, 128, 32768, 16, BF16, 512) == 512
    assert f(5000, 8, 32, 128, 4096, 16, BF16, 0) == split(5000, 8, 4096, 16)
    assert f(8, 8, 64, 128, 32768, 16, 7, 0) == DTYPE
    assert f(8, 8, 60, 128, 32768, 16, BF16, 0) == SHAPE
    assert f(2, 2, 8, 128, 100, 16, BF16, -1) == SHAPE
    assert f(2, 2, 8, 128, 100, 16, F32, -1) == SHAPE


def test_read_blocks_argument_checks(lib):
    f = lib.kv_read_blocks
    by = ctypes.byref
    assert f(None, 0, A, 4, A, None) == NULL
    assert f(by(pool()), 2, A, 4, A, None) == LAYER
    assert f(by(pool()), 0, A, -1, A, None) == SHAPE
    assert f(by(pool()), 0, A, 0, A, None) == OK            # nothing to read
    assert f(by(pool()), 0, None, 4, A, None) == NULL
    assert f(by(pool()), 0, A, 4, None, None) == NULL
    assert f(by(pool(bs=12)), 0, A, 4, A, None) == SHAPE


def test_validate_argument_checks(lib):
    f = lib.kv_validate
    by = ctypes.byref
    assert f(None, A, 4, A, A, 2, 10, A, 3, A, None) == NULL
    assert f(by(pool()), A, 4, A, A, 2, 10, A, 3, None, None) == NULL
    assert f(by(pool(bs=6)), A, 4, A, A, 2, 10, A, 3, A, None) == SHAPE
    assert f(by(pool()), None, 4, A, A, 2, 10, A, 3, A, None) == NULL
    assert f(by(pool()), A, 4, A, A, 2, 10, None, 3, A, None) == NULL


def test_block_stride_checks(lib):
    """A nonzero block stride is at least one dense block (2 layers x 16 x
    8 x 128 bf16 = 64 KiB here) and a multiple of 16 bytes."""
    f = lib.kv_scatter
    by = ctypes.byref
    dense = 2 * 16 * 8 * 128 * 2
    assert f(by(pool(stride=dense - 16)), 0, A, A, A, 4, None) == SHAPE
    assert f(by(pool(stride=dense + 8)), 0, A, A, A, 4, None) == ALIGN
    assert f(by(pool(stride=2 * dense)), 0, A, A, A, 0, None) == OK
    assert f(by(pool(stride=dense)), 0, A, A, A, 0, None) == OK


def test_copy_blocks_argument_checks(lib):
    f = lib.kv_copy_blocks
    by = ctypes.byref
    assert f(None, A, A, 3, None) == NULL
    assert f(by(pool(k=None)), A, A, 3, None) == NULL
    assert f(by(pool(dtype=5)), A, A, 3, None) == DTYPE
    assert f(by(pool(bs=3)), A, A, 3, None) == SHAPE
    assert f(by(pool()), A, A, -1, None) == SHAPE
    assert f(by(pool()), A, A, 0, None) == OK
    assert f(by(pool()), None, A, 3, None) == NULL
    assert f(by(pool()), A, None, 3, None) == NULL
    assert f(by(pool(stride=100)), A, A, 3, None) == SHAPE


def test_swap_argument_checks(lib):
    """Host block ids are checked before any copy: one id outside
    [0, num_blocks) rejects the whole call."""
    import numpy as np

    by = ctypes.byref
    good = np.array([0, 1, 15], np.int32)
    for f in (lib.kv_swap_out, lib.kv_swap_in):
        for bad in ([0, 16], [-1], [3, 2, 99]):
            ids = np.array(bad, np.int32)
            assert f(by(pool()), ids.ctypes.data, len(bad), A, A, None) == -11
        assert f(by(pool()), good.ctypes.data, 0, A, A, None) == OK
        assert f(by(pool()), good.ctypes.data, -1, A, A, None) == SHAPE
        assert f(by(pool()), None, 3, A, A, None) == NULL
        assert f(by(pool()), good.ctypes.data, 3, None, A, None) == NULL
        assert f(by(pool()), good.ctypes.data, 3, A, None, None) == NULL   # V pool set, no V buffer
        assert f(None, good.ctypes.data, 3, A, A, None) == NULL
        assert f(by(pool(dtype=9)), good.ctypes.data, 3, A, A, None) == DTYPE


def test_make_pool_combined_layout():
    """The K and V views of a combined (num_blocks, 2, layers, block_size,
    heads, head_dim) cache: V starts one dense block after K, and both step
    two dense blocks per block."""
    import torch

    kv = torch.zeros(5, 2, 3, 16, 2, 64, dtype=torch.bfloat16)
    k, v = N.combined_views(kv)
    p = N.make_pool(k, v)
    dense = 3 * 16 * 2 * 64 * 2
    assert p.block_stride == 2 * dense
    assert p.v - p.k == dense
    assert (p.num_blocks, p.num_layers, p.block_size, p.num_kv_heads, p.head_dim) == (5, 3, 16, 2, 64)
    assert N.make_pool(torch.zeros(5, 3, 16, 2, 64, dtype=torch.bfloat16)).block_stride == 0
    with pytest.raises(ValueError):
        N.make_pool(kv[:, :, 0])                      # not dense within a block
    with pytest.raises(ValueError):
        N.make_pool(k, torch.zeros(5, 3, 16, 2, 64, dtype=torch.bfloat16))   # strides differ
    with pytest.raises(ValueError):
        N.combined_views(torch.zeros(5, 3, 3, 16, 2, 64))


def test_quantized_pool_checks(lib):
    """An int8 pool needs 16-byte aligned scale arrays; prefill refuses it;
    decode and decode with append take it (checked like a float pool)."""
    by = ctypes.byref
    I8 = 2
    sc = lib.kv_scatter
    assert sc(by(pool(dtype=I8, ks=None)), 0, A, A, A, 4, None) == NULL
    assert sc(by(pool(dtype=I8, vs=None)), 0, A, A, A, 4, None) == NULL
    assert sc(by(pool(dtype=I8, v=None, vs=None)), 0, A, None, A, 0, None) == OK
    assert sc(by(pool(dtype=I8, ks=0x3004)), 0, A, A, A, 4, None) == ALIGN
    assert sc(by(pool(dtype=I8, d=96)), 0, A, A, A, 4, None) == UNSUP
    assert sc(by(pool(dtype=I8)), 0, A, A, A, 0, None) == OK
    assert sc(by(pool(dtype=0, ks=None, vs=None)), 0, A, A, A, 0, None) == OK   # float: ignored

    dec = lib.paged_attn_decode

    def decode(p, split=0, hq=32):
        return dec(by(p), 0, A, hq, A, 8, A, A, 4, 100, 0.1, split, A, A, 1 << 30, None)

    assert decode(pool(dtype=I8), split=-1) == SHAPE
    assert decode(pool(dtype=I8, d=96)) == UNSUP
    assert decode(pool(dtype=I8), hq=24) == UNSUP
    assert decode(pool(dtype=I8, ks=None)) == NULL
    app = lib.paged_attn_decode_append
    assert app(by(pool(dtype=I8)), 0, A, 32, None, A, A, 8, A, A, 4, 100, 0.1, 0, A, A, 1 << 30,
               None) == NULL                                # accepted: the new rows are checked
    assert app(by(pool(dtype=I8)), 0, A, 32, A + 4, A, A, 8, A, A, 4, 100, 0.1, 0, A, A, 1 << 30,
               None) == ALIGN
    assert app(by(pool(dtype=I8, d=96)), 0, A, 32, A, A, A, 8, A, A, 4, 100, 0.1, 0, A, A, 1 << 30,
               None) == UNSUP
    pre = lib.paged_attn_prefill
    assert pre(by(pool(dtype=I8)), 0, A, 32, A, 64, 16, A, 8, A, A, 4, 0.1, A, None) == UNSUP
    f = lib.paged_attn_decode_schedule
    split = lib.paged_attn_decode_split_tokens
    assert f(32, 8, 32, 128, 2048, 16, I8, 0) == 1            # the device-planned split
    assert f(65, 8, 32, 128, 2048, 16, I8, 0) == 256      # 520 pairs: up to 32 items per CU
    assert f(32, 8, 32, 128, 2048, 16, I8, -1) == SHAPE


def test_int4_pool_checks(lib):
    """An int4 pool (two codes per byte) needs an even head_dim and its scale
    arrays; decode, decode with append and the copies take it like int8;
    prefill refuses it."""
    by = ctypes.byref
    I4 = 3
    sc = lib.kv_scatter
    assert sc(by(pool(dtype=I4, ks=None)), 0, A, A, A, 4, None) == NULL
    assert sc(by(pool(dtype=I4, d=63)), 0, A, A, A, 4, None) == SHAPE
    assert sc(by(pool(dtype=I4, d=96)), 0, A, A, A, 4, None) == UNSUP
    assert sc(by(pool(dtype=I4)), 0, A, A, A, 0, None) == OK
    dec = lib.paged_attn_decode

    def decode(p, split=0, hq=32):
        return dec(by(p), 0, A, hq, A, 8, A, A, 4, 100, 0.1, split, A, A, 1 << 30, None)

    assert decode(pool(dtype=I4), split=-1) == SHAPE
    assert decode(pool(dtype=I4, d=96)) == UNSUP
    assert decode(pool(dtype=I4, vs=None)) == NULL
    app = lib.paged_attn_decode_append
    assert app(by(pool(dtype=I4)), 0, A, 32, A, None, A, 8, A, A, 4, 100, 0.1, 0, A, A, 1 << 30,
               None) == NULL
    assert app(by(pool(dtype=I4, d=63)), 0, A, 32, A, A, A, 8, A, A, 4, 100, 0.1, 0, A, A, 1 << 30,
               None) == SHAPE
    pre = lib.paged_attn_prefill
    assert pre(by(pool(dtype=I4)), 0, A, 32, A, 64, 16, A, 8, A, A, 4, 0.1, A, None) == UNSUP
    f = lib.paged_attn_decode_schedule
    assert f(32, 8, 32, 128, 2048, 16, I4, 0) == 1
    assert f(65, 8, 32, 128, 2048, 16, I4, 0) == 256


def test_quantized_pool_binding():
    """QuantizedPool pairs describe an int8 pool (scale pointers set, dtype
    PKV_I8); their rows, queries and outputs are bf16; a quantised K with a
    float V is refused."""
    import torch

    k = N.QuantizedPool.empty(6, 2, 16, 2, 64, "cpu")
    v = N.QuantizedPool.empty(6, 2, 16, 2, 64, "cpu")
    p = N.make_pool(k, v)
    assert p.dtype == 2 and p.k_scale == k.scales.data_ptr() and p.v_scale == v.scales.data_ptr()
    assert p.block_stride == 0 and N._row_dtype(k) == torch.bfloat16
    with pytest.raises(TypeError):
        N.make_pool(k, torch.zeros(6, 2, 16, 2, 64))
    with pytest.raises(ValueError):
        N.QuantizedPool(k.codes, torch.zeros(6, 2, 16, 2))
    buf = torch.zeros(3 * (2 * 16 * 2 * 64 + 2 * 2 * 16 * 4), dtype=torch.uint8)
    codes, scales = N.split_swapped_q8(buf, k, 3)
    assert codes.shape == (3, 2, 16, 2, 64) and scales.shape == (3, 2, 2, 16)
    k4 = N.QuantizedPool.empty(6, 2, 16, 2, 64, "cpu", bits=4)
    v4 = N.QuantizedPool.empty(6, 2, 16, 2, 64, "cpu", bits=4)
    assert k4.codes.shape == (6, 2, 16, 2, 32) and k4.codes.dtype == torch.uint8
    assert tuple(k4.shape) == (6, 2, 16, 2, 64) and k4.bits == 4
    p4 = N.make_pool(k4, v4)
    assert p4.dtype == 3 and p4.head_dim == 64
    with pytest.raises(TypeError):
        N.make_pool(k4, v)                            # int4 K with int8 V
    buf4 = torch.zeros(3 * (2 * 16 * 2 * 32 + 2 * 2 * 16 * 4), dtype=torch.uint8)
    codes, scales = N.split_swapped_q8(buf4, k4, 3)
    assert codes.shape == (3, 2, 16, 2, 32) and codes.dtype == torch.uint8
