"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: slot mapping, scatter and gather bit-exact (compared as integer bit
patterns, so NaN payloads count); decode attention within max abs error 2e-2
for bf16 inputs and 1e-5 for fp32 inputs against the float64 oracle.

Small cases run the oracle on the whole pool and span several 16-token
chunks, several splits and ragged tails; the full-size cases (the five
workload presets) hand the oracle a compact copy of the referenced blocks.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import (TOL, as_f64, bits, compact, host, max_abs_err, oracle_decode_for,
                               oracle_threads, row_starts)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


_FULL = {}


def full(name, dev):
    """Full-size preset workloads, built once; at most one kept alive."""
    if name not in _FULL:
        _FULL.clear()
        torch.cuda.empty_cache()
        _FULL[name] = W.PRESETS[name](device=dev)
    return _FULL[name]


def small_decode(dev, dtype=torch.bfloat16, head_dim=128, group=4, num_kv_heads=2, seed=11,
                 num_seqs=6, min_len=1, max_len=700, offsets="random", num_blocks=512):
    return W.decode_batch(device=dev, seed=seed, num_seqs=num_seqs, min_len=min_len,
                          max_len=max_len, num_blocks=num_blocks, num_layers=3,
                          num_kv_heads=num_kv_heads, head_dim=head_dim,
                          num_q_heads=num_kv_heads * group, dtype=dtype, layer=1,
                          offsets=offsets)


def set_lens(w, lens, offsets):
    """Replace lengths/offsets (tables already cover up to max_len + 15)."""
    w.seq_lens = torch.tensor(lens, dtype=torch.int32, device=w.seq_lens.device)
    w.offsets = torch.tensor(offsets, dtype=torch.int32, device=w.offsets.device)
    return w


def run_decode(w, split=0, q=None, workspace=None):
    """Decode through the C ABI into an output prefilled with NaN, so any
    element the kernels fail to write shows up."""
    q = w.q if q is None else q
    out = torch.full_like(q, float("nan"))
    return N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, q, w.block_tables, w.seq_lens,
                               w.offsets, w.max_seq_len, w.scale, split_tokens=split, out=out,
                               workspace=workspace)


# ---------------------------------------------------------------------------
# slot mapping
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "prefill", "prefill_randpad", "decode_batch",
                                  "prefix_sharing", "long_context"])
def test_slot_mapping_bit_exact(dev, name):
    if name == "tiny":
        w = W.tiny(device=dev)
    elif name.startswith("prefill"):
        w = W.prefill(device=dev, random_padding=name.endswith("randpad"), with_pools=False)
    else:
        w = W.decode_tokens(W.PRESETS[name](device=dev, with_pools=False))
    got = N.kv_slot_mapping(w.block_tables, w.offsets, w.token_seq, w.token_pos, w.block_size)
    ref = O.slot_mapping(host(w.block_tables), host(w.offsets), host(w.token_seq),
                         host(w.token_pos), w.block_size)
    assert np.array_equal(host(got), ref)


def test_slot_mapping_outside_table_is_padding(dev):
    bt = torch.tensor([[3, 1]], dtype=torch.int32, device=dev)
    off = torch.tensor([4], dtype=torch.int32, device=dev)
    ts = torch.tensor([0, 0, -1, 0, 7], dtype=torch.int32, device=dev)
    tp = torch.tensor([27, 28, 0, -1, 0], dtype=torch.int32, device=dev)
    got = host(N.kv_slot_mapping(bt, off, ts, tp, 16))
    ref = O.slot_mapping(host(bt), host(off), host(ts[:1]), host(tp[:1]), 16)
    assert got[0] == ref[0]
    assert list(got[1:]) == [-1, -1, -1, -1]


# ---------------------------------------------------------------------------
# scatter
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,hkv,d,bs", [(torch.float32, 2, 64, 16), (torch.bfloat16, 8, 128, 16),
                                            (torch.bfloat16, 2, 64, 4), (torch.float32, 1, 32, 1)])
def test_scatter_small_pool_bit_exact(dev, dtype, hkv, d, bs):
    g = torch.Generator().manual_seed(5)
    nb, nl, layer = 64, 3, 2
    shape = (nb, nl, bs, hkv, d)
    # random bit patterns (NaN payloads included) for pool and new rows
    ity = torch.int16 if dtype == torch.bfloat16 else torch.int32
    lo, hi = (-(1 << 15), 1 << 15) if ity == torch.int16 else (-(1 << 31), 1 << 31)
    k = torch.randint(lo, hi, shape, generator=g, dtype=ity).view(dtype).to(dev)
    v = torch.randint(lo, hi, shape, generator=g, dtype=ity).view(dtype).to(dev)
    n = min(300, nb * bs - 8)
    slots = torch.randperm(nb * bs, generator=g)[:n].to(torch.int64)
    slots[torch.randperm(n, generator=g)[:n // 8]] = -1
    ks = torch.randint(lo, hi, (n, hkv, d), generator=g, dtype=ity).view(dtype).to(dev)
    vs = torch.randint(lo, hi, (n, hkv, d), generator=g, dtype=ity).view(dtype).to(dev)
    ref_k, ref_v = host(k).copy(), host(v).copy()
    O.scatter(ref_k, layer, host(ks), slots.numpy())
    O.scatter(ref_v, layer, host(vs), slots.numpy())
    N.kv_scatter(k, v, layer, ks, vs, slots.to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(k)), bits(ref_k))
    assert np.array_equal(bits(host(v)), bits(ref_v))


def test_scatter_all_padding_leaves_pool(dev):
    w = W.prefill(device=dev, num_blocks=256, num_layers=2, layer=1, num_requests=2,
                  prompt_len=64)
    before_k, before_v = w.k_pool.clone(), w.v_pool.clone()
    slots = torch.full((w.k_new.shape[0],), -1, dtype=torch.int64, device=dev)
    N.kv_scatter(w.k_pool, w.v_pool, w.layer, w.k_new, w.v_new, slots)
    torch.cuda.synchronize()
    assert torch.equal(w.k_pool.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(w.v_pool.view(torch.int16), before_v.view(torch.int16))


@pytest.mark.parametrize("random_padding", [False, True])
def test_scatter_prefill_full_size(dev, random_padding):
    """8 x 1024 rows, 10% padding, into the 16384-block 32-layer pool at layer
    17: the touched blocks match the oracle byte for byte (all layers), every
    other block is untouched."""
    w = W.prefill(device=dev, random_padding=random_padding)
    slots_np = O.slot_mapping(host(w.block_tables), host(w.offsets), host(w.token_seq),
                              host(w.token_pos), w.block_size)
    assert int((slots_np < 0).sum()) == w.meta["padding_rows"]
    bt = w.block_tables.cpu()
    ids = torch.unique(bt[bt >= 0]).to(torch.int64)
    dev_ids = ids.to(dev)
    k_before = host(w.k_pool.index_select(0, dev_ids))
    v_before = host(w.v_pool.index_select(0, dev_ids))
    untouched = torch.ones(w.num_blocks, dtype=torch.bool)
    untouched[ids] = False
    untouched = untouched.to(dev)
    ku_before = w.k_pool[untouched].clone()
    # oracle on the compact copy: same tables renumbered into `ids`
    pos = torch.searchsorted(ids, bt.clamp(min=0).to(torch.int64)).to(torch.int32)
    bt_c = torch.where(bt >= 0, pos, torch.full_like(pos, -1)).numpy()
    slots_c = O.slot_mapping(bt_c, host(w.offsets), host(w.token_seq), host(w.token_pos),
                             w.block_size)
    O.scatter(k_before, w.layer, host(w.k_new), slots_c)
    O.scatter(v_before, w.layer, host(w.v_new), slots_c)

    N.kv_scatter(w.k_pool, w.v_pool, w.layer, w.k_new, w.v_new,
                 torch.from_numpy(slots_np).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(w.k_pool.index_select(0, dev_ids))), bits(k_before))
    assert np.array_equal(bits(host(w.v_pool.index_select(0, dev_ids))), bits(v_before))
    assert torch.equal(w.k_pool[untouched].view(torch.int16), ku_before.view(torch.int16))
    if not random_padding:
        # gather(scatter(K)) == K on the valid rows, in request order
        total = int(w.seq_lens.sum())
        k_out = torch.empty((total, w.num_kv_heads, w.head_dim), dtype=w.dtype, device=dev)
        v_out = torch.empty_like(k_out)
        N.kv_gather(w.k_pool, w.v_pool, w.layer, w.block_tables, w.seq_lens, w.offsets,
                    row_starts(w.seq_lens), w.max_seq_len, k_out, v_out)
        valid = (w.token_seq >= 0)
        assert torch.equal(k_out.view(torch.int16), w.k_new[valid].view(torch.int16))
        assert torch.equal(v_out.view(torch.int16), w.v_new[valid].view(torch.int16))


# ---------------------------------------------------------------------------
# append (slot mapping + scatter in one kernel)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "prefill_randpad", "decode_batch"])
def test_append_bit_exact(dev, name):
    """kv_append writes exactly what the oracle's slot mapping followed by
    its scatter writes (compact copy of the touched blocks, all layers) and
    returns the oracle's slots; untouched blocks keep their bytes."""
    if name == "tiny":
        w = W.tiny(device=dev)
    elif name == "prefill_randpad":
        w = W.prefill(device=dev, random_padding=True)
    else:
        w = W.decode_tokens(W.decode_batch(device=dev, offsets="random"))
    # rows past the table and padding rows must be skipped, too
    ts, tp = w.token_seq.clone(), w.token_pos.clone()
    past = None
    if ts.shape[0] > 4:
        ts[1] = -1
        past = 2
        tp[past] = w.block_tables.shape[1] * w.block_size
    # the oracle refuses a position outside the table; the kernel marks it -1
    keep = np.ones(ts.shape[0], dtype=bool)
    if past is not None:
        keep[past] = False

    def oracle_slots(bt_np):
        out = np.full(ts.shape[0], -1, dtype=np.int64)
        out[keep] = O.slot_mapping(bt_np, host(w.offsets), host(ts)[keep], host(tp)[keep],
                                   w.block_size)
        return out

    slots_np = oracle_slots(host(w.block_tables))
    bt = w.block_tables.cpu()
    ids = torch.unique(bt[bt >= 0]).to(torch.int64)
    dev_ids = ids.to(dev)
    k_ref = host(w.k_pool.index_select(0, dev_ids))
    v_ref = host(w.v_pool.index_select(0, dev_ids))
    untouched = torch.ones(w.num_blocks, dtype=torch.bool)
    untouched[ids] = False
    untouched = untouched.to(dev)
    ku_before = w.k_pool[untouched].clone()
    pos = torch.searchsorted(ids, bt.clamp(min=0).to(torch.int64)).to(torch.int32)
    bt_c = torch.where(bt >= 0, pos, torch.full_like(pos, -1)).numpy()
    slots_c = oracle_slots(bt_c)
    O.scatter(k_ref, w.layer, host(w.k_new), slots_c)
    O.scatter(v_ref, w.layer, host(w.v_new), slots_c)

    got = torch.full((ts.shape[0],), 12345, dtype=torch.int64, device=dev)
    N.kv_append(w.k_pool, w.v_pool, w.layer, w.k_new, w.v_new, w.block_tables, w.offsets, ts, tp,
                slot_mapping_out=got)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), slots_np)
    assert np.array_equal(bits(host(w.k_pool.index_select(0, dev_ids))), bits(k_ref))
    assert np.array_equal(bits(host(w.v_pool.index_select(0, dev_ids))), bits(v_ref))
    ity = torch.int16 if w.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(w.k_pool[untouched].view(ity), ku_before.view(ity))


def test_append_k_only_without_slots_out(dev):
    w = W.tiny(device=dev)
    k_ref = host(w.k_pool).copy()
    slots = O.slot_mapping(host(w.block_tables), host(w.offsets), host(w.token_seq),
                           host(w.token_pos), w.block_size)
    O.scatter(k_ref, w.layer, host(w.k_new), slots)
    v_before = w.v_pool.clone()
    N.kv_append(w.k_pool, None, w.layer, w.k_new, None, w.block_tables, w.offsets, w.token_seq,
                w.token_pos)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(w.k_pool)), bits(k_ref))
    assert torch.equal(w.v_pool.view(torch.int32), v_before.view(torch.int32))


# ---------------------------------------------------------------------------
# gather
# ---------------------------------------------------------------------------
def gather_both(w):
    total = int(w.seq_lens.sum())
    k_out = torch.empty((max(total, 1), w.num_kv_heads, w.head_dim), dtype=w.dtype, device=w.k_pool.device)
    v_out = torch.empty_like(k_out)
    N.kv_gather(w.k_pool, w.v_pool, w.layer, w.block_tables, w.seq_lens, w.offsets,
                row_starts(w.seq_lens), w.max_seq_len, k_out, v_out)
    torch.cuda.synchronize()
    return k_out[:total], v_out[:total]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_gather_small_bit_exact(dev, dtype, d):
    w = small_decode(dev, dtype=dtype, head_dim=d, seed=21)
    k_out, v_out = gather_both(w)
    ref_k = O.gather(host(w.k_pool), w.layer, host(w.block_tables), host(w.seq_lens), host(w.offsets))
    ref_v = O.gather(host(w.v_pool), w.layer, host(w.block_tables), host(w.seq_lens), host(w.offsets))
    assert np.array_equal(bits(host(k_out)), bits(ref_k))
    assert np.array_equal(bits(host(v_out)), bits(ref_v))


def test_gather_edge_lengths_and_offsets(dev):
    w = small_decode(dev, seed=22, num_seqs=18, min_len=40, max_len=40, offsets=None)
    lens = [0, 1, 15, 16, 17, 33] * 3
    offs = [0] * 6 + [1] * 6 + [15] * 6
    set_lens(w, lens, offs)
    k_out, v_out = gather_both(w)
    ref_k = O.gather(host(w.k_pool), w.layer, host(w.block_tables), host(w.seq_lens), host(w.offsets))
    assert np.array_equal(bits(host(k_out)), bits(ref_k))


@pytest.mark.parametrize("name", ["tiny", "decode_batch", "prefix_sharing", "long_context"])
def test_gather_full_size_bit_exact(dev, name):
    w = W.tiny(device=dev) if name == "tiny" else full(name, dev)
    k_out, v_out = gather_both(w)
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, w.block_tables)
    ref_k = O.gather(k_c, 0, bt_c, host(w.seq_lens), host(w.offsets))
    ref_v = O.gather(v_c, 0, bt_c, host(w.seq_lens), host(w.offsets))
    assert np.array_equal(bits(host(k_out)), bits(ref_k))
    assert np.array_equal(bits(host(v_out)), bits(ref_v))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_small_grid(dev, dtype, head_dim, group):
    w = small_decode(dev, dtype=dtype, head_dim=head_dim, group=group, seed=30 + group)
    ref = oracle_decode_for(w)
    for split in (16, 64, 0) + ((N.SPLIT_PLANNED,) if dtype == torch.bfloat16 else ()):
        got = run_decode(w, split)
        err = max_abs_err(got, ref)
        assert err <= TOL[dtype], (split, err)


@pytest.mark.parametrize("bs", [1, 4, 32])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_other_block_sizes(dev, bs, dtype):
    """block_size below 16 (a 16-position chunk spans several blocks) and
    above it (a chunk is part of one block), with random offsets."""
    w = W.decode_batch(device=dev, seed=60 + bs, num_seqs=5, min_len=1, max_len=300,
                       num_blocks=2048 // bs + 64, num_layers=2, num_kv_heads=2, head_dim=128,
                       num_q_heads=8, dtype=dtype, layer=1, offsets="random", block_size=bs)
    ref = oracle_decode_for(w)
    for split in (16, 64, 0) + ((N.SPLIT_PLANNED,) if dtype == torch.bfloat16 else ()):
        if split > 0 and split // bs + 2 > 1024:
            continue
        got = run_decode(w, split)
        assert max_abs_err(got, ref) <= TOL[dtype], split


@pytest.mark.parametrize("split", [16, 32, 0, N.SPLIT_PLANNED])
def test_decode_edge_lengths_and_offsets(dev, split):
    w = small_decode(dev, seed=40, num_seqs=18, min_len=40, max_len=40, offsets=None)
    set_lens(w, [0, 1, 15, 16, 17, 33] * 3, [0] * 6 + [1] * 6 + [15] * 6)
    ref = oracle_decode_for(w)
    got = run_decode(w, split)
    assert max_abs_err(got, ref) <= TOL[w.dtype]
    assert torch.all(got[0] == 0) and torch.all(got[6] == 0) and torch.all(got[12] == 0)


def test_decode_single_token_is_v_row(dev):
    w = small_decode(dev, seed=41, num_seqs=4, min_len=1, max_len=1)
    got = run_decode(w)
    ref = oracle_decode_for(w)  # exact V rows in float64
    assert np.array_equal(as_f64(got), ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_ignores_unowned_nan_slots(dev, dtype):
    """Every pool slot at the tested layer that no sequence owns is NaN:
    masked positions (before the offset, after seq_len, other blocks) must
    not reach the output."""
    w = small_decode(dev, dtype=dtype, seed=42, head_dim=64 if dtype == torch.float32 else 128)
    lens = host(w.seq_lens)
    tseq = np.concatenate([np.full(l, s, np.int32) for s, l in enumerate(lens)])
    tpos = np.concatenate([np.arange(l, dtype=np.int32) for l in lens])
    owned = O.slot_mapping(host(w.block_tables), host(w.offsets), tseq, tpos, w.block_size)
    mask = torch.ones(w.num_blocks * w.block_size, dtype=torch.bool)
    mask[torch.from_numpy(owned)] = False
    mask = mask.view(w.num_blocks, w.block_size).to(dev)
    for pool in (w.k_pool, w.v_pool):
        lay = pool[:, w.layer]
        lay[mask] = float("nan")
    ref = oracle_decode_for(w)
    assert np.all(np.isfinite(ref))
    for split in (16, 0):
        got = run_decode(w, split)
        assert max_abs_err(got, ref) <= TOL[dtype]


def test_decode_tiny_config(dev):
    w = W.tiny(device=dev)
    assert w.scale == 1 / math.sqrt(64)
    got = run_decode(w)
    ref = oracle_decode_for(w)
    assert max_abs_err(got, ref) <= TOL[torch.float32]


@pytest.mark.parametrize("name", ["decode_batch", "prefix_sharing", "long_context"])
def test_decode_full_size(dev, name):
    w = full(name, dev)
    got = run_decode(w)
    ref = oracle_decode_for(w)   # every sequence
    err = max_abs_err(got, ref)
    print(f"{name}: split={N.paged_attn_decode_split_tokens(w.num_seqs, w.num_kv_heads, w.max_seq_len, w.block_size)} max_abs_err={err:.3e}")
    assert err <= TOL[w.dtype]
    # bitwise reproducible run to run
    again = run_decode(w)
    assert torch.equal(got.view(torch.int16), again.view(torch.int16))


def test_decode_long_context_other_splits(dev):
    """All 8 sequences of the long-context batch at explicit splits: 2048
    (16 splits per sequence, the merge kernel) and 8192 (4 splits, merged in
    the kernel)."""
    w = full("long_context", dev)
    ref = oracle_decode_for(w)
    for split in (2048, 8192):
        got = run_decode(w, split)
        assert max_abs_err(got, ref) <= TOL[w.dtype], split


def test_decode_block_relabelling_is_bitwise_invariant(dev):
    w = small_decode(dev, seed=43, num_blocks=400)
    a = run_decode(w, 64)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(1)).to(dev)
    k2 = torch.empty_like(w.k_pool)
    v2 = torch.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    bt = w.block_tables
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].to(torch.int32), bt)
    b = N.paged_attn_decode(k2, v2, w.layer, w.q, bt2, w.seq_lens, w.offsets, w.max_seq_len,
                            w.scale, split_tokens=64)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# validation and argument errors
# ---------------------------------------------------------------------------
def test_validate_counts_violations(dev):
    w = small_decode(dev, seed=50, num_seqs=4, min_len=20, max_len=60)
    assert N.kv_validate(w.k_pool, w.block_tables, w.seq_lens, w.offsets, w.max_seq_len) == 0
    bt = w.block_tables.clone()
    bt[1, 0] = w.num_blocks            # out of range, used
    offs = w.offsets.clone()
    offs[2] = w.block_size              # offset not < block_size
    lens = w.seq_lens.clone()
    lens[3] = bt.shape[1] * w.block_size + 1  # beyond capacity (and max_seq_len)
    slots = torch.tensor([-1, 0, w.num_blocks * w.block_size, -5], dtype=torch.int64, device=dev)
    n = N.kv_validate(w.k_pool, bt, lens, offs, w.max_seq_len, slots)
    # bad id (1) + bad offset (1) + seq 3 over capacity and max_seq_len (1)
    # + seq 3 now uses every entry of its row, so its -1 padding entries
    # count too + 2 bad slots
    pad3 = int((bt[3] < 0).sum())
    assert n == 5 + pad3, (n, pad3)


@pytest.mark.parametrize("split", [64, 16, 0, N.SPLIT_PLANNED])
def test_decode_workspace_reuse_leaves_counters_zero(dev, split):
    """One zeroed workspace serves successive calls of different shapes: each
    call gives the same bits as a call with a fresh workspace and leaves the
    split counters (the first bytes of the workspace) zero again.  Split 64
    keeps every sequence within 16 splits (merged by the last split's
    workgroup); split 16 goes past that (merged by the merge kernel)."""
    cases = [small_decode(dev, seed=60, num_seqs=12, max_len=300),
             small_decode(dev, seed=61, num_seqs=5, min_len=100, max_len=500, num_kv_heads=8,
                          group=1),
             set_lens(small_decode(dev, seed=62, num_seqs=6, min_len=300, max_len=300),
                      [0, 300, 1, 17, 0, 250], [3, 0, 15, 2, 0, 9])]
    need = max(N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                                  w.head_dim, w.max_seq_len, w.block_size, split)
               for w in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for w in cases:
        for _ in range(2):
            got = run_decode(w, split, workspace=ws)
            ref = run_decode(w, split)
            itype = torch.int16 if got.element_size() == 2 else torch.int32
            assert torch.equal(got.view(itype), ref.view(itype))
            cnt = (w.num_seqs * w.num_kv_heads * 4 + 255) // 256 * 256
            assert int(torch.count_nonzero(ws[:cnt])) == 0
        assert max_abs_err(got, oracle_decode_for(w)) <= TOL[w.dtype]


@pytest.mark.parametrize("num_seqs,max_len,num_blocks", [(300, 90, 2400), (96, 700, 4400)])
def test_decode_many_sequences_auto_split(dev, num_seqs, max_len, num_blocks):
    """Batches of more sequences than the device-planned schedule takes (at
    most 64) run the split schedule with the automatic split (with many
    (sequence, kv head) pairs: up to 32 work items per compute unit), every
    7th sequence empty.  A second call on the same workspace gives the same
    bits and the merge counters are zero after each call."""
    w = small_decode(dev, seed=70 + num_seqs, num_seqs=num_seqs, min_len=1, max_len=max_len,
                     num_blocks=num_blocks)
    lens = host(w.seq_lens).copy()
    lens[::7] = 0
    set_lens(w, lens.tolist(), host(w.offsets).tolist())
    sched = N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                         w.max_seq_len, w.block_size, w.dtype, 0)
    assert sched > 0 and sched != N.SCHEDULE_PLANNED and sched % 16 == 0
    need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                              w.head_dim, w.max_seq_len, w.block_size, 0)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    cnt = (w.num_seqs * w.num_kv_heads * 4 + 255) // 256 * 256
    got = run_decode(w, 0, workspace=ws)
    assert int(torch.count_nonzero(ws[:cnt])) == 0
    again = run_decode(w, 0, workspace=ws)
    assert int(torch.count_nonzero(ws[:cnt])) == 0
    assert torch.equal(got.view(torch.int16), again.view(torch.int16))
    assert max_abs_err(got, oracle_decode_for(w)) <= TOL[w.dtype]
    empty = np.flatnonzero(host(w.seq_lens) == 0)
    assert torch.all(got[torch.from_numpy(empty).to(dev)] == 0)


@pytest.mark.parametrize("num_seqs,max_len,num_kv_heads,num_blocks,empty_every",
                         [(1, 3000, 2, 256, 0), (64, 700, 2, 4096, 7), (40, 2048, 2, 5400, 0),
                          (64, 90, 8, 1024, 3), (32, 2048, 8, 4400, 0), (3, 40, 8, 64, 2)])
def test_decode_planned_schedule(dev, num_seqs, max_len, num_kv_heads, num_blocks, empty_every):
    """The device-planned split schedule (the automatic one for these bf16
    batches): every workgroup reads all lengths, picks the split and takes
    one (sequence, split, head group) piece -- full pieces from the front of
    the grid, first/last pieces from the back.  Cases cover a grid that holds
    every piece at the smallest split (1 and 3 sequences), the bound on the
    split that fits 2 workgroups per compute unit (64 x 700), head groups of
    4 kv heads (8 kv heads), random offsets, and empty sequences, whose
    outputs must be zero.  A second call on the same workspace gives the
    same bits and leaves the merge counters zero."""
    w = small_decode(dev, seed=90 + num_seqs, num_seqs=num_seqs, min_len=1, max_len=max_len,
                     num_kv_heads=num_kv_heads, num_blocks=num_blocks)
    lens = host(w.seq_lens).copy()
    if empty_every:
        lens[1::empty_every] = 0
    set_lens(w, lens.tolist(), host(w.offsets).tolist())
    pl = N.SPLIT_PLANNED
    for split in (0, pl):
        assert N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                            w.max_seq_len, w.block_size, w.dtype,
                                            split) == N.SCHEDULE_PLANNED
    need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                              w.head_dim, w.max_seq_len, w.block_size, pl)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    cnt = (w.num_seqs * w.num_kv_heads * 4 + 255) // 256 * 256
    got = run_decode(w, pl, workspace=ws)
    assert int(torch.count_nonzero(ws[:cnt])) == 0
    again = run_decode(w, pl, workspace=ws)
    assert int(torch.count_nonzero(ws[:cnt])) == 0
    assert torch.equal(got.view(torch.int16), again.view(torch.int16))
    assert max_abs_err(got, oracle_decode_for(w)) <= TOL[w.dtype]
    empty = np.flatnonzero(host(w.seq_lens) == 0)
    assert torch.all(got[torch.from_numpy(empty).to(dev)] == 0)
    # the same function as a fixed split
    assert float((got.float() - run_decode(w, 64).float()).abs().max()) <= TOL[w.dtype]


def test_decode_planned_refused_past_its_limits(dev):
    """More than 64 sequences (or fp32 pools): an explicit planned request is
    refused, and split_tokens = 0 takes another schedule."""
    w = small_decode(dev, seed=97, num_seqs=65, max_len=50, num_blocks=512)
    assert N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                        w.max_seq_len, w.block_size, w.dtype,
                                        0) != N.SCHEDULE_PLANNED
    with pytest.raises(N.PagedKVError) as e:
        run_decode(w, N.SPLIT_PLANNED)
    assert e.value.status == -8
    w32 = small_decode(dev, dtype=torch.float32, seed=98, num_seqs=4, max_len=50)
    with pytest.raises(N.PagedKVError) as e:
        run_decode(w32, N.SPLIT_PLANNED)
    assert e.value.status == -8
    got = run_decode(w, 0)
    assert max_abs_err(got, oracle_decode_for(w)) <= TOL[w.dtype]


def test_decode_rejects_unsupported_group(dev):
    w = small_decode(dev, seed=51, group=1, num_kv_heads=2, num_seqs=2)
    q3 = torch.zeros((2, 6, w.head_dim), dtype=w.dtype, device=dev)  # G = 3
    with pytest.raises(N.PagedKVError) as e:
        N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, q3, w.block_tables, w.seq_lens,
                            w.offsets, w.max_seq_len, w.scale)
    assert e.value.status == -8
