"""Parity of the one-launch decode step (paged_attn_decode_append) with the
oracle: each sequence's new K/V row lands at logical position seq_len - 1
(the oracle's slot mapping followed by its scatter, bit for bit; no other
byte of the pool changes), and the output is the oracle's decode over the
updated pool (max abs error 2e-2 for bf16 inputs, 1e-5 for fp32).  The
output is also bitwise the output of kv_append followed by
paged_attn_decode with the same schedule.
"""
import numpy as np
import pytest
import torch

import oracle as O
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import TOL, bits, compact, host, max_abs_err, oracle_threads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def small(dev, dtype=torch.bfloat16, head_dim=128, group=4, seed=300, num_seqs=6, min_len=1,
          max_len=700, block_size=16, num_kv_heads=2):
    nb = (num_seqs * (max_len + 2 * block_size)) // block_size + 64
    w = W.decode_batch(device=dev, seed=seed, num_seqs=num_seqs, min_len=min_len,
                       max_len=max_len, num_blocks=nb, num_layers=3, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, num_q_heads=num_kv_heads * group, dtype=dtype, layer=1,
                       offsets="random", block_size=block_size)
    return W.decode_tokens(w)   # k_new/v_new: one row per sequence with seq_len > 0


def new_rows_for_all(w):
    """k_new/v_new indexed by sequence (decode_tokens gives rows only for
    sequences with tokens; the entry point takes one row per sequence)."""
    shape = (w.num_seqs, w.num_kv_heads, w.head_dim)
    kn = torch.zeros(shape, dtype=w.dtype, device=w.k_pool.device)
    vn = torch.zeros_like(kn)
    seqs = w.token_seq.long()
    kn[seqs] = w.k_new
    vn[seqs] = w.v_new
    return kn, vn


def oracle_step(w, kn, vn):
    """Oracle: slot mapping + scatter of the new rows into a host copy of
    the pool at the layer (all blocks), then decode over it."""
    k = host(w.k_pool).copy()
    v = host(w.v_pool).copy()
    lens = host(w.seq_lens)
    live = np.flatnonzero(lens > 0).astype(np.int32)
    slots = O.slot_mapping(host(w.block_tables), host(w.offsets), live,
                           (lens[live] - 1).astype(np.int32), w.block_size)
    O.scatter(k, w.layer, host(kn)[live], slots)
    O.scatter(v, w.layer, host(vn)[live], slots)
    out = O.decode(k, v, w.layer, host(w.q), host(w.block_tables), lens, host(w.offsets),
                   w.scale, num_threads=oracle_threads())
    return k, v, out


def run_append(w, kn, vn, split=0, ws=None):
    out = torch.full_like(w.q, float("nan"))
    return N.paged_attn_decode_append(w.k_pool, w.v_pool, w.layer, w.q, kn, vn, w.block_tables,
                                      w.seq_lens, w.offsets, w.max_seq_len, w.scale,
                                      split_tokens=split, out=out, workspace=ws)


CASES = [(torch.bfloat16, 16), (torch.bfloat16, 64), (torch.bfloat16, 0),
         (torch.bfloat16, N.SPLIT_PLANNED), (torch.float32, 16), (torch.float32, 0)]


@pytest.mark.parametrize("dtype,split", CASES)
def test_decode_append_small(dev, dtype, split):
    w = small(dev, dtype=dtype, seed=300 + split % 97, min_len=40)
    # an empty sequence, and lengths ending on a chunk / block edge (the
    # tables cover at least 40 tokens)
    lens = host(w.seq_lens).copy()
    lens[1], lens[2], lens[3] = 0, 16 - int(host(w.offsets)[2]), 17
    w.seq_lens = torch.from_numpy(lens).to(dev)
    w = W.decode_tokens(w)
    kn, vn = new_rows_for_all(w)
    k_ref, v_ref, ref = oracle_step(w, kn, vn)
    got = run_append(w, kn, vn, split)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(w.k_pool)), bits(k_ref))
    assert np.array_equal(bits(host(w.v_pool)), bits(v_ref))
    assert max_abs_err(got, ref) <= TOL[dtype]
    assert torch.all(got[1] == 0)


@pytest.mark.parametrize("bs", [1, 4, 32])
def test_decode_append_other_block_sizes(dev, bs):
    for dtype in (torch.bfloat16, torch.float32):
        w = small(dev, dtype=dtype, seed=310 + bs, block_size=bs, max_len=300)
        kn, vn = new_rows_for_all(w)
        k_ref, v_ref, ref = oracle_step(w, kn, vn)
        got = run_append(w, kn, vn)
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(w.k_pool)), bits(k_ref))
        assert np.array_equal(bits(host(w.v_pool)), bits(v_ref))
        assert max_abs_err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("split", [0, 64, N.SPLIT_PLANNED])
def test_decode_append_equals_append_then_decode(dev, split):
    """Same schedule, same bits: the fused step's output is the two-call
    step's output, and both leave the same pool."""
    w = small(dev, seed=320, num_seqs=9, max_len=1500)
    kn, vn = new_rows_for_all(w)
    k0, v0 = w.k_pool.clone(), w.v_pool.clone()
    fused = run_append(w, kn, vn, split)
    k1, v1 = w.k_pool.clone(), w.v_pool.clone()
    w.k_pool.copy_(k0)
    w.v_pool.copy_(v0)
    N.kv_append(w.k_pool, w.v_pool, w.layer, w.k_new, w.v_new, w.block_tables, w.offsets,
                w.token_seq, w.token_pos)
    plain = N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables, w.seq_lens,
                                w.offsets, w.max_seq_len, w.scale, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), plain.view(torch.int16))
    assert torch.equal(k1.view(torch.int16), w.k_pool.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), w.v_pool.view(torch.int16))


def test_decode_append_missing_block_writes_nothing(dev):
    """A -1 table entry at the new position: nothing is written into the
    sequence's blocks (the position is masked, as in decode); the other
    sequences are unaffected."""
    w = small(dev, seed=330, num_seqs=3, min_len=40, max_len=40)
    bt = w.block_tables.clone()
    lens, offs = host(w.seq_lens), host(w.offsets)
    j = (int(offs[0]) + int(lens[0]) - 1) // w.block_size
    bt[0, j] = -1
    w.block_tables = bt
    kn, vn = new_rows_for_all(w)
    k0, v0 = w.k_pool.clone(), w.v_pool.clone()
    got = run_append(w, kn, vn)
    torch.cuda.synchronize()
    ids0 = torch.from_numpy(host(bt[0][bt[0] >= 0]).astype(np.int64)).to(dev)
    assert torch.equal(w.k_pool[ids0].view(torch.int16), k0[ids0].view(torch.int16))
    assert torch.equal(w.v_pool[ids0].view(torch.int16), v0[ids0].view(torch.int16))
    assert torch.isfinite(got[0]).all()
    sel = torch.tensor([1, 2], device=dev)
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, bt[sel])
    ref = O.decode(k_c, v_c, 0, host(w.q[sel]), bt_c, lens[1:], offs[1:], w.scale)
    assert max_abs_err(got[sel], ref) <= TOL[w.dtype]


def test_decode_append_full_size_decode_batch(dev):
    """The bench's step at full size: 32 sequences, 16384-block pool of 32
    layers.  The new rows land at the oracle's slots, and the output meets
    the oracle's decode over the updated pool (compact copy)."""
    w = W.decode_tokens(W.decode_batch(device=dev, offsets="random"))
    kn, vn = new_rows_for_all(w)
    lens = host(w.seq_lens)
    live = np.flatnonzero(lens > 0).astype(np.int32)
    slots = O.slot_mapping(host(w.block_tables), host(w.offsets), live,
                           (lens[live] - 1).astype(np.int32), w.block_size)
    got = run_append(w, kn, vn)
    torch.cuda.synchronize()
    b = torch.from_numpy(slots // w.block_size).to(dev)
    r = torch.from_numpy(slots % w.block_size).to(dev)
    assert torch.equal(w.k_pool[b, w.layer, r].view(torch.int16), kn[live].view(torch.int16))
    assert torch.equal(w.v_pool[b, w.layer, r].view(torch.int16), vn[live].view(torch.int16))
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, w.block_tables)
    ref = O.decode(k_c, v_c, 0, host(w.q), bt_c, lens, host(w.offsets), w.scale,
                   num_threads=oracle_threads())
    assert max_abs_err(got, ref) <= TOL[w.dtype]


def oracle_partial_step(w, kn, vn, lens_attend, write):
    """Oracle pool after writing the new rows of the sequences in `write`
    (slot mapping + scatter), and its decode over lens_attend tokens."""
    k = host(w.k_pool).copy()
    v = host(w.v_pool).copy()
    lens = host(w.seq_lens)
    live = np.array([s for s in range(w.num_seqs) if lens[s] > 0 and write[s]], np.int32)
    if live.size:
        slots = O.slot_mapping(host(w.block_tables), host(w.offsets), live,
                               (lens[live] - 1).astype(np.int32), w.block_size)
        O.scatter(k, w.layer, host(kn)[live], slots)
        O.scatter(v, w.layer, host(vn)[live], slots)
    out = O.decode(k, v, w.layer, host(w.q), host(w.block_tables),
                   np.asarray(lens_attend, np.int32), host(w.offsets), w.scale,
                   num_threads=oracle_threads())
    return k, v, out


STALE_CASES = [(torch.bfloat16, 0), (torch.bfloat16, 64), (torch.bfloat16, 16),
               (torch.bfloat16, N.SPLIT_PLANNED),
               (torch.float32, 64), (torch.float32, 0)]


@pytest.mark.parametrize("dtype,split", STALE_CASES)
def test_stale_max_seq_len_then_correct_call(dev, dtype, split):
    """A caller's max_seq_len one below the longest sequence breaks the
    contract: that sequence is attended over its first max_seq_len tokens
    and its new row is not written (it would land on a cached token's slot
    under the clamped length), every other sequence is computed exactly,
    and the workspace is left reusable -- a correct call on the same
    workspace afterwards matches the oracle.  Sequence 0 has offset 15 and
    690 tokens, so at 64-token splits its last split index is one past the
    splits a 689-token bound provides."""
    nb = 6 * 46 + 64
    w = W.decode_batch(device=dev, seed=340, num_seqs=6, min_len=690, max_len=690, num_blocks=nb,
                       num_layers=3, num_kv_heads=2, head_dim=128, num_q_heads=8, dtype=dtype,
                       layer=1, offsets=[15, 3, 0, 7, 15, 9])
    lens = host(w.seq_lens).copy()
    lens[1:] = [689, 300, 17, 512, 641]
    w.seq_lens = torch.from_numpy(lens).to(dev)
    w = W.decode_tokens(w)
    kn, vn = new_rows_for_all(w)
    mx = int(lens.max())
    need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                              w.head_dim, mx, w.block_size, split)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    k0, v0 = w.k_pool.clone(), w.v_pool.clone()

    clamp = np.minimum(lens, mx - 1)
    k_ref, v_ref, ref = oracle_partial_step(w, kn, vn, clamp, lens <= mx - 1)
    out = torch.full_like(w.q, float("nan"))
    N.paged_attn_decode_append(w.k_pool, w.v_pool, w.layer, w.q, kn, vn, w.block_tables,
                               w.seq_lens, w.offsets, mx - 1, w.scale, split_tokens=split,
                               out=out, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(w.k_pool)), bits(k_ref))
    assert np.array_equal(bits(host(w.v_pool)), bits(v_ref))
    assert max_abs_err(out, ref) <= TOL[dtype]

    # the correct call, same workspace, from the original pool
    w.k_pool.copy_(k0)
    w.v_pool.copy_(v0)
    k_ref, v_ref, ref = oracle_step(w, kn, vn)
    out = torch.full_like(w.q, float("nan"))
    N.paged_attn_decode_append(w.k_pool, w.v_pool, w.layer, w.q, kn, vn, w.block_tables,
                               w.seq_lens, w.offsets, mx, w.scale, split_tokens=split, out=out,
                               workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(w.k_pool)), bits(k_ref))
    assert np.array_equal(bits(host(w.v_pool)), bits(v_ref))
    assert max_abs_err(out, ref) <= TOL[dtype]
