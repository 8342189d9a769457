"""Quantised int4 pools on the GPU, through the C ABI, against the oracle
(oracle/quant.py: the int8 reading at four bits, two codes per byte).

  * the quantising scatter and append write exactly the oracle's packed
    codes and scales (bit for bit), and nothing else;
  * the dequantising gather writes exactly bf16(code * scale);
  * decode over an int4 pool meets the oracle's float64 decode of the stored
    values within 2e-2 (the bf16 bar; queries and outputs are bf16), on
    random pool bytes (every code, -8 included);
  * whole-block copies and swaps move packed codes and scales bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import quant as Q
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import host, max_abs_err, row_starts

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def qpools(dev, nb, nl, bs, h, d, seed):
    kc, ks = W.int4_pool_tensors(nb, nl, bs, h, d, dev, seed)
    vc, vs = W.int4_pool_tensors(nb, nl, bs, h, d, dev, seed + 1)
    return N.QuantizedPool(kc, ks), N.QuantizedPool(vc, vs)


def bf16_rows(dev, n, h, d, seed, spread=True):
    x = torch.empty((n, h, d), dtype=torch.float32, device=dev)
    W.fill_normal_(x, seed)
    if not spread:
        return x.to(torch.bfloat16)
    g = torch.Generator(device=dev).manual_seed(seed + 7)
    mag = 10.0 ** (torch.rand((n, h, 1), generator=g, device=dev) * 4 - 2)
    return (x * mag).to(torch.bfloat16)


def workload(dev, seed, num_seqs=6, max_len=500, bs=16, hkv=2, group=4, d=128, min_len=1):
    nb = (num_seqs * (max_len + 2 * bs)) // bs + 64
    w = W.decode_batch(device=dev, seed=seed, num_seqs=num_seqs, min_len=min_len,
                       max_len=max_len, num_blocks=nb, num_layers=3, num_kv_heads=hkv,
                       head_dim=d, num_q_heads=hkv * group, dtype=torch.bfloat16, layer=1,
                       offsets="random", block_size=bs, with_pools=False)
    k, v = qpools(dev, nb, 3, bs, hkv, d, seed * 3)
    return w, k, v


def test_int4_pool_geometry(dev):
    k, v = qpools(dev, 10, 2, 16, 2, 128, 1)
    assert tuple(k.shape) == (10, 2, 16, 2, 128) and k.codes.shape[-1] == 64 and k.bits == 4
    p = N.make_pool(k, v)
    assert p.dtype == N.PKV_I4 and p.head_dim == 128


@pytest.mark.parametrize("d,h,bs", [(128, 8, 16), (64, 2, 4), (128, 2, 1), (64, 8, 32)])
def test_int4_quantising_scatter_is_the_oracles(dev, d, h, bs):
    nb = 80 // bs + 8
    k, v = qpools(dev, nb, 2, bs, h, d, 800 + d + bs)
    rows = 70
    ks = bf16_rows(dev, rows, h, d, 810)
    vs = bf16_rows(dev, rows, h, d, 811)
    ks[5] = 0                                       # a zero row: scale 0, codes 0
    rng = np.random.default_rng(812)
    slots = rng.permutation(nb * bs)[:rows].astype(np.int64)
    slots[[3, 17]] = -1
    kc, ksc = host(k.codes).copy(), host(k.scales).copy()
    vc, vsc = host(v.codes).copy(), host(v.scales).copy()
    Q.scatter_q4(kc, ksc, 1, host(ks), slots)
    Q.scatter_q4(vc, vsc, 1, host(vs), slots)
    N.kv_scatter(k, v, 1, ks, vs, torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(host(k.codes), kc) and np.array_equal(host(v.codes), vc)
    assert np.array_equal(host(k.scales).view(np.uint32), ksc.view(np.uint32))
    assert np.array_equal(host(v.scales).view(np.uint32), vsc.view(np.uint32))


def test_int4_quantising_append_is_the_oracles(dev):
    w, k, v = workload(dev, 820, num_seqs=5, max_len=200)
    w = W.decode_tokens(w)
    kn = bf16_rows(dev, w.token_seq.shape[0], w.num_kv_heads, w.head_dim, 821)
    vn = bf16_rows(dev, w.token_seq.shape[0], w.num_kv_heads, w.head_dim, 822)
    slots = O.slot_mapping(host(w.block_tables), host(w.offsets), host(w.token_seq),
                           host(w.token_pos), w.block_size)
    kc, ksc = host(k.codes).copy(), host(k.scales).copy()
    vc, vsc = host(v.codes).copy(), host(v.scales).copy()
    Q.scatter_q4(kc, ksc, w.layer, host(kn), slots)
    Q.scatter_q4(vc, vsc, w.layer, host(vn), slots)
    out = torch.empty(slots.shape[0], dtype=torch.int64, device=dev)
    N.kv_append(k, v, w.layer, kn, vn, w.block_tables, w.offsets, w.token_seq, w.token_pos,
                slot_mapping_out=out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), slots)
    assert np.array_equal(host(k.codes), kc) and np.array_equal(host(v.codes), vc)
    assert np.array_equal(host(k.scales).view(np.uint32), ksc.view(np.uint32))
    assert np.array_equal(host(v.scales).view(np.uint32), vsc.view(np.uint32))


@pytest.mark.parametrize("d,bs", [(128, 16), (64, 4), (128, 1), (64, 32)])
def test_int4_dequantising_gather_is_the_oracles(dev, d, bs):
    w, k, v = workload(dev, 830 + bs, d=d, bs=bs, max_len=300)
    rows = int(w.seq_lens.sum())
    ko = torch.full((rows, w.num_kv_heads, d), float("nan"), dtype=torch.bfloat16, device=dev)
    vo = torch.full_like(ko, float("nan"))
    N.kv_gather(k, v, w.layer, w.block_tables, w.seq_lens, w.offsets, row_starts(w.seq_lens),
                w.max_seq_len, ko, vo)
    torch.cuda.synchronize()
    args = (w.layer, host(w.block_tables), host(w.seq_lens), host(w.offsets))
    assert np.array_equal(host(ko), Q.gather_q4(host(k.codes), host(k.scales), *args))
    assert np.array_equal(host(vo), Q.gather_q4(host(v.codes), host(v.scales), *args))


def oracle_decode(w, k, v, q=None):
    bt, sl, off = host(w.block_tables), host(w.seq_lens), host(w.offsets)
    q = host(w.q if q is None else q)
    return Q.decode_q4(host(k.codes), host(k.scales), host(v.codes), host(v.scales), w.layer, q,
                       bt, sl, off, w.scale)


def run(w, k, v, split=0):
    out = torch.full_like(w.q, float("nan"))
    return N.paged_attn_decode(k, v, w.layer, w.q, w.block_tables, w.seq_lens, w.offsets,
                               w.max_seq_len, w.scale, split_tokens=split, out=out)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_int4_decode_grid(dev, d, group):
    """split 0 takes the device-planned schedule for these batches, 16 and
    64 fixed splits."""
    w, k, v = workload(dev, 840 + group, d=d, group=group)
    assert N.paged_attn_decode_schedule(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                        w.max_seq_len, w.block_size, torch.uint8,
                                        0) == N.SCHEDULE_PLANNED
    ref = oracle_decode(w, k, v)
    for split in (0, 16, 64):
        got = run(w, k, v, split)
        err = max_abs_err(got, ref)
        assert err <= TOL, (split, err)


@pytest.mark.parametrize("bs", [1, 4, 32])
def test_int4_decode_other_block_sizes(dev, bs):
    w, k, v = workload(dev, 850 + bs, bs=bs, max_len=300)
    ref = oracle_decode(w, k, v)
    for split in (0, 32):
        assert max_abs_err(run(w, k, v, split), ref) <= TOL


def test_int4_decode_edges(dev):
    """Empty sequences give zeros; lengths on chunk and block edges; NaN in
    the scales of slots no sequence owns never reaches an output; many
    splits (merged by the second kernel)."""
    w, k, v = workload(dev, 860, num_seqs=8, max_len=80, min_len=80)
    w.seq_lens = torch.tensor([0, 1, 15, 16, 17, 33, 0, 64], dtype=torch.int32, device=dev)
    w.offsets = torch.tensor([3, 0, 1, 15, 0, 7, 0, 2], dtype=torch.int32, device=dev)
    lens, offs, bt = host(w.seq_lens), host(w.offsets), host(w.block_tables)
    for s in range(w.num_seqs):
        for p in range(bt.shape[1] * w.block_size):
            b = int(bt[s, p // w.block_size])
            if b >= 0 and not (offs[s] <= p < offs[s] + lens[s]):
                k.scales[b, w.layer, :, p % w.block_size] = float("nan")
                v.scales[b, w.layer, :, p % w.block_size] = float("nan")
    ref = oracle_decode(w, k, v)
    for split in (0, 16):
        got = run(w, k, v, split)
        assert max_abs_err(got, ref) <= TOL
        assert torch.all(got[0] == 0) and torch.all(got[6] == 0)
    w2, k2, v2 = workload(dev, 861, num_seqs=2, max_len=700, min_len=600)
    assert max_abs_err(run(w2, k2, v2, 16), oracle_decode(w2, k2, v2)) <= TOL


def test_int4_write_then_decode(dev):
    """Rows written with the quantising append are what decode attends to."""
    w, k, v = workload(dev, 880, num_seqs=7, max_len=400)
    w = W.decode_tokens(w)
    kn = bf16_rows(dev, w.token_seq.shape[0], w.num_kv_heads, w.head_dim, 881, spread=False)
    vn = bf16_rows(dev, w.token_seq.shape[0], w.num_kv_heads, w.head_dim, 882, spread=False)
    kc, ksc = host(k.codes).copy(), host(k.scales).copy()
    vc, vsc = host(v.codes).copy(), host(v.scales).copy()
    slots = O.slot_mapping(host(w.block_tables), host(w.offsets), host(w.token_seq),
                           host(w.token_pos), w.block_size)
    Q.scatter_q4(kc, ksc, w.layer, host(kn), slots)
    Q.scatter_q4(vc, vsc, w.layer, host(vn), slots)
    N.kv_append(k, v, w.layer, kn, vn, w.block_tables, w.offsets, w.token_seq, w.token_pos)
    got = run(w, k, v)
    ref = Q.decode_q4(kc, ksc, vc, vsc, w.layer, host(w.q), host(w.block_tables),
                      host(w.seq_lens), host(w.offsets), w.scale)
    assert max_abs_err(got, ref) <= TOL


def test_int4_copy_and_swap(dev):
    nb = 20
    k, v = qpools(dev, nb, 3, 16, 2, 128, 890)
    src = np.array([1, 2, 3, -1], np.int32)
    dst = np.array([10, 11, 12, 4], np.int32)
    ref = [host(t).copy() for t in (k.codes, k.scales, v.codes, v.scales)]
    for a in ref:
        O.copy_blocks(a, src, dst)
    N.kv_copy_blocks(k, v, torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev))
    torch.cuda.synchronize()
    for t, a in zip((k.codes, k.scales, v.codes, v.scales), ref):
        assert np.array_equal(host(t).view(np.uint8), a.view(np.uint8))
    ids = np.array([5, 6, 7, 0, 19], np.int32)
    kh, vh = N.kv_swap_out(k, v, ids)
    torch.cuda.synchronize()
    for buf, t in ((kh, k), (vh, v)):
        c, s = N.split_swapped_q8(buf, t, len(ids))
        assert np.array_equal(c.numpy(), O.swap_out(host(t.codes), ids))
        assert np.array_equal(s.numpy().view(np.uint32), O.swap_out(host(t.scales), ids).view(np.uint32))
    into = np.array([13, 14, 15, 16, 2], np.int32)
    before = [host(t).copy() for t in (k.codes, k.scales, v.codes, v.scales)]
    N.kv_swap_in(k, v, into, kh, vh)
    torch.cuda.synchronize()
    for t, a in zip((k.codes, k.scales, v.codes, v.scales), before):
        O.swap_in(a, into, O.swap_out(a.copy(), ids))
        assert np.array_equal(host(t).view(np.uint8), a.view(np.uint8))


def test_int4_decode_batch_full_size(dev):
    """The decode batch (32 sequences, U[128, 2048], 8 kv heads, head_dim
    128, G 4) on a full-size int4 pool (16384 blocks x 32 layers): every
    sequence against the oracle over the referenced blocks."""
    w = W.decode_batch(device=dev, offsets="random", with_pools=False)
    k, v = qpools(dev, w.num_blocks, w.num_layers, w.block_size, w.num_kv_heads, w.head_dim,
                  901)
    got = run(w, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    bt = w.block_tables
    ids = torch.unique(bt[bt >= 0]).to(torch.int64)
    pos = torch.searchsorted(ids.cpu(), bt.cpu().clamp(min=0).to(torch.int64)).to(torch.int32)
    bt_c = torch.where(bt.cpu() >= 0, pos, torch.full_like(pos, -1)).numpy()
    sub = lambda t: host(t[ids][:, w.layer:w.layer + 1])
    ref = Q.decode_q4(sub(k.codes), sub(k.scales), sub(v.codes), sub(v.scales), 0,
                      host(w.q), bt_c, host(w.seq_lens), host(w.offsets), w.scale)
    err = max_abs_err(got, ref)
    print(f"int4 decode batch, all {w.num_seqs} sequences: max abs err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("d,group", [(64, 1), (128, 8)])
def test_int4_partials_at_high_workspace_addresses(dev, d, group):
    """Split partials written through a workspace whose address has bit 31
    of its low word set, and one where it is clear: the int4 partial writer
    builds a buffer resource from the workspace address, so both halves of
    that address must reach it unchanged."""
    w, k, v = workload(dev, 910 + group, d=d, group=group, num_seqs=4, max_len=300)
    ref = oracle_decode(w, k, v)
    need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                              w.max_seq_len, w.block_size, 16)
    big = torch.zeros((1 << 32) + need + 4096, dtype=torch.uint8, device=dev)
    base = big.data_ptr()
    for want_bit in (True, False):
        # the first 256-byte aligned offset whose address has bit 31 set (or clear)
        off = 0
        while bool((base + off) & 0x80000000) != want_bit:
            off += 1 << 28
        off += (-(base + off)) % 256
        assert bool((base + off) & 0x80000000) == want_bit and off + need <= big.numel()
        ws = big[off:off + need]
        got = N.paged_attn_decode(k, v, w.layer, w.q, w.block_tables, w.seq_lens, w.offsets,
                                  w.max_seq_len, w.scale, split_tokens=16,
                                  out=torch.full_like(w.q, float("nan")), workspace=ws)
        assert max_abs_err(got, ref) <= TOL, want_bit
    del big
    torch.cuda.empty_cache()


def _clone(pool):
    return N.QuantizedPool(pool.codes.clone(), pool.scales.clone())


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("split", [0, 16])
def test_quantised_decode_append_is_append_then_decode(dev, bits, split):
    """paged_attn_decode_append on a quantised pool leaves the pool bit for
    bit as kv_append writes it (each sequence's new token at position
    len - 1) and gives paged_attn_decode's output over that pool, bit for
    bit, within 2e-2 of the oracle.  Sequences with length 0, with no block
    at the new position (-1), or with a length above max_seq_len write
    nothing."""
    make = W.int8_pool_tensors if bits == 8 else W.int4_pool_tensors
    w = W.decode_batch(device=dev, seed=930 + bits, num_seqs=7, min_len=1, max_len=400,
                       num_blocks=260, num_layers=3, num_kv_heads=2, head_dim=128,
                       num_q_heads=8, dtype=torch.bfloat16, layer=1, offsets="random",
                       block_size=16, with_pools=False)
    shape = (260, 3, 16, 2, 128)
    k = N.QuantizedPool(*make(*shape, dev, 931))
    v = N.QuantizedPool(*make(*shape, dev, 932))
    lens = host(w.seq_lens).copy()
    offs = host(w.offsets)
    bt = host(w.block_tables).copy()
    mx = int(lens.max())
    lens[0] = 0                                            # empty: nothing written
    bt[1, (offs[1] + lens[1] - 1) // 16] = -1              # no block at the new position
    lens[2] = mx + 5                                       # above max_seq_len: clamped, nothing written
    w.seq_lens = torch.from_numpy(lens).to(dev)
    w.block_tables = torch.from_numpy(bt).to(dev)
    kn = bf16_rows(dev, w.num_seqs, 2, 128, 933, spread=False)
    vn = bf16_rows(dev, w.num_seqs, 2, 128, 934, spread=False)
    k2, v2 = _clone(k), _clone(v)
    got = N.paged_attn_decode_append(k, v, w.layer, w.q, kn, vn, w.block_tables, w.seq_lens,
                                     w.offsets, mx, w.scale, split_tokens=split,
                                     out=torch.full_like(w.q, float("nan")))
    write = [s for s in range(w.num_seqs) if 1 <= lens[s] <= mx]
    ts = torch.tensor(write, dtype=torch.int32, device=dev)
    tp = torch.tensor([int(lens[s]) - 1 for s in write], dtype=torch.int32, device=dev)
    N.kv_append(k2, v2, w.layer, kn[ts.long()].contiguous(), vn[ts.long()].contiguous(),
                w.block_tables, w.offsets, ts, tp)
    ref = N.paged_attn_decode(k2, v2, w.layer, w.q, w.block_tables, w.seq_lens, w.offsets, mx,
                              w.scale, split_tokens=split, out=torch.full_like(w.q, float("nan")))
    torch.cuda.synchronize()
    for a, b in ((k, k2), (v, v2)):
        assert torch.equal(a.codes, b.codes)
        assert torch.equal(a.scales.view(torch.int32), b.scales.view(torch.int32))
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # the oracle over the written pool, for the sequences whose tables cover
    # their (clamped) lengths
    keep = [s for s in range(w.num_seqs) if s not in (1, 2)]
    dec = Q.decode_q8 if bits == 8 else Q.decode_q4
    want = dec(host(k.codes), host(k.scales), host(v.codes), host(v.scales), w.layer,
               host(w.q)[keep], bt[keep], np.minimum(lens, mx)[keep], offs[keep], w.scale)
    assert max_abs_err(got[keep], want) <= TOL
