"""paged_attn_decode_noalloc (the decode entry point that allocates nothing
and keeps its partials in the library's fixed per-device scratch) against
paged_attn_decode with a caller workspace: bitwise the same output, and
within the decode tolerance of the oracle, on two calls in a row, the
second with a smaller batch -- so the second call runs on scratch that still
holds the first call's partials and counters region.
"""
import numpy as np
import pytest
import torch

from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import TOL, max_abs_err, oracle_decode_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def batch(dev, dtype, num_seqs, max_len, seed, group=4, head_dim=128, num_kv_heads=2):
    nb = (num_seqs * (max_len + 32)) // 16 + 64
    return W.decode_batch(device=dev, seed=seed, num_seqs=num_seqs, min_len=1, max_len=max_len,
                          num_blocks=nb, num_layers=3, num_kv_heads=num_kv_heads,
                          head_dim=head_dim, num_q_heads=num_kv_heads * group, dtype=dtype,
                          layer=1, offsets="random")


def both(w, split):
    """(noalloc output, paged_attn_decode output with a fresh zeroed
    workspace), same arguments."""
    got = N.paged_attn_decode_noalloc(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables,
                                      w.seq_lens, w.offsets, w.max_seq_len, w.scale,
                                      split_tokens=split,
                                      out=torch.full_like(w.q, float("nan")))
    ref = N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables, w.seq_lens,
                              w.offsets, w.max_seq_len, w.scale, split_tokens=split,
                              out=torch.full_like(w.q, float("nan")))
    torch.cuda.synchronize()
    return got, ref


def same_bits(a, b):
    ia = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
    ib = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
    return torch.equal(ia, ib)


CASES = [(torch.bfloat16, 0), (torch.bfloat16, 64), (torch.bfloat16, 16),
         (torch.bfloat16, N.SPLIT_PLANNED), (torch.float32, 16), (torch.float32, 0)]


@pytest.mark.parametrize("dtype,split", CASES)
def test_noalloc_matches_decode_two_calls(dev, dtype, split):
    big = batch(dev, dtype, num_seqs=9, max_len=1500, seed=410)
    small = batch(dev, dtype, num_seqs=4, max_len=300, seed=411)
    for w in (big, small):
        got, ref = both(w, split)
        assert same_bits(got, ref)
        assert max_abs_err(got, oracle_decode_for(w)) <= TOL[dtype]


def test_noalloc_full_size_decode_batch_then_small(dev):
    """The decode batch at full size (32 sequences, 16384-block pool of 32
    layers), then a small batch, through the automatic schedule."""
    w = W.decode_batch(device=dev, offsets="random")
    got, ref = both(w, 0)
    assert same_bits(got, ref)
    seqs = [0, 7, 19, 31]
    assert max_abs_err(got[seqs], oracle_decode_for(w, seqs=seqs)) <= TOL[w.dtype]
    del w
    torch.cuda.empty_cache()
    s = batch(dev, torch.bfloat16, num_seqs=3, max_len=200, seed=412)
    got, ref = both(s, 0)
    assert same_bits(got, ref)
    assert max_abs_err(got, oracle_decode_for(s)) <= TOL[s.dtype]


def test_noalloc_rejects_sizes_beyond_the_scratch(dev):
    """A bound of 65440 tokens at 16-token splits needs 4090 partial
    records per sequence, more than the scratch holds for two sequences:
    refused before anything is enqueued, and the out buffer is untouched."""
    w = batch(dev, torch.bfloat16, num_seqs=2, max_len=64, seed=413)
    mx = 4090 * 16
    need = N.paged_attn_decode_workspace_size(w.num_seqs, w.num_kv_heads, w.num_q_heads,
                                              w.head_dim, mx, w.block_size, 16)
    assert N.NOALLOC_SCRATCH_BYTES < need < (1 << 62)
    out = torch.full_like(w.q, float("nan"))
    with pytest.raises(N.PagedKVError) as e:
        N.paged_attn_decode_noalloc(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables, w.seq_lens,
                                    w.offsets, mx, w.scale, split_tokens=16, out=out)
    assert e.value.status == -13
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


def qbatch(dev, bits, num_seqs, max_len, seed, group=4, head_dim=128, num_kv_heads=2):
    """A decode batch over a quantised pool (int8 or int4 codes, one float32
    scale per token and kv head), bf16 queries."""
    nb = (num_seqs * (max_len + 32)) // 16 + 64
    w = W.decode_batch(device=dev, seed=seed, num_seqs=num_seqs, min_len=1, max_len=max_len,
                       num_blocks=nb, num_layers=3, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, num_q_heads=num_kv_heads * group,
                       dtype=torch.bfloat16, layer=1, offsets="random", with_pools=False)
    make = W.int8_pool_tensors if bits == 8 else W.int4_pool_tensors
    shape = (nb, 3, 16, num_kv_heads, head_dim)
    w.k_pool = N.QuantizedPool(*make(*shape, dev, seed * 3))
    w.v_pool = N.QuantizedPool(*make(*shape, dev, seed * 3 + 1))
    return w


@pytest.mark.parametrize("bits,split", [(8, 0), (8, 16), (4, 0), (4, 16)])
def test_noalloc_quantised_pools_two_calls(dev, bits, split):
    """Quantised pools through the scratch: the int4 partials are written by
    buffer stores whose resource is built from the partials' address, here
    the library's scratch."""
    from oracle import quant as Q
    from tests.pkv_testlib import host

    dec = Q.decode_q8 if bits == 8 else Q.decode_q4
    for w in (qbatch(dev, bits, 9, 1500, 420 + bits), qbatch(dev, bits, 4, 300, 421 + bits)):
        got, ref = both(w, split)
        assert same_bits(got, ref)
        want = dec(host(w.k_pool.codes), host(w.k_pool.scales), host(w.v_pool.codes),
                   host(w.v_pool.scales), w.layer, host(w.q), host(w.block_tables),
                   host(w.seq_lens), host(w.offsets), w.scale)
        assert max_abs_err(got, want) <= 2e-2
