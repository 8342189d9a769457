"""Split records of the in-kernel merge at extreme value ranges.

The MFMA decode kernels at head_dim 128 keep each split's accumulator rows
in half precision, every row re-referenced by a power of two so that its
largest element sits just below the top of the half-precision range (the
record (m + k, l 2^-k, acc 2^-k) merges like (m, l, acc)).  Without that
shift, values scaled by 2^20 overflow half precision and values scaled by
2^-20 keep only a few significant bits.  These cases scale V (the bf16
pool, or the quantised pools' row scales) by powers of two, which scales
the exact result by the same factor, and require multi-split decode through
the in-kernel merge to stay within the usual bar times that factor.
"""
import numpy as np
import pytest
import torch

from oracle import quant as Q
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import TOL, host, max_abs_err, oracle_decode_for

pytestmark = pytest.mark.gpu

QTOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def build(dev, dtype, seed):
    bs, max_len, n, hkv, g = 16, 700, 6, 2, 4
    nb = n * ((max_len + bs - 1) // bs + 1) + 16
    quant = dtype in ("i8", "i4")
    w = W.decode_batch(device=dev, seed=9000 + seed, num_seqs=n, min_len=200, max_len=max_len,
                       num_blocks=nb, num_layers=2, num_kv_heads=hkv, head_dim=128,
                       num_q_heads=hkv * g, dtype=torch.bfloat16, layer=1, offsets="random",
                       block_size=bs, with_pools=not quant)
    if quant:
        make = W.int8_pool_tensors if dtype == "i8" else W.int4_pool_tensors
        shape = (nb, 2, bs, hkv, 128)
        w.k_pool = N.QuantizedPool(*make(*shape, dev, 9100 + seed))
        w.v_pool = N.QuantizedPool(*make(*shape, dev, 9200 + seed))
    return w


@pytest.mark.parametrize("split", [64, N.SPLIT_PLANNED])
@pytest.mark.parametrize("log2_scale", [20, -20, 100])
@pytest.mark.parametrize("dtype", ["bf16", "i8", "i4"])
def test_records_keep_range(dev, dtype, log2_scale, split):
    w = build(dev, dtype, abs(log2_scale) + (1 if split == 64 else 2))
    scale = 2.0 ** log2_scale
    if dtype == "bf16":
        w.v_pool.mul_(scale)  # exact: a power of two, within bf16's range
    else:
        w.v_pool.scales.mul_(scale)
    print(dtype, log2_scale, split, flush=True)
    out = torch.full_like(w.q, float("nan"))
    got = N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables, w.seq_lens, w.offsets,
                              w.max_seq_len, w.scale, split_tokens=split, out=out)
    torch.cuda.synchronize()
    if dtype == "bf16":
        want = oracle_decode_for(w)
        bar = TOL[torch.bfloat16]
    else:
        dq = Q.decode_q8 if dtype == "i8" else Q.decode_q4
        want = dq(host(w.k_pool.codes), host(w.k_pool.scales), host(w.v_pool.codes), host(w.v_pool.scales),
                  w.layer, host(w.q), host(w.block_tables), host(w.seq_lens), host(w.offsets), w.scale)
        bar = QTOL
    assert np.all(np.isfinite(want))
    err = max_abs_err(got, want)
    assert err <= bar * scale, (err / scale, bar)
