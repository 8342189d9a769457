"""Quantised KV pools in the oracle: int8 codes with one scale per (token,
kv head) row, written by a quantising scatter and read back dequantised by
gather and decode.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Source: [P3] mini-runtime, chapter 12 "Paged KV Cache", the evolution
diagram of sec. 6 names quantised KV (int8 / int4) as the next compression
step of a paged cache, and gives no method.  The reading taken (the plainest
symmetric scheme):

  * one row = the head_dim values of one token at one kv head; its scale is
    s = amax / 127 (amax = max |x| over the row), a float32 division;
  * code = round-half-to-even(x / s) in float32, clamped to [-127, 127];
    a row of zeros has s = 0 and codes 0;
  * the stored value is code * s (float32 product where a float32 value is
    needed; exact float64 product in the float64 decode).

Layouts (host numpy):
  codes   int8    (num_blocks, num_layers, block_size, num_kv_heads, head_dim)
  scales  float32 (num_blocks, num_layers, num_kv_heads, block_size)
Input rows are float32 or uint16 bfloat16 bit patterns; rows must be finite.

int4 (the other width the diagram names), the same reading at 4 bits:
  * s = amax / 7, code = round-half-to-even(x / s) clamped to [-7, 7]
    (-8 is not used, so the code range stays symmetric like int8's);
  * two codes per byte, four-bit two's complement, element 2i of a row in
    the low nibble of byte i and element 2i + 1 in the high nibble:
  packed  uint8   (num_blocks, num_layers, block_size, num_kv_heads, head_dim / 2)
  scales  as for int8.

Gather and decode over a quantised pool are the plain gather and decode of
the pages (P1 "Problem", P3 sec. 2.2, P2 sec. 2.3) applied to the stored
values: the codes and scales are gathered with the oracle's own gather, then
dequantised.
"""
import numpy as np

from .oracle import gather

QMAX = 127
QMAX4 = 7


def as_f32(rows):
    """float32 values of float32 rows or of uint16 bfloat16 bit patterns."""
    rows = np.asarray(rows)
    if rows.dtype == np.uint16:
        return (rows.astype(np.uint32) << 16).view(np.float32)
    return rows.astype(np.float32)


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest even (values here
    are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def quantize_rows(x, qmax=QMAX):
    """(codes int8 [..., D], scales float32 [...]) of rows x [..., D]: the
    symmetric per-row reading stated in the module header, with codes in
    [-qmax, qmax] (127 for int8, 7 for int4)."""
    x = as_f32(x)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(qmax)).astype(np.float32)
    live = s > 0
    div = np.where(live, s, np.float32(1.0)).astype(np.float32)
    c = np.rint((x / div[..., None]).astype(np.float32))
    c = np.clip(c, -qmax, qmax)
    c = np.where(live[..., None], c, 0)
    return c.astype(np.int8), s


def quantize_rows_q4(x):
    """(codes int8 in [-7, 7] [..., D], scales float32 [...]): the int4
    reading (amax / 7)."""
    return quantize_rows(x, QMAX4)


def pack_q4(codes):
    """int4 codes [..., D] (int8 values in [-8, 7]) -> bytes [..., D / 2]:
    element 2i in the low nibble of byte i, element 2i + 1 in the high
    nibble, each as four-bit two's complement."""
    c = np.asarray(codes).astype(np.int16)
    if c.shape[-1] % 2:
        raise ValueError("head_dim must be even")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_q4(packed):
    """bytes [..., D / 2] -> int4 codes [..., D] as int8 (sign-extended from
    four bits), the inverse of pack_q4."""
    b = np.asarray(packed).astype(np.int16)
    nib = np.stack([b & 0xF, (b >> 4) & 0xF], axis=-1)
    nib = np.where(nib >= 8, nib - 16, nib)
    return nib.reshape(*b.shape[:-1], b.shape[-1] * 2).astype(np.int8)


def dequantize_f32(codes, scales):
    """code * scale, a float32 product per element."""
    return (codes.astype(np.float32) * scales.astype(np.float32)[..., None]).astype(np.float32)


def dequantize_f64(codes, scales):
    """code * scale in float64 (exact: 8-bit code times 24-bit scale)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def scatter_q8(codes, scales, layer, src, slots):
    """In place: row i of src ([n, H, D], float32 or bf16 bits) is quantised
    per kv head and stored at slot slots[i] of `layer` (codes at
    [slot // bs, layer, slot % bs], scales at [slot // bs, layer, :,
    slot % bs]); slot -1 is skipped.  The scatter of P1 "relation to
    step14_1" / P2 sec. 2.2 with quantisation on write."""
    nb, nl, bs, h, d = codes.shape
    c, s = quantize_rows(np.asarray(src).reshape(-1, h, d))
    slots = np.asarray(slots, dtype=np.int64)
    if slots.shape[0] != c.shape[0]:
        raise ValueError("src must hold one row per slot")
    for i, sl in enumerate(slots.tolist()):
        if sl == -1:
            continue
        if sl < 0 or sl >= nb * bs:
            raise ValueError("slot outside the pool")
        codes[sl // bs, layer, sl % bs] = c[i]
        scales[sl // bs, layer, :, sl % bs] = s[i]
    return codes, scales


def _gather_scales(scales, layer, block_tables, seq_lens, offsets):
    # scales as a (nb, nl, bs, H, 1) pool, gathered by the oracle's gather
    pool = np.ascontiguousarray(np.transpose(scales, (0, 1, 3, 2))[..., None])
    return gather(pool, layer, block_tables, seq_lens, offsets)[..., 0]


def gather_q8(codes, scales, layer, block_tables, seq_lens, offsets):
    """Gather of the stored values as bfloat16 bit patterns (sum seq_lens,
    H, D): the codes and scales gathered with the first-block offset, then
    code * scale (float32) rounded to bfloat16."""
    c = gather(codes, layer, block_tables, seq_lens, offsets)
    s = _gather_scales(scales, layer, block_tables, seq_lens, offsets)
    return bf16_bits(dequantize_f32(c, s))


def attention_f64(q, k, v, scale):
    """Standard softmax attention of one decode query, float64: q [Hq, D],
    k / v [L, Hkv, D]; query head h reads kv head h // (Hq / Hkv).  [P2
    sec. 2.3]  L = 0 gives zeros."""
    hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    if k.shape[0] == 0:
        return out
    for h in range(hq):
        s = scale * (k[:, h // g, :] @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p @ v[:, h // g, :]) / p.sum()
    return out


def decode_q8(k_codes, k_scales, v_codes, v_scales, layer, q, block_tables, seq_lens, offsets,
              scale):
    """Decode over a quantised pool, float64 (num_seqs, Hq, D): each
    sequence's codes and scales gathered through its table, dequantised
    exactly, then attention_f64.  q: float32 or bf16 bits."""
    qf = as_f32(q).astype(np.float64)
    bt = np.asarray(block_tables, np.int32)
    sl = np.asarray(seq_lens, np.int32)
    off = np.asarray(offsets, np.int32)
    out = np.empty(qf.shape, dtype=np.float64)
    for s in range(sl.shape[0]):
        args = (layer, bt[s:s + 1], sl[s:s + 1], off[s:s + 1])
        k = dequantize_f64(gather(k_codes, *args), _gather_scales(k_scales, *args))
        v = dequantize_f64(gather(v_codes, *args), _gather_scales(v_scales, *args))
        out[s] = attention_f64(qf[s], k, v, scale)
    return out


def scatter_q4(packed, scales, layer, src, slots):
    """scatter_q8 for an int4 pool: row i of src ([n, H, D]) is quantised
    per kv head (the int4 reading), packed two codes per byte and stored at
    slot slots[i] of `layer`; slot -1 is skipped."""
    nb, nl, bs, h, d2 = packed.shape
    c, s = quantize_rows_q4(np.asarray(src).reshape(-1, h, 2 * d2))
    pk = pack_q4(c)
    slots = np.asarray(slots, dtype=np.int64)
    if slots.shape[0] != pk.shape[0]:
        raise ValueError("src must hold one row per slot")
    for i, sl in enumerate(slots.tolist()):
        if sl == -1:
            continue
        if sl < 0 or sl >= nb * bs:
            raise ValueError("slot outside the pool")
        packed[sl // bs, layer, sl % bs] = pk[i]
        scales[sl // bs, layer, :, sl % bs] = s[i]
    return packed, scales


def gather_q4(packed, scales, layer, block_tables, seq_lens, offsets):
    """gather_q8 for an int4 pool: the packed codes and the scales gathered
    with the first-block offset, unpacked, then code * scale (float32)
    rounded to bfloat16 bit patterns (sum seq_lens, H, D)."""
    c = unpack_q4(gather(packed, layer, block_tables, seq_lens, offsets))
    s = _gather_scales(scales, layer, block_tables, seq_lens, offsets)
    return bf16_bits(dequantize_f32(c, s))


def decode_q4(k_packed, k_scales, v_packed, v_scales, layer, q, block_tables, seq_lens, offsets,
              scale):
    """decode_q8 for an int4 pool: each sequence's packed codes and scales
    gathered through its table, unpacked and dequantised exactly, then
    attention_f64."""
    qf = as_f32(q).astype(np.float64)
    bt = np.asarray(block_tables, np.int32)
    sl = np.asarray(seq_lens, np.int32)
    off = np.asarray(offsets, np.int32)
    out = np.empty(qf.shape, dtype=np.float64)
    for s in range(sl.shape[0]):
        args = (layer, bt[s:s + 1], sl[s:s + 1], off[s:s + 1])
        k = dequantize_f64(unpack_q4(gather(k_packed, *args)), _gather_scales(k_scales, *args))
        v = dequantize_f64(unpack_q4(gather(v_packed, *args)), _gather_scales(v_scales, *args))
        out[s] = attention_f64(qf[s], k, v, scale)
    return out
