"""Pins of the int4 quantised-KV oracle (oracle/quant.py: quantize_rows_q4,
pack_q4 / unpack_q4, scatter_q4, gather_q4, decode_q4).

The pages name int4 beside int8 as a quantised KV width (mini-runtime
ch. 12, sec. 6 evolution diagram) with no method.  The oracle takes the int8
reading at four bits: one float32 scale amax / 7 per (token, kv head) row,
codes round-half-even(x / scale) in [-7, 7], two codes per byte (element 2i
in the low nibble, four-bit two's complement).  Pinned here by mathematics
and by the already pinned gather and decode:

  * the reading's facts: the scale is amax / 7 in float32, every stored
    value is within half a step of its input, the codes stay in [-7, 7],
    the row's largest magnitude maps to +-7, integer rows of amax 7 come
    back exactly and ties go to even; zero rows, odd symmetry and
    power-of-two scaling;
  * packing against hand-worked bytes and, exhaustively over all 256 code
    pairs, against the arithmetic definition of four-bit two's complement
    (c mod 16) -- a formulation other than the bit masks pack_q4 uses;
  * gather over the int4 pool equals a per-token loop over the stated
    layouts, scatter-then-gather returns bf16(code * scale) of the rows
    written, and decode equals the C oracle's decode of a float32 pool
    holding the stored values (exactly, with power-of-two scales).

Planted mistakes (floor rounding, amax / 8, the nibbles swapped,
sign-magnitude nibbles, ties away from zero) each fail a pin.
"""
import numpy as np
import pytest

import oracle as O
from oracle import quant as Q


def rows(rng, n, h, d, lo=-3, hi=3):
    mag = 10.0 ** rng.uniform(lo, hi, size=(n, h, 1))
    return (rng.standard_normal((n, h, d)) * mag).astype(np.float32)


def check_reading(quantize, x):
    """The facts the int4 reading fixes, for one quantiser; returns failures."""
    bad = []
    c, s = quantize(x)
    amax = np.max(np.abs(x), axis=-1)
    if not np.array_equal(s, (amax / np.float32(7)).astype(np.float32)):
        bad.append("scale")
    err = np.abs(Q.dequantize_f64(c, s) - x.astype(np.float64))
    if np.any(err > s.astype(np.float64)[..., None] * (0.5 + 2.0 ** -20)):
        bad.append("half-step bound")
    if np.any(np.abs(c.astype(np.int32)) > 7):
        bad.append("code range")
    top = np.take_along_axis(np.abs(c.astype(np.int32)), np.argmax(np.abs(x), -1)[..., None], -1)
    if np.any(top[..., 0][amax > 0] != 7):
        bad.append("amax code")
    ints = np.array([[7, 2.5, -3.5, 0.5, -0.5, 1.5, -7, 4]], np.float32)
    ci, si = quantize(ints)
    if not (si[0] == 1.0 and list(ci[0]) == [7, 2, -4, 0, 0, 2, -7, 4]):
        bad.append("ties to even / exact integers")
    return bad


def test_quantize_q4_meets_the_reading():
    rng = np.random.default_rng(41)
    x = rows(rng, 300, 4, 128)
    assert check_reading(Q.quantize_rows_q4, x) == []
    b = Q.bf16_bits(x)
    c1, s1 = Q.quantize_rows_q4(b)
    c2, s2 = Q.quantize_rows_q4(Q.as_f32(b))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_quantize_q4_zero_rows_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(42)
    x = rows(rng, 50, 2, 64)
    x[3, 1] = 0.0
    c, s = Q.quantize_rows_q4(x)
    assert s[3, 1] == 0 and not c[3, 1].any()
    cn, sn = Q.quantize_rows_q4(-x)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    for k in (-7, 5):
        ck, sk = Q.quantize_rows_q4(x * np.float32(2.0 ** k))
        assert np.array_equal(ck, c) and np.array_equal(sk, s * np.float32(2.0 ** k))


def _floor(x):
    c, s = Q.quantize_rows_q4(x)
    div = np.where(s > 0, s, 1)[..., None]
    return np.clip(np.floor(x / div), -7, 7).astype(np.int8), s


def _over_8(x):
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(8)).astype(np.float32)
    div = np.where(s > 0, s, 1)[..., None]
    return np.clip(np.rint(x / div), -7, 7).astype(np.int8), s


def _ties_away(x):
    c, s = Q.quantize_rows_q4(x)
    div = np.where(s > 0, s, 1)[..., None].astype(np.float32)
    t = (x / div).astype(np.float32)
    return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -7, 7).astype(np.int8), s


@pytest.mark.parametrize("mutant", [_floor, _over_8, _ties_away], ids=lambda f: f.__name__)
def test_planted_q4_quantiser_mistake_fails(mutant):
    rng = np.random.default_rng(43)
    x = rows(rng, 40, 4, 64)
    assert check_reading(mutant, x)


def two_complement_bytes(codes):
    """Reference packing from the definition: a four-bit two's complement
    nibble holds c mod 16; byte i = nibble(c[2i]) + 16 * nibble(c[2i+1])."""
    c = [int(v) for v in np.asarray(codes).reshape(-1)]
    return [(c[2 * i] % 16) + 16 * (c[2 * i + 1] % 16) for i in range(len(c) // 2)]


def test_pack_q4_worked_bytes():
    # element 2i in the low nibble: (1, -1) -> 0xF1; (-7, 7) -> 0x79;
    # (0, -7) -> 0x90; (3, -3) -> 0xD3
    codes = np.array([1, -1, -7, 7, 0, -7, 3, -3], np.int8)
    assert list(Q.pack_q4(codes)) == [0xF1, 0x79, 0x90, 0xD3]
    assert list(Q.unpack_q4(np.array([0xF1, 0x79, 0x90, 0xD3], np.uint8))) == list(codes)


def test_pack_q4_all_pairs_against_the_definition():
    a, b = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    codes = np.stack([a.reshape(-1), b.reshape(-1)], axis=-1).astype(np.int8)   # 256 pairs
    packed = Q.pack_q4(codes)
    assert packed.shape == (256, 1)
    assert list(packed[:, 0]) == two_complement_bytes(codes)
    assert sorted(set(packed[:, 0].tolist())) == list(range(256))
    assert np.array_equal(Q.unpack_q4(packed), codes)


def _swapped(codes):
    c = np.asarray(codes).astype(np.int16)
    return ((c[..., 1::2] & 0xF) | ((c[..., 0::2] & 0xF) << 4)).astype(np.uint8)


def _sign_magnitude(codes):
    c = np.asarray(codes).astype(np.int16)
    nib = np.where(c < 0, 8 | (-c), c) & 0xF
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("mutant", [_swapped, _sign_magnitude], ids=lambda f: f.__name__)
def test_planted_packing_mistake_fails(mutant):
    codes = np.array([1, -1, -7, 7, 0, -7, 3, -3], np.int8)
    assert list(mutant(codes)) != [0xF1, 0x79, 0x90, 0xD3]


def make_pool4(rng, nb, nl, bs, h, d, pow2):
    codes = rng.integers(-7, 8, size=(nb, nl, bs, h, d)).astype(np.int8)
    if pow2:
        scales = (2.0 ** rng.integers(-12, 4, size=(nb, nl, h, bs))).astype(np.float32)
    else:
        scales = (10.0 ** rng.uniform(-3, 0, size=(nb, nl, h, bs))).astype(np.float32)
    return codes, Q.pack_q4(codes), scales


def tables(rng, nseq, bs, nb, max_len):
    lens = rng.integers(0, max_len + 1, size=nseq).astype(np.int32)
    offs = rng.integers(0, bs, size=nseq).astype(np.int32)
    need = [O.blocks_needed(int(l) + int(o), bs) for l, o in zip(lens, offs)]
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((nseq, max(max(need), 1)), -1, np.int32)
    at = 0
    for i, c in enumerate(need):
        bt[i, :c] = perm[at:at + c]
        at += c
    return bt, lens, offs


def test_gather_q4_is_the_per_token_definition():
    """Token t of a sequence sits at flat position off + t of its table
    (P3 sec. 2.2); its stored row at kv head h is its unpacked codes times
    scales[b, l, h, r] (float32), rounded to bf16."""
    rng = np.random.default_rng(44)
    bs, h, d, nl = 4, 3, 64, 2
    bt, lens, offs = tables(rng, 4, bs, 64, 30)
    codes, packed, scales = make_pool4(rng, 64, nl, bs, h, d, pow2=False)
    got = Q.gather_q4(packed, scales, 1, bt, lens, offs)
    want = []
    for s in range(4):
        for t in range(int(lens[s])):
            p = int(offs[s]) + t
            b, r = int(bt[s, p // bs]), p % bs
            row = codes[b, 1, r].astype(np.float32) * scales[b, 1, :, r][:, None]
            want.append(Q.bf16_bits(row.astype(np.float32)))
    assert np.array_equal(got, np.array(want).reshape(got.shape))


def test_scatter_q4_then_gather_q4():
    """Rows scattered with int4 quantisation come back as bf16(code * scale)
    of their own quantisation; slot -1 rows are dropped; every other byte of
    the pool is unchanged."""
    rng = np.random.default_rng(45)
    nb, nl, bs, h, d = 12, 2, 4, 2, 64
    _, packed, scales = make_pool4(rng, nb, nl, bs, h, d, pow2=False)
    p0, s0 = packed.copy(), scales.copy()
    x = rows(rng, 9, h, d)
    slots = np.array([5, 6, -1, 7, 8, 9, 10, 11, 40], np.int64)
    Q.scatter_q4(packed, scales, 1, x, slots)
    cq, sq = Q.quantize_rows_q4(x)
    for i, sl in enumerate(slots.tolist()):
        if sl >= 0:
            assert np.array_equal(Q.unpack_q4(packed[sl // bs, 1, sl % bs]), cq[i])
            assert np.array_equal(scales[sl // bs, 1, :, sl % bs], sq[i])
    touched = np.zeros((nb, nl, bs), bool)
    for sl in slots[slots >= 0].tolist():
        touched[sl // bs, 1, sl % bs] = True
    assert np.array_equal(packed[~touched], p0[~touched])
    assert np.array_equal(scales.transpose(0, 1, 3, 2)[~touched], s0.transpose(0, 1, 3, 2)[~touched])
    bt = np.array([[1, 2]], np.int32)
    got = Q.gather_q4(packed, scales, 1, bt, np.array([7], np.int32), np.array([1], np.int32))
    keep = [0, 1, 3, 4, 5, 6, 7]
    assert np.array_equal(got, Q.bf16_bits(Q.dequantize_f32(cq[keep], sq[keep])))
    with pytest.raises(ValueError):
        Q.scatter_q4(packed, scales, 0, x[:1], np.array([nb * bs], np.int64))


@pytest.mark.parametrize("G", [1, 4])
def test_decode_q4_is_decode_of_the_stored_values(G):
    """With power-of-two scales the stored values are exact in float32, so
    decode over the int4 pool must equal the C oracle's decode of a float32
    pool holding them; with other scales they differ only by the float32
    rounding of the stored values."""
    rng = np.random.default_rng(46 + G)
    nb, nl, bs, hkv, d = 48, 2, 4, 2, 64
    bt, lens, offs = tables(rng, 5, bs, nb, 30)
    q = rng.standard_normal((5, hkv * G, d)).astype(np.float32)
    for pow2 in (True, False):
        kc, kp, ks = make_pool4(rng, nb, nl, bs, hkv, d, pow2)
        vc, vp, vs = make_pool4(rng, nb, nl, bs, hkv, d, pow2)
        kf = Q.dequantize_f32(kc, ks.transpose(0, 1, 3, 2))
        vf = Q.dequantize_f32(vc, vs.transpose(0, 1, 3, 2))
        got = Q.decode_q4(kp, ks, vp, vs, 1, q, bt, lens, offs, 0.125)
        ref = O.decode(kf, vf, 1, q, bt, lens, offs, 0.125)
        tol = 1e-12 if pow2 else 1e-5
        assert np.max(np.abs(got - ref)) <= tol * max(1.0, np.max(np.abs(ref)))
    assert not got[lens == 0].any()
