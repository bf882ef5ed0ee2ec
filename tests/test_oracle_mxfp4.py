"""Pins of the oracle's 4-bit cache codec, OCP MXFP4 (CPU only): the E2M1 code table from the
format definition against the magnitudes the MX specification lists, the encoder against a
brute-force nearest search with the tie rule, the shared-exponent rule, exact round trips,
the error bound, NaN blocks, the nibble order, and the cache write + gather path."""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import codecs as C
from oracle.allocator import Allocator


def test_e2m1_table_is_the_listed_magnitudes():
    """E2M1 represents +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} (codes 0..7 positive, 8..15 negative)."""
    assert list(C.E2M1_DECODE[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(C.E2M1_DECODE[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert np.signbit(C.E2M1_DECODE[8])


def _brute_encode(v):
    """Nearest of the 8 magnitudes by explicit distance, ties to the code whose mantissa bit is
    0, magnitudes past 6 to 6, sign kept."""
    a = min(abs(v), 6.0)
    best = None
    for code in range(8):
        dist = abs(C.E2M1_DECODE[code] - a)
        if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0):
            best = (dist, code)
    return best[1] | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_encode_vs_bruteforce():
    vals = np.concatenate([np.linspace(-9, 9, 36001), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9, 100.0, -0.0]])
    got = C.e2m1_encode(vals)
    want = np.array([_brute_encode(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)
    # the ties, worked out from the rule
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, y in ties.items():
        assert C.E2M1_DECODE[C.e2m1_encode(np.array([x]))[0]] == y


def test_block_exponent_rule():
    """2^E is the largest power of two with amax / 2^E >= 4, i.e. amax / 2^E in [4, 8)."""
    rng = np.random.default_rng(5)
    amax = np.ldexp(rng.uniform(0.5, 1.0, 2000), rng.integers(-100, 100, 2000))
    E = C.mx_block_exponent(amax)
    r = amax / np.ldexp(1.0, E)
    assert np.all((r >= 4) & (r < 8))
    assert C.mx_block_exponent(np.array([0.0]))[0] == -127
    assert C.mx_block_exponent(np.array([2.0 ** -130]))[0] == -127          # clamped to the E8M0 range
    assert C.mx_block_exponent(np.array([1.0, 4.0, 6.0, 7.99]))[:].tolist() == [-2, 0, 0, 0]


def test_round_trip_of_representable_blocks():
    """Blocks made of E2M1 values times 2^E, with a magnitude of 4 or 6 present, quantize back to
    the same codes and scale."""
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, size=(300, 32)).astype(np.uint8)
    codes[:, 0] = rng.choice([6, 7, 14, 15], size=300)
    E = rng.integers(-120, 120, size=300)
    x = C.E2M1_DECODE[codes] * np.ldexp(1.0, E)[:, None]
    qc, qs = C.mxfp4_quantize(x)
    assert np.array_equal(C.E2M1_DECODE[qc], C.E2M1_DECODE[codes])          # -0 and +0 both decode to 0
    assert np.array_equal(qs[:, 0].astype(np.int64), E + 127)
    assert np.array_equal(C.mxfp4_dequantize(qc, qs), x)


def test_error_bound():
    """|dequant - x| <= 2^E where |x| / 2^E <= 6 (half the widest spacing) and <= 2 * 2^E where
    it saturates (|x| / 2^E in (6, 8))."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((500, 64)) * np.ldexp(1.0, rng.integers(-20, 20, size=(500, 1)))
    qc, qs = C.mxfp4_quantize(x)
    y = C.mxfp4_dequantize(qc, qs)
    unit = np.repeat(np.ldexp(1.0, qs.astype(np.int64) - 127), 32, axis=-1)
    err = np.abs(y - x)
    sat = np.abs(x) / unit > 6
    assert np.all(err[~sat] <= unit[~sat]) and np.all(err[sat] <= 2 * unit[sat])


def test_nonfinite_block_is_nan_and_isolated():
    x = np.ones((2, 64))
    x[0, 40] = np.nan
    x[1, 3] = np.inf
    qc, qs = C.mxfp4_quantize(x)
    assert qs.tolist() == [[125, C.E8M0_NAN], [C.E8M0_NAN, 125]]
    y = C.mxfp4_dequantize(qc, qs)
    assert np.isnan(y[0, 32:]).all() and np.isnan(y[1, :32]).all()
    assert np.array_equal(y[0, :32], np.ones(32)) and np.array_equal(y[1, 32:], np.ones(32))


def test_nibble_order():
    codes = np.arange(16, dtype=np.uint8)
    p = C.pack_nibbles(codes)
    assert p.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(C.unpack_nibbles(p), codes)


@pytest.mark.parametrize("d,bs", [(128, 16), (64, 8), (128, 128)])
def test_cache_write_gather_and_decode(d, bs):
    """Rows written into an MXFP4 cache through slots and gathered through the table are the
    codec's dequantized rows; decode over that cache equals attention over those rows."""
    rng = np.random.default_rng(8 + d + bs)
    Hkv, Hq, lens = 2, 8, [5, 40, 17]
    N = sum(-(-L // bs) for L in lens) + 2
    al = Allocator(N, bs, np.random.default_rng(9).permutation(N))
    slots, rows_k, rows_v = [], [], []
    for b, L in enumerate(lens):
        al.add(b)
        s, _ = al.append(b, L)
        slots += s
        rows_k.append(C.f32_to_bf16_bits(rng.standard_normal((L, Hkv, d)).astype(np.float32)))
        rows_v.append(C.f32_to_bf16_bits(rng.standard_normal((L, Hkv, d)).astype(np.float32)))
    tb = bs * (d // 2 + d // 32)
    kc = np.zeros((N, Hkv, tb), np.uint8)
    vc = np.zeros_like(kc)
    A.kv_write(np.concatenate(rows_k), np.concatenate(rows_v), np.array(slots), kc, vc, bs, "mxfp4")
    tables, seq_lens = al.block_table(range(3), max(-(-L // bs) for L in lens))
    q = rng.standard_normal((3, Hq, d)).astype(np.float32)
    got = A.decode(q, kc, vc, np.array(tables), np.array(seq_lens), np.float32(0.1), bs, "mxfp4", "f32")
    for b, L in enumerate(lens):
        for g in range(Hkv):
            K = A.gather(kc, tables[b], L, g, bs, "mxfp4", head_dim=d)
            Kq = C.mxfp4_dequantize(*C.mxfp4_quantize(C.bf16_bits_to_f64(rows_k[b][:, g])))
            assert np.array_equal(K, Kq)
            V = C.mxfp4_dequantize(*C.mxfp4_quantize(C.bf16_bits_to_f64(rows_v[b][:, g])))
            for h in range(g * 4, g * 4 + 4):
                np.testing.assert_allclose(got[b, h], A.attend(q[b, h].astype(np.float64), Kq, V, float(np.float32(0.1))),
                                           rtol=0, atol=1e-12)
