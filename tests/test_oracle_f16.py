"""Pins for the oracle's own IEEE-754 binary16 conversions against numpy's
float16 casts (an independent library routine).  Widening is checked on all
65536 patterns; narrowing on a stratified sample that covers every binary32
exponent, every rounding-relevant low-bit pattern around the binary16
subnormal/normal/overflow boundaries, and the exact ties."""
import numpy as np


def _np_f16(x):
    with np.errstate(over="ignore", invalid="ignore"):
        return x.astype(np.float16).view(np.uint16)


def test_widening_all_patterns(oracle):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f32_from_f16(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _check_narrowing(oracle, bits):
    x = bits.view(np.float32)
    ours = oracle.f16_from_f32(x)
    ref = _np_f16(x)
    nan = np.isnan(x)
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x3FF) != 0)
    bad = np.nonzero(ours[~nan] != ref[~nan])[0]
    assert bad.size == 0, [(hex(int(b)), hex(int(o)), hex(int(r))) for b, o, r in
                           zip(bits[~nan][bad[:5]], ours[~nan][bad[:5]], ref[~nan][bad[:5]])]


def test_narrowing_every_exponent(oracle):
    rng = np.random.default_rng(1234)
    exps = np.repeat(np.arange(256, dtype=np.uint32), 1 << 16)
    mant = rng.integers(0, 1 << 23, exps.size, dtype=np.uint32)
    sign = rng.integers(0, 2, exps.size, dtype=np.uint32)
    _check_narrowing(oracle, (sign << 31) | (exps << 23) | mant)


def test_narrowing_rounding_bits_near_boundaries(oracle):
    # binary16 keeps 10 fraction bits of a normal value and fewer of a
    # subnormal: exhaust the low 15 fraction bits at every binary32 exponent
    # from below the smallest subnormal (2^-26) to past the overflow (2^16).
    rng = np.random.default_rng(99)
    low = np.arange(1 << 15, dtype=np.uint32)
    parts = []
    for e in range(127 - 27, 127 + 17):
        for _ in range(2):
            high = np.uint32(rng.integers(0, 1 << 8)) << np.uint32(15)
            parts.append((np.uint32(e) << np.uint32(23)) | high | low)
    bits = np.concatenate(parts)
    _check_narrowing(oracle, bits)
    _check_narrowing(oracle, bits | np.uint32(0x80000000))


def test_narrowing_named_values(oracle):
    vals = np.array([0.0, -0.0, 1.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30,
                     2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -25 + 2.0 ** -40,
                     2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
                     np.inf, -np.inf, np.float32(0.1), np.finfo(np.float32).tiny], np.float32)
    _check_narrowing(oracle, vals.view(np.uint32))
    # ties go to even: 1 + 2^-11 -> 1.0 ; 1 + 3*2^-11 -> 1 + 2^-9
    got = oracle.f16_from_f32(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], np.float32))
    assert list(got) == [0x3C00, 0x3C02]


def test_round_trip_is_identity_on_binary16(oracle):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    back = oracle.f16_from_f32(oracle.f32_from_f16(h))
    assert np.array_equal(back[finite], h[finite])
