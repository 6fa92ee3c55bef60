"""Pins for the oracle's element formats (E2M1, E4M3, bf16, nibble packing).

Each check compares against something other than the oracle itself: the
hand-written value table of the pages' E2M1 format, torch's float8_e4m3fn and
bfloat16 casts (library routines, round-to-nearest-even), hand-derived cases,
or a brute-force nearest search.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats


def test_e2m1_table_matches_format(golden):
    g = golden("e2m1_values.txt")
    want = np.array([float(v) for v in g["magnitudes"]])
    assert np.array_equal(oracle.E2M1_VALUES, want)


def test_e2m1_ties_by_hand():
    # nearest-even on the E2M1 grid; ties go to the code with mantissa bit 0
    cases = {0.0: 0, 0.25: 0, 0.2500001: 1, 0.75: 2, 0.7499999: 1, 1.25: 2, 1.2500001: 3,
             1.75: 4, 2.5: 4, 2.5000002: 5, 3.5: 6, 3.4999998: 5, 5.0: 6, 5.0000005: 7,
             6.0: 7, 7.0: 7, 1e30: 7, 0.1: 0, 0.4: 1, 2.9: 5}
    q = np.array(list(cases), dtype=np.float64)
    assert list(oracle.e2m1_rne_sat(q)) == list(cases.values())


def test_e2m1_brute_force_nearest():
    rng = np.random.default_rng(123)
    vals = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    q = list(rng.uniform(0, 8, 4000).astype(np.float32))
    for m in mids + vals:
        f = np.float32(m)
        q += [f, np.nextafter(f, np.float32(10)), np.nextafter(f, np.float32(-10))]
    q = np.abs(np.array(q, dtype=np.float32)).astype(np.float64)
    got = oracle.e2m1_rne_sat(q)
    for qi, gi in zip(q, got):
        d = [abs(qi - v) for v in vals]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        if qi >= 6:
            want = 7
        elif len(cands) == 1:
            want = cands[0]
        else:
            want = [c for c in cands if c % 2 == 0][0]
        assert gi == want, (qi, gi, want)


def test_e4m3_decode_exhaustive_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    finite = got[np.isfinite(got)]
    assert len(finite) == 254 and finite.max() == 448.0
    assert np.min(finite[finite > 0]) == 2.0 ** -9


def test_e4m3_decode_by_hand():
    d = oracle.e4m3_decode
    assert d(0x7E) == 448.0 and d(0x38) == 1.0 and d(0x01) == 2.0 ** -9
    assert d(0x08) == 2.0 ** -6 and d(0x35) == 0.8125 and d(0x39) == 1.125
    assert d(0x28) == 0.25 and d(0x03) == 3 * 2.0 ** -9 and d(0xB8) == -1.0


def test_e4m3_encode_vs_torch_dense():
    # dense sweep of [0, 464) plus every midpoint between neighbours ±1 ulp (f32)
    rng = np.random.default_rng(7)
    vals = oracle.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    xs = [np.linspace(0, 463.99, 200001, dtype=np.float32),
          rng.uniform(0, 2.0 ** -5, 20000).astype(np.float32),
          vals.astype(np.float32), mids.astype(np.float32)]
    m32 = mids.astype(np.float32)
    xs += [np.nextafter(m32, np.float32(1e9)), np.nextafter(m32, np.float32(-1e9))]
    x = np.abs(np.concatenate(xs)).astype(np.float32)
    x = x[x < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode_rne_satfinite(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_by_hand():
    f = oracle.e4m3_encode_rne_satfinite
    assert list(f(np.array([448.0, 460.0, 464.0, 470.0, 1e6]))) == [0x7E] * 5
    assert list(f(np.array([2.0 ** -10, 2.0 ** -10 * 1.0000001, 0.0]))) == [0, 1, 0]
    assert f(np.array([5.0 / 6.0]))[0] == 0x35        # 0.8125 nearer than 0.875
    assert f(np.array([7.0 / 6.0]))[0] == 0x39        # 1.125 nearer than 1.25
    assert f(np.array([7.5 * 2.0 ** -9]))[0] == 0x08  # tie between 0x07 and 0x08 → even


def test_bf16_rne_vs_torch_on_f32_inputs():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    ties = np.array([0x3F808000, 0x3F818000, 0x3F80C000, 0x00008000, 0x80018000,
                     0x00000001, 0x007FFFFF], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne_from_f64(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rne_single_rounding_by_hand():
    # 1 + 2^-8 + 2^-30 is just above the bf16 midpoint 1 + 2^-8: one rounding
    # gives 1 + 2^-7 (0x3F81); rounding through binary32 first would give 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.bf16_rne_from_f64(np.array([x]))[0] == 0x3F81
    assert oracle.bf16_rne_from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80  # tie → even
    assert oracle.bf16_rne_from_f64(np.array([-0.0]))[0] == 0x8000
    assert oracle.bf16_rne_from_f64(np.array([2.0 ** -133]))[0] == 0x0001
    assert oracle.bf16_rne_from_f64(np.array([2.0 ** -134]))[0] == 0x0000  # tie → even (0)


def test_bf16_bits_roundtrip():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(b)
    ok = np.isfinite(f)
    assert np.array_equal(oracle.bf16_rne_from_f64(f[ok].astype(np.float64)), b[ok])


def test_nibble_order_by_hand():
    assert list(oracle.pack_nibbles(np.array([1, 2, 3, 4, 0xF, 0x8]))) == [0x21, 0x43, 0x8F]
    assert list(oracle.unpack_nibbles(np.array([0x21, 0x8F], dtype=np.uint8))) == [1, 2, 0xF, 0x8]


def test_input_validation():
    with pytest.raises(ValueError):
        oracle.e2m1_rne_sat(np.array([-1.0]))
    with pytest.raises(ValueError):
        oracle.e4m3_encode_rne_satfinite(np.array([np.nan]))
    with pytest.raises(ValueError):
        formats.pack_nibbles(np.array([1, 2, 3]))
