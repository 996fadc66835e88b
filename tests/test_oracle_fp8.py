"""Pins of the FP8 (OCP E4M3) cache oracle (no GPU).

The oracle's code table, encoder and quantiser are checked against a
library routine (torch's float8_e4m3fn conversions), the format's closed
forms, a hand-worked fixture, round trips, tie and saturation cases, and
invariants of the attention over a quantised cache."""

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_code_values_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(ours[ok]))


def test_code_values_closed_forms():
    v = fp8.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6            # smallest normal
    assert v(0x07) == 7 / 8 * 2.0 ** -6    # largest subnormal
    assert v(0x01) == 2.0 ** -9            # smallest subnormal
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x30) == 0.5
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert not math.isnan(v(0x7E)) and not math.isnan(v(0x78))   # e=15 is finite except f=7
    assert v(0x78) == 256.0


def test_finite_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_value(codes)), codes)


def test_encoder_matches_torch_rounding_in_range():
    """torch's float32 -> float8_e4m3fn conversion rounds to nearest even;
    inside the finite range it must agree with the oracle everywhere,
    midpoints and subnormals included."""
    rng = np.random.default_rng(0)
    mags = fp8.e4m3_value(np.arange(0, 0x7F))
    mids = (mags[1:] + mags[:-1]) / 2
    x = np.concatenate([
        rng.standard_normal(20000) * 4,
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000)),
        mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        mags, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -10 * 3],
    ]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448.0]
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = fp8.e4m3_encode(x.astype(np.float64))
    bad = np.nonzero(lib != ours)[0]
    assert bad.size == 0, (x[bad[:5]], lib[bad[:5]], ours[bad[:5]])


def test_ties_go_to_the_even_code():
    for c in range(0, 0x7E):
        lo, hi = fp8.e4m3_value(c), fp8.e4m3_value(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(mid) == even
        assert fp8.e4m3_encode(-mid) == even | 0x80
        assert fp8.e4m3_encode(np.nextafter(mid, -1)) == c
        assert fp8.e4m3_encode(np.nextafter(mid, 1000)) == c + 1


def test_saturation_and_nan():
    x = np.array([449.0, 464.0, 480.0, 1e9, np.inf, -449.0, -np.inf, np.nan])
    assert fp8.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]


def test_encoder_is_monotone():
    x = np.sort(np.random.default_rng(1).uniform(-500, 500, 50000))
    v = fp8.e4m3_value(fp8.e4m3_encode(x))
    assert np.all(np.diff(v) >= 0)


def test_quantise_golden():
    fx = json.load(open(os.path.join(GOLDEN, "fp8_e4m3_quantise.json")))
    x = np.array([float(c["x"]) for c in fx["cases"]], dtype=np.float32)
    want = [int(c["code"], 16) for c in fx["cases"]]
    assert fp8.quantize(x, fx["k_scale"]).tolist() == want
    for c in fx["float32_quotient_cases"]:
        assert fp8.quantize(np.float32(c["x"]), c["scale"]) == int(c["code"], 16), c["why"]


def test_quantise_divides_in_float32():
    """The quotient is a float32: scaling by a power of two is exact, and a
    source from a 16-bit type is widened exactly."""
    x = torch.randn(4096, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    base = fp8.quantize(x, 1.0)
    assert np.array_equal(fp8.quantize(x.float() * 8, 8.0), base)
    assert np.array_equal(fp8.quantize(x, 0.25), fp8.quantize(x.float() * 4, 1.0))
    assert np.array_equal(base, fp8.e4m3_encode(x.double().numpy()))


def test_reshape_and_cache_fp8_places_codes():
    k = np.array([[[1.0, -0.3, 300.0, 0.001]], [[4.5, 0.0, -0.0, 0.53125]]], np.float32)
    v = -k
    kc = np.full((3, 1, 2, 4), 0xAA, np.uint8)
    vc = kc.copy()
    fp8.reshape_and_cache_fp8(k, v, kc, vc, np.array([5, -1]), 0.5, 2.0)
    assert kc[2, 0, 1].tolist() == [0x40, 0xB2, 0x7E, 0x01]
    assert (kc[:2] == 0xAA).all() and (kc[2, 0, 0] == 0xAA).all()
    # V row -k[0] under scale 2: -1/2 = -0.5 is 0xB0 (e=6, f=0, sign)
    assert vc[2, 0, 1, 0] == 0xB0
    assert vc[2, 0, 1].tolist() == fp8.quantize(-k[0, 0], 2.0).tolist()


def test_decode_fp8_scales_factor_out():
    """A K scale multiplies every score (the same as a larger attention
    scale on the raw code values), and a power-of-two V scale multiplies the
    output exactly."""
    rng = np.random.default_rng(5)
    nb, hkv, bs, hd, B, hq = 12, 2, 8, 16, 3, 4
    kc = rng.integers(0, 256, (nb, hkv, bs, hd)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, hkv, bs, hd)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    q = rng.standard_normal((B, hq, hd))
    tables = rng.permutation(nb)[:B * 4].reshape(B, 4)
    lens = np.array([30, 1, 17])
    a = fp8.decode_fp8(q, kc, vc, tables, lens, 0.1, 0.25, 1.0, hkv)
    b = oracle.decode(q, fp8.e4m3_value(kc), fp8.e4m3_value(vc), tables, lens, 0.025, hkv)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    c = fp8.decode_fp8(q, kc, vc, tables, lens, 0.1, 0.25, 4.0, hkv)
    assert np.array_equal(c, 4.0 * a)
    # one token: the output is that token's dequantised V row
    assert np.array_equal(a[1], np.repeat(fp8.e4m3_value(vc[tables[1, 0], :, 0, :]), 2, axis=0))


def test_prefill_fp8_one_query_per_sequence_is_decode_fp8():
    """Prefill over codes with one query per sequence is decode over codes;
    with every token queried, the last row of each sequence is too."""
    rng = np.random.default_rng(9)
    nb, hkv, bs, hd = 10, 2, 4, 8
    kc = rng.integers(0, 0x7F, (nb, hkv, bs, hd)).astype(np.uint8)
    vc = rng.integers(0, 0x7F, (nb, hkv, bs, hd)).astype(np.uint8)
    tables = rng.permutation(nb)[:8].reshape(2, 4)
    lens = np.array([13, 6])
    q = rng.standard_normal((2, 4, hd))
    one = fp8.prefill_fp8(q, kc, vc, tables, lens, np.arange(3), 0.2, 0.5, 0.25, hkv)
    assert np.array_equal(one, fp8.decode_fp8(q, kc, vc, tables, lens, 0.2, 0.5, 0.25, hkv))
    qa = rng.standard_normal((19, 4, hd))
    qs = np.array([0, 13, 19])
    full = fp8.prefill_fp8(qa, kc, vc, tables, lens, qs, 0.2, 0.5, 0.25, hkv)
    last = fp8.decode_fp8(qa[[12, 18]], kc, vc, tables, lens, 0.2, 0.5, 0.25, hkv)
    assert np.allclose(full[[12, 18]], last, rtol=0, atol=1e-13)
