"""Pins of the oracle's codecs (FP8 e4m3 and bf16) against things other than the oracle itself.

The pages name the KV storage format only as "FP8 (e4m3)" (Cloudflare, "Smaller, faster, safer",
section 量化 KV cache).  The oracle's encoder/decoder implement the OCP E4M3FN format with
round-to-nearest-even and saturation at +-448; the checks below pin that against
  * closed forms of the format (code table values, hand-derived ties, saturation),
  * torch's own float8_e4m3fn and bfloat16 conversions (independent library routines),
  * an independent nearest-neighbour search over the sorted table of code values,
  * the theorem that fp64 division rounded to fp32 equals correctly rounded fp32 division.
"""
import numpy as np
import pytest
import torch


def _torch_decode_table():
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_code_table_closed_forms(orc):
    d = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])           # -0 kept
    assert d[0x01] == 2.0**-9                                # smallest subnormal
    assert d[0x07] == 7 * 2.0**-9                            # largest subnormal
    assert d[0x08] == 2.0**-6                                # smallest normal
    assert d[0x38] == 1.0                                    # exponent field 7 = bias
    assert d[0x39] == 1.125
    assert d[0x7E] == 448.0                                  # largest finite
    assert d[0xFE] == -448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])           # the only NaN patterns
    assert np.isfinite(np.delete(d, [0x7F, 0xFF])).all()     # no infinities in E4M3FN


def test_decode_matches_torch_float8_e4m3fn(orc):
    ref = _torch_decode_table()
    d = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert (nan == np.isnan(d)).all()
    assert (ref[~nan] == d[~nan]).all()
    assert (np.signbit(ref[~nan]) == np.signbit(d[~nan])).all()


def test_round_trip_all_finite_codes(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    assert (orc.e4m3_encode(vals) == codes).all()


@pytest.mark.parametrize("t,code", [
    (1.0625, 0x38),          # halfway 1.0 (m=0) / 1.125 (m=1): even mantissa m=0
    (1.1875, 0x3A),          # halfway 1.125 (m=1) / 1.25 (m=2): even m=2
    (2.0**-10, 0x00),        # halfway 0 / 2^-9: even -> 0
    (3 * 2.0**-10, 0x02),    # halfway 2^-9 (m=1) / 2^-8 (m=2): even m=2
    (15 * 2.0**-10, 0x08),   # halfway 7*2^-9 / 2^-6: rounds up into the first normal (m=0 even)
    (-1.0625, 0xB8),
    (240.0, 0x77),           # exact: 1.875 * 2^7
    (232.0, 0x76),           # halfway 224 (m=6) / 240 (m=7): even m=6
    (447.0, 0x7E),
    (440.0, 0x7E),           # above the 416/448 midpoint (432)
])
def test_hand_derived_ties(orc, t, code):
    assert orc.e4m3_encode(np.float32(t))[0] == code


def test_midpoint_416_448(orc):
    # 416 = (8+5)*2^5 (code 0x7D), 448 = (8+6)*2^5 (code 0x7E); the midpoint 432 ties to the
    # even mantissa 6.
    assert orc.e4m3_encode(np.float32(432.0))[0] == 0x7E
    assert orc.e4m3_encode(np.nextafter(np.float32(432.0), np.float32(0)))[0] == 0x7D


def test_saturation_nan_and_signed_zero(orc):
    vals = np.array([448.0, 449.0, 464.0, 1e9, np.inf, -449.0, -np.inf, np.float32(3.4e38)], np.float32)
    assert list(orc.e4m3_encode(vals)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E]
    assert orc.e4m3_encode(np.float32(np.nan))[0] == 0x7F
    assert orc.e4m3_encode(np.float32(-np.nan))[0] == 0xFF
    assert orc.e4m3_encode(np.float32(-0.0))[0] == 0x80
    assert orc.e4m3_encode(np.float32(0.0))[0] == 0x00
    assert orc.e4m3_encode(np.float32(-1e-30))[0] == 0x80     # underflow keeps the sign


def _nearest_by_search(t):
    """Independent nearest-code search on the sorted positive code values (ties -> even code)."""
    tab = _torch_decode_table()[:0x7F]                 # codes 0..126, strictly increasing values
    a = np.abs(t.astype(np.float64))
    idx = np.clip(np.searchsorted(tab, a), 1, 126)
    lo, hi = idx - 1, idx
    dlo, dhi = a - tab[lo], tab[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= tab[126], 126, pick)          # saturate at 448
    return (pick | np.where(np.signbit(t), 0x80, 0)).astype(np.uint8)


def test_encode_matches_independent_nearest_search(orc):
    rng = np.random.default_rng(12345)
    log_uniform = np.exp2(rng.uniform(-14, 10, 1_000_000)) * rng.choice([-1, 1], 1_000_000)
    uniform = rng.uniform(-500, 500, 500_000)
    tab = _torch_decode_table()[:0x7F]
    mids = (tab[1:] + tab[:-1]) / 2                    # every midpoint (exact in fp32)
    m32 = mids.astype(np.float32)
    assert (m32.astype(np.float64) == mids).all()
    edge = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           tab.astype(np.float32)])
    edge = np.concatenate([edge, -edge])
    t = np.concatenate([log_uniform.astype(np.float32), uniform.astype(np.float32), edge])
    assert (orc.e4m3_encode(t) == _nearest_by_search(t)).all()


def test_encode_matches_torch_cast_below_448(orc):
    rng = np.random.default_rng(7)
    t = (np.exp2(rng.uniform(-14, 8.8, 400_000)) * rng.choice([-1, 1], 400_000)).astype(np.float32)
    t = t[np.abs(t) < 448]
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (orc.e4m3_encode(t) == ref).all()


def test_quantize_is_fp32_division_then_encode(orc):
    # fp64 division rounded once to fp32 equals the correctly rounded fp32 quotient (53 >= 2*24+2),
    # so this route to fp32(x/s) shares nothing with the oracle's single-precision division.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(300_000) * 4).astype(np.float32)
    for s in [np.float32(4.0 / 448), np.float32(0.0123456), np.float32(1.0), np.float32(37.5 / 448)]:
        t = (x.astype(np.float64) / np.float64(s)).astype(np.float32)
        assert (orc.quantize_fp8(x, s) == orc.e4m3_encode(t)).all()


def test_bf16_matches_torch_cast(orc):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        (rng.standard_normal(500_000) * np.exp2(rng.uniform(-30, 30, 500_000))).astype(np.float32),
        rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (orc.bf16_from_f32(x) == ref).all()


def test_bf16_closed_forms(orc):
    u = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x7F7FFFFF, 0x7F7F7FFF, 0x80000000, 0x00000001,
                  0x7F800000, 0xFF800000], np.uint32)
    # tie -> even 0x3F80; tie -> even 0x3F82; above tie -> 0x3F81; overflow past the top
    # midpoint -> inf; just below it -> max finite; -0; smallest denormal -> +0; +-inf kept
    exp = [0x3F80, 0x3F82, 0x3F81, 0x7F80, 0x7F7F, 0x8000, 0x0000, 0x7F80, 0xFF80]
    assert list(orc.bf16_from_f32(u.view(np.float32))) == exp
    assert orc.bf16_from_f32(np.float32(np.nan))[0] == 0x7FC0
