"""fp8 (e4m3) state cache: the oracle's rounding pinned to the format's definition, and the
library's geometry rules for the compressed cache (CPU only).

The compressed cache follows DiTango, "Significato e Claim" (cache compression named as the
way to ease the state cache's memory cost); the format is OCP fp8 e4m3fn."""
import numpy as np
import pytest

from oracle.attention import round_fp8_e4m3


def _format_values():
    """Every finite e4m3fn value, enumerated from the bit fields: sign, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 is subnormal, (15, 7) is NaN."""
    vals = set()
    for sign in (1.0, -1.0):
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue
                mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
                vals.add(sign * mag)
    return np.array(sorted(vals))


FMT = _format_values()


def test_format_enumeration():
    assert len(FMT) == 253                       # 2 x 127 finite values, +0 and -0 merged
    assert FMT.max() == 448.0 and FMT.min() == -448.0
    assert np.min(FMT[FMT > 0]) == 2.0 ** -9


def test_representable_values_are_fixed_points():
    assert np.array_equal(round_fp8_e4m3(FMT), FMT)


@pytest.mark.parametrize("x, want", [
    (0.1, 13 / 128),              # 0.1 lies in [2^-4, 2^-3): spacing 2^-7; 12.8 -> 13
    (1.0625, 1.0),                # tie between 1.0 (mantissa 0) and 1.125 (1): even wins
    (1.1875, 1.25),               # tie between 1.125 (1) and 1.25 (2): even wins
    (3.3, 3.25),                  # spacing 0.25 in [2, 4)
    (-5.1, -5.0),
    (449.0, 448.0),               # saturation
    (1e4, 448.0),
    (2.0 ** -10, 0.0),            # tie between 0 and the smallest subnormal 2^-9: even (0)
    (3 * 2.0 ** -10, 2.0 ** -8),  # tie between 2^-9 (m=1) and 2^-8 (m=2): even
    (0.0015, 2.0 ** -9),
])
def test_hand_worked_values(x, want):
    assert round_fp8_e4m3(np.array([x]))[0] == want


def test_nearest_value_brute_force():
    """Against a search over the enumerated format: the nearest value, halfway cases to the
    one with an even mantissa (even bit pattern)."""
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-500, 500, 3000), rng.uniform(-0.05, 0.05, 3000),
                        rng.normal(0, 2, 3000), (FMT[1:] + FMT[:-1]) / 2])
    got = round_fp8_e4m3(x)
    codes = {}
    for sign_bit, sign in ((0, 1.0), (1, -1.0)):
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue
                mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
                codes.setdefault(sign * mag, (e << 3) | m)
    for xi, gi in zip(x, got):
        if abs(xi) >= 448:
            assert gi == np.copysign(448.0, xi)
            continue
        d = np.abs(FMT - xi)
        best = FMT[d == d.min()]
        if len(best) == 1:
            assert gi == best[0], (xi, gi, best)
        else:
            even = [b for b in best if codes[b] % 2 == 0]
            assert gi == even[0], (xi, gi, best)


def test_symmetric_and_monotonic():
    x = np.linspace(-460, 460, 20001)
    r = round_fp8_e4m3(x)
    assert np.array_equal(round_fp8_e4m3(-x), -r)
    assert np.all(np.diff(r) >= 0)


@pytest.fixture(scope="module")
def dita():
    return pytest.importorskip("partial_state_reuse_amd")


def test_library_accepts_fp8_cache_with_bf16_inputs_only(dita):
    g8 = dita.make_geometry(1, 2, 64, 64, 2, 4, 8, 4, dtype="bf16", cache_dtype="fp8")
    g16 = dita.make_geometry(1, 2, 64, 64, 2, 4, 8, 4, dtype="bf16")
    b8, b16 = dita.dita_cache_required_bytes(g8), dita.dita_cache_required_bytes(g16)
    assert b8 < b16
    bad = dita.make_geometry(1, 2, 64, 64, 2, 4, 8, 4, dtype="f32", cache_dtype="fp8")
    with pytest.raises(dita.DitaError, match="UNSUPPORTED"):
        dita.dita_cache_required_bytes(bad)
