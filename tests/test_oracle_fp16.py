"""The C++ oracle's hand-written binary16 <-> binary32 conversions, over every
binary16 bit pattern (CPU only).

Pins: numpy's IEEE conversions (an independent implementation), and, for the
rounding direction, every midpoint between neighbouring binary16 values (the
ties), the binary32 neighbours of each midpoint, the overflow edge 65520 and
the underflow edge 2^-25.
"""
import numpy as np

from oracle import _native as nat


def _f16_to_f32_all():
    h = np.arange(65536, dtype=np.uint16)
    out = np.empty(65536, dtype=np.float32)
    nat.lib().orc_f16_to_f32_array(nat.ptr(h), 65536, nat.ptr(out))
    return h, out


def _f32_to_f16(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.size, dtype=np.uint16)
    nat.lib().orc_f32_to_f16_array(nat.ptr(f), f.size, nat.ptr(out))
    return out


def test_f16_to_f32_every_pattern():
    h, got = _f16_to_f32_all()
    want = h.view(np.float16).astype(np.float32)
    finite = np.isfinite(want)
    assert np.array_equal(got[finite].view(np.uint32), want[finite].view(np.uint32))   # incl. -0, subnormals
    assert np.array_equal(np.isinf(got), np.isinf(want)) and np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_f32_to_f16_round_trips_every_pattern():
    h, f = _f16_to_f32_all()
    back = _f32_to_f16(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], h[~nan])
    assert np.all((back[nan] & 0x7C00) == 0x7C00) and np.all(back[nan] & 0x3FF)


def test_f32_to_f16_ties_and_neighbours():
    h = np.arange(0, 0x7C00, dtype=np.uint16)                    # every finite non-negative binary16
    lo = h[:-1].view(np.float16).astype(np.float64)
    hi = h[1:].view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)                       # exact: one more bit than binary16
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    for vals in (mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))):
        for sign in (1, -1):
            v = (sign * vals).astype(np.float32)
            assert np.array_equal(_f32_to_f16(v), v.astype(np.float16).view(np.uint16))
    # ties go to the even pattern
    assert np.all(_f32_to_f16(mid) % 2 == 0)


def test_f32_to_f16_edges_and_random():
    edges = np.array([65504, 65519.996, 65520, 1e6, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -24,
                      2.0 ** -14 * (1 - 2.0 ** -11), 1e-30, 0.0, -0.0, np.inf, -np.inf], dtype=np.float32)
    rng = np.random.default_rng(0)
    r = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 18, 200000))).astype(np.float32)
    with np.errstate(over="ignore"):        # numpy warns on the values that overflow to infinity
        assert np.array_equal(_f32_to_f16(edges), edges.astype(np.float16).view(np.uint16))
        assert np.array_equal(_f32_to_f16(r), r.astype(np.float16).view(np.uint16))


def test_scalar_entry_points_agree_with_arrays():
    lib = nat.lib()
    for hbits in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF):
        f = lib.orc_f16_to_f32(hbits)
        assert np.float32(f) == np.uint16(hbits).view(np.float16).astype(np.float32)
        assert lib.orc_f32_to_f16(f) == hbits
