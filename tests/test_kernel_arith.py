"""CPU checks of arithmetic sequences the kernels use in place of the exact
operations the method defines (no GPU; numpy emulation of fp32 steps).

* Re-quantization to power-of-two block scales multiplies an E4M3 value by
  the 24-bit ratio s / s' in fp32 and converts the product to E4M3 with
  round-to-nearest-even.  The plain fp32 product can land on an E4M3
  midpoint the exact product is not on; the kernel rounds the product to odd
  (fp32 nearest product, its exact FMA remainder as a sticky bit).  Checked
  here for every finite code against 2^12 random ratios and ratios next to
  2/3, 0.7 and 0.9 (where plain fp32 products of small codes fall exactly on
  an E4M3 midpoint that the exact product misses), and the plain product
  shown to fail there (so the check has teeth).
"""
import numpy as np

from oracle import e4m3


def _round_odd_product(a32, m32):
    p = (a32 * m32).astype(np.float32)
    err = a32.astype(np.float64) * m32.astype(np.float64) - p.astype(np.float64)   # exact (<= 28 bits)
    bits = p.view(np.uint32).copy()
    fix = (err != 0) & ((bits & 1) == 0)
    up = np.sign(err) == np.sign(p)
    bits[fix & up] += np.uint32(1)
    bits[fix & ~up] -= np.uint32(1)
    return bits.view(np.float32), p


def test_requant_product_round_to_odd_is_exact_rounding():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    a = e4m3.decode(codes).astype(np.float32)
    rng = np.random.default_rng(0)
    # ratios s / s' in (1/2, 1]: 0.1f in binary with a random 23-bit f, plus
    # short mantissas (which make exact ties likely)
    f = rng.integers(0, 1 << 23, 1 << 12, dtype=np.uint32)
    f[:512] &= np.uint32(0x7FF000)
    m = ((np.uint32(126) << np.uint32(23)) | f).view(np.float32)
    m[0] = np.float32(1.0)
    near = [float.fromhex(h) for h in ("0x1.aaaaaap-1", "0x1.aaaaacp-1", "0x1.666666p-1", "0x1.ccccccp-1",
                                       "0x1.cccccep-1")]
    m = np.concatenate([m, np.array(near, np.float32)])
    A, Mm = np.meshgrid(a, m, indexing="ij")
    exact = e4m3.encode(A.astype(np.float64) * Mm.astype(np.float64))
    ro, rn = _round_odd_product(A, Mm)
    assert np.array_equal(e4m3.encode(ro.astype(np.float64)), exact)
    assert not np.array_equal(e4m3.encode(rn.astype(np.float64)), exact)


# --------------------------------------------------------------------------
# Group scale and its reciprocal without a division.  The quantizers compute,
# in every lane, s = fp32(max(amax, 1e-10) / 448) and r = fp32(1 / s) for the
# group whose maximum the lane holds, as
#     s0 = RN(a * C), C = RN(1/448);  e = RN(a - s0 * 448)  (one FMA);
#     s  = RN(s0 + e * C)                                    (one FMA);
#     r0 = hardware reciprocal of s (within an ulp or two);
#     t  = RN(1 - s * r0) (one FMA);  r = RN(r0 + r0 * t)   (one FMA).
# amax is a bf16 value (the maximum of bf16 inputs) or the fp32 floor, so
# the check below covers every input the sequence can see: each positive
# finite bf16 value >= 1e-10 and the floor, with every reciprocal estimate
# within 2 ulp of RN(1/s).  Rationals are exact; RN is round-to-nearest-even
# to fp32.

from fractions import Fraction as _Fr
import math as _math


def _rn32(q: _Fr) -> _Fr:
    """q rounded to the nearest fp32 value (ties to even), q in the normal range."""
    if q == 0:
        return _Fr(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = _math.floor(_math.log2(q.numerator) - _math.log2(q.denominator))
    while _Fr(2) ** e > q:
        e -= 1
    while _Fr(2) ** (e + 1) <= q:
        e += 1
    ulp = _Fr(2) ** (e - 23)
    m = q / ulp
    lo = _math.floor(m)
    rem = m - lo
    if rem > _Fr(1, 2) or (rem == _Fr(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


def _amax_values():
    vals = {np.float32(1e-10)}
    for e in range(-40, 128):
        for m in range(128):
            a = np.float32((1 + m / 128) * 2.0 ** e)
            if a >= np.float32(1e-10) and np.isfinite(a):
                vals.add(a)
    return sorted(vals)


def _neighbours(x: np.float32, k: int):
    out, up, dn = [x], x, x
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up, dn]
    return out


def test_group_scale_and_reciprocal_without_division_are_exact():
    C = _rn32(_Fr(1, 448))
    vals = _amax_values()
    assert len(vals) > 20000 and max(vals) == np.float32(3.3895314e38)
    plain_wrong = 0
    for a32 in vals:
        a = _Fr(float(a32))
        s_ref = _rn32(a / 448)
        s0 = _rn32(a * C)
        plain_wrong += s0 != s_ref
        e = _rn32(a - s0 * 448)
        s = _rn32(s0 + e * C)
        assert s == s_ref, float(a32)
        r_ref = _rn32(1 / s)
        for r0_32 in _neighbours(np.float32(float(r_ref)), 2):
            r0 = _Fr(float(r0_32))
            t = _rn32(1 - s * r0)
            assert _rn32(r0 + r0 * t) == r_ref, (float(a32), float(r0_32))
    # the refinement step is needed: the plain product is wrong for many amax
    assert plain_wrong > 1000
