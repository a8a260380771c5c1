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
