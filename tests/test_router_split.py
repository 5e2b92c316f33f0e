"""The matrix-core router splits each fp32 router weight into three bf16 parts
by truncation (w1 = w with its low 16 bits cleared, w2 the same of w - w1,
w3 = the rest).  That is exact only if w1 + w2 + w3 == w and every part is a
bf16 value; checked here on the host with the same bit operations, for random
weights of the generator's distribution and for edge values.  The domain is
w == 0 or |w| >= 2^-102: below that the last part falls under fp32's normal
range (N(0, 0.02) weights never get there)."""
import numpy as np


def split3(w):
    u = w.view(np.uint32)
    a1 = (u & np.uint32(0xFFFF0000)).view(np.float32)
    r1 = (w - a1).astype(np.float32)                    # fp32 subtraction, as on the device
    a2 = (r1.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    r2 = (r1 - a2).astype(np.float32)
    return a1, a2, r2


def is_bf16(v):
    return np.all((v.view(np.uint32) & np.uint32(0xFFFF)) == 0)


def check(w):
    a1, a2, a3 = split3(w)
    assert is_bf16(a1) and is_bf16(a2) and is_bf16(a3)
    exact = a1.astype(np.float64) + a2.astype(np.float64) + a3.astype(np.float64)
    assert np.array_equal(exact, w.astype(np.float64))


def test_split_exact_random_router_weights():
    rng = np.random.default_rng(7)
    check((rng.standard_normal(1 << 20) * 0.02).astype(np.float32))
    check(rng.standard_normal(1 << 16).astype(np.float32) * np.float32(1e30))


def test_split_exact_edge_values():
    bits = np.array([0x00000000, 0x80000000, 0x3F800000, 0x3F800001, 0x3FFFFFFF, 0x7F7FFFFF, 0xFF7FFFFF,
                     0x0C800000, 0x0C800001, 0x8C8FFFFF, 0x0E800001, 0x3DA3D70A, 0xBDA3D70A, 0x33FFFFFF],
                    dtype=np.uint32)   # 0x0C800000 = 2^-102
    check(bits.view(np.float32))
    # every low-16-bit pattern under one exponent and sign
    low = np.arange(1 << 16, dtype=np.uint32)
    check((np.uint32(0x3C2A0000) | low).view(np.float32))
    check((np.uint32(0xBC2A0000) | low).view(np.float32))


def test_split_products_with_bf16_are_exact():
    """x (bf16) times each part has at most 16 significant bits: exact in fp32."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(4096).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    w = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    for part in split3(w):
        p32 = (x * part).astype(np.float32)
        assert np.array_equal(p32.astype(np.float64), x.astype(np.float64) * part.astype(np.float64))
