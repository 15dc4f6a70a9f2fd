"""The key decode of the local-window kernel's fast path, checked on the CPU.

For a grid with rows of W >= 8 tokens and key indices below 2^22, the kernel
splits a key index k into row k // W as trunc(fma(k, 1/W, 1/(2W))) in fp32,
with 1/W rounded from fp64 (and the row into frame and row-in-frame the same
way with H). The exact value k/W + 1/(2W) lies at least 1/(2W) from the next
integer and the fp32 error of the product stays below that while k < 2^22.
This test evaluates that expression exactly as the hardware does (the fp64
sum k * invW + invW / 2 is exact here, so rounding it once to fp32 is the
fused multiply-add) for every k below 2^22 and a spread of divisors. The
kernel writes it as trunc((k + 1/2) * invW): k + 1/2 is exact in fp32 below
2^23 and the product rounds the same exact value once, so the two forms give
the same bits, which the test checks as well."""
import numpy as np
import pytest

LIMIT = 1 << 22
DIVISORS = sorted(set(list(range(1, 65)) + [79, 80, 81, 96, 100, 127, 128, 129, 255, 256, 257, 1000, 1023,
                                            1025, 4095, 4096, 65535, 65537, (1 << 21) - 1, 1 << 21,
                                            LIMIT - 1]))


def fast_quotient(k: np.ndarray, w: int) -> np.ndarray:
    inv = np.float32(1.0 / float(w))
    half = np.float32(inv * np.float32(0.5))  # exact: a power-of-two scaling
    exact = k.astype(np.float64) * np.float64(inv) + np.float64(half)  # fits in 53 bits
    return exact.astype(np.float32).astype(np.int64)  # one rounding, then truncation


def kernel_quotient(k: np.ndarray, w: int) -> np.ndarray:
    """The form the kernel evaluates: fp32 k + 0.5 (exact), times 1/W rounded once."""
    inv = np.float32(1.0 / float(w))
    x = (k.astype(np.float32) + np.float32(0.5)).astype(np.float64)
    assert np.all(x == k.astype(np.float64) + 0.5)
    return (x * np.float64(inv)).astype(np.float32).astype(np.int64)  # the product fits in 53 bits


@pytest.fixture(scope="module")
def keys():
    return np.arange(LIMIT, dtype=np.int64)


@pytest.mark.parametrize("w", DIVISORS)
def test_fast_decode_is_exact_below_2_pow_22(keys, w):
    q = fast_quotient(keys, w)
    bad = np.nonzero(q != keys // w)[0]
    assert bad.size == 0, f"W={w}: first wrong k={bad[:5]}"
    assert np.array_equal(kernel_quotient(keys, w), q)


def test_the_bound_is_needed():
    """Past 2^22 the same expression goes wrong for some divisor, so the
    host must keep the fast path below it."""
    k = np.arange(LIMIT, 1 << 25, 7, dtype=np.int64)
    assert any(np.any(fast_quotient(k, w) != k // w) for w in (3, 7, 11, 79, 80, 81, 1023))
