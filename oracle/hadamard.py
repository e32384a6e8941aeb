"""The 128-point orthonormal Hadamard matrix used by the codec.

[GR] "The four-stage pipeline", stage 1 and [TSM] "What KVarN does differently": each tile is
rotated along the channel dimension by an orthonormal Hadamard transform, which spreads a few
large channels over all channels and leaves attention scores unchanged.

Reading R2: the transform has 128 points (the head dimension; other head dimensions are not
supported, [GR] "Frequently Asked Questions"), is the Sylvester matrix in natural order scaled
by 1/sqrt(128), carries no random signs, and is the same for keys, values, every head and
every layer. Entry (i, j) is (-1)^popcount(i & j) / sqrt(128); the matrix is symmetric and
its own inverse.

Test infrastructure only (see the package header).
"""

import numpy as np

D = 128


def hadamard(n: int = D) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order n (a power of two), float64."""
    if n <= 0 or n & (n - 1):
        raise ValueError("order must be a power of two")
    i = np.arange(n)
    parity = np.zeros((n, n), dtype=np.int64)
    both = i[:, None] & i[None, :]
    while np.any(both):
        parity ^= both & 1
        both = both >> 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(float(n))


H128 = hadamard(D)
SIGNS128 = np.rint(H128 * np.sqrt(float(D)))  # the +-1 matrix, exact


def sign_vector(words) -> np.ndarray:
    """Per-channel signs (+-1, float64) from four 32-bit words: channel j is negated when bit
    j % 32 of word j // 32 is set (reading R27: the optional sign flips before the rotation;
    all-zero words give the plain Hadamard of R2)."""
    w = np.asarray(words, dtype=np.uint64).reshape(4)
    j = np.arange(D)
    bits = (w[j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(bits == 1, -1.0, 1.0)


def rotate(x: np.ndarray, signs=None) -> np.ndarray:
    """(x * signs) @ H along the last axis (channels), float64; signs None means all +1.

    The +-1 sums are formed first and scaled once: for fp16 inputs every partial sum is exact
    in float64, so an exactly zero rotated value comes out as exactly zero."""
    x = np.asarray(x, dtype=np.float64)
    if signs is not None:
        x = x * signs
    return (x @ SIGNS128) / np.sqrt(float(D))
