"""The orthonormal Hadamard matrices used by the codec (64, 128 and 256 points).

[GR] "The four-stage pipeline", stage 1 and [TSM] "What KVarN does differently": each tile is
rotated along the channel dimension by an orthonormal Hadamard transform, which spreads a few
large channels over all channels and leaves attention scores unchanged.

Reading R2: the transform has as many points as the head dimension, is the Sylvester matrix in
natural order scaled by 1/sqrt(n), carries no random signs, and is the same for keys, values,
every head and every layer. Entry (i, j) is (-1)^popcount(i & j) / sqrt(n); the matrix is
symmetric and its own inverse. The pages' preset has 128 points; reading R29 takes 64 and 256
for the other head dimensions ([GR] "Frequently Asked Questions" says the preset covers only
128 and that another geometry needs its own layout).

Test infrastructure only (see the package header).
"""

import numpy as np

D = 128
HEAD_DIMS = (64, 128, 256)


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


H_OF = {d: hadamard(d) for d in HEAD_DIMS}
SIGNS_OF = {d: np.rint(H_OF[d] * np.sqrt(float(d))) for d in HEAD_DIMS}  # +-1 matrices, exact
H64, H128, H256 = H_OF[64], H_OF[128], H_OF[256]
SIGNS128 = SIGNS_OF[128]


def check_head_dim(d: int) -> int:
    if d not in HEAD_DIMS:
        raise ValueError("head dimension must be 64, 128 or 256")
    return d


def sign_vector(words, d: int = D) -> np.ndarray:
    """Per-channel signs (+-1, float64) of a head dimension d from d / 32 32-bit words
    (longer arrays: the first d / 32 words count): channel j is negated when bit j % 32 of
    word j // 32 is set (reading R27: the optional sign flips before the rotation; all-zero
    words give the plain Hadamard of R2)."""
    check_head_dim(d)
    w = np.asarray(words, dtype=np.uint64).reshape(-1)
    if w.shape[0] < d // 32:
        raise ValueError("need d / 32 sign words")
    j = np.arange(d)
    bits = (w[j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(bits == 1, -1.0, 1.0)


def rotate(x: np.ndarray, signs=None) -> np.ndarray:
    """(x * signs) @ H along the last axis (channels; 64, 128 or 256 of them), float64; signs
    None means all +1.

    The +-1 sums are formed first and scaled once: for fp16 inputs every partial sum is exact
    in float64, so an exactly zero rotated value comes out as exactly zero."""
    x = np.asarray(x, dtype=np.float64)
    d = check_head_dim(x.shape[-1])
    if signs is not None:
        x = x * signs
    return (x @ SIGNS_OF[d]) / np.sqrt(float(d))
