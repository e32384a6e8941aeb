"""One-tile KVarN quantisation, the packed tile record, and dequantisation (fp64).

A tile is 128 tokens x 128 channels of one KV head, keys or values, rows = tokens,
columns = channels (reading R1). [GR] "What KVarN changes in vLLM's serving path": the preset
kvarn_k4v2_g128 stores keys with 4 bits and values with 2 bits per element, per 128-token tile
(one paged-cache block), with FP8 scales and FP16 zero-points. [GR] "The four-stage pipeline"
gives the order of the write-path stages: Hadamard rotation along channels, an iterative
Sinkhorn-like normalisation that alternates column and row standard deviations in log space,
then asymmetric round-to-nearest on a uniform grid; the scales are applied again only when the
tile is read for attention. [TSM] "What KVarN does differently" describes the same two
conditioning steps.

The steps below follow that order. Readings taken where the pages are silent (R-numbers as in
the design notes): R4 centred population standard deviation; R5 column step first; R6 a fixed
number N of rounds (default 4); R7 log-space scales with the gauge mean_j log c_j = 0; R8 a
floor on every standard deviation, relative to the largest magnitude of the matrix being
normalised; R9 one asymmetric grid per token over the channel-equalised values; R12 FP8 scales
per channel (c-hat) and per token (s-hat), FP16 zero-point per token (z-hat); R13 codes and
c-hat round to nearest-even, s-hat rounds up and z-hat rounds down so that the grid covers
every value of its token; R14 codes come from the stored, rounded scales; R15 overflow
saturates and is flagged.

Test infrastructure only (see the package header).
"""

import numpy as np

from .formats import (E4M3_MAX, E4M3_MIN_SUBNORMAL, FP16_MAX, e4m3_rne, e4m3_ru, e4m3_value,
                      fp16_rd, fp16_value)
from .hadamard import H128, rotate

T = 128           # tokens per tile = tokens per cache block
D = 128           # head dimension = channels per token
K_BITS = 4
V_BITS = 2
DEFAULT_ITERS = 4

# ------------------------------------------------------------------ tile record layout
# One record per (block, KV head), 13312 bytes, little-endian:
#   [0, 8192)       key codes, token-major: token t at byte 64*t; channel j in byte j//2,
#                   low nibble for even j, high nibble for odd j
#   [8192, 12288)   value codes, 2 bits each, at the position given by v_code_position()
#   [12288, 12416)  key   per-channel scale c-hat, FP8 E4M3, channel j at byte j
#   [12416, 12544)  key   per-token scale s-hat, FP8 E4M3, token t at byte t
#   [12544, 12800)  key   per-token zero-point z-hat, FP16, token t at bytes 2t, 2t+1
#   [12800, 12928)  value c-hat;  [12928, 13056) value s-hat;  [13056, 13312) value z-hat
K_CODES_OFF = 0
V_CODES_OFF = 8192
K_META_OFF = 12288
V_META_OFF = 12800
C_REL, S_REL, Z_REL = 0, 128, 256
TILE_BYTES = 13312


def v_code_position(t, j):
    """Bit address of the 2-bit value code of token t, channel j inside the value-code section.

    The section is 1024 little-endian 32-bit words. With nb = j // 16, n = j % 16,
    kb = t // 32, h = (t // 16) % 2, s = (t // 4) % 4, i = t % 4:
        word = 256*kb + 4*(16*s + n) + (2*h + i // 2),   bit = 2*nb + 16*(i % 2).
    Returns (byte offset within the section, bit shift within that byte)."""
    t = np.asarray(t)
    j = np.asarray(j)
    nb, n = j // 16, j % 16
    kb, h, s, i = t // 32, (t // 16) % 2, (t // 4) % 4, t % 4
    word = 256 * kb + 4 * (16 * s + n) + (2 * h + i // 2)
    bit = 2 * nb + 16 * (i % 2)
    return 4 * word + bit // 8, bit % 8


_VT, _VJ = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
_V_BYTE, _V_SHIFT = v_code_position(_VT, _VJ)


# ------------------------------------------------------------------ normalisation


def normalise(xt: np.ndarray, iters: int = DEFAULT_ITERS, ddof: int = 0):
    """Log-space alternating standard-deviation normalisation of a rotated tile xt (T x D).

    lr (per token) starts at 0. Each round first sets every column's log scale to the log of
    the standard deviation over tokens of xt * exp(-lr), then every row's log scale to the log
    of the standard deviation over channels of xt * exp(-lc). A standard deviation is floored
    at 2^-16 times the largest magnitude of xt times the largest of the multipliers applied.
    The final row step does not change the output; it is returned for checking. The column
    log scales are then shifted to mean zero over channels (the gauge).

    ddof selects the population (0, reading R4) or sample (1) standard deviation; the gauge
    makes the result independent of it. Returns (lc_gauged, lc_raw, lr) as float64 arrays;
    iters = 0 returns all zeros."""
    xt = np.asarray(xt, dtype=np.float64)
    big = np.max(np.abs(xt))
    lr = np.zeros(xt.shape[0])
    lc = np.zeros(xt.shape[1])
    for _ in range(iters):
        u = np.exp(-lr)
        col_sd = np.std(xt * u[:, None], axis=0, ddof=ddof)
        lc = np.log(np.maximum(col_sd, 2.0 ** -16 * big * np.max(u)))
        v = np.exp(-lc)
        row_sd = np.std(xt * v[None, :], axis=1, ddof=ddof)
        lr = np.log(np.maximum(row_sd, 2.0 ** -16 * big * np.max(v)))
    return lc - np.mean(lc), lc, lr


# ------------------------------------------------------------------ one tile


def quantize_tile(x: np.ndarray, bits: int, iters: int = DEFAULT_ITERS, signs=None) -> dict:
    """Quantise one T x D tile of fp16 values with `bits`-bit codes.

    Returns a dict with c_hat, s_hat, z_hat (float64 values), c_code, s_code (E4M3 bytes),
    z_bits (FP16 patterns), codes (T x D int), and the intermediates xt (rotated tile),
    c (pre-rounding per-channel scale), step (pre-rounding per-token scale), y (xt / c_hat),
    flags (count of saturations)."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape != (T, D):
        raise ValueError("tile must be 128 x 128")
    qmax = (1 << bits) - 1
    xt = rotate(x, signs)                                 # stage 1: Hadamard along channels
    if np.max(np.abs(xt)) == 0.0:                         # all-zero tile (reading R8)
        one, one_code = e4m3_rne(np.ones(D))
        zero = np.zeros(T)
        return dict(c_hat=one, c_code=one_code, s_hat=zero, s_code=np.zeros(T, np.uint8),
                    z_hat=zero.copy(), z_bits=np.zeros(T, np.uint16),
                    codes=np.zeros((T, D), np.int64), xt=xt, c=np.ones(D), step=zero.copy(),
                    y=np.zeros((T, D)), flags=0)
    lc, _, _ = normalise(xt, iters)                       # stage 2: variance normalisation
    c = np.exp(lc)
    c_hat, c_code = e4m3_rne(np.clip(c, E4M3_MIN_SUBNORMAL, E4M3_MAX))
    y = xt / c_hat[None, :]                               # stage 3: asymmetric RTN per token
    mn = y.min(axis=1)
    mx = y.max(axis=1)
    flags = int(np.sum(mn < -FP16_MAX))
    z_hat, z_bits = fp16_rd(np.maximum(mn, -FP16_MAX))
    step = (mx - z_hat) / qmax
    flags += int(np.sum(step > E4M3_MAX))
    s_hat, s_code = e4m3_ru(np.minimum(step, E4M3_MAX))
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((y - z_hat[:, None]) / s_hat[:, None])
    codes = np.where(s_hat[:, None] > 0, np.clip(q, 0, qmax), 0).astype(np.int64)
    return dict(c_hat=c_hat, c_code=c_code, s_hat=s_hat, s_code=s_code, z_hat=z_hat,
                z_bits=z_bits, codes=codes, xt=xt, c=c, step=step, y=y, flags=flags)


def dequantize_rotated(c_hat, s_hat, z_hat, codes) -> np.ndarray:
    """Stage 4 values in the rotated space: c_hat_j * (s_hat_t * code_tj + z_hat_t)."""
    return np.asarray(c_hat)[None, :] * (np.asarray(s_hat)[:, None] * codes
                                         + np.asarray(z_hat)[:, None])


def dequantize(c_hat, s_hat, z_hat, codes, signs=None) -> np.ndarray:
    """Dequantised tile in the original space: rotated values times H (H is its own inverse),
    then the sign flips of the rotation (R27) undone."""
    out = dequantize_rotated(c_hat, s_hat, z_hat, codes) @ H128
    return out if signs is None else out * signs


# ------------------------------------------------------------------ record pack / unpack


def pack_record(kq: dict, vq: dict) -> np.ndarray:
    """The 13312-byte record of one (block, KV head) from the key and value tile results."""
    rec = np.zeros(TILE_BYTES, dtype=np.uint8)
    kc = np.asarray(kq["codes"], dtype=np.uint8)
    rec[K_CODES_OFF:V_CODES_OFF] = (kc[:, 0::2] | (kc[:, 1::2] << 4)).reshape(-1)
    vsec = np.zeros(K_META_OFF - V_CODES_OFF, dtype=np.uint8)
    vc = np.asarray(vq["codes"], dtype=np.uint8)
    np.bitwise_or.at(vsec, _V_BYTE.reshape(-1), (vc << _V_SHIFT).reshape(-1).astype(np.uint8))
    rec[V_CODES_OFF:K_META_OFF] = vsec
    for off, q in ((K_META_OFF, kq), (V_META_OFF, vq)):
        rec[off + C_REL:off + C_REL + D] = q["c_code"]
        rec[off + S_REL:off + S_REL + T] = q["s_code"]
        rec[off + Z_REL:off + Z_REL + 2 * T] = np.asarray(q["z_bits"], "<u2").view(np.uint8)
    return rec


def unpack_record(rec: np.ndarray) -> dict:
    """Codes and scales of both halves of a record: dict(k=..., v=...), each with
    codes (T x D int), c_code, s_code, z_bits and their float64 values."""
    rec = np.asarray(rec, dtype=np.uint8)
    if rec.shape != (TILE_BYTES,):
        raise ValueError("record must be 13312 bytes")
    kb = rec[K_CODES_OFF:V_CODES_OFF].reshape(T, D // 2).astype(np.int64)
    kcodes = np.empty((T, D), np.int64)
    kcodes[:, 0::2] = kb & 0xF
    kcodes[:, 1::2] = kb >> 4
    vsec = rec[V_CODES_OFF:K_META_OFF].astype(np.int64)
    vcodes = (vsec[_V_BYTE] >> _V_SHIFT) & 0x3
    out = {}
    for name, off, codes in (("k", K_META_OFF, kcodes), ("v", V_META_OFF, vcodes)):
        c_code = rec[off + C_REL:off + C_REL + D].copy()
        s_code = rec[off + S_REL:off + S_REL + T].copy()
        z_bits = rec[off + Z_REL:off + Z_REL + 2 * T].copy().view("<u2").astype(np.uint16)
        out[name] = dict(codes=codes, c_code=c_code, s_code=s_code, z_bits=z_bits,
                         c_hat=e4m3_value(c_code), s_hat=e4m3_value(s_code),
                         z_hat=fp16_value(z_bits))
    return out


def encode_record(k_tile, v_tile, iters: int = DEFAULT_ITERS, signs=None) -> np.ndarray:
    """Quantise the key and value tiles of one (block, KV head) and pack them."""
    return pack_record(quantize_tile(k_tile, K_BITS, iters, signs),
                       quantize_tile(v_tile, V_BITS, iters, signs))


def decode_record(rec, signs=None) -> tuple:
    """Dequantised (K-hat, V-hat) of a record in the original (unrotated) space."""
    u = unpack_record(rec)
    return tuple(dequantize(u[n]["c_hat"], u[n]["s_hat"], u[n]["z_hat"], u[n]["codes"], signs)
                 for n in ("k", "v"))
