"""One-tile KVarN quantisation, the packed tile record, and dequantisation (fp64).

A tile is 128 tokens x D channels of one KV head, keys or values, rows = tokens, columns =
channels (reading R1); D is the head dimension, 128 in the pages' preset, 64 or 256 under
reading R29. [GR] "What KVarN changes in vLLM's serving path": the preset kvarn_k4v2_g128
stores keys with 4 bits and values with 2 bits per element, per 128-token tile (one
paged-cache block), with FP8 scales and FP16 zero-points. [GR] "The four-stage pipeline" gives
the order of the write-path stages: Hadamard rotation along channels, an iterative
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
saturates and is flagged; R28 a second preset with 4-bit values (kvarn_k4v4_g128) beside the
pages' kvarn_k4v2_g128, same stages, its own record layout; R29 head dimensions 64 and 256
with the same stages, the same number of rounds and the same floor, a D-point rotation, D
per-channel scales, and the record layout below scaled with D ([GR] "Frequently Asked
Questions": other geometries are not covered by the preset and need their own scale layout).

Test infrastructure only (see the package header).
"""

import numpy as np

from .formats import (E4M3_MAX, E4M3_MIN_SUBNORMAL, FP16_MAX, e4m3_rne, e4m3_ru, e4m3_value,
                      fp16_rd, fp16_value)
from .hadamard import H_OF, HEAD_DIMS, check_head_dim, rotate

T = 128           # tokens per tile = tokens per cache block
D = 128           # head dimension of the pages' preset = channels per token
K_BITS = 4
V_BITS = 2        # value bits of the default preset kvarn_k4v2_g128
V_BITS_ALLOWED = (2, 4)
DEFAULT_ITERS = 4

# ------------------------------------------------------------------ tile record layout
# One record per (block, KV head), little-endian. With head dimension d, value bits vb (2 or
# 4) and V = 16 d vb bytes of value codes:
#   [0, 64 d)            key codes, token-major: token t at byte (d / 2) t; channel j in byte
#                        j // 2, low nibble for even j, high nibble for odd j
#   [64 d, 64 d + V)     value codes, vb bits each, at the position given by
#                        v_code_position() (vb = 2) or v4_code_position() (vb = 4)
#   then d + 384 bytes of key metadata and d + 384 of value metadata, each:
#     +0        per-channel scale c-hat, FP8 E4M3, channel j at byte j
#     +d        per-token scale s-hat, FP8 E4M3, token t at byte t
#     +d + 128  per-token zero-point z-hat, FP16, token t at bytes 2t, 2t+1
# d = 128, vb = 2: 13312 bytes (metadata at 12288 and 12800); vb = 4: 17408 (16384, 16896).
# d = 64: 7040 (vb = 2) and 9088 (vb = 4); d = 256: 25856 and 34048.
K_CODES_OFF = 0
V_CODES_OFF = 8192
K_META_OFF = 12288
V_META_OFF = 12800
C_REL, S_REL, Z_REL = 0, 128, 256
TILE_BYTES = 13312


def meta_rel(d: int = D) -> tuple:
    """Offsets of c-hat, s-hat and z-hat inside a metadata half of a record of head dim d."""
    return 0, d, d + 128


def layout(v_bits: int = V_BITS, d: int = D) -> dict:
    """Byte offsets and size of the record for `v_bits`-bit values and head dimension d."""
    if v_bits not in V_BITS_ALLOWED:
        raise ValueError("value bits must be 2 or 4")
    check_head_dim(d)
    v_codes = 64 * d
    k_meta = v_codes + 16 * d * v_bits
    half = d + 384
    return dict(k_codes=0, v_codes=v_codes, k_meta=k_meta, v_meta=k_meta + half,
                tile_bytes=k_meta + 2 * half)


def tile_bytes(v_bits: int = V_BITS, d: int = D) -> int:
    return layout(v_bits, d)["tile_bytes"]


def geometry_of_record(n_bytes: int) -> tuple:
    """(head dim, value bits) of a record of n_bytes bytes; the six sizes are distinct."""
    for d in HEAD_DIMS:
        for vb in V_BITS_ALLOWED:
            if tile_bytes(vb, d) == n_bytes:
                return d, vb
    raise ValueError("not a record size: " + str(n_bytes))


def v_bits_of_record(n_bytes: int) -> int:
    """The value bits a record of n_bytes bytes holds (13312: 2, 17408: 4, and so on)."""
    return geometry_of_record(n_bytes)[1]


def _token_split(t):
    t = np.asarray(t)
    return t // 32, (t // 16) % 2, (t // 4) % 4, t % 4


def v_code_position(t, j, d: int = D):
    """Bit address of the 2-bit value code of token t, channel j inside the value-code section.

    With nb = j // 16, n = j % 16, kb = t // 32, h = (t // 16) % 2, s = (t // 4) % 4, i = t % 4
    and e = 2 h + i // 2, the section is 2 d little-endian 32-bit words per token block kb.
    d >= 128 (one field of 2 bits per channel block of a 128-channel half hb = nb // 8):
        word = 2 d kb + (d / 32)(16 s + n) + 4 hb + e,   bit = 2 (nb % 8) + 16 (i % 2).
    d = 64 (two token pairs per word):
        word = 128 kb + 2 (16 s + n) + e // 2,   bit = 2 nb + 8 (e % 2) + 16 (i % 2).
    Returns (byte offset within the section, bit shift within that byte)."""
    check_head_dim(d)
    j = np.asarray(j)
    nb, n = j // 16, j % 16
    kb, h, s, i = _token_split(t)
    e = 2 * h + i // 2
    if d >= 128:
        word = 2 * d * kb + (d // 32) * (16 * s + n) + 4 * (nb // 8) + e
        bit = 2 * (nb % 8) + 16 * (i % 2)
    else:
        word = 128 * kb + 2 * (16 * s + n) + e // 2
        bit = 2 * nb + 8 * (e % 2) + 16 * (i % 2)
    return 4 * word + bit // 8, bit % 8


def v4_code_position(t, j, d: int = D):
    """Bit address of the 4-bit value code of token t, channel j (preset kvarn_k4v4_g128).

    The section is 4 d words per token block; the same token grouping as the 2-bit layout,
    with the channel blocks split into quarters hb = nb // 4 of four nibble fields each:
        word = 4 d kb + 256 hb + 4 (16 s + n) + (2 h + i // 2),   bit = 4 (nb % 4) + 16 (i % 2).
    Returns (byte offset within the section, bit shift within that byte)."""
    check_head_dim(d)
    j = np.asarray(j)
    nb, n = j // 16, j % 16
    kb, h, s, i = _token_split(t)
    word = 4 * d * kb + 256 * (nb // 4) + 4 * (16 * s + n) + (2 * h + i // 2)
    bit = 4 * (nb % 4) + 16 * (i % 2)
    return 4 * word + bit // 8, bit % 8


_V_POS = {}


def _v_pos(vb: int, d: int):
    if (vb, d) not in _V_POS:
        tt, jj = np.meshgrid(np.arange(T), np.arange(d), indexing="ij")
        _V_POS[(vb, d)] = (v_code_position if vb == 2 else v4_code_position)(tt, jj, d)
    return _V_POS[(vb, d)]


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
    """Quantise one T x D tile of fp16 values with `bits`-bit codes (D = 64, 128 or 256).

    Returns a dict with c_hat, s_hat, z_hat (float64 values), c_code, s_code (E4M3 bytes),
    z_bits (FP16 patterns), codes (T x D int), bits, and the intermediates xt (rotated tile),
    c (pre-rounding per-channel scale), step (pre-rounding per-token scale), y (xt / c_hat),
    flags (count of saturations)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[0] != T or x.shape[1] not in HEAD_DIMS:
        raise ValueError("tile must be 128 tokens x 64, 128 or 256 channels")
    d = x.shape[1]
    qmax = (1 << bits) - 1
    xt = rotate(x, signs)                                 # stage 1: Hadamard along channels
    if np.max(np.abs(xt)) == 0.0:                         # all-zero tile (reading R8)
        one, one_code = e4m3_rne(np.ones(d))
        zero = np.zeros(T)
        return dict(c_hat=one, c_code=one_code, s_hat=zero, s_code=np.zeros(T, np.uint8),
                    z_hat=zero.copy(), z_bits=np.zeros(T, np.uint16),
                    codes=np.zeros((T, d), np.int64), xt=xt, c=np.ones(d), step=zero.copy(),
                    y=np.zeros((T, d)), flags=0, bits=bits)
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
                z_bits=z_bits, codes=codes, xt=xt, c=c, step=step, y=y, flags=flags, bits=bits)


def dequantize_rotated(c_hat, s_hat, z_hat, codes) -> np.ndarray:
    """Stage 4 values in the rotated space: c_hat_j * (s_hat_t * code_tj + z_hat_t)."""
    return np.asarray(c_hat)[None, :] * (np.asarray(s_hat)[:, None] * codes
                                         + np.asarray(z_hat)[:, None])


def dequantize(c_hat, s_hat, z_hat, codes, signs=None) -> np.ndarray:
    """Dequantised tile in the original space: rotated values times H (H is its own inverse),
    then the sign flips of the rotation (R27) undone."""
    codes = np.asarray(codes)
    out = dequantize_rotated(c_hat, s_hat, z_hat, codes) @ H_OF[check_head_dim(codes.shape[1])]
    return out if signs is None else out * signs


# ------------------------------------------------------------------ record pack / unpack


def pack_record(kq: dict, vq: dict) -> np.ndarray:
    """The record of one (block, KV head) from the key and value tile results; its size
    follows the head dimension and the value bits vq["bits"] (d = 128: 13312 bytes for 2-bit
    values, 17408 for 4-bit)."""
    if kq.get("bits", K_BITS) != K_BITS:
        raise ValueError("keys are 4-bit in every preset")
    vb = vq.get("bits", V_BITS)
    kc = np.asarray(kq["codes"], dtype=np.uint8)
    vc = np.asarray(vq["codes"], dtype=np.uint8)
    d = check_head_dim(kc.shape[1])
    if vc.shape != kc.shape:
        raise ValueError("key and value tiles differ in shape")
    lay = layout(vb, d)
    rec = np.zeros(lay["tile_bytes"], dtype=np.uint8)
    rec[lay["k_codes"]:lay["v_codes"]] = (kc[:, 0::2] | (kc[:, 1::2] << 4)).reshape(-1)
    vsec = np.zeros(lay["k_meta"] - lay["v_codes"], dtype=np.uint8)
    vbyte, vshift = _v_pos(vb, d)
    np.bitwise_or.at(vsec, vbyte.reshape(-1), (vc << vshift).reshape(-1).astype(np.uint8))
    rec[lay["v_codes"]:lay["k_meta"]] = vsec
    c_rel, s_rel, z_rel = meta_rel(d)
    for off, q in ((lay["k_meta"], kq), (lay["v_meta"], vq)):
        rec[off + c_rel:off + c_rel + d] = q["c_code"]
        rec[off + s_rel:off + s_rel + T] = q["s_code"]
        rec[off + z_rel:off + z_rel + 2 * T] = np.asarray(q["z_bits"], "<u2").view(np.uint8)
    return rec


def unpack_record(rec: np.ndarray) -> dict:
    """Codes and scales of both halves of a record: dict(k=..., v=...), each with
    codes (T x D int), c_code, s_code, z_bits and their float64 values. The head dimension and
    value bits are those of the record's size (geometry_of_record)."""
    rec = np.asarray(rec, dtype=np.uint8)
    if rec.ndim != 1:
        raise ValueError("one record at a time")
    d, vb = geometry_of_record(rec.shape[0])
    lay = layout(vb, d)
    kb = rec[lay["k_codes"]:lay["v_codes"]].reshape(T, d // 2).astype(np.int64)
    kcodes = np.empty((T, d), np.int64)
    kcodes[:, 0::2] = kb & 0xF
    kcodes[:, 1::2] = kb >> 4
    vsec = rec[lay["v_codes"]:lay["k_meta"]].astype(np.int64)
    vbyte, vshift = _v_pos(vb, d)
    vcodes = (vsec[vbyte] >> vshift) & ((1 << vb) - 1)
    c_rel, s_rel, z_rel = meta_rel(d)
    out = {}
    for name, off, codes in (("k", lay["k_meta"], kcodes), ("v", lay["v_meta"], vcodes)):
        c_code = rec[off + c_rel:off + c_rel + d].copy()
        s_code = rec[off + s_rel:off + s_rel + T].copy()
        z_bits = rec[off + z_rel:off + z_rel + 2 * T].copy().view("<u2").astype(np.uint16)
        out[name] = dict(codes=codes, c_code=c_code, s_code=s_code, z_bits=z_bits,
                         c_hat=e4m3_value(c_code), s_hat=e4m3_value(s_code),
                         z_hat=fp16_value(z_bits))
    out["v_bits"] = vb
    out["head_dim"] = d
    return out


def encode_record(k_tile, v_tile, iters: int = DEFAULT_ITERS, signs=None,
                  v_bits: int = V_BITS) -> np.ndarray:
    """Quantise the key and value tiles of one (block, KV head) and pack them."""
    if v_bits not in V_BITS_ALLOWED:
        raise ValueError("value bits must be 2 or 4")
    return pack_record(quantize_tile(k_tile, K_BITS, iters, signs),
                       quantize_tile(v_tile, v_bits, iters, signs))


def decode_record(rec, signs=None) -> tuple:
    """Dequantised (K-hat, V-hat) of a record in the original (unrotated) space."""
    u = unpack_record(rec)
    return tuple(dequantize(u[n]["c_hat"], u[n]["s_hat"], u[n]["z_hat"], u[n]["codes"], signs)
                 for n in ("k", "v"))
