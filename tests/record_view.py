"""Reads packed tile records (as laid out in include/kvarn.h) into arrays, and compares a
library-written record with the oracle's for the same input tile.

This parser is test code of its own (it shares nothing with the library or the oracle): it
only decodes the documented byte layout so that records can be compared field by field."""

import numpy as np

T = 128
# record bytes -> (head dimension D, value bits): 64 D key-code bytes, 16 D vbits value-code
# bytes, two metadata halves of D + 384 bytes
SIZES = {64 * d + 16 * d * vb + 2 * (d + 384): (d, vb) for d in (64, 128, 256) for vb in (2, 4)}


def _v_index(vbits, d):
    t, j = np.meshgrid(np.arange(T), np.arange(d), indexing="ij")
    nb, n = j // 16, j % 16
    kb, h, s, i = t // 32, (t // 16) % 2, (t // 4) % 4, t % 4
    e = 2 * h + i // 2
    if vbits == 2 and d >= 128:
        word = 2 * d * kb + (d // 32) * (16 * s + n) + 4 * (nb // 8) + e
        bit = 2 * (nb % 8) + 16 * (i % 2)
    elif vbits == 2:
        word = 128 * kb + 2 * (16 * s + n) + e // 2
        bit = 2 * nb + 8 * (e % 2) + 16 * (i % 2)
    else:
        word = 4 * d * kb + 256 * (nb // 4) + 4 * (16 * s + n) + e
        bit = 4 * (nb % 4) + 16 * (i % 2)
    return word, bit


_VIDX = {(vb, d): _v_index(vb, d) for vb in (2, 4) for d in (64, 128, 256)}


def parse(rec: np.ndarray) -> dict:
    rec = np.asarray(rec, np.uint8)
    d, vbits = SIZES[rec.shape[0]]
    kcode = 64 * d
    k_meta = kcode + 16 * d * vbits
    kb = rec[:kcode].reshape(T, d // 2).astype(np.int64)
    kc = np.stack([kb & 15, kb >> 4], axis=-1).reshape(T, d)
    words = rec[kcode:k_meta].view("<u4").astype(np.int64)
    vw, vbit = _VIDX[(vbits, d)]
    vc = (words[vw] >> vbit) & ((1 << vbits) - 1)
    out = dict(k_codes=kc, v_codes=vc, v_bits=vbits, head_dim=d)
    for name, off in (("k", k_meta), ("v", k_meta + d + 384)):
        out[name + "_c"] = rec[off:off + d].copy()
        out[name + "_s"] = rec[off + d:off + d + 128].copy()
        out[name + "_z"] = rec[off + d + 128:off + d + 384].view("<u2").copy()
    return out


def e4m3(code):
    code = np.asarray(code, np.int64)
    e, m = (code >> 3) & 15, code & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def fp16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


class Budget:
    """Counts of tolerated differences between library and oracle records."""

    def __init__(self):
        self.values = 0
        self.scale_flips = 0
        self.elements = 0
        self.code_off_by_one = 0
        self.flipped_rows = 0
        self.flipped_cols = 0

    def check(self, flip_rate=1e-4, code_rate=1e-4):
        # at most 1e-4 of the scale values and of the codes, and never more than one of each
        # when fewer than 10,000 were compared (a tile holds 2 (D + 256) scale values)
        assert self.scale_flips <= max(1, int(flip_rate * self.values)), vars(self)
        assert self.code_off_by_one <= max(1, int(code_rate * self.elements)), vars(self)

    def exact(self):
        return self.scale_flips == 0 and self.code_off_by_one == 0


def _near(x, boundary, rel=1e-5):
    return np.abs(x - boundary) <= rel * np.abs(boundary)


def compare_half(gpu: dict, ora: dict, name: str, bits: int, budget: Budget):
    """Compare the key ('k') or value ('v') half of a library record (parsed) with the oracle's
    quantize_tile result for the same tile. Scale/zero-point differences are allowed only where
    the oracle's pre-rounding value lies within 1e-5 (relative) of the rounding boundary between
    the two stored values; rows and columns carrying such a flip are checked for validity (the
    library's codes reproduce its own grid within half a step) instead of equality."""
    qmax = 2 ** bits - 1
    gc, gs, gz = gpu[name + "_c"].astype(np.int64), gpu[name + "_s"].astype(np.int64), gpu[name + "_z"]
    oc, os_, oz = ora["c_code"].astype(np.int64), ora["s_code"].astype(np.int64), ora["z_bits"]
    budget.values += len(gc) + 2 * 128
    # per-channel scale (round to nearest): boundary = midpoint of the two codes
    dc = gc != oc
    if dc.any():
        assert np.all(np.abs(gc[dc] - oc[dc]) == 1), (name, "c-hat off by more than one step")
        mid = (e4m3(gc[dc]) + e4m3(oc[dc])) / 2
        pre = np.clip(ora["c"][dc], 2.0 ** -9, 448.0)
        assert np.all(_near(pre, mid)), (name, "c-hat flip away from a rounding boundary")
    # per-token zero-point (round down): boundary = the larger of the two fp16 values
    # a token whose minimum or maximum sits in a column whose c-hat moved has a different
    # grid legitimately; its z-hat and s-hat are then only checked for validity below
    moved = dc[ora["y"].argmin(axis=1)] | dc[ora["y"].argmax(axis=1)]
    dz = gz != oz
    if dz.any():
        gzv, ozv = fp16(gz[dz]), fp16(oz[dz])
        mn = ora["y"].min(axis=1)[dz]
        bound = np.maximum(gzv, ozv)
        row_scale = np.abs(ora["y"]).max(axis=1)[dz]
        # fp32 noise can move a minimum that is exactly 0 across zero: an absolute margin of
        # 1e-6 of the token's largest magnitude covers it
        near = np.abs(mn - bound) <= 1e-5 * np.abs(bound) + 1e-6 * row_scale
        between = (np.minimum(gzv, ozv) <= mn + 1e-6 * row_scale)
        assert np.all((near & between) | moved[dz]), (name, "z-hat flip away from a boundary")
    # per-token scale (round up): boundary = the smaller of the two E4M3 values, unless the
    # zero-point moved (then the pre-rounding value moved with it)
    ds = gs != os_
    if ds.any():
        one = np.abs(gs[ds] - os_[ds]) == 1
        near = _near(ora["step"][ds], np.minimum(e4m3(gs[ds]), e4m3(os_[ds])))
        assert np.all((one & (near | dz[ds])) | moved[ds]), \
            (name, "s-hat flip away from a rounding boundary")
    budget.scale_flips += int(dc.sum() + dz.sum() + ds.sum())
    rows = dz | ds
    cols = dc
    budget.flipped_rows += int(rows.sum())
    budget.flipped_cols += int(cols.sum())
    codes_g = gpu[name + "_codes"]
    codes_o = ora["codes"]
    assert codes_g.min() >= 0 and codes_g.max() <= qmax
    same = ~rows[:, None] & ~cols[None, :]
    diff = (codes_g != codes_o) & same
    if diff.any():
        assert np.all(np.abs(codes_g[diff] - codes_o[diff]) == 1), (name, "code off by > 1")
    budget.elements += int(same.sum())
    budget.code_off_by_one += int(diff.sum())
    if rows.any() or cols.any():
        # validity of the library's codes on its own grid, in the rows/columns that moved
        chat = e4m3(gc)
        shat = e4m3(gs)
        zhat = fp16(gz)
        y = ora["xt"] / chat[None, :]
        deq = shat[:, None] * codes_g + zhat[:, None]
        sel = ~same
        err = np.abs(y - deq)[sel]
        lim = (shat[:, None] / 2 * (1 + 1e-4) + 1e-6 * np.abs(y))[sel]
        assert np.all(err <= lim), (name, "codes invalid on the library's own grid")
