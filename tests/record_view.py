"""Reads packed tile records (as laid out in include/kvarn.h) into arrays, and compares a
library-written record with the oracle's for the same input tile.

This parser is test code of its own (it shares nothing with the library or the oracle): it
only decodes the documented byte layout so that records can be compared field by field."""

import numpy as np

T = D = 128
SIZES = {13312: 2, 17408: 4}          # record bytes -> value bits


def _v_index(vbits):
    t, j = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
    nb, n = j // 16, j % 16
    kb, h, s, i = t // 32, (t // 16) % 2, (t // 4) % 4, t % 4
    if vbits == 2:
        word = 256 * kb + 4 * (16 * s + n) + 2 * h + i // 2
        bit = 2 * nb + 16 * (i % 2)
    else:
        word = 512 * kb + 256 * (nb // 4) + 4 * (16 * s + n) + 2 * h + i // 2
        bit = 4 * (nb % 4) + 16 * (i % 2)
    return word, bit


_VIDX = {vb: _v_index(vb) for vb in (2, 4)}


def parse(rec: np.ndarray) -> dict:
    rec = np.asarray(rec, np.uint8)
    vbits = SIZES[rec.shape[0]]
    k_meta = 8192 + 2048 * vbits
    kb = rec[:8192].reshape(T, 64).astype(np.int64)
    kc = np.stack([kb & 15, kb >> 4], axis=-1).reshape(T, D)
    words = rec[8192:k_meta].view("<u4").astype(np.int64)
    vw, vbit = _VIDX[vbits]
    vc = (words[vw] >> vbit) & ((1 << vbits) - 1)
    out = dict(k_codes=kc, v_codes=vc, v_bits=vbits)
    for name, off in (("k", k_meta), ("v", k_meta + 512)):
        out[name + "_c"] = rec[off:off + 128].copy()
        out[name + "_s"] = rec[off + 128:off + 256].copy()
        out[name + "_z"] = rec[off + 256:off + 512].view("<u2").copy()
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
        # when fewer than 10,000 were compared (a single tile holds 768 scale values)
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
    budget.values += 3 * 128
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
