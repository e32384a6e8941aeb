"""Pins of the oracle at head dimensions 64 and 256 (reading R29): the D-point Hadamard matrix
against scipy and a radix-2 butterfly, closed-form tiles worked by hand for each D, the
normalisation and rounding invariants, the record layout (sizes, bijection, hand positions),
and the attention forms against each other and against torch's SDPA."""

import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import attention, codec, formats, hadamard
from workloads import gen

T = 128
DIMS = (64, 256)


def _tile(seed, d, drift=False):
    rng = np.random.default_rng([seed, d])
    mult = np.exp(rng.standard_normal(d))
    mult[rng.choice(d, 3, replace=False)] *= 15
    x = rng.standard_normal((T, d)) * mult
    if drift:
        x *= np.exp(0.5 * rng.standard_normal((T, 1)))
    return x.astype(np.float16).astype(np.float64)


# ------------------------------------------------------------------ the rotation


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_equals_scipy_sylvester(d):
    assert np.array_equal(hadamard.H_OF[d] * np.sqrt(float(d)),
                          scipy.linalg.hadamard(d).astype(float))
    h = hadamard.H_OF[d]
    assert np.array_equal(h, h.T)
    assert np.allclose(h @ h, np.eye(d), atol=1e-14, rtol=0)


@pytest.mark.parametrize("d", DIMS)
def test_rotation_matches_radix2_butterflies(d):
    x = np.random.default_rng(d).standard_normal(d)
    y = x.copy()
    half = 1
    while half < d:
        for start in range(0, d, 2 * half):
            for i in range(start, start + half):
                a, b = y[i], y[i + half]
                y[i], y[i + half] = a + b, a - b
        half *= 2
    assert np.allclose(y / np.sqrt(float(d)), hadamard.rotate(x), atol=1e-13, rtol=0)


def test_sign_words_per_head_dim():
    s = hadamard.sign_vector([1, 0x80000000], 64)
    assert s.shape == (64,) and s[0] == -1 and s[63] == -1 and np.sum(s < 0) == 2
    w = [0] * 8
    w[7] = 1 << 31
    w[4] = 1 << 3
    s = hadamard.sign_vector(w, 256)
    assert np.flatnonzero(s < 0).tolist() == [131, 255]
    with pytest.raises(ValueError):
        hadamard.sign_vector([0, 0, 0, 0], 256)


def test_other_head_dims_rejected():
    with pytest.raises(ValueError):
        codec.quantize_tile(np.zeros((T, 96)), 4)
    with pytest.raises(ValueError):
        codec.layout(2, 32)


# ------------------------------------------------------------------ closed-form tiles


def _closed_form_tile(d, seed):
    """fp16-exact tile whose rotation has one nonzero value per (token, channel pair) (d = 256)
    or two equal nonzero tokens per channel (d = 64), magnitudes 2^e with sum e = 0.

    d = 256: token t = sign_t 2^e_t (S[pi(2t)] + S[pi(2t + 1)]), S the +-1 Sylvester matrix.
    d = 64:  tokens tau(2j), tau(2j + 1) = sign_j 2^e_j S[j]."""
    rng = np.random.default_rng(seed)
    pm1 = hadamard.SIGNS_OF[d]
    x = np.zeros((T, d))
    if d == 256:
        pi = rng.permutation(d)
        sign = np.where(rng.random(T) < 0.5, -1.0, 1.0)
        half = rng.integers(-5, 6, T // 2)
        e = rng.permutation(np.concatenate([half, -half]))
        for t in range(T):
            x[t] = sign[t] * 2.0 ** e[t] * (pm1[pi[2 * t]] + pm1[pi[2 * t + 1]])
        chan_e = np.empty(d)
        chan_e[pi[0::2]] = e
        chan_e[pi[1::2]] = e
        tok_sign = sign
        nz = [(t, [pi[2 * t], pi[2 * t + 1]]) for t in range(T)]
    else:
        tau = rng.permutation(T)
        sign = np.where(rng.random(d) < 0.5, -1.0, 1.0)
        half = rng.integers(-5, 6, d // 2)
        chan_e = rng.permutation(np.concatenate([half, -half])).astype(float)
        tok_sign = np.empty(T)
        nz = []
        for j in range(d):
            for k in range(2):
                t = tau[2 * j + k]
                x[t] = sign[j] * 2.0 ** chan_e[j] * pm1[j]
                tok_sign[t] = sign[j]
                nz.append((t, [j]))
    return x, chan_e, tok_sign, sorted(nz)


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("seed", [0, 1])
def test_closed_form_tiles(d, seed):
    # Worked by hand (r = sqrt(d); a column or row of n entries holding k equal nonzeros w has
    # standard deviation w sqrt(k n - k^2) / n).
    # d = 256: the rotated token t holds sign_t 2^e_t r at its two channels and nothing else;
    #   each channel holds one nonzero among 128 tokens: c_j = 2^e_t r sqrt(127) / 128. The row
    #   step then sees two entries 128 / sqrt(127) among 256 channels: std
    #   (128 / sqrt(127)) sqrt(508) / 256 = 1 exactly, so the rows stay at 1 and every round
    #   repeats the columns. Gauge (mean log c = 0 with sum e = 0): c-hat_j = 2^e_t.
    #   y = xt / c-hat: two entries sign * 16 per token.
    #     sign +1: z = 0; K s = RU(16 / 15 = 1.0667) = 1.125, codes 14 at the two channels
    #              (16 / 1.125 = 14.2), 0 elsewhere; V s = RU(16 / 3 = 5.333) = 5.5, codes 3.
    #     sign -1: z = -16; the two channels 0, the rest 14 (K) and 3 (V).
    # d = 64: each channel holds two equal entries sign_j 2^e_j r among 128 tokens:
    #   c_j = 2^e_j r sqrt(252) / 128; the row step sees one entry 128 / sqrt(252) among 64
    #   channels: std (128 / sqrt(252)) sqrt(63) / 64 = 1 exactly. c-hat_j = 2^e_j.
    #   y: one entry sign * 8 per token.
    #     sign +1: z = 0; K s = RU(8 / 15 = 0.5333) = 0.5625, code 14 (8 / 0.5625 = 14.2);
    #              V s = RU(8 / 3 = 2.667) = 2.75, code 3 (2.91).
    #     sign -1: z = -8; the channel 0, the rest 14 (K) and 3 (V).
    x, chan_e, tok_sign, nz = _closed_form_tile(d, seed)
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
    r = math.sqrt(d)
    s_exp = {256: {4: 1.125, 2: 5.5}, 64: {4: 0.5625, 2: 2.75}}[d]
    for bits, top in ((4, 14), (2, 3)):
        q = codec.quantize_tile(x, bits)
        assert np.array_equal(q["c_hat"], 2.0 ** chan_e)
        assert np.array_equal(q["s_hat"], np.full(T, s_exp[bits]))
        assert np.array_equal(q["z_hat"], np.where(tok_sign > 0, 0.0, -r))
        codes = np.where(tok_sign[:, None] > 0, 0, top) * np.ones((T, d), int)
        for t, chans in nz:
            codes[t, chans] = top if tok_sign[t] > 0 else 0
        assert np.array_equal(q["codes"], codes)


# ------------------------------------------------------------------ invariants


@pytest.mark.parametrize("d", DIMS)
def test_normalisation_invariants(d):
    xt = hadamard.rotate(_tile(3, d, drift=True))
    for iters in (1, 4):
        _, lc, lr = codec.normalise(xt, iters)
        z = xt * np.exp(-lr)[:, None] * np.exp(-lc)[None, :]
        assert np.allclose(z.std(axis=1), 1.0, rtol=0, atol=1e-12)
    _, lc_prev, lr_prev = codec.normalise(xt, 3)
    _, lc, _ = codec.normalise(xt, 4)
    z = xt * np.exp(-lr_prev)[:, None] * np.exp(-lc)[None, :]
    assert np.allclose(z.std(axis=0), 1.0, rtol=0, atol=1e-12)
    lc0, _, _ = codec.normalise(xt, 4, ddof=0)
    lc1, _, _ = codec.normalise(xt, 4, ddof=1)
    assert abs(lc0.mean()) < 1e-14 and np.allclose(lc0, lc1, rtol=0, atol=1e-13)


@pytest.mark.parametrize("d", DIMS)
def test_scaling_and_permutation(d):
    x = _tile(6, d, drift=True)
    perm = np.random.default_rng(0).permutation(T)
    for bits in (4, 2):
        a = codec.quantize_tile(x, bits)
        b = codec.quantize_tile(x * 4.0, bits)
        c = codec.quantize_tile(x[perm], bits)
        assert np.array_equal(a["c_hat"], b["c_hat"]) and np.array_equal(a["codes"], b["codes"])
        assert np.array_equal(a["s_hat"] * 4.0, b["s_hat"])
        assert np.array_equal(a["z_hat"] * 4.0, b["z_hat"])
        assert np.array_equal(a["c_hat"], c["c_hat"])
        assert np.array_equal(a["codes"][perm], c["codes"])


@pytest.mark.parametrize("d", DIMS)
def test_rtn_bounds_and_bypass(d):
    x = _tile(9, d, drift=True)
    for bits in (4, 2):
        q = codec.quantize_tile(x, bits)
        qmax = 2 ** bits - 1
        codes, s, z, y = q["codes"], q["s_hat"], q["z_hat"], q["y"]
        assert codes.min() >= 0 and codes.max() <= qmax
        deq = s[:, None] * codes + z[:, None]
        assert np.all(np.abs(y - deq) <= s[:, None] / 2 * (1 + 1e-12))
        assert np.all(z <= y.min(axis=1)) and np.all(z + qmax * s >= y.max(axis=1))
        prev = formats.E4M3_DECODE[q["s_code"].astype(int) - 1]
        assert np.all(z + qmax * prev < y.max(axis=1))
        back = (q["c_hat"][None, :] * q["y"]) @ hadamard.H_OF[d]
        assert np.abs(back - x).max() <= 1e-13 * np.abs(x).max()


@pytest.mark.parametrize("d", DIMS)
def test_zero_iterations_is_textbook_per_token_minmax(d):
    x = _tile(12, d)
    xt = hadamard.rotate(x)
    for bits in (4, 2):
        q = codec.quantize_tile(x, bits, iters=0)
        qmax = 2 ** bits - 1
        assert np.all(q["c_hat"] == 1.0)
        mn = xt.min(axis=1)
        expect_z = np.array([np.float16(m) if np.float16(m) <= m else
                             np.nextafter(np.float16(m), np.float16(-np.inf)) for m in mn], float)
        assert np.array_equal(q["z_hat"], expect_z)
        expect_codes = np.clip(np.rint((xt - expect_z[:, None]) / q["s_hat"][:, None]), 0, qmax)
        assert np.array_equal(q["codes"], expect_codes)


@pytest.mark.parametrize("d", DIMS)
def test_all_zero_tile(d):
    q = codec.quantize_tile(np.zeros((T, d)), 2)
    assert q["c_hat"].shape == (d,) and np.all(q["c_code"] == 0x38)
    assert np.all(q["s_hat"] == 0) and np.all(q["z_hat"] == 0) and np.all(q["codes"] == 0)


# ------------------------------------------------------------------ record layout


@pytest.mark.parametrize("d,vb,size", [(64, 2, 7040), (64, 4, 9088), (256, 2, 25856),
                                       (256, 4, 34048)])
def test_record_sizes_and_round_trip(d, vb, size):
    assert codec.tile_bytes(vb, d) == size
    assert codec.geometry_of_record(size) == (d, vb)
    kq = codec.quantize_tile(_tile(16, d), 4)
    vq = codec.quantize_tile(_tile(17, d), vb)
    rec = codec.pack_record(kq, vq)
    assert rec.shape == (size,)
    u = codec.unpack_record(rec)
    assert u["head_dim"] == d and u["v_bits"] == vb
    for name, q in (("k", kq), ("v", vq)):
        for key in ("codes", "c_hat", "s_hat", "z_hat"):
            assert np.array_equal(u[name][key], q[key])


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("vb", [2, 4])
def test_value_layout_is_a_bijection(d, vb):
    tt, jj = np.meshgrid(np.arange(T), np.arange(d), indexing="ij")
    pos = codec.v_code_position if vb == 2 else codec.v4_code_position
    byte, shift = pos(tt, jj, d)
    bitaddr = (8 * byte + shift).ravel()
    assert np.all(shift % vb == 0)
    assert len(np.unique(bitaddr)) == T * d
    assert bitaddr.min() == 0 and bitaddr.max() == 16 * d * vb * 8 - vb


def test_layout_hand_positions():
    # d = 64, 2-bit values: token 37 (kb 1, h 0, s 1, i 1), channel 51 (nb 3, n 3), e = 0:
    #   word 128 + 2 (16 + 3) + 0 = 166, bit 2*3 + 0 + 16 = 22 -> byte 666, shift 6;
    #   key token 3, channel 5 -> byte 3 * 32 + 2; z-hat^K token 7 at 6144 + 64 + 128 + 14;
    #   s-hat^V token 100 at 6592 + 64 + 100.
    # d = 256, 2-bit values: token 37, channel 211 (nb 13: half 1, field 5; n 3):
    #   word 512 + 8 (16 + 3) + 4 + 0 = 668, bit 10 + 16 = 26 -> byte 2675, shift 2;
    #   key byte 3 * 128 + 2; z-hat^K token 7 at 24576 + 256 + 128 + 14; s-hat^V token 100 at
    #   25216 + 256 + 100.
    # d = 256, 4-bit values: word 1024 + 256 * 3 + 4 * 19 + 0 = 1868, bit 4 + 16 = 20 ->
    #   byte 7474, shift 4.
    # A second value code 1 at token 38 (kb 1, h 0, s 1, i 2, e = 1), same channel:
    #   d = 64: word 128 + 38 + 0 = 166, bit 6 + 8 + 0 = 14 -> byte 665, shift 6;
    #   d = 256, 2-bit: word 512 + 152 + 4 + 1 = 669, bit 10 -> byte 2677, shift 2;
    #   d = 256, 4-bit: word 1024 + 768 + 76 + 1 = 1869, bit 4 -> byte 7476, shift 4.
    cases = [(64, 2, 4096 + 666, 2 << 6, 4096 + 665, 1 << 6, 98, 6350, 6756),
             (256, 2, 16384 + 2675, 2 << 2, 16384 + 2677, 1 << 2, 386, 24974, 25572),
             (256, 4, 16384 + 7474, 2 << 4, 16384 + 7476, 1 << 4, 386, 32768 + 398,
              33408 + 356)]
    for d, vb, vbyte, vval, vbyte2, vval2, kbyte, zoff, soff in cases:
        kq = dict(codes=np.zeros((T, d), int), c_code=np.zeros(d, np.uint8),
                  s_code=np.zeros(T, np.uint8), z_bits=np.zeros(T, np.uint16))
        vq = {k: v.copy() for k, v in kq.items()}
        vq["bits"] = vb
        kq["codes"][3, 5] = 0xB
        vq["codes"][37, 51 if d == 64 else 211] = 2
        vq["codes"][38, 51 if d == 64 else 211] = 1
        kq["z_bits"][7] = 0xABCD
        vq["s_code"][100] = 0x42
        rec = codec.pack_record(kq, vq)
        assert rec[kbyte] == 0xB0
        assert rec[vbyte] == vval and rec[vbyte2] == vval2
        assert rec[zoff] == 0xCD and rec[zoff + 1] == 0xAB
        assert rec[soff] == 0x42
        assert np.count_nonzero(rec) == 6


# ------------------------------------------------------------------ attention


def _cache(sp, tails, vb=2, seed=0):
    st = gen.prefill(sp, max_new_tokens=T)
    d = sp.head_dim
    pool = np.zeros((st["num_blocks"], sp.hkv, codec.tile_bytes(vb, d)), np.uint8)
    attention.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool)
    lens = st["seq_lens"].copy()
    stg_k = np.zeros((sp.batch, sp.hkv, T, d), np.float16)
    stg_v = np.zeros_like(stg_k)
    rng = np.random.default_rng(seed)
    for b, tail in enumerate(tails):
        stg_k[b, :, :tail] = rng.standard_normal((sp.hkv, tail, d)) * 3
        stg_v[b, :, :tail] = rng.standard_normal((sp.hkv, tail, d)) * 3
        lens[b] += tail
    return pool, st["block_table"], lens, stg_k, stg_v


@pytest.mark.parametrize("d", DIMS)
def test_folded_equals_plain_and_sdpa(d):
    sp = gen.spec("qwen3-4b", batch=2, ctx=256, hkv=2, hq=4, head_dim=d)
    pool, bt, lens, sk, sv = _cache(sp, tails=[0, 37])
    q = gen.query(sp, dense=True)
    sm = 1 / math.sqrt(d)
    a = attention.decode_attention(q, pool, bt, lens, sk, sv, sm)
    b = attention.decode_attention_folded(q, pool, bt, lens, sk, sv, sm)
    assert a.shape == (2, 4, d)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())
    for bb in range(sp.batch):
        for g in range(sp.hkv):
            kv = [codec.decode_record(pool[bt[bb, i], g]) for i in range(lens[bb] // T)]
            tail = lens[bb] % T
            kk = torch.from_numpy(np.concatenate([k for k, _ in kv]
                                                 + [sk[bb, g, :tail].astype(np.float64)]))
            vv = torch.from_numpy(np.concatenate([v for _, v in kv]
                                                 + [sv[bb, g, :tail].astype(np.float64)]))
            for h in range(g * 2, g * 2 + 2):
                qq = torch.from_numpy(q[bb, h].astype(np.float64))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, kk[None], vv[None], scale=sm)[0, 0].numpy()
                assert np.allclose(a[bb, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", DIMS)
def test_sign_flips_fold_through_attention(d):
    sp = gen.spec("qwen3-4b", batch=1, ctx=128, hkv=1, hq=2, head_dim=d)
    st = gen.prefill(sp, max_new_tokens=T)
    signs = hadamard.sign_vector(gen.rotation_sign_words(sp), d)
    pool = np.zeros((st["num_blocks"], 1, codec.tile_bytes(2, d)), np.uint8)
    attention.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool, signs=signs)
    z = np.zeros((1, 1, T, d), np.float16)
    q = gen.query(sp)
    a = attention.decode_attention(q, pool, st["block_table"], st["seq_lens"], z, z, 0.1,
                                   signs)
    b = attention.decode_attention_folded(q, pool, st["block_table"], st["seq_lens"], z, z, 0.1,
                                          signs)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())
    # the flips before the rotation are undone on the way back: the dequantised tile is close
    # to the input in the original space
    kh, _ = codec.decode_record(pool[st["dst_blocks"][0], 0], signs)
    k0 = st["k"][:T, 0].astype(np.float64)
    assert np.linalg.norm(kh - k0) / np.linalg.norm(k0) < 0.12
