"""Pins of the oracle's second preset, kvarn_k4v4_g128 (4-bit values; reading R28).

The value codes use the same per-token grid construction as every other bit width (stage 3 of
[GR] "The four-stage pipeline"), so the pins are: the grid relation between 2-bit and 4-bit
scales of one tile (step ratio exactly 5 before FP8 rounding up), the rounding bound, the
record layout (a bijection onto its section, hand-computed positions, size), independence of
the key half from the value preset, and the folded attention equal to the plain one over the
dequantised tiles."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, codec, formats
from workloads import gen

T, D = 128, 128


def _tile(seed, drift=True):
    rng = np.random.default_rng(seed)
    mult = np.exp(rng.standard_normal(D))
    mult[rng.choice(D, 3, replace=False)] *= 15
    x = rng.standard_normal((T, D)) * mult
    if drift:
        x *= np.exp(0.5 * rng.standard_normal((T, 1)))
    return x.astype(np.float16).astype(np.float64)


def test_layout_sizes():
    assert codec.tile_bytes(2) == 13312 and codec.tile_bytes(4) == 17408
    lay = codec.layout(4)
    assert lay["k_meta"] == 16384 and lay["v_meta"] == 16896
    assert codec.v_bits_of_record(13312) == 2 and codec.v_bits_of_record(17408) == 4
    with pytest.raises(ValueError):
        codec.layout(3)
    with pytest.raises(ValueError):
        codec.v_bits_of_record(13313)


def test_v4_layout_is_a_bijection_onto_the_section():
    tt, jj = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
    byte, shift = codec.v4_code_position(tt, jj)
    bitaddr = (8 * byte + shift).ravel()
    assert np.all(shift % 4 == 0)
    assert len(np.unique(bitaddr)) == T * D and bitaddr.min() == 0
    assert bitaddr.max() == 8 * 8192 - 4


def test_v4_layout_hand_positions():
    kq = dict(codes=np.zeros((T, D), int), c_code=np.zeros(D, np.uint8),
              s_code=np.zeros(T, np.uint8), z_bits=np.zeros(T, np.uint16), bits=4)
    vq = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in kq.items()}
    # token 37: kb 1, h 0, s 1, i 1; channel 83: nb 5 (half 1, field 1), n 3
    # word 512 + 256 + 4 * (16 + 3) + 0 = 844, bit 4 * 1 + 16 = 20 -> byte 3378, shift 4
    vq["codes"][37, 83] = 0xA
    # token 127: kb 3, h 1, s 3, i 3; channel 0: nb 0, n 0
    # word 1536 + 0 + 4 * 48 + 3 = 1731, bit 16 -> byte 6926, shift 0
    vq["codes"][127, 0] = 0x7
    kq["z_bits"][7] = 0xABCD
    vq["s_code"][100] = 0x42
    vq["c_code"][5] = 0x11
    rec = codec.pack_record(kq, vq)
    assert rec.shape == (17408,)
    assert rec[8192 + 3378] == 0xA << 4
    assert rec[8192 + 6926] == 0x7
    assert rec[16384 + 256 + 14] == 0xCD and rec[16384 + 256 + 15] == 0xAB
    assert rec[16896 + 128 + 100] == 0x42
    assert rec[16896 + 5] == 0x11
    assert np.count_nonzero(rec) == 6


def test_record_round_trip():
    kq = codec.quantize_tile(_tile(20), 4)
    vq = codec.quantize_tile(_tile(21), 4)
    rec = codec.pack_record(kq, vq)
    assert rec.shape == (17408,)
    u = codec.unpack_record(rec)
    assert u["v_bits"] == 4
    for name, q in (("k", kq), ("v", vq)):
        assert np.array_equal(u[name]["codes"], q["codes"])
        assert np.array_equal(u[name]["c_code"], q["c_code"])
        assert np.array_equal(u[name]["s_code"], q["s_code"])
        assert np.array_equal(u[name]["z_bits"], q["z_bits"])
    assert u["v"]["codes"].max() > 3          # really four bits wide


@pytest.mark.parametrize("seed", [22, 23])
def test_value_grid_relation_between_presets(seed):
    """Same tile, same c-hat and z-hat: the unrounded step of the 4-bit grid is exactly 1/5 of
    the 2-bit one ((max - z) / 15 vs / 3), and each s-hat is the smallest E4M3 value at or
    above its step."""
    x = _tile(seed)
    q2 = codec.quantize_tile(x, 2)
    q4 = codec.quantize_tile(x, 4)
    assert np.array_equal(q2["c_hat"], q4["c_hat"]) and np.array_equal(q2["z_hat"], q4["z_hat"])
    assert np.allclose(q2["step"], 5 * q4["step"], rtol=1e-15, atol=0)
    for q in (q2, q4):
        assert np.all(q["s_hat"] >= q["step"])
        prev = formats.E4M3_DECODE[q["s_code"].astype(int) - 1]
        assert np.all(prev < q["step"])
    # rounding bound on the rotated, channel-equalised values
    y = q4["y"]
    deq = q4["s_hat"][:, None] * q4["codes"] + q4["z_hat"][:, None]
    assert np.all(np.abs(y - deq) <= q4["s_hat"][:, None] / 2 * (1 + 1e-12))
    assert q4["codes"].min() == 0 and q4["codes"].max() == 15
    # and the 4-bit reconstruction is the closer one
    e2 = np.linalg.norm(codec.dequantize(q2["c_hat"], q2["s_hat"], q2["z_hat"], q2["codes"]) - x)
    e4 = np.linalg.norm(codec.dequantize(q4["c_hat"], q4["s_hat"], q4["z_hat"], q4["codes"]) - x)
    assert e4 < 0.3 * e2


def test_key_half_does_not_depend_on_the_value_preset():
    k, v = _tile(24), _tile(25)
    r2 = codec.encode_record(k, v, v_bits=2)
    r4 = codec.encode_record(k, v, v_bits=4)
    assert np.array_equal(r2[:8192], r4[:8192])                 # key codes
    assert np.array_equal(r2[12288:12800], r4[16384:16896])     # key metadata
    # value c-hat and z-hat are those of the same normalisation and token minima; only the
    # step, s-hat, depends on the bit width
    assert np.array_equal(r2[12800:12928], r4[16896:17024])
    assert np.array_equal(r2[13056:], r4[17152:])
    with pytest.raises(ValueError):
        codec.encode_record(k, v, v_bits=8)


def _cache(sp, v_bits):
    st = gen.prefill(sp, max_new_tokens=T)
    pool = np.zeros((st["num_blocks"], sp.hkv, codec.tile_bytes(v_bits)), np.uint8)
    attention.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool)
    stg_k = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    stg_v = np.zeros_like(stg_k)
    rng = np.random.default_rng(5)
    lens = st["seq_lens"].copy()
    for b, tail in enumerate([3, 100][:sp.batch]):
        stg_k[b, :, :tail] = rng.standard_normal((sp.hkv, tail, D)) * 3
        stg_v[b, :, :tail] = rng.standard_normal((sp.hkv, tail, D)) * 3
        lens[b] += tail
    return st, pool, lens, stg_k, stg_v


def test_attention_over_k4v4_cache():
    sp = gen.spec("qwen3-4b", batch=2, ctx=256, hkv=2, hq=4)
    st, pool, lens, sk, sv = _cache(sp, 4)
    q = gen.query(sp)
    sm = 1 / math.sqrt(D)
    plain = attention.decode_attention(q, pool, st["block_table"], lens, sk, sv, sm)
    folded = attention.decode_attention_folded(q, pool, st["block_table"], lens, sk, sv, sm)
    assert np.abs(plain - folded).max() <= 1e-12 * max(1.0, np.abs(plain).max())
    # plain form = SDPA over the dequantised tiles plus the staging tokens
    bt = st["block_table"]
    for b in range(sp.batch):
        for g in range(sp.hkv):
            kv = [codec.decode_record(pool[bt[b, i], g]) for i in range(lens[b] // T)]
            tail = lens[b] % T
            kk = torch.from_numpy(np.concatenate([k for k, _ in kv]
                                                 + [sk[b, g, :tail].astype(np.float64)]))
            vv = torch.from_numpy(np.concatenate([v for _, v in kv]
                                                 + [sv[b, g, :tail].astype(np.float64)]))
            for h in range(g * 2, g * 2 + 2):
                qq = torch.from_numpy(q[b, h].astype(np.float64))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, kk[None], vv[None], scale=sm)[0, 0].numpy()
                assert np.allclose(plain[b, h], ref, rtol=1e-12, atol=1e-12)


def test_k4v4_attention_closer_to_fp16_than_k4v2():
    sp = gen.spec("qwen3-4b", batch=2, ctx=256, hkv=2, hq=4)
    q = gen.query(sp, dense=True)
    sm = 1 / math.sqrt(D)
    outs = {}
    for vb in (2, 4):
        st, pool, lens, sk, sv = _cache(sp, vb)
        outs[vb] = attention.decode_attention(q, pool, st["block_table"], lens, sk, sv, sm)
    # exact attention over the unquantised fp16 tiles
    st, _, lens, sk, sv = _cache(sp, 2)
    kt, vt = gen.tiles_by_block(st, sp.hkv)
    ref = attention.decode_attention_fp16(q, kt, vt, st["block_table"], lens, sk, sv, sm)
    # the keys are 4-bit in both presets, so part of the error stays
    e2 = np.sqrt(np.mean((outs[2] - ref) ** 2))
    e4 = np.sqrt(np.mean((outs[4] - ref) ** 2))
    assert e4 < 0.75 * e2, (e4, e2)
