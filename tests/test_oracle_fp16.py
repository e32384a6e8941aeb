"""Pins of the oracle's attention over an unquantised paged fp16 cache (the comparison path):
closed forms (zero query, equal keys, one dominant key, two tokens, one token, empty),
block-permutation invariance, and agreement with the packed-cache oracle when the fp16 tiles
hold exactly the dequantised packed tiles."""

import math

import numpy as np

from oracle import attention, codec
from workloads import gen

T, D = 128, 128


def _fp16_cache(sp, tails, seed=0):
    st = gen.prefill(sp, max_new_tokens=T)
    kt, vt = gen.tiles_by_block(st, sp.hkv)
    lens = st["seq_lens"].copy()
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    sv = np.zeros_like(sk)
    rng = np.random.default_rng(seed)
    for b, tail in enumerate(tails):
        sk[b, :, :tail] = rng.standard_normal((sp.hkv, tail, D)) * 2
        sv[b, :, :tail] = rng.standard_normal((sp.hkv, tail, D)) * 2
        lens[b] += tail
    return st, kt, vt, lens, sk, sv, gen.query(sp)


def test_zero_query_gives_mean_of_all_values():
    sp = gen.spec("qwen3-4b", batch=1, ctx=256, hkv=1, hq=1)
    st, kt, vt, lens, sk, sv, _ = _fp16_cache(sp, [11])
    q = np.zeros((1, 1, D), np.float16)
    out = attention.decode_attention_fp16(q, kt, vt, st["block_table"], lens, sk, sv, 0.3)
    rows = [vt[st["block_table"][0, i], 0].astype(np.float64) for i in range(2)]
    mean = np.concatenate(rows + [sv[0, 0, :11].astype(np.float64)]).mean(axis=0)
    assert np.allclose(out[0, 0], mean, rtol=1e-12, atol=1e-12)


def test_equal_keys_give_mean_whatever_the_query():
    kt = np.zeros((1, 1, T, D), np.float16)
    kt[0, 0] = np.linspace(-1, 1, D)            # every token the same key
    vt = (np.random.default_rng(1).standard_normal((1, 1, T, D))).astype(np.float16)
    q = np.random.default_rng(2).standard_normal((1, 2, D)).astype(np.float16)
    sk = np.zeros((1, 1, T, D), np.float16)
    out = attention.decode_attention_fp16(q, kt, vt, np.zeros((1, 1), np.int32),
                                          np.array([T]), sk, sk, 0.2)
    mean = vt[0, 0].astype(np.float64).mean(axis=0)
    assert np.allclose(out[0], mean[None, :], rtol=1e-12, atol=1e-12)


def test_dominant_key_returns_its_value():
    kt = np.zeros((2, 1, T, D), np.float16)
    vt = (np.random.default_rng(3).standard_normal((2, 1, T, D))).astype(np.float16)
    kt[1, 0, 77, 5] = 8.0                       # block 1, token 77: the only non-zero key
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, 5] = 60.0                           # score 480 * scale 1 vs 0 elsewhere
    sk = np.zeros((1, 1, T, D), np.float16)
    out = attention.decode_attention_fp16(q, kt, vt, np.array([[0, 1]], np.int32),
                                          np.array([2 * T]), sk, sk, 1.0)
    assert np.array_equal(out[0, 0], vt[1, 0, 77].astype(np.float64))


def test_two_tokens_logistic_weight():
    sk = np.zeros((1, 1, T, D), np.float16)
    sv = np.zeros_like(sk)
    sk[0, 0, 0, 0], sk[0, 0, 1, 0] = 1.0, -0.5
    sv[0, 0, 0] = 2.0
    sv[0, 0, 1] = -4.0
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, 0] = 1.5
    scale = 0.8
    out = attention.decode_attention_fp16(q, np.zeros((1, 1, T, D), np.float16),
                                          np.zeros((1, 1, T, D), np.float16),
                                          np.zeros((1, 1), np.int32), np.array([2]), sk, sv, scale)
    w1 = 1.0 / (1.0 + math.exp(scale * 1.5 * (-0.5 - 1.0)))   # weight of token 0
    expect = w1 * 2.0 + (1.0 - w1) * (-4.0)
    assert np.allclose(out[0, 0], expect, rtol=1e-13, atol=1e-13)


def test_single_token_and_empty():
    sk = np.zeros((2, 1, T, D), np.float16)
    sv = np.zeros_like(sk)
    sv[0, 0, 0] = np.arange(D) / 5
    q = np.ones((2, 1, D), np.float16)
    z = np.zeros((1, 1, T, D), np.float16)
    out = attention.decode_attention_fp16(q, z, z, np.zeros((2, 1), np.int32), np.array([1, 0]),
                                          sk, sv, 0.1)
    assert np.array_equal(out[0, 0], sv[0, 0, 0].astype(np.float64))
    assert np.all(out[1] == 0)


def test_block_permutation_invariance():
    sp = gen.spec("qwen3-4b", batch=2, ctx=384, hkv=2, hq=4)
    st, kt, vt, lens, sk, sv, q = _fp16_cache(sp, [5, 0])
    perm = np.random.default_rng(6).permutation(kt.shape[0])
    kt2, vt2 = np.empty_like(kt), np.empty_like(vt)
    kt2[perm], vt2[perm] = kt, vt
    bt2 = perm[st["block_table"]].astype(np.int32)
    a = attention.decode_attention_fp16(q, kt, vt, st["block_table"], lens, sk, sv, 0.09)
    b = attention.decode_attention_fp16(q, kt2, vt2, bt2, lens, sk, sv, 0.09)
    assert np.array_equal(a, b)


def test_agrees_with_packed_oracle_on_dequantised_tiles():
    sp = gen.spec("qwen3-4b", batch=2, ctx=256, hkv=1, hq=2)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = np.zeros((st["num_blocks"], sp.hkv, codec.TILE_BYTES), np.uint8)
    attention.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool)
    kt = np.zeros((st["num_blocks"], sp.hkv, T, D))
    vt = np.zeros_like(kt)
    for blk in st["dst_blocks"]:
        for h in range(sp.hkv):
            kt[blk, h], vt[blk, h] = codec.decode_record(pool[blk, h])
    lens = st["seq_lens"]
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    q = gen.query(sp)
    a = attention.decode_attention(q, pool, st["block_table"], lens, sk, sk, 0.088)
    b = attention.decode_attention_fp16(q, kt, vt, st["block_table"], lens, sk, sk, 0.088)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
