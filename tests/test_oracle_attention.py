"""Pins of the oracle's decode attention and cache-level operations: folded form equals the
plain form, brute force on tiny inputs, torch's SDPA on staging-only sequences, closed-form
special cases, block-permutation invariance, and append/quantise agreement."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, codec
from workloads import gen

T, D = 128, 128


def _cache(sp, tails=None, seed=0):
    """Oracle cache for a (small) workload spec: pool, block table, lens, staging, queries."""
    st = gen.prefill(sp, max_new_tokens=T)
    pool = np.zeros((st["num_blocks"], sp.hkv, codec.TILE_BYTES), np.uint8)
    attention.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool)
    lens = st["seq_lens"].copy()
    stg_k = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    stg_v = np.zeros_like(stg_k)
    rng = np.random.default_rng(seed)
    if tails is not None:
        for b, tail in enumerate(tails):
            stg_k[b, :, :tail] = rng.standard_normal((sp.hkv, tail, D)) * 3
            stg_v[b, :, :tail] = rng.standard_normal((sp.hkv, tail, D)) * 3
            lens[b] += tail
    q = gen.query(sp)
    return pool, st["block_table"], lens, stg_k, stg_v, q


@pytest.mark.parametrize("dense", [False, True])
def test_folded_equals_plain(dense):
    sp = gen.spec("qwen3-4b", batch=3, ctx=384, hkv=2, hq=8)
    pool, bt, lens, sk, sv, _ = _cache(sp, tails=[0, 5, 127])
    q = gen.query(sp, dense=dense)
    sm = 1 / math.sqrt(D)
    a = attention.decode_attention(q, pool, bt, lens, sk, sv, sm)
    b = attention.decode_attention_folded(q, pool, bt, lens, sk, sv, sm)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    for L in (1, 2, 3, 4):
        k = rng.standard_normal((L, D)).astype(np.float16)
        v = rng.standard_normal((L, D)).astype(np.float16)
        q = rng.standard_normal(D).astype(np.float16)
        sk = np.zeros((1, 1, T, D), np.float16)
        sv = np.zeros_like(sk)
        sk[0, 0, :L], sv[0, 0, :L] = k, v
        out = attention.decode_attention(q[None, None], None, np.zeros((1, 1), np.int32),
                                         np.array([L]), sk, sv, 0.125)[0, 0]
        s = [0.125 * sum(float(q[j]) * float(k[t, j]) for j in range(D)) for t in range(L)]
        w = [math.exp(x - max(s)) for x in s]
        ref = [sum(w[t] * float(v[t, j]) for t in range(L)) / sum(w) for j in range(D)]
        assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_staging_only_equals_torch_sdpa():
    rng = np.random.default_rng(4)
    B, hkv, G = 3, 2, 4
    lens = np.array([1, 77, 127])
    sk = (rng.standard_normal((B, hkv, T, D)) * 2).astype(np.float16)
    sv = (rng.standard_normal((B, hkv, T, D)) * 2).astype(np.float16)
    q = rng.standard_normal((B, hkv * G, D)).astype(np.float16)
    out = attention.decode_attention(q, None, np.zeros((B, 1), np.int32), lens, sk, sv,
                                     1 / math.sqrt(D))
    for b in range(B):
        L = lens[b]
        kk = torch.from_numpy(sk[b, :, :L].astype(np.float64)).repeat_interleave(G, 0)
        vv = torch.from_numpy(sv[b, :, :L].astype(np.float64)).repeat_interleave(G, 0)
        qq = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0].numpy()
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_packed_equals_sdpa_over_dequantised_tiles():
    sp = gen.spec("qwen3-4b", batch=2, ctx=256, hkv=2, hq=4)
    pool, bt, lens, sk, sv, q = _cache(sp)
    out = attention.decode_attention(q, pool, bt, lens, sk, sv, 0.1)
    for b in range(sp.batch):
        for g in range(sp.hkv):
            kv = [codec.decode_record(pool[bt[b, i], g]) for i in range(lens[b] // T)]
            kk = torch.from_numpy(np.concatenate([k for k, _ in kv]))
            vv = torch.from_numpy(np.concatenate([v for _, v in kv]))
            for h in range(g * 2, g * 2 + 2):
                qq = torch.from_numpy(q[b, h].astype(np.float64))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, kk[None], vv[None], scale=0.1)[0, 0].numpy()
                assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    sp = gen.spec("qwen3-4b", batch=1, ctx=256, hkv=1, hq=1)
    pool, bt, lens, sk, sv, _ = _cache(sp, tails=[9])
    q = np.zeros((1, 1, D), np.float16)
    out = attention.decode_attention(q, pool, bt, lens, sk, sv, 0.1)[0, 0]
    vs = [codec.decode_record(pool[bt[0, i], 0])[1] for i in range(2)]
    mean = np.concatenate(vs + [sv[0, 0, :9].astype(np.float64)]).mean(axis=0)
    assert np.allclose(out, mean, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value_and_empty_gives_zero():
    sk = np.zeros((2, 1, T, D), np.float16)
    sv = np.zeros_like(sk)
    sv[0, 0, 0] = np.arange(D) / 7
    q = np.ones((2, 1, D), np.float16)
    out = attention.decode_attention(q, None, np.zeros((2, 1), np.int32), np.array([1, 0]),
                                     sk, sv, 0.1)
    assert np.array_equal(out[0, 0], sv[0, 0, 0].astype(np.float64))
    assert np.all(out[1] == 0)


def test_block_permutation_invariance():
    sp = gen.spec("qwen3-4b", batch=2, ctx=384, hkv=2, hq=4)
    pool, bt, lens, sk, sv, q = _cache(sp, tails=[3, 0])
    perm = np.random.default_rng(5).permutation(pool.shape[0])
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    bt2 = perm[bt].astype(np.int32)
    a = attention.decode_attention(q, pool, bt, lens, sk, sv, 0.09)
    b = attention.decode_attention(q, pool2, bt2, lens, sk, sv, 0.09)
    assert np.array_equal(a, b)


def test_append_completes_tile_like_prefill():
    sp = gen.spec("write-stream", batch=2, ctx=128, hkv=2, hq=4)
    st = gen.prefill(sp, max_new_tokens=256)
    pool = np.zeros((st["num_blocks"], sp.hkv, codec.TILE_BYTES), np.uint8)
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    sv = np.zeros_like(sk)
    toks_k, toks_v = [], []
    for step in range(T):
        k, v = gen.append_tokens(sp, step)
        toks_k.append(k)
        toks_v.append(v)
        pos = np.array([128 + step, 128 + step])
        attention.append_token(k, v, pos, st["block_table"], sk, sv, pool)
    kk = np.stack(toks_k, 0)   # [128, B, Hkv, D]
    vv = np.stack(toks_v, 0)
    ref = np.zeros_like(pool)
    for b in range(sp.batch):
        attention.quantize_tiles(kk[:, b], vv[:, b], [st["block_table"][b, 1]], ref)
    for b in range(sp.batch):
        blk = st["block_table"][b, 1]
        assert np.array_equal(pool[blk], ref[blk])
    assert np.array_equal(sk[0].transpose(1, 0, 2), kk[:, 0])


def test_skipped_rows_untouched():
    sk = np.zeros((2, 1, T, D), np.float16)
    sv = np.zeros_like(sk)
    k = np.ones((2, 1, D), np.float16)
    pool = np.zeros((2, 1, codec.TILE_BYTES), np.uint8)
    attention.append_token(k, k, np.array([-1, 5]), np.array([[0], [1]]), sk, sv, pool)
    assert np.all(sk[0] == 0) and np.all(sk[1, 0, 5] == 1) and np.count_nonzero(sk) == D
