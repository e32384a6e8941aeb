"""Pins of oracle.attention.decode_attention_multi (several query tokens per sequence, causal
over the last Q positions; reading R25). Each pin ties it to something other than itself: the
one-token oracle (already pinned by its own tests) on the cases where the two must agree, the
causal structure, and a closed form."""

import numpy as np

from oracle import attention as oatt
from oracle import codec

T, D = codec.T, codec.D


def _case(lens, hkv=2, hq=4, nq=3, seed=0):
    """Random keys/values quantised into one block per (sequence, tile), random staging."""
    max_tiles = max(1, max(l // T for l in lens))
    bt = np.zeros((len(lens), max_tiles), np.int32)
    pool = np.zeros((max(1, len(lens) * max_tiles), hkv, 13312), np.uint8)
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((len(lens) * max_tiles * T, hkv, D)) * 2).astype(np.float16)
    v = (rng.standard_normal((len(lens) * max_tiles * T, hkv, D)) * 2).astype(np.float16)
    ids = np.arange(len(lens) * max_tiles, dtype=np.int32)
    oatt.quantize_tiles(k[: len(ids) * T], v[: len(ids) * T], ids, pool)
    bt[:] = ids.reshape(len(lens), max_tiles)
    sk = (rng.standard_normal((len(lens), hkv, T, D)) * 2).astype(np.float16)
    sv = (rng.standard_normal((len(lens), hkv, T, D)) * 2).astype(np.float16)
    q = rng.standard_normal((len(lens), nq, hq, D)).astype(np.float16)
    return q, pool, bt, np.array(lens, np.int32), sk, sv


def test_one_query_token_is_the_one_token_decode():
    q, pool, bt, lens, sk, sv = _case([5, 130, 256], nq=1)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.1)
    b = oatt.decode_attention(q[:, 0], pool, bt, lens, sk, sv, 0.1)
    assert np.array_equal(a[:, 0], b)


def test_last_query_token_sees_the_whole_sequence():
    q, pool, bt, lens, sk, sv = _case([7, 129, 250], nq=4)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.1)
    b = oatt.decode_attention(q[:, -1], pool, bt, lens, sk, sv, 0.1)
    assert np.array_equal(a[:, -1], b)


def test_query_token_equals_decode_of_the_shorter_sequence():
    # all Q tokens in staging (L mod 128 >= Q): query token i is the one-token decode of a
    # sequence of L - Q + i + 1 tokens over the same blocks and staging tile
    q, pool, bt, lens, sk, sv = _case([10, 140, 200], nq=5)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.1)
    for i in range(5):
        b = oatt.decode_attention(q[:, i], pool, bt, lens - 5 + i + 1, sk, sv, 0.1)
        assert np.allclose(a[:, i], b, rtol=0, atol=1e-12)


def test_causality():
    # changing the staging token at position p changes exactly the queries that see it
    q, pool, bt, lens, sk, sv = _case([140], nq=4)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.1)
    sk2, sv2 = sk.copy(), sv.copy()
    p = 140 - 2                                      # seen by query tokens 2 and 3 only
    sk2[0, :, p - T] += np.float16(1.5)
    sv2[0, :, p - T] -= np.float16(3.0)
    b = oatt.decode_attention_multi(q, pool, bt, lens, sk2, sv2, 0.1)
    assert np.array_equal(a[:, :2], b[:, :2])
    assert not np.allclose(a[:, 2:], b[:, 2:])


def test_causal_mask_reaches_into_the_last_packed_tile():
    # L = 129, Q = 4: positions 125..128; tokens 126 and 127 sit in packed tile 0 and must be
    # hidden from query token 0, which then equals attention over tokens 0..125 only
    q, pool, bt, lens, sk, sv = _case([129], nq=4)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.1)
    kh, vh = codec.decode_record(pool[bt[0, 0], 0])
    ref = oatt.softmax_attend(np.asarray(q[0, 0, 0], np.float64), kh[:126], vh[:126], 0.1)
    assert np.allclose(a[0, 0, 0], ref, rtol=0, atol=1e-12)


def test_too_short_sequence_gives_zeros_for_the_early_tokens():
    q, pool, bt, lens, sk, sv = _case([2], nq=4)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.1)
    assert np.all(a[0, :2] == 0) and np.all(np.abs(a[0, 2:]).sum(axis=-1) > 0)


def test_two_tokens_closed_form():
    # L = 2 (staging only), Q = 2: token 0 sees only itself (output = v0 exactly); token 1 mixes
    # v0 and v1 with the logistic weight of its score difference
    q, pool, bt, lens, sk, sv = _case([2], hkv=1, hq=1, nq=2)
    a = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, 0.25)
    k0, k1 = sk[0, 0, 0].astype(np.float64), sk[0, 0, 1].astype(np.float64)
    v0, v1 = sv[0, 0, 0].astype(np.float64), sv[0, 0, 1].astype(np.float64)
    assert np.allclose(a[0, 0, 0], v0, rtol=0, atol=1e-12)
    q1 = q[0, 1, 0].astype(np.float64)
    w1 = 1.0 / (1.0 + np.exp(0.25 * (q1 @ k0 - q1 @ k1)))
    assert np.allclose(a[0, 1, 0], (1 - w1) * v0 + w1 * v1, rtol=0, atol=1e-12)
