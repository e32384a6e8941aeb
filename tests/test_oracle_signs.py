"""Pins of the optional sign flips before the rotation (reading R27): the sign words' bit
order, orthonormality of the signed rotation, its equivalence with flipping the input's signs,
the per-row rounding bound of the round trip, and the folded decode equal to the plain one."""

import math

import numpy as np
import pytest

from oracle import attention, codec
from oracle.hadamard import H128, rotate, sign_vector
from workloads import gen

T, D = 128, 128


def test_sign_words_bit_order():
    assert np.all(sign_vector([0, 0, 0, 0]) == 1.0)
    s = sign_vector([1, 0, 0, 0x80000000])
    assert s[0] == -1 and s[127] == -1 and np.sum(s == -1) == 2
    s = sign_vector([0, 1 << 5, 0, 0])
    assert s[37] == -1 and np.sum(s == -1) == 1


def test_signed_rotation_is_orthonormal():
    s = sign_vector(gen.rotation_sign_words(gen.spec("tiny")))
    r = rotate(np.eye(D), s)                       # rows: the signed rotation of each basis vector
    assert np.abs(r @ r.T - np.eye(D)).max() < 1e-14
    assert not np.allclose(r, H128)
    x = np.random.default_rng(1).standard_normal((4, D))
    assert np.allclose(np.linalg.norm(rotate(x, s), axis=1), np.linalg.norm(x, axis=1),
                       rtol=1e-14)


def test_signs_equal_flipped_input():
    sp = gen.spec("qwen3-4b", batch=1, ctx=128, hkv=1)
    st = gen.prefill(sp)
    s = sign_vector(gen.rotation_sign_words(sp))
    x = st["k"][:, 0].astype(np.float64)
    a = codec.quantize_tile(x, 4, signs=s)
    b = codec.quantize_tile(x * s, 4)              # exact: fp16 values times +-1
    for key in ("codes", "c_code", "s_code", "z_bits"):
        assert np.array_equal(a[key], b[key])
    c = codec.quantize_tile(x, 4)
    assert not np.array_equal(a["codes"], c["codes"])


def test_signed_round_trip_bound():
    sp = gen.spec("qwen3-4b", batch=1, ctx=128, hkv=1)
    st = gen.prefill(sp)
    s = sign_vector(gen.rotation_sign_words(sp))
    k, v = st["k"][:, 0], st["v"][:, 0]
    rec = codec.encode_record(k, v, signs=s)
    u = codec.unpack_record(rec)
    for x, xh, half in zip((k, v), codec.decode_record(rec, signs=s), ("k", "v")):
        bound = np.sqrt(np.sum((u[half]["c_hat"][None, :] * u[half]["s_hat"][:, None] / 2) ** 2,
                               axis=1))
        err = np.linalg.norm(x.astype(np.float64) - xh, axis=1)
        assert np.all(err <= bound * (1 + 1e-9))
    # without the signs the same record decodes to something else
    assert not np.allclose(codec.decode_record(rec)[0], codec.decode_record(rec, signs=s)[0])


@pytest.mark.parametrize("dense", [False, True])
def test_signed_folded_equals_plain(dense):
    sp = gen.spec("qwen3-4b", batch=2, ctx=256, hkv=2, hq=4)
    s = sign_vector(gen.rotation_sign_words(sp))
    st = gen.prefill(sp, max_new_tokens=T)
    pool = np.zeros((st["num_blocks"], sp.hkv, codec.TILE_BYTES), np.uint8)
    attention.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool, signs=s)
    lens = st["seq_lens"] + np.array([5, 0], np.int32)
    rng = np.random.default_rng(2)
    sk = (rng.standard_normal((sp.batch, sp.hkv, T, D)) * 3).astype(np.float16)
    sv = (rng.standard_normal((sp.batch, sp.hkv, T, D)) * 3).astype(np.float16)
    q = gen.query(sp, dense=dense)
    sm = 1 / math.sqrt(D)
    a = attention.decode_attention(q, pool, st["block_table"], lens, sk, sv, sm, signs=s)
    b = attention.decode_attention_folded(q, pool, st["block_table"], lens, sk, sv, sm, signs=s)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())
