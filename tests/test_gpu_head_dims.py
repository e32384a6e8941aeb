"""Parity of the HIP library with the fp64 oracle at head dimensions 64 and 256 (reading R29):
quantiser records, append completion, one-token and several-token decode, dequantisation,
sign flips, and the degenerate rows, for both value widths.

The rules are those of the head-dimension-128 tests: records within the rounding-boundary
budget (record_view), staging bit-exact, decode outputs against the oracle's fp64 attention
over the same oracle-written cache within 2e-3, dequantised tiles within 4e-6 relative."""

import math
import sys

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from oracle import attention as oatt
from oracle import codec, hadamard
from workloads import gen

from record_view import Budget, compare_half, parse
from test_oracle_head_dims import _closed_form_tile

pytestmark = pytest.mark.gpu
T = 128
TOL = 2e-3
CASES = [(64, 2), (64, 4), (256, 2), (256, 4)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _spec(d, **over):
    base = dict(batch=2, ctx=384, hkv=2, hq=8, head_dim=d)
    base.update(over)
    return gen.spec("qwen3-4b", **base)


def gpu_pool(cfg, st, hkv):
    pool = torch.zeros(st["num_blocks"], hkv, kv.tile_bytes(cfg), dtype=torch.uint8,
                       device="cuda")
    if len(st["dst_blocks"]):
        kd, vd = dev(st["k"]), dev(st["v"])
        kv.quantize_tiles(cfg, kd.view(kd.shape[0], -1), vd.view(vd.shape[0], -1),
                          dev(st["dst_blocks"]), pool)
    torch.cuda.synchronize()
    return pool


def oracle_pool(st, hkv, d, vb, signs=None):
    pool = np.zeros((st["num_blocks"], hkv, codec.tile_bytes(vb, d)), np.uint8)
    oatt.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool, signs=signs)
    return pool


def staging(sp, tails, seed=0):
    d = sp.head_dim
    sk = np.zeros((sp.batch, sp.hkv, T, d), np.float16)
    sv = np.zeros_like(sk)
    rng = np.random.default_rng([seed, d])
    for b, n in enumerate(tails):
        sk[b, :, :n] = rng.standard_normal((sp.hkv, n, d)) * 2
        sv[b, :, :n] = rng.standard_normal((sp.hkv, n, d)) * 2
    return sk, sv


def gpu_decode(cfg, q, pool, bt, lens, sk, sv, sm, noalloc=False):
    b, hq, d = q.shape
    out = torch.full((b, hq, d), -7.0, dtype=torch.float32, device="cuda")
    pool_d = pool if isinstance(pool, torch.Tensor) else dev(pool)
    if noalloc:
        kv.decode_attention_noalloc(cfg, dev(q), pool_d, dev(bt), dev(lens), dev(sk), dev(sv),
                                    sm, out)
    else:
        ws = torch.empty(max(kv.decode_workspace_bytes(cfg, b, hq, bt.shape[1]), 256),
                         dtype=torch.uint8, device="cuda")
        kv.decode_attention(cfg, dev(q), pool_d, dev(bt), dev(lens), dev(sk), dev(sv), sm, out,
                            ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def compare_pool(pool_g, k, v, dst, hkv, vb, signs=None):
    budget = Budget()
    for i in range(len(dst)):
        for h in range(hkv):
            rows = slice(T * i, T * i + T)
            rec = parse(pool_g[dst[i], h])
            assert rec["head_dim"] == k.shape[2] and rec["v_bits"] == vb
            compare_half(rec, codec.quantize_tile(k[rows, h].astype(np.float64), 4, signs=signs),
                         "k", 4, budget)
            compare_half(rec, codec.quantize_tile(v[rows, h].astype(np.float64), vb,
                                                  signs=signs), "v", vb, budget)
    return budget


# ------------------------------------------------------------------ quantiser


@pytest.mark.parametrize("d,vb", CASES)
def test_quantize_matches_oracle(d, vb):
    _say(f"quantize d={d} vb={vb}")
    sp = _spec(d)
    st = gen.prefill(sp)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    pool = gpu_pool(cfg, st, sp.hkv)
    b = compare_pool(pool.cpu().numpy(), st["k"], st["v"], st["dst_blocks"], sp.hkv, vb)
    _say(f"  {vars(b)}")
    b.check()


@pytest.mark.parametrize("d,vb", CASES)
def test_quantize_special_tiles(d, vb):
    # closed-form tiles (worked by hand in the oracle pins), an all-zero tile, identical
    # tokens (the floor decides the columns) and a tile with one nonzero element
    _say(f"special tiles d={d} vb={vb}")
    tiles = [_closed_form_tile(d, 0)[0], _closed_form_tile(d, 1)[0], np.zeros((T, d))]
    row = np.random.default_rng(d).standard_normal(d) * 3
    tiles.append(np.repeat(row[None, :], T, axis=0))
    one = np.zeros((T, d))
    one[5, 9] = 3.0
    tiles.append(one)
    x = np.stack([t.astype(np.float16) for t in tiles])            # [n, T, d]
    n = len(tiles)
    k = np.ascontiguousarray(x.reshape(n * T, 1, d))
    v = np.ascontiguousarray(x[::-1].reshape(n * T, 1, d))
    st = dict(k=k, v=v, dst_blocks=np.arange(n, dtype=np.int32), num_blocks=n)
    cfg = kv.default_config(1, v_bits=vb, head_dim=d)
    pool = gpu_pool(cfg, st, 1).cpu().numpy()
    b = compare_pool(pool, k, v, st["dst_blocks"], 1, vb)
    assert b.exact(), vars(b)
    for i in range(2):                                             # the closed forms exactly
        assert np.array_equal(pool[i, 0], codec.encode_record(k[T * i:T * i + T, 0],
                                                              v[T * i:T * i + T, 0], v_bits=vb))


@pytest.mark.parametrize("d", [64, 256])
def test_quantize_with_sign_flips(d):
    _say(f"quantize signs d={d}")
    sp = _spec(d, batch=1, ctx=256)
    st = gen.prefill(sp)
    words = gen.rotation_sign_words(sp)
    assert len(words) == d // 32
    signs = hadamard.sign_vector(words, d)
    cfg = kv.default_config(sp.hkv, head_dim=d, rotation_signs=words)
    pool = gpu_pool(cfg, st, sp.hkv)
    b = compare_pool(pool.cpu().numpy(), st["k"], st["v"], st["dst_blocks"], sp.hkv, 2, signs)
    b.check()


# ------------------------------------------------------------------ append


@pytest.mark.parametrize("d,vb", [(64, 2), (256, 4)])
def test_append_matches_oracle(d, vb):
    _say(f"append d={d} vb={vb}")
    sp = _spec(d, batch=3, ctx=128)
    st = gen.prefill(sp, max_new_tokens=T)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    pool_g = gpu_pool(cfg, st, sp.hkv)
    pool_o = np.zeros((st["num_blocks"], sp.hkv, codec.tile_bytes(vb, d)), np.uint8)
    sk_o = np.zeros((sp.batch, sp.hkv, T, d), np.float16)
    sv_o = np.zeros_like(sk_o)
    sk_g, sv_g = dev(sk_o), dev(sv_o)
    bt = st["block_table"]
    # sequence 0 fills its second tile completely, 1 stops short, 2 is skipped
    for step in range(T):
        kn, vn = gen.append_tokens(sp, step)
        pos = np.array([T + step, T + step if step < 70 else -1, -1], np.int32)
        oatt.append_token(kn, vn, pos, bt, sk_o, sv_o, pool_o)
        kv.append_token(cfg, dev(kn), dev(vn), dev(pos), dev(bt), sk_g, sv_g, pool_g)
    torch.cuda.synchronize()
    assert np.array_equal(sk_g.cpu().numpy(), sk_o) and np.array_equal(sv_g.cpu().numpy(), sv_o)
    blk = bt[0, 1]
    rec = parse(pool_g.cpu().numpy()[blk, 0])
    ko = np.ascontiguousarray(sk_o[0, 0]).astype(np.float64)
    vo = np.ascontiguousarray(sv_o[0, 0]).astype(np.float64)
    b = Budget()
    compare_half(rec, codec.quantize_tile(ko, 4), "k", 4, b)
    compare_half(rec, codec.quantize_tile(vo, vb), "v", vb, b)
    b.check()
    assert not pool_g.cpu().numpy()[bt[1, 1]].any()               # never completed


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("d,vb", CASES)
@pytest.mark.parametrize("hq", [8, 16])
def test_decode_matches_oracle(d, vb, hq):
    _say(f"decode d={d} vb={vb} hq={hq}")
    sp = _spec(d, batch=3, ctx=640, hq=hq)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = oracle_pool(st, sp.hkv, d, vb)
    sk, sv = staging(sp, [0, 37, 127])
    lens = st["seq_lens"] + np.array([0, 37, 127], np.int32)
    q = gen.query(sp, dense=True)
    sm = 1 / math.sqrt(d)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    out = gpu_decode(cfg, q, pool, st["block_table"], lens, sk, sv, sm)
    ref = oatt.decode_attention(q, pool, st["block_table"], lens, sk, sv, sm)
    err = np.abs(out - ref).max()
    _say(f"  max |err| {err:.2e} (max |ref| {np.abs(ref).max():.2f})")
    assert err <= TOL


@pytest.mark.parametrize("d", [64, 256])
def test_decode_many_splits_and_ragged_lengths(d):
    # 40 tiles per sequence (several splits each), lengths 0 .. 40 tiles with ragged tails
    _say(f"decode splits d={d}")
    sp = _spec(d, batch=4, ctx=40 * T, hq=8)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = oracle_pool(st, sp.hkv, d, 2)
    lens = np.array([0, 1, 17 * T + 5, 40 * T + 99], np.int32)
    sk, sv = staging(sp, [0, 1, 5, 99], seed=3)
    q = gen.query(sp, dense=True)
    cfg = kv.default_config(sp.hkv, head_dim=d)
    assert kv.decode_workspace_bytes(cfg, 4, 8, st["block_table"].shape[1]) > 0
    out = gpu_decode(cfg, q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(d))
    ref = oatt.decode_attention(q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(d))
    assert np.all(out[0] == 0.0)
    err = np.abs(out - ref).max()
    _say(f"  max |err| {err:.2e}")
    assert err <= TOL
    # the allocation-free entry point gives the same result
    out2 = gpu_decode(cfg, q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(d),
                      noalloc=True)
    assert np.abs(out2 - ref).max() <= TOL


@pytest.mark.parametrize("d", [64, 256])
def test_decode_invalid_rows(d):
    sp = _spec(d, batch=3, ctx=256, hq=8)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = oracle_pool(st, sp.hkv, d, 2)
    bt = st["block_table"].copy()
    bt[1, 0] = st["num_blocks"] + 5                   # a block id outside the pool
    lens = st["seq_lens"].copy()
    lens[2] = -1                                      # a negative length
    sk, sv = staging(sp, [0, 0, 0])
    q = gen.query(sp)
    cfg = kv.default_config(sp.hkv, head_dim=d)
    out = gpu_decode(cfg, q, pool, bt, lens, sk, sv, 0.1)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    ref = oatt.decode_attention(q[:1], pool, bt[:1], lens[:1], sk[:1], sv[:1], 0.1)
    assert np.abs(out[0] - ref[0]).max() <= TOL


@pytest.mark.parametrize("d", [64, 256])
def test_decode_with_sign_flips(d):
    sp = _spec(d, batch=2, ctx=256, hq=8)
    st = gen.prefill(sp, max_new_tokens=T)
    words = gen.rotation_sign_words(sp)
    signs = hadamard.sign_vector(words, d)
    pool = oracle_pool(st, sp.hkv, d, 2, signs)
    sk, sv = staging(sp, [3, 64])
    lens = st["seq_lens"] + np.array([3, 64], np.int32)
    q = gen.query(sp, dense=True)
    cfg = kv.default_config(sp.hkv, head_dim=d, rotation_signs=words)
    out = gpu_decode(cfg, q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(d))
    ref = oatt.decode_attention(q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(d),
                                signs)
    assert np.abs(out - ref).max() <= TOL


@pytest.mark.parametrize("d,vb", [(64, 2), (256, 4)])
@pytest.mark.parametrize("nq", [2, 5])
def test_multi_token_decode(d, vb, nq):
    _say(f"multi d={d} vb={vb} nq={nq}")
    sp = _spec(d, batch=2, ctx=384, hq=8)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = oracle_pool(st, sp.hkv, d, vb)
    sk, sv = staging(sp, [2, 90])
    lens = st["seq_lens"] + np.array([2, 90], np.int32)
    q = gen.query_tokens(sp, nq, dense=True)
    sm = 1 / math.sqrt(d)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    ws = torch.empty(max(kv.decode_multi_workspace_bytes(cfg, 2, 8, nq, st["block_table"].shape[1]),
                         256), dtype=torch.uint8, device="cuda")
    out = torch.full((2, nq, 8, d), -7.0, dtype=torch.float32, device="cuda")
    kv.decode_attention_multi(cfg, dev(q), dev(pool), dev(st["block_table"]), dev(lens), dev(sk),
                              dev(sv), sm, out, ws)
    torch.cuda.synchronize()
    ref = oatt.decode_attention_multi(q, pool, st["block_table"], lens, sk, sv, sm)
    assert np.abs(out.cpu().numpy() - ref).max() <= TOL


@pytest.mark.parametrize("d,vb", [(64, 2), (256, 4)])
@pytest.mark.parametrize("nq", [2, 5])
def test_multi_token_decode_tile_list(d, vb, nq):
    """The same several-token decodes on a wide block table: the tile kernel's list schedule,
    one unit per (sequence, KV head, head group of 8), so more than 8 virtual heads per KV head
    make several units."""
    from test_gpu_parity import widen
    _say(f"multi tile list d={d} vb={vb} nq={nq}")
    sp = _spec(d, batch=2, ctx=384, hq=8)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = oracle_pool(st, sp.hkv, d, vb)
    sk, sv = staging(sp, [2, 90])
    lens = st["seq_lens"] + np.array([2, 90], np.int32)
    q = gen.query_tokens(sp, nq, dense=True)
    sm = 1 / math.sqrt(d)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    bt = widen(st["block_table"], sp.hkv)
    ws = torch.empty(max(kv.decode_multi_workspace_bytes(cfg, 2, 8, nq, bt.shape[1]), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((2, nq, 8, d), -7.0, dtype=torch.float32, device="cuda")
    kv.decode_attention_multi(cfg, dev(q), dev(pool), dev(bt), dev(lens), dev(sk), dev(sv), sm,
                              out, ws)
    torch.cuda.synchronize()
    ref = oatt.decode_attention_multi(q, pool, st["block_table"], lens, sk, sv, sm)
    assert np.abs(out.cpu().numpy() - ref).max() <= TOL


# ------------------------------------------------------------------ dequantisation


@pytest.mark.parametrize("d,vb", CASES)
def test_dequantize_matches_oracle(d, vb):
    sp = _spec(d, batch=1, ctx=256)
    st = gen.prefill(sp)
    pool = oracle_pool(st, sp.hkv, d, vb)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    ids = list(st["dst_blocks"][::-1]) + [st["num_blocks"] + 3]   # last: outside the pool
    n = len(ids)
    ko = torch.full((n * T, sp.hkv, d), -5.0, dtype=torch.float32, device="cuda")
    vo = torch.full_like(ko, -5.0)
    kv.dequantize_tiles(cfg, dev(pool), dev(np.asarray(ids, np.int32)), ko, vo)
    torch.cuda.synchronize()
    ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
    worst = 0.0
    for i, blk in enumerate(ids[:-1]):
        for h in range(sp.hkv):
            rk, rv = codec.decode_record(pool[blk, h])
            for got, ref in ((ko[T * i:T * i + T, h], rk), (vo[T * i:T * i + T, h], rv)):
                worst = max(worst, np.abs(got - ref).max() / (1.0 + np.abs(ref).max()))
    assert worst <= 4e-6, worst
    assert np.all(np.isnan(ko[-T:])) and np.all(np.isnan(vo[-T:]))
