"""Parity of the optional sign flips before the rotation (reading R27) with the oracle, through
the C ABI: records of seeded tiles, decode over an oracle-written signed cache (one and
several query tokens), dequantisation, and the append path."""

import math

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from oracle import attention as oatt
from oracle import codec
from oracle.hadamard import sign_vector
from workloads import gen

from record_view import Budget, compare_half, parse
from test_gpu_parity import TOL, dev, gpu_quantize

pytestmark = pytest.mark.gpu
T = D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def _setup(name="qwen3-4b", **over):
    sp = gen.spec(name, **over)
    words = gen.rotation_sign_words(sp)
    return sp, words, sign_vector(words), kv.default_config(sp.hkv, rotation_signs=words)


def test_signed_records_match_oracle():
    sp, words, s, cfg = _setup(batch=2, ctx=256, hkv=2)
    st = gen.prefill(sp)
    pool = gpu_quantize(cfg, st["k"], st["v"], st["dst_blocks"], st["num_blocks"], sp.hkv)
    pool_h = pool.cpu().numpy()
    budget = Budget()
    for i, blk in enumerate(st["dst_blocks"]):
        for h in range(sp.hkv):
            rows = slice(T * i, T * i + T)
            rec = parse(pool_h[blk, h])
            compare_half(rec, codec.quantize_tile(st["k"][rows, h].astype(np.float64), 4,
                                                  signs=s), "k", 4, budget)
            compare_half(rec, codec.quantize_tile(st["v"][rows, h].astype(np.float64), 2,
                                                  signs=s), "v", 2, budget)
    budget.check()
    # the plain preset writes different records for the same tiles
    plain = gpu_quantize(kv.default_config(sp.hkv), st["k"], st["v"], st["dst_blocks"],
                         st["num_blocks"], sp.hkv)
    assert not torch.equal(plain, pool)


@pytest.mark.parametrize("nq", [1, 3])
def test_signed_decode_matches_oracle(nq):
    sp, words, s, cfg = _setup(batch=3, ctx=384, hkv=2, hq=8)
    st = gen.prefill(sp, max_new_tokens=T)
    pool = np.zeros((st["num_blocks"], sp.hkv, 13312), np.uint8)
    oatt.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool, signs=s)
    lens = (st["seq_lens"] + np.array([0, 5, 127])).astype(np.int32)
    rng = np.random.default_rng(4)
    sk = (rng.standard_normal((sp.batch, sp.hkv, T, D)) * 3).astype(np.float16)
    sv = (rng.standard_normal((sp.batch, sp.hkv, T, D)) * 3).astype(np.float16)
    q = gen.query_tokens(sp, nq)
    sm = 1 / math.sqrt(D)
    ws = torch.empty(max(kv.decode_multi_workspace_bytes(cfg, sp.batch, sp.hq, nq,
                                                         st["block_table"].shape[1]), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((sp.batch, nq, sp.hq, D), -7.0, dtype=torch.float32, device="cuda")
    kv.decode_attention_multi(cfg, dev(q), dev(pool), dev(st["block_table"]), dev(lens),
                              dev(sk), dev(sv), sm, out, ws)
    torch.cuda.synchronize()
    ref = oatt.decode_attention_multi(q, pool, st["block_table"], lens, sk, sv, sm, signs=s)
    assert np.abs(out.cpu().numpy() - ref).max() <= TOL


def test_signed_dequantize_matches_oracle():
    sp, words, s, cfg = _setup(batch=1, ctx=256, hkv=2)
    st = gen.prefill(sp)
    pool = np.zeros((st["num_blocks"], sp.hkv, 13312), np.uint8)
    oatt.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool, signs=s)
    ids = st["dst_blocks"]
    ko = torch.empty(len(ids) * T, sp.hkv, D, dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    kv.dequantize_tiles(cfg, dev(pool), dev(ids), ko, vo)
    torch.cuda.synchronize()
    ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
    for i, blk in enumerate(ids):
        for h in range(sp.hkv):
            rk, rv = codec.decode_record(pool[blk, h], signs=s)
            for got, ref in ((ko[T * i:T * i + T, h], rk), (vo[T * i:T * i + T, h], rv)):
                assert np.abs(got - ref).max() <= 4e-6 * (1 + np.abs(ref).max())


def test_signed_append_completes_tiles_like_the_oracle():
    sp, words, s, cfg = _setup("write-stream", batch=2, ctx=120, hkv=2, hq=4)
    st = gen.prefill(sp, max_new_tokens=16)
    bt = st["block_table"]
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    for b in range(sp.batch):
        sk[b, :, :120] = st["tail_k"][b].transpose(1, 0, 2)
    sv = np.zeros_like(sk)
    for b in range(sp.batch):
        sv[b, :, :120] = st["tail_v"][b].transpose(1, 0, 2)
    pool_g = torch.zeros(st["num_blocks"], sp.hkv, 13312, dtype=torch.uint8, device="cuda")
    skg, svg = dev(sk), dev(sv)
    pool_o = np.zeros((st["num_blocks"], sp.hkv, 13312), np.uint8)
    sko, svo = sk.copy(), sv.copy()
    for step in range(8):                       # positions 120..127: the tile completes
        kn, vn = gen.append_tokens(sp, step)
        pos = np.full(sp.batch, 120 + step, np.int32)
        kv.append_token(cfg, dev(kn), dev(vn), dev(pos), dev(bt), skg, svg, pool_g)
        oatt.append_token(kn, vn, pos, bt, sko, svo, pool_o, signs=s)
    torch.cuda.synchronize()
    got = pool_g.cpu().numpy()
    budget = Budget()
    for b in range(sp.batch):
        for h in range(sp.hkv):
            rec = parse(got[bt[b, 0], h])
            compare_half(rec, codec.quantize_tile(sko[b, h].astype(np.float64), 4, signs=s),
                         "k", 4, budget)
            compare_half(rec, codec.quantize_tile(svo[b, h].astype(np.float64), 2, signs=s),
                         "v", 2, budget)
    budget.check()
    assert np.array_equal(skg.cpu().numpy(), sko) and np.array_equal(svg.cpu().numpy(), svo)
