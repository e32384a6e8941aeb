"""Parity of the library's unquantised fp16-cache decode (the comparison path) with the fp64
oracle's attention over the same fp16 tiles: max-abs <= 2e-3 on fp32 outputs, as for the
packed decode. The library writes its fp16 pool from the workload's prefill tiles with its own
kernel; the oracle reads the same tiles as plain arrays (workloads.tiles_by_block)."""

import sys

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from oracle import attention as oatt
from workloads import gen

pytestmark = pytest.mark.gpu
T = D = 128
TOL = 2e-3


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


def _case(sp, tails, seed=0):
    st = gen.prefill(sp, max_new_tokens=T)
    kt, vt = gen.tiles_by_block(st, sp.hkv)
    lens = st["seq_lens"].copy()
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    sv = np.zeros_like(sk)
    rng = np.random.default_rng(seed)
    for b, tail in enumerate(tails):
        sk[b, :, :tail] = (rng.standard_normal((sp.hkv, tail, D)) * 3).astype(np.float16)
        sv[b, :, :tail] = (rng.standard_normal((sp.hkv, tail, D)) * 3).astype(np.float16)
        lens[b] += tail
    return st, kt, vt, lens.astype(np.int32), sk, sv, gen.query(sp)


def _gpu_pool(cfg, st, hkv):
    pool = torch.zeros(st["num_blocks"], hkv, kv.FP16_RECORD_BYTES, dtype=torch.uint8,
                       device="cuda")
    if len(st["dst_blocks"]):
        kd, vd = dev(st["k"]), dev(st["v"])
        kv.fp16_write_tiles(cfg, kd.view(kd.shape[0], -1), vd.view(vd.shape[0], -1),
                            dev(st["dst_blocks"]), pool)
    torch.cuda.synchronize()
    return pool


def _gpu_decode(cfg, q, pool, bt, lens, sk, sv, sm):
    b, hq, _ = q.shape
    ws = torch.empty(max(kv.decode_workspace_bytes(cfg, b, hq, bt.shape[1]), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((b, hq, D), -7.0, dtype=torch.float32, device="cuda")
    kv.decode_attention_fp16(cfg, dev(q), pool, dev(bt), dev(lens), dev(sk), dev(sv), sm, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name,over,tails", [
    ("qwen3-4b", dict(batch=3, ctx=384, hkv=2, hq=8), [0, 5, 127]),
    ("qwen3-32b-16k", dict(batch=2, ctx=640, hkv=2, hq=16), [0, 100]),
    ("tiny", dict(), [0]),
    ("qwen3-4b", dict(batch=2, ctx=256, hkv=1, hq=16), [17, 0]),      # group 16
    ("phi4-ragged", dict(batch=4, ragged=(128, 1024), hkv=2, hq=8), [0, 1, 2, 126]),
])
def test_fp16_decode_matches_oracle(name, over, tails):
    sp = gen.spec(name, **over)
    st, kt, vt, lens, sk, sv, q = _case(sp, tails)
    cfg = kv.default_config(sp.hkv)
    pool = _gpu_pool(cfg, st, sp.hkv)
    sm = 1 / np.sqrt(D)
    got = _gpu_decode(cfg, q, pool, st["block_table"], lens, sk, sv, sm)
    ref = oatt.decode_attention_fp16(q, kt, vt, st["block_table"], lens, sk, sv, sm)
    err = np.abs(got - ref).max()
    _say(f"fp16 decode {name} {over} tails={tails}: max abs err {err:.3g}, "
         f"max |o| {np.abs(ref).max():.3g}")
    assert err <= TOL


def test_fp16_decode_edge_lengths_and_invalid_rows():
    sp = gen.spec("qwen3-4b", batch=6, ctx=256, hkv=2, hq=4)
    st, kt, vt, _, _, _, q = _case(sp, [0] * 6)
    rng = np.random.default_rng(9)
    sk = (rng.standard_normal((sp.batch, sp.hkv, T, D)) * 2).astype(np.float16)
    sv = (rng.standard_normal((sp.batch, sp.hkv, T, D)) * 2).astype(np.float16)
    cfg = kv.default_config(sp.hkv)
    pool = _gpu_pool(cfg, st, sp.hkv)
    bt = st["block_table"].copy()
    # row 4 negative, row 5 more tiles than the table holds
    lens = np.array([0, 1, 129, 256, -2, (bt.shape[1] + 1) * T], np.int32)
    got = _gpu_decode(cfg, q, pool, bt, lens, sk, sv, 0.1)
    ok = slice(0, 4)
    ref = oatt.decode_attention_fp16(q[ok], kt, vt, bt[ok], lens[ok], sk[ok], sv[ok], 0.1)
    assert np.all(got[0] == 0)
    assert np.abs(got[ok] - ref).max() <= TOL
    assert np.isnan(got[4:]).all()


def test_fp16_decode_full_size_sampled():
    # the long-context layer at full size (1 GB fp16 pool), shuffled blocks; heads sampled
    sp = gen.spec("qwen3-32b-16k")
    st = gen.prefill(sp, max_new_tokens=T)
    cfg = kv.default_config(sp.hkv)
    pool = _gpu_pool(cfg, st, sp.hkv)
    lens = st["seq_lens"].astype(np.int32)
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    q = gen.query(sp)
    sm = 1 / np.sqrt(D)
    got = _gpu_decode(cfg, q, pool, st["block_table"], lens, sk, sk, sm)
    kt, vt = gen.tiles_by_block(st, sp.hkv)
    rng = np.random.default_rng(4)
    worst = 0.0
    for b in rng.choice(sp.batch, 3, replace=False):
        g = int(rng.integers(sp.hkv))
        hs = range(g * sp.group, (g + 1) * sp.group)
        sub = slice(b, b + 1)
        ref = oatt.decode_attention_fp16(q[sub], kt, vt, st["block_table"][sub], lens[sub],
                                         sk[sub], sk[sub], sm)
        worst = max(worst, float(np.abs(got[b, list(hs)] - ref[0, list(hs)]).max()))
    _say(f"fp16 decode full size sampled: max abs err {worst:.3g}")
    assert worst <= TOL
