"""Parity of the several-token decode (kvarn_decode_attention_multi) with the oracle's
decode_attention_multi (reading R25: the last Q tokens of each sequence, causal) on seeded
inputs, through the C ABI. Same bar as the one-token decode: max-abs <= 2e-3."""

import math

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from oracle import attention as oatt
from oracle import codec
from workloads import gen

from test_gpu_parity import TOL, _decode_case, _say, dev, gpu_decode

pytestmark = pytest.mark.gpu
T = D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def gpu_multi(cfg, q, pool, bt, lens, sk, sv, sm):
    b, nq, hq, _ = q.shape
    ws = torch.empty(max(kv.decode_multi_workspace_bytes(cfg, b, hq, nq, bt.shape[1]), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((b, nq, hq, D), -7.0, dtype=torch.float32, device="cuda")
    pool_d = pool if isinstance(pool, torch.Tensor) else dev(pool)
    kv.decode_attention_multi(cfg, dev(q), pool_d, dev(bt), dev(lens), dev(sk), dev(sv), sm,
                              out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name,over,tails,nq", [
    # tails 0: every query token inside the last packed tile; 5 < Q = 8: the tokens straddle
    # the tile boundary; 127: all in staging
    ("qwen3-4b", dict(batch=3, ctx=384, hkv=2, hq=8), [0, 5, 127], 2),
    ("qwen3-4b", dict(batch=3, ctx=384, hkv=2, hq=8), [0, 5, 127], 8),
    ("qwen3-32b-16k", dict(batch=2, ctx=640, hkv=2, hq=16), [3, 0], 4),
    ("qwen3-32b-16k", dict(batch=2, ctx=640, hkv=2, hq=16), [100, 9], 16),   # 16 x 8 rows
    ("qwen3-4b", dict(batch=2, ctx=256, hkv=1, hq=16), [17, 0], 3),          # group 16
    ("phi4-ragged", dict(batch=4, ragged=(128, 1024), hkv=2, hq=8), [0, 1, 2, 126], 5),
    ("qwen3-4b", dict(batch=2, ctx=384, hkv=2, hq=6), [0, 33], 3),          # 9 rows: 8 + 1
    ("qwen3-4b", dict(batch=2, ctx=256, hkv=2, hq=24), [90, 1], 2),         # 24 rows: 3 groups
    ("qwen3-4b", dict(batch=1, ctx=128, hkv=5, hq=10), [127], 16),          # 32 rows, one tile
])
def test_multi_matches_oracle(name, over, tails, nq):
    sp = gen.spec(name, **over)
    pool, bt, lens, sk, sv, _, sm = _decode_case(sp, tails)
    q = gen.query_tokens(sp, nq)
    cfg = kv.default_config(sp.hkv)
    got = gpu_multi(cfg, q, pool, bt, lens, sk, sv, sm)
    ref = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, sm)
    err = np.abs(got - ref).max()
    _say(f"multi {name} {over} tails={tails} Q={nq}: max abs err {err:.3g}")
    assert err <= TOL


def test_one_query_token_equals_the_one_token_decode():
    sp = gen.spec("qwen3-4b", batch=3, ctx=384, hkv=2, hq=8)
    pool, bt, lens, sk, sv, q, sm = _decode_case(sp, [0, 5, 127])
    cfg = kv.default_config(sp.hkv)
    a = gpu_multi(cfg, q[:, None], pool, bt, lens, sk, sv, sm)
    b = gpu_decode(cfg, q, pool, bt, lens, sk, sv, sm)
    assert np.array_equal(a[:, 0], b)


def test_multi_short_sequences_and_invalid_rows():
    # lengths 0, 1, 2 with Q = 4 (early tokens see nothing: zeros), one valid row, and rows
    # with a negative length or an out-of-range block id (NaN in every query token)
    sp = gen.spec("qwen3-4b", batch=6, ctx=256, hkv=2, hq=4)
    pool, bt, lens, sk, sv, _, sm = _decode_case(sp, [0, 0, 0, 0, 9, 0])
    lens = lens.copy()
    lens[:3] = [0, 1, 2]
    lens[4] = -1
    bt = bt.copy()
    bt[5, 0] = pool.shape[0] + 3
    q = gen.query_tokens(sp, 4)
    cfg = kv.default_config(sp.hkv)
    got = gpu_multi(cfg, q, pool, bt, lens, sk, sv, sm)
    ref = oatt.decode_attention_multi(q[:4], pool, bt[:4], lens[:4], sk[:4], sv[:4], sm)
    assert np.all(got[0] == 0) and np.all(got[1, :3] == 0) and np.all(got[2, :2] == 0)
    assert np.abs(got[:4] - ref).max() <= TOL
    assert np.isnan(got[4:]).all()


def test_multi_full_size_sampled():
    """The 16K workload at full size with Q = 4, launched as the benchmark launches it: one
    (sequence, KV head) holds oracle records, the rest library-quantised device-generated
    tiles; that pair's query rows are compared with the oracle."""
    sp = gen.spec("qwen3-32b-16k")
    sample_b, sample_g, nq = 5, 2, 4
    st_s = gen.prefill(sp, sequences=[sample_b])
    lens = st_s["seq_lens"]
    bt = st_s["block_table"]
    cfg = kv.default_config(sp.hkv)
    pool = torch.zeros(st_s["num_blocks"], sp.hkv, 13312, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(sp.seed + 1)
    for b in range(sp.batch):
        n = int(lens[b]) // T
        kd = (torch.randn(n * T, sp.hkv, D, device="cuda", generator=g) * 4).half()
        vd = (torch.randn(n * T, sp.hkv, D, device="cuda", generator=g) * 4).half()
        kv.quantize_tiles(cfg, kd.view(n * T, -1), vd.view(n * T, -1), dev(bt[b, :n]), pool)
    n_s = int(lens[sample_b]) // T
    recs = np.stack([codec.encode_record(st_s["k"][T * i:T * i + T, sample_g],
                                         st_s["v"][T * i:T * i + T, sample_g])
                     for i in range(n_s)])
    idx = torch.from_numpy(bt[sample_b, :n_s].astype(np.int64)).cuda()
    pool[idx, sample_g] = dev(recs)
    q = gen.query_tokens(sp, nq)
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    got = gpu_multi(cfg, q, pool, bt, lens, sk, sk, 1 / math.sqrt(D))
    G = sp.group
    sub_pool = np.zeros((st_s["num_blocks"], 1, 13312), np.uint8)
    sub_pool[bt[sample_b, :n_s], 0] = recs
    ref = oatt.decode_attention_multi(q[sample_b:sample_b + 1, :, sample_g * G:(sample_g + 1) * G],
                                      sub_pool, bt[sample_b:sample_b + 1],
                                      lens[sample_b:sample_b + 1], sk[:1, :1], sk[:1, :1],
                                      1 / math.sqrt(D))
    err = np.abs(got[sample_b, :, sample_g * G:(sample_g + 1) * G] - ref[0]).max()
    _say(f"multi full-size Q={nq}: max abs err {err:.3g}")
    assert err <= TOL
    assert np.isfinite(got).all()


def test_multi_at_the_split_limit():
    """Sixteen query tokens of eight heads (128 rows per KV head) on one long sequence whose
    split plan reaches 64 splits, with the last tokens straddling the staging tile."""
    sp = gen.spec("qwen3-32b-16k", batch=1, ctx=64000, hkv=1, hq=8)
    st = gen.prefill(sp, max_new_tokens=1200)
    pool = np.zeros((st["num_blocks"], 1, codec.TILE_BYTES), np.uint8)
    oatt.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool)
    rng = np.random.default_rng(13)
    sk = np.zeros((1, 1, T, D), np.float16)
    sv = np.zeros_like(sk)
    sk[0, 0, :9] = rng.standard_normal((9, D)).astype(np.float16)
    sv[0, 0, :9] = rng.standard_normal((9, D)).astype(np.float16)
    lens = st["seq_lens"].astype(np.int32) + 9               # 9 < 16 query tokens
    q = gen.query_tokens(sp, 16)
    cfg = kv.default_config(sp.hkv)
    assert kv.decode_multi_workspace_bytes(cfg, 1, sp.hq, 16, 510) == 16 * sp.hq * 64 * 130 * 4
    got = gpu_multi(cfg, q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(D))
    ref = oatt.decode_attention_multi(q, pool, st["block_table"], lens, sk, sv, 1 / math.sqrt(D))
    err = np.abs(got - ref).max()
    _say(f"multi at 64 splits, Q=16: max abs err {err:.3g}")
    assert err <= TOL


@pytest.mark.parametrize("name,over,tails,nq", [
    ("qwen3-4b", dict(batch=3, ctx=1024, hkv=2, hq=4), [0, 5, 127], 2),      # 2 x 2 rows
    ("qwen3-4b", dict(batch=2, ctx=640, hkv=2, hq=2), [100, 9], 4),          # 1 x 4 rows
    ("qwen3-4b", dict(batch=2, ctx=768, hkv=2, hq=2), [0, 1], 3),            # 1 x 3 rows
])
def test_multi_pair_kernel_matches_oracle(name, over, tails, nq):
    """Several query tokens with at most four virtual heads per KV head in the paired-tile
    kernel (a wide block table selects it), causal masks included."""
    from test_gpu_parity import widen
    sp = gen.spec(name, **over)
    pool, bt, lens, sk, sv, _, sm = _decode_case(sp, tails)
    q = gen.query_tokens(sp, nq)
    cfg = kv.default_config(sp.hkv)
    got = gpu_multi(cfg, q, pool, widen(bt, sp.hkv), lens, sk, sv, sm)
    ref = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, sm)
    err = np.abs(got - ref).max()
    _say(f"multi pair kernel {name} {over} tails={tails} nq={nq}: max abs err {err:.3g}")
    assert err <= TOL


@pytest.mark.parametrize("name,over,tails,nq,v_bits", [
    ("qwen3-4b", dict(batch=3, ctx=1024, hkv=2, hq=8), [0, 5, 127], 2, 2),     # 4 x 2 rows
    ("qwen3-4b", dict(batch=2, ctx=896, hkv=2, hq=4), [100, 9], 4, 4),         # 2 x 4 rows
    ("qwen3-4b", dict(batch=4, ctx=640, hkv=2, hq=2), [0, 1, 64, 127], 3, 4),  # 1 x 3 rows, 4-bit
])
def test_multi_tile_list_matches_oracle(name, over, tails, nq, v_bits):
    """Several query tokens with five to eight virtual heads per KV head (or 4-bit values) on
    a wide block table: the four-wave tile kernel's list schedule, causal masks included."""
    from test_gpu_parity import widen
    sp = gen.spec(name, **over)
    pool, bt, lens, sk, sv, _, sm = _decode_case(sp, tails, v_bits=v_bits)
    q = gen.query_tokens(sp, nq)
    cfg = kv.default_config(sp.hkv, v_bits=v_bits)
    got = gpu_multi(cfg, q, pool, widen(bt, sp.hkv), lens, sk, sv, sm)
    ref = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, sm)
    err = np.abs(got - ref).max()
    _say(f"multi tile list {name} {over} tails={tails} nq={nq} v_bits={v_bits}: "
         f"max abs err {err:.3g}")
    assert err <= TOL


@pytest.mark.parametrize("name,over,tails,nq", [
    ("qwen3-32b-16k", dict(batch=2, ctx=640, hkv=2, hq=16), [3, 0], 4),     # 32 rows: 2 groups
    ("qwen3-4b", dict(batch=2, ctx=768, hkv=2, hq=24), [90, 1], 2),         # 24 rows: 16 + 8
    ("qwen3-4b", dict(batch=3, ctx=512, hkv=1, hq=16), [0, 17, 127], 3),    # 48 rows: 3 groups
])
def test_multi_wide_list_head_groups_matches_oracle(name, over, tails, nq):
    """More than 16 virtual heads per KV head on a wide block table: the 16-head kernel's list
    schedule with one list unit per (sequence, KV head, head group of 16), causal masks
    included."""
    from test_gpu_parity import widen
    sp = gen.spec(name, **over)
    pool, bt, lens, sk, sv, _, sm = _decode_case(sp, tails)
    q = gen.query_tokens(sp, nq)
    cfg = kv.default_config(sp.hkv)
    got = gpu_multi(cfg, q, pool, widen(bt, sp.hkv), lens, sk, sv, sm)
    ref = oatt.decode_attention_multi(q, pool, bt, lens, sk, sv, sm)
    err = np.abs(got - ref).max()
    _say(f"multi wide list {name} {over} tails={tails} nq={nq}: max abs err {err:.3g}")
    assert err <= TOL
