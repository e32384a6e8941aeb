"""kvarn_decode_attention_noalloc (the decode for callers that cannot allocate: the library's
static per-device scratch instead of a caller workspace) against kvarn_decode_attention on the
same inputs, through the C ABI: identical outputs (same kernels, same split plan), both within
the decode bar of the oracle, on two calls in a row, the second smaller than the first (the
scratch still holds the first call's partials)."""

import math

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from oracle import attention as oatt
from workloads import gen

pytestmark = pytest.mark.gpu
T = D = 128
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(sp, tails, seed):
    st = gen.prefill(sp, max_new_tokens=T)
    pool = np.zeros((st["num_blocks"], sp.hkv, kv.TILE_BYTES), np.uint8)
    oatt.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool)
    lens = st["seq_lens"].copy()
    rng = np.random.default_rng(seed)
    sk = np.zeros((sp.batch, sp.hkv, T, D), np.float16)
    sv = np.zeros_like(sk)
    for b, tail in enumerate(tails):
        sk[b, :, :tail] = (rng.standard_normal((sp.hkv, tail, D)) * 2).astype(np.float16)
        sv[b, :, :tail] = (rng.standard_normal((sp.hkv, tail, D)) * 2).astype(np.float16)
        lens[b] += tail
    return pool, st["block_table"], lens.astype(np.int32), sk, sv, gen.query(sp, dense=True)


def _both(cfg, pool, bt, lens, sk, sv, q, sm):
    b, hq, _ = q.shape
    args = [dev(q), dev(pool), dev(bt), dev(lens), dev(sk), dev(sv)]
    ws = torch.empty(max(kv.decode_workspace_bytes(cfg, b, hq, bt.shape[1]), 256),
                     dtype=torch.uint8, device="cuda")
    out_ws = torch.full((b, hq, D), -3.0, dtype=torch.float32, device="cuda")
    out_na = torch.full((b, hq, D), -5.0, dtype=torch.float32, device="cuda")
    kv.decode_attention(cfg, *args, sm, out_ws, ws)
    kv.decode_attention_noalloc(cfg, *args, sm, out_na)
    torch.cuda.synchronize()
    return out_ws.cpu().numpy(), out_na.cpu().numpy()


def test_noalloc_matches_the_workspace_decode_on_two_calls():
    sm = 1 / math.sqrt(D)
    # first call: 6 sequences of 1,536 tokens plus staging tails, 4 KV heads, 16 query heads
    sp1 = gen.spec("qwen3-4b", batch=6, ctx=1536, hkv=4, hq=16)
    c1 = _case(sp1, [0, 5, 127, 64, 1, 99], 1)
    cfg1 = kv.default_config(sp1.hkv)
    a1, n1 = _both(cfg1, *c1, sm)
    ref1 = oatt.decode_attention(c1[5], c1[0], c1[1], c1[2], c1[3], c1[4], sm)
    print(f"no-alloc call 1: max |ws - noalloc| {np.abs(a1 - n1).max():.3g}, vs oracle "
          f"{np.abs(n1 - ref1).max():.3g}", flush=True)
    assert np.array_equal(a1, n1)
    assert np.abs(n1 - ref1).max() <= TOL
    # second call, smaller (2 sequences of 384 tokens, 2 KV heads): the scratch still holds the
    # first call's partials
    sp2 = gen.spec("qwen3-32b-16k", batch=2, ctx=384, hkv=2, hq=8)
    c2 = _case(sp2, [17, 0], 2)
    cfg2 = kv.default_config(sp2.hkv)
    a2, n2 = _both(cfg2, *c2, sm)
    ref2 = oatt.decode_attention(c2[5], c2[0], c2[1], c2[2], c2[3], c2[4], sm)
    print(f"no-alloc call 2: max |ws - noalloc| {np.abs(a2 - n2).max():.3g}, vs oracle "
          f"{np.abs(n2 - ref2).max():.3g}", flush=True)
    assert np.array_equal(a2, n2)
    assert np.abs(n2 - ref2).max() <= TOL


def test_noalloc_rejects_sizes_beyond_its_scratch():
    cfg = kv.default_config(8)
    q = torch.zeros(4096, 64, D, dtype=torch.float16, device="cuda")
    bt = torch.zeros(4096, 8, dtype=torch.int32, device="cuda")
    assert kv.decode_workspace_bytes(cfg, 4096, 64, 8) > kv.STATIC_SCRATCH_BYTES
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kv.KvarnError) as e:
        kv.decode_attention_noalloc(cfg, q, small, bt, bt[:, 0], small, small, 0.1,
                                    torch.empty(1, device="cuda"))
    assert e.value.code == 6
