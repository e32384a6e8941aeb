"""Parity of kvarn_dequantize_tiles (stage 4 written out) with the oracle's decode_record on
oracle-written records, and the rounding bound on records the library wrote itself."""

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from oracle import codec
from workloads import gen

from record_view import e4m3, parse
from test_gpu_parity import dev, gpu_quantize

pytestmark = pytest.mark.gpu
T = D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def gpu_dequant(cfg, pool, ids, hkv):
    n = len(ids)
    ko = torch.full((n * T, hkv, D), -5.0, dtype=torch.float32, device="cuda")
    vo = torch.full_like(ko, -5.0)
    kv.dequantize_tiles(cfg, pool, dev(np.asarray(ids, np.int32)), ko, vo)
    torch.cuda.synchronize()
    return ko.cpu().numpy(), vo.cpu().numpy()


@pytest.mark.parametrize("name,over", [("tiny", {}), ("qwen3-4b", dict(batch=2, ctx=256, hkv=2)),
                                       ("qwen3-32b-16k", dict(batch=1, ctx=384, hkv=3))])
def test_dequantize_matches_oracle(name, over):
    sp = gen.spec(name, **over)
    st = gen.prefill(sp)
    n = len(st["dst_blocks"])
    pool = np.zeros((st["num_blocks"], sp.hkv, 13312), np.uint8)
    refs = {}
    for i, blk in enumerate(st["dst_blocks"]):
        for h in range(sp.hkv):
            rows = slice(T * i, T * i + T)
            pool[blk, h] = codec.encode_record(st["k"][rows, h], st["v"][rows, h])
            refs[i, h] = codec.decode_record(pool[blk, h])
    cfg = kv.default_config(sp.hkv)
    ids = list(st["dst_blocks"][::-1])                     # any order, any blocks
    ko, vo = gpu_dequant(cfg, dev(pool), ids, sp.hkv)
    worst = 0.0
    for i, blk in enumerate(ids):
        src = int(np.where(st["dst_blocks"] == blk)[0][0])
        for h in range(sp.hkv):
            rk, rv = refs[src, h]
            for got, ref in ((ko[T * i:T * i + T, h], rk), (vo[T * i:T * i + T, h], rv)):
                err = np.abs(got - ref).max() / (1.0 + np.abs(ref).max())
                worst = max(worst, err)
    assert worst <= 4e-6, worst


def test_dequantize_invalid_ids_give_nan():
    sp = gen.spec("tiny")
    cfg = kv.default_config(1)
    pool = torch.zeros(2, 1, 13312, dtype=torch.uint8, device="cuda")
    ko, vo = gpu_dequant(cfg, pool, [-1, 2, 1], 1)
    assert np.isnan(ko[:2 * T]).all() and np.isnan(vo[:2 * T]).all()
    assert np.all(ko[2 * T:] == 0) and np.all(vo[2 * T:] == 0)     # an all-zero record


def test_round_trip_error_bound_on_library_records():
    # rotated-space rounding bound |y - y-hat| <= s-hat / 2 per element, carried through the
    # per-channel scale and the orthonormal rotation: per token,
    # ||x_t - x-hat_t||^2 <= sum_j (c-hat_j s-hat_t / 2)^2 (+ fp32 slack)
    sp = gen.spec("qwen3-4b", batch=2, ctx=512, hkv=2)
    st = gen.prefill(sp)
    cfg = kv.default_config(sp.hkv)
    pool = gpu_quantize(cfg, st["k"], st["v"], st["dst_blocks"], st["num_blocks"], sp.hkv)
    ko, vo = gpu_dequant(cfg, pool, list(st["dst_blocks"]), sp.hkv)
    pool_h = pool.cpu().numpy()
    for i, blk in enumerate(st["dst_blocks"]):
        for h in range(sp.hkv):
            rec = parse(pool_h[blk, h])
            for half, x, xh in (("k", st["k"], ko), ("v", st["v"], vo)):
                c_hat, s_hat = e4m3(rec[half + "_c"]), e4m3(rec[half + "_s"])
                bound = np.sqrt(np.sum((c_hat[None, :] * s_hat[:, None] / 2) ** 2, axis=1))
                rows = slice(T * i, T * i + T)
                err = np.sqrt(np.sum((x[rows, h].astype(np.float64) - xh[rows, h]) ** 2, axis=1))
                assert np.all(err <= bound * (1 + 1e-5) + 1e-4), (half, i, h)
