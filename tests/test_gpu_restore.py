"""Save and restore of a live cache: the block pool, the staging tiles and the block table of
a decode batch written to host files and read back (into the same block ids, and into other
block ids with the table rewritten) give bitwise-identical attention. A record carries
everything its tile needs ([TSM] "Where the bill lands": the per-tile statistics are state that
must stay consistent between the writes and the reads), so nothing else has to be saved."""

import math
import os

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from workloads import gen

pytestmark = pytest.mark.gpu
T = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _decode(cfg, q, pool, bt, lens, sk, sv, d):
    b, hq = q.shape[0], q.shape[1]
    ws = torch.empty(max(kv.decode_workspace_bytes(cfg, b, hq, bt.shape[1]), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(b, hq, d, dtype=torch.float32, device="cuda")
    kv.decode_attention(cfg, q, pool, bt, lens, sk, sv, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,vb", [(128, 2), (128, 4), (64, 2), (256, 2)])
def test_saved_cache_restores_bitwise(tmp_path, d, vb):
    sp = gen.spec("phi4-ragged", batch=5, ragged=(256, 1400), head_dim=d)
    st = gen.prefill(sp, max_new_tokens=2 * T)
    cfg = kv.default_config(sp.hkv, v_bits=vb, head_dim=d)
    pool = torch.zeros(st["num_blocks"], sp.hkv, kv.tile_bytes(cfg), dtype=torch.uint8,
                       device="cuda")
    kd, vd = dev(st["k"]), dev(st["v"])
    kv.quantize_tiles(cfg, kd.view(kd.shape[0], -1), vd.view(vd.shape[0], -1),
                      dev(st["dst_blocks"]), pool)
    # a live decode state: staging written by appends (one of them completes a tile)
    sk = torch.zeros(sp.batch, sp.hkv, T, d, dtype=torch.float16, device="cuda")
    sv = torch.zeros_like(sk)
    bt = dev(st["block_table"])
    lens = st["seq_lens"].astype(np.int32).copy()
    for step in range(T + 3):
        kn, vn = gen.append_tokens(sp, step)
        kv.append_token(cfg, dev(kn), dev(vn), dev(lens), bt, sk, sv, pool)
        lens += 1
    q = dev(gen.query(sp, dense=True))
    lens_d = dev(lens)
    ref = _decode(cfg, q, pool, bt, lens_d, sk, sv, d)

    # save: plain arrays in one .npz (no pickled objects), then drop every device buffer
    path = os.path.join(tmp_path, "cache.npz")
    np.savez(path, pool=pool.cpu().numpy(), staging_k=sk.cpu().numpy(),
             staging_v=sv.cpu().numpy(), block_table=st["block_table"], seq_lens=lens)
    del pool, sk, sv, bt
    torch.cuda.synchronize()

    saved = np.load(path)
    assert saved["pool"].shape[-1] == kv.tile_bytes(cfg)
    # restore into the same block ids
    out = _decode(cfg, q, dev(saved["pool"]), dev(saved["block_table"]), dev(saved["seq_lens"]),
                  dev(saved["staging_k"]), dev(saved["staging_v"]), d)
    assert np.array_equal(out, ref)
    # restore into other block ids of a larger pool, with the table rewritten to match
    nb = saved["pool"].shape[0]
    perm = np.random.default_rng(7).permutation(2 * nb)[:nb].astype(np.int32)
    big = np.zeros((2 * nb,) + saved["pool"].shape[1:], np.uint8)
    big[perm] = saved["pool"]
    table = perm[saved["block_table"]]
    out2 = _decode(cfg, q, dev(big), dev(table), dev(saved["seq_lens"]),
                   dev(saved["staging_k"]), dev(saved["staging_v"]), d)
    assert np.array_equal(out2, ref)
