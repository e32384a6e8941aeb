"""HIP graph capture of the library's calls. A serving loop that cannot afford one launch per
kernel captures its append + decode steps once and replays them: the calls issue only kernel
launches on the caller's stream (no allocation, no memset, no host synchronisation), so every
replay of a captured step gives bitwise the eager results. Each replay is checked, with eager
work and synchronisations between the replays. The cases cover the split-grid decode of a small
table, the paired-tile list schedule of a large one (its end marks live in the workspace), the
4-bit value preset, head dimension 256, the several-token decode on the 16-head list, and the
allocation-free decode (its static scratch in place of the workspace) on both schedules."""

import math

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


def _state(name, v_bits, **over):
    sp = gen.spec(name, **over)
    st = gen.prefill(sp, max_new_tokens=T)
    cfg = kv.default_config(sp.hkv, v_bits=v_bits, head_dim=sp.head_dim)
    pool = torch.zeros(st["num_blocks"], sp.hkv, kv.tile_bytes(cfg), dtype=torch.uint8,
                       device="cuda")
    kd, vd = dev(st["k"]), dev(st["v"])
    kv.quantize_tiles(cfg, kd.view(kd.shape[0], -1), vd.view(vd.shape[0], -1),
                      dev(st["dst_blocks"]), pool)
    return sp, st, cfg, pool


@pytest.mark.parametrize("name,over,steps,v_bits,nq,noalloc", [
    ("qwen3-4b", dict(batch=3, ctx=1024, hkv=2, hq=8), 3, 2, 1, False),          # split grid
    ("qwen3-32b-16k", dict(batch=16, ctx=8192, hkv=16, hq=64), 2, 2, 1, False),  # paired list
    ("qwen3-4b", dict(batch=3, ctx=1024, hkv=2, hq=8), 2, 4, 1, False),          # 4-bit values
    ("qwen3-4b", dict(batch=2, ctx=640, hkv=2, hq=8, head_dim=256), 2, 2, 1, False),
    ("qwen3-32b-16k", dict(batch=16, ctx=8192, hkv=8, hq=64), 2, 2, 4, False),   # 32 heads
    ("qwen3-4b", dict(batch=3, ctx=1024, hkv=2, hq=8), 2, 2, 1, True),           # static scratch
    ("qwen3-32b-16k", dict(batch=16, ctx=8192, hkv=8, hq=32), 2, 2, 1, True),
])
def test_captured_steps_replay_bitwise(name, over, steps, v_bits, nq, noalloc):
    sp, st, cfg, pool = _state(name, v_bits, **over)
    b, hq, D = sp.batch, sp.hq, sp.head_dim
    bt = dev(st["block_table"])
    mb = st["block_table"].shape[1]
    sk = torch.zeros(b, sp.hkv, T, D, dtype=torch.float16, device="cuda")
    sv = torch.zeros_like(sk)
    lens0 = st["seq_lens"].astype(np.int32)
    toks = [gen.append_tokens(sp, i) for i in range(steps)]
    kn = [dev(t[0]) for t in toks]
    vn = [dev(t[1]) for t in toks]
    pos = [dev(lens0 + i) for i in range(steps)]
    lens = [dev(lens0 + i + 1) for i in range(steps)]
    if nq == 1:
        q = dev(gen.query(sp))
        ws_bytes = kv.decode_workspace_bytes(cfg, b, hq, mb)
    else:
        q = dev(gen.query_tokens(sp, nq))
        ws_bytes = kv.decode_multi_workspace_bytes(cfg, b, hq, nq, mb)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(*q.shape, dtype=torch.float32, device="cuda") for _ in range(steps)]
    sm = 1.0 / math.sqrt(D)
    pool0, sk0, sv0 = pool.clone(), sk.clone(), sv.clone()

    def decode(lens_i, scale, out):
        if noalloc:
            kv.decode_attention_noalloc(cfg, q, pool, bt, lens_i, sk, sv, scale, out)
        elif nq == 1:
            kv.decode_attention(cfg, q, pool, bt, lens_i, sk, sv, scale, out, ws)
        else:
            kv.decode_attention_multi(cfg, q, pool, bt, lens_i, sk, sv, scale, out, ws)

    def step_all():
        for i in range(steps):
            kv.append_token(cfg, kn[i], vn[i], pos[i], bt, sk, sv, pool)
            decode(lens[i], sm, outs[i])

    step_all()                                   # eager reference (also warms the plan caches)
    torch.cuda.synchronize()
    ref = [o.cpu().numpy().copy() for o in outs]
    assert all(np.isfinite(r).all() for r in ref)
    pool.copy_(pool0); sk.copy_(sk0); sv.copy_(sv0)
    for o in outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all()
    torch.cuda.synchronize()
    other = torch.empty_like(outs[0])
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            got = outs[i].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref[i].view(np.uint32)), (rep, i)
        # eager work between the replays: a different decode through the same workspace, and
        # the outputs scribbled over
        decode(lens[0], 0.5 * sm, other)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
