"""HIP graph capture of the library's calls. A serving loop that cannot afford one launch per
kernel captures its append + decode steps once and replays them: the calls issue only kernel
launches on the caller's stream (no allocation, no memset, no host synchronisation), so every
replay of a captured step gives bitwise the eager results. Each replay is checked, with eager
work and synchronisations between the replays; the cases cover the split-grid decode of a small
table and the paired-tile list schedule of a large one (its end marks live in the workspace)."""

import math

import numpy as np
import pytest
import torch

import decode_attention_tok_amd as kv
from workloads import gen

pytestmark = pytest.mark.gpu
T, D = 128, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _state(name, **over):
    sp = gen.spec(name, **over)
    st = gen.prefill(sp, max_new_tokens=T)
    cfg = kv.default_config(sp.hkv)
    pool = torch.zeros(st["num_blocks"], sp.hkv, kv.TILE_BYTES, dtype=torch.uint8, device="cuda")
    kd, vd = dev(st["k"]), dev(st["v"])
    kv.quantize_tiles(cfg, kd.view(kd.shape[0], -1), vd.view(vd.shape[0], -1),
                      dev(st["dst_blocks"]), pool)
    return sp, st, cfg, pool


@pytest.mark.parametrize("name,over,steps", [
    ("qwen3-4b", dict(batch=3, ctx=1024, hkv=2, hq=8), 3),          # split grid
    ("qwen3-32b-16k", dict(batch=16, ctx=8192, hkv=16, hq=64), 2),  # paired-tile list
])
def test_captured_steps_replay_bitwise(name, over, steps):
    sp, st, cfg, pool = _state(name, **over)
    b, hq = sp.batch, sp.hq
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
    q = dev(gen.query(sp))
    ws = torch.empty(max(kv.decode_workspace_bytes(cfg, b, hq, mb), 256), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty(b, hq, D, dtype=torch.float32, device="cuda") for _ in range(steps)]
    sm = 1.0 / math.sqrt(D)
    pool0, sk0, sv0 = pool.clone(), sk.clone(), sv.clone()

    def step_all():
        for i in range(steps):
            kv.append_token(cfg, kn[i], vn[i], pos[i], bt, sk, sv, pool)
            kv.decode_attention(cfg, q, pool, bt, lens[i], sk, sv, sm, outs[i], ws)

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
        kv.decode_attention(cfg, q, pool, bt, lens[0], sk, sv, 0.5 * sm, other, ws)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
