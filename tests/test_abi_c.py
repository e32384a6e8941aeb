"""The C ABI from a plain C99 program (tests/c/kvarn_c_client.c, built by build()): the header
compiles as C, the library links, host-side validation answers as documented; on a GPU the
same program quantises a small prefill and decodes one step through nothing but the C ABI and
the HIP runtime's C API, and its records and outputs are checked against the oracle."""

import math
import os
import subprocess

import numpy as np
import pytest

from decode_attention_tok_amd import build as kbuild

T = D = 128


def _client(path):
    if not os.path.exists(path):
        pytest.skip("C client not built (run build())")
    return path


def test_c_client_host_checks():
    out = subprocess.run([_client(kbuild.C_CLIENT)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "ok" in out.stdout


def test_c_client_host_checks_under_address_sanitizer():
    """The same host checks against a copy of the library whose host code is built with
    AddressSanitizer: every validation path runs without an invalid access or a leak."""
    exe = _client(kbuild.C_CLIENT_ASAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stderr[-4000:]
    assert "ok" in out.stdout and "AddressSanitizer" not in out.stderr


def _write_input(path, st, sp, q, sk, sv, lens, sm, v_bits):
    hdr = np.array([0x4B56524E, v_bits, len(st["dst_blocks"]), sp.hkv, sp.hq, sp.batch,
                    st["block_table"].shape[1], st["num_blocks"], sp.head_dim], np.int32)
    with open(path, "wb") as f:
        for a in (hdr, st["k"].astype(np.float16), st["v"].astype(np.float16),
                  st["dst_blocks"].astype(np.int32), st["block_table"].astype(np.int32),
                  lens.astype(np.int32), q.astype(np.float16), sk, sv,
                  np.array([sm], np.float32)):
            f.write(np.ascontiguousarray(a).tobytes())


@pytest.mark.gpu
@pytest.mark.parametrize("v_bits,d", [(2, 128), (4, 128), (2, 64), (4, 256)])
def test_c_client_gpu_round_trip(tmp_path, v_bits, d):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import attention as oatt
    from oracle import codec
    from workloads import gen
    from record_view import Budget, compare_half, parse

    client = _client(kbuild.C_CLIENT_GPU)
    sp = gen.spec("qwen3-4b", batch=2, ctx=384, hkv=2, hq=8, head_dim=d)
    st = gen.prefill(sp, max_new_tokens=T)
    lens = st["seq_lens"].astype(np.int32)
    rng = np.random.default_rng(3)
    sk = np.zeros((sp.batch, sp.hkv, T, d), np.float16)
    sv = np.zeros_like(sk)
    for b, tail in enumerate([0, 40]):
        sk[b, :, :tail] = rng.standard_normal((sp.hkv, tail, d)).astype(np.float16)
        sv[b, :, :tail] = rng.standard_normal((sp.hkv, tail, d)).astype(np.float16)
        lens[b] += tail
    q = gen.query(sp, dense=True)
    sm = 1 / math.sqrt(d)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_input(fin, st, sp, q, sk, sv, lens, sm, v_bits)
    print(f"C client on the GPU: v_bits={v_bits} head_dim={d}", flush=True)
    res = subprocess.run([client, "run", str(fin), str(fout)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    raw = np.fromfile(fout, np.uint8)
    n_out = sp.batch * sp.hq * d * 4
    got = raw[:n_out].view(np.float32).reshape(sp.batch, sp.hq, d)
    rb = codec.tile_bytes(v_bits, d)
    pool_g = raw[n_out:].reshape(st["num_blocks"], sp.hkv, rb)
    # the records the C program had the library write, against the oracle's quantisation
    budget = Budget()
    for i, blk in enumerate(st["dst_blocks"]):
        for h in range(sp.hkv):
            rows = slice(T * i, T * i + T)
            rec = parse(pool_g[blk, h])
            compare_half(rec, codec.quantize_tile(st["k"][rows, h].astype(np.float64), 4), "k",
                         4, budget)
            compare_half(rec, codec.quantize_tile(st["v"][rows, h].astype(np.float64), v_bits),
                         "v", v_bits, budget)
    budget.check()
    # its decode output against the oracle's attention over the oracle's own records of the
    # same tiles. When every record matches the oracle's exactly (no rounding-boundary flip,
    # the measured case), the two caches are byte-identical and the decode bar of 2e-3 holds;
    # a tolerated flip may move outputs by a fraction of the quantisation error instead
    pool_o = np.zeros((st["num_blocks"], sp.hkv, rb), np.uint8)
    oatt.quantize_tiles(st["k"], st["v"], st["dst_blocks"], pool_o)
    ref = oatt.decode_attention(q, pool_o, st["block_table"], lens, sk, sv, sm)
    err = float(np.abs(got - ref).max())
    scale = float(np.abs(ref).max())
    print(f"C client v_bits={v_bits}: {vars(budget)}; decode max abs err {err:.3g} "
          f"(|o| max {scale:.3g})", flush=True)
    assert np.isfinite(got).all()
    if budget.exact():
        assert np.array_equal(pool_g, pool_o)
        assert err <= 2e-3
    else:
        assert err <= 0.02 * scale
