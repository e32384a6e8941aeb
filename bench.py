"""Benchmark of the KVarN K4V2 g128 hot path on one MI355X.

One step = the whole path on one batch: quantise every full prefill tile of the batch into the
paged block pool (kvarn_quantize_tiles), append one new key/value token per sequence into the
fp16 staging tile (kvarn_append_token), and one decode-attention step over the packed tiles plus
the staging token (kvarn_decode_attention). Default workload: the Qwen3-4B-like layer (8 KV
heads, 32 query heads, batch 8, 4096-token context = 32 tiles per sequence, then token 4097).

All inputs are resident in HBM before timing starts. Each step uses the next of several
identical input/cache replicas so that the 256 MB last-level (Infinity) cache cannot serve a
step from the previous one.

Printed: one JSON line. value = whole-step effective HBM GB/s (algorithmic bytes of all three
calls / step time). Also per call: decode-attention GB/s and fraction of the 8 TB/s peak,
tiles quantised per second; the roofline of the dominant kernel (HIP events around each call
on the launch stream); the fp64 oracle timed on a bounded sample on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
T = D = 128
TILE = 13312

WORKLOADS = {
    # name: (spec name, spec overrides)
    "qwen3-4b": ("qwen3-4b", {}),
    "qwen3-32b-16k": ("qwen3-32b-16k", {}),
    "phi4-ragged": ("phi4-ragged", {}),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qwen3-4b", choices=sorted(WORKLOADS))
    p.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 1 GB")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run one device copy of this many MiB (counter calibration)")
    p.add_argument("--no-fp16-decode", action="store_true",
                   help="skip the comparison decode over an unquantised fp16 cache")
    p.add_argument("--no-multi-decode", action="store_true",
                   help="skip the several-token (Q = 4) decode measurement")
    p.add_argument("--no-k4v4", action="store_true",
                   help="skip the measurement of the 4-bit value preset")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the copy-bandwidth, layer-stream and write-stream measurements")
    return p.parse_args()


KERNEL_SOURCES = {
    "quantise": ("kvarn_quantize.hip", "kvarn_device.hpp"),
    "append": ("kvarn_quantize.hip", "kvarn_device.hpp"),
    "decode": ("kvarn_decode.hip", "kvarn_device.hpp"),
}


def source_digest(part=None):
    """Digest of the HIP sources (of one part of the path, or all of them)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_tok_amd", "csrc")
    names = sorted(os.listdir(csrc)) if part is None else KERNEL_SOURCES[part]
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(lens, hkv, hq, appended, tile_bytes=TILE):
    """Bytes the method must move (not what an implementation happens to move); tile_bytes is
    the size of one (block, KV head) record: 13,312 packed, 65,536 for the fp16 cache."""
    n_full = [int(l) // T for l in lens]
    n_stage = [int(l) % T for l in lens]
    decode = sum(n * hkv * tile_bytes + s * hkv * 2 * D * 2 + 4 * n + 4
                 for n, s in zip(n_full, n_stage))
    decode += len(lens) * hq * D * (2 + 4)                       # q in (fp16), out (fp32)
    return decode


def fp16_decode_comparison(args, kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R, sm,
                           ws_bytes, td, torch, np, dev):
    """The same decode over an unquantised fp16 paged cache of the same tiles (the comparison
    path), timed separately after the main loop: its own pools (replicas beyond 1.2 GB), the
    main run's queries, staging tiles and lengths."""
    import ctypes
    V = ctypes.c_void_p
    fp16_bytes = int(lib.kvarn_fp16_block_bytes(ctypes.byref(cfg)))
    per = st["num_blocks"] * fp16_bytes
    reps = max(2, min(16, math.ceil(1.2e9 / per)))
    dst = dev(st["dst_blocks"])
    k0, v0 = dev(st["k"]), dev(st["v"])
    k0, v0 = k0.view(k0.shape[0], -1), v0.view(v0.shape[0], -1)
    pools = []
    for _ in range(reps):
        pool = torch.zeros(st["num_blocks"] * fp16_bytes, dtype=torch.uint8, device="cuda")
        kv.fp16_write_tiles(cfg, k0, v0, dst, pool)
        pools.append(pool)
    del k0, v0
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    f = lib.kvarn_decode_attention_fp16
    calls = [(ctypes.byref(cfg), V(R[i % len(R)]["q"].data_ptr()), sp.hq, V(pools[i].data_ptr()),
              st["num_blocks"], V(bt.data_ptr()), bt_np.shape[1], V(lens.data_ptr()),
              V(R[i % len(R)]["sk"].data_ptr()), V(R[i % len(R)]["sv"].data_ptr()),
              ctypes.c_float(sm), V(R[i % len(R)]["out"].data_ptr()),
              V(R[i % len(R)]["ws"].data_ptr()), max(ws_bytes, 256), sp.batch,
              V(stream.cuda_stream)) for i in range(reps)]
    steps = max(10, args.steps // 4)
    for i in range(max(2, args.warmup // 4)):
        assert f(*calls[i % reps]) == 0
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        assert f(*calls[i % reps]) == 0
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t16 = sum(a.elapsed_time(b) for a, b in evs) / steps * 1e-3
    b16 = algorithmic_bytes(lens_np, sp.hkv, sp.hq, True, tile_bytes=65536)
    print(f"# fp16-cache decode {t16 * 1e6:.1f} us over {reps} pools", file=sys.stderr,
          flush=True)
    return {"us": round(t16 * 1e6, 2), "gbps": round(b16 / t16 / 1e9, 1),
            "frac_of_peak": round(b16 / t16 / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": b16,
            "packed_speedup": round(t16 / td, 3)}


def multi_decode_measure(args, kv, lib, cfg, sp, bt, bt_np, lens, lens_np, R, sm, td, torch,
                         np, dev, n_query=4):
    """The several-token decode (query tokens = the last n_query cached tokens of each
    sequence, causal) over the main run's packed pools, staging tiles and lengths, timed
    separately after the main loop."""
    import ctypes
    from workloads import gen
    V = ctypes.c_void_p
    ws_m = kv.decode_multi_workspace_bytes(cfg, sp.batch, sp.hq, n_query, bt_np.shape[1])
    qm = dev(gen.query_tokens(sp, n_query))
    om = torch.empty(sp.batch, n_query, sp.hq, D, dtype=torch.float32, device="cuda")
    wsm = torch.empty(max(ws_m, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    f = lib.kvarn_decode_attention_multi
    reps = len(R)
    calls = [(ctypes.byref(cfg), V(qm.data_ptr()), sp.hq, n_query, V(r["pool"].data_ptr()),
              r["pool"].shape[0], V(bt.data_ptr()), bt_np.shape[1], V(lens.data_ptr()),
              V(r["sk"].data_ptr()), V(r["sv"].data_ptr()), ctypes.c_float(sm), V(om.data_ptr()),
              V(wsm.data_ptr()), max(ws_m, 256), sp.batch, V(stream.cuda_stream)) for r in R]
    steps = max(10, args.steps // 4)
    for i in range(max(2, args.warmup // 4)):
        assert f(*calls[i % reps]) == 0
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        assert f(*calls[i % reps]) == 0
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    tm = sum(a.elapsed_time(b) for a, b in evs) / steps * 1e-3
    bm = algorithmic_bytes(lens_np, sp.hkv, sp.hq, True) + \
        (n_query - 1) * len(lens_np) * sp.hq * D * (2 + 4)
    print(f"# {n_query}-token decode {tm * 1e6:.1f} us", file=sys.stderr, flush=True)
    return {"n_query": n_query, "us": round(tm * 1e6, 2), "gbps": round(bm / tm / 1e9, 1),
            "frac_of_peak": round(bm / tm / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": bm,
            "query_tokens_per_s": round(sp.batch * n_query / tm, 1),
            "time_vs_one_token": round(tm / td, 3)}


def k4v4_measure(args, kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R, sm, torch, dev):
    """The 4-bit value preset (kvarn_k4v4_g128) on the same workload: quantise the same prefill
    tiles into pools of 17,408-byte records, then the one-token decode over them with the main
    run's queries, staging tiles and lengths. Each call is timed on its own after the main loop,
    and the default preset is timed again in the same loops for the ratios."""
    import ctypes
    V = ctypes.c_void_p
    cfg4 = kv.default_config(sp.hkv, v_bits=4)
    rb = kv.tile_bytes(cfg4)
    n_tiles = int(st["dst_blocks"].shape[0])
    tile_heads = n_tiles * sp.hkv
    dst = dev(st["dst_blocks"])
    pools4 = [torch.zeros(st["num_blocks"], sp.hkv, rb, dtype=torch.uint8, device="cuda")
              for _ in R]
    ws_bytes = kv.decode_workspace_bytes(cfg4, sp.batch, sp.hq, bt_np.shape[1])
    stream = torch.cuda.current_stream()

    def calls(c, pools):
        cp = ctypes.byref(c)
        qc = [(cp, V(r["k"].data_ptr()), V(r["v"].data_ptr()), r["k"].stride(0), n_tiles,
               V(dst.data_ptr()), V(p.data_ptr()), st["num_blocks"], V(stream.cuda_stream))
              for r, p in zip(R, pools)]
        dc = [(cp, V(r["q"].data_ptr()), sp.hq, V(p.data_ptr()), st["num_blocks"],
               V(bt.data_ptr()), bt_np.shape[1], V(lens.data_ptr()), V(r["sk"].data_ptr()),
               V(r["sv"].data_ptr()), ctypes.c_float(sm), V(r["out"].data_ptr()),
               V(r["ws"].data_ptr()), max(ws_bytes, 256), sp.batch, V(stream.cuda_stream))
              for r, p in zip(R, pools)]
        return qc, dc

    reps = len(R)
    steps = max(10, args.steps // 4)

    def timed(f, cl):
        for i in range(max(reps, args.warmup // 4)):       # every pool is written first
            assert f(*cl[i % reps]) == 0
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record(stream)
            assert f(*cl[i % reps]) == 0
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps * 1e-3

    res = {}
    for key, c, pools in (("k4v2", cfg, [r["pool"] for r in R]), ("k4v4", cfg4, pools4)):
        qc, dc = calls(c, pools)
        res[key] = (timed(lib.kvarn_quantize_tiles, qc), timed(lib.kvarn_decode_attention, dc))
    qb = tile_heads * (2 * T * D * 2 + rb)
    db = algorithmic_bytes(lens_np, sp.hkv, sp.hq, True, tile_bytes=rb)
    (t2q, t2d), (t4q, t4d) = res["k4v2"], res["k4v4"]
    print(f"# k4v4: quantise {t4q * 1e6:.1f} us (k4v2 {t2q * 1e6:.1f}), decode "
          f"{t4d * 1e6:.1f} us (k4v2 {t2d * 1e6:.1f})", file=sys.stderr, flush=True)
    return {"v_bits": 4, "record_bytes": rb,
            "quantise": {"us": round(t4q * 1e6, 2), "tiles_per_s": round(tile_heads / t4q, 1),
                         "gbps": round(qb / t4q / 1e9, 1),
                         "frac_of_peak": round(qb / t4q / 1e9 / HBM_PEAK_GBPS, 4),
                         "algorithmic_bytes": qb, "k4v2_us_same_loop": round(t2q * 1e6, 2)},
            "decode_attn": {"us": round(t4d * 1e6, 2), "gbps": round(db / t4d / 1e9, 1),
                            "frac_of_peak": round(db / t4d / 1e9 / HBM_PEAK_GBPS, 4),
                            "algorithmic_bytes": db, "k4v2_us_same_loop": round(t2d * 1e6, 2)}}


def hbm_copy_measure(torch, n_bytes=1 << 30, repeats=5):
    """Achievable HBM bandwidth of a plain device-to-device copy (read + write bytes / time),
    median of a few repeats: context for the roofline fractions, never their denominator."""
    a = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(ts)[len(ts) // 2]
    del a, b
    return {"copy_bytes": n_bytes, "gbps": round(2 * n_bytes / t / 1e9, 1),
            "frac_of_peak": round(2 * n_bytes / t / 1e9 / HBM_PEAK_GBPS, 4)}


def layer_stream_measure(kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R, sm, torch, dev,
                         layers=36, repeats=5):
    """Decode of one token through `layers` layers back to back: the same step's decode over
    `layers` separate packed pools (one per layer, written by the quantiser from the same
    prefill), launched one after another; per-layer time = stream time / layers (median of
    repeats). The launch-amortised figure beside the per-launch one."""
    import ctypes
    V = ctypes.c_void_p
    n_tiles = int(st["dst_blocks"].shape[0])
    dst = dev(st["dst_blocks"])
    r0 = R[0]
    pools = []
    for _ in range(layers):
        p = torch.zeros(st["num_blocks"], sp.hkv, TILE, dtype=torch.uint8, device="cuda")
        kv.quantize_tiles(cfg, r0["k"], r0["v"], dst, p)
        pools.append(p)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    cp = ctypes.byref(cfg)
    ws_bytes = kv.decode_workspace_bytes(cfg, sp.batch, sp.hq, bt_np.shape[1])
    calls = [(cp, V(r0["q"].data_ptr()), sp.hq, V(p.data_ptr()), st["num_blocks"],
              V(bt.data_ptr()), bt_np.shape[1], V(lens.data_ptr()), V(r0["sk"].data_ptr()),
              V(r0["sv"].data_ptr()), ctypes.c_float(sm), V(r0["out"].data_ptr()),
              V(r0["ws"].data_ptr()), max(ws_bytes, 256), sp.batch, V(stream.cuda_stream))
             for p in pools]
    f = lib.kvarn_decode_attention
    for c in calls:
        assert f(*c) == 0
    torch.cuda.synchronize()
    ts = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for c in calls:
            assert f(*c) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(ts)[len(ts) // 2] / layers
    db = algorithmic_bytes(lens_np, sp.hkv, sp.hq, True)
    del pools
    print(f"# {layers}-layer decode stream: {t * 1e6:.1f} us per layer", file=sys.stderr,
          flush=True)
    return {"layers": layers, "us_per_layer": round(t * 1e6, 2), "gbps": round(db / t / 1e9, 1),
            "frac_of_peak": round(db / t / 1e9 / HBM_PEAK_GBPS, 4)}


def write_stream_measure(kv, lib, torch, np, dev, steps=None):
    """The write-path stream workload: batch 64, 8 KV heads, 32 query heads, 1024-token
    prefill; every step appends one key/value token per sequence into the fp16 staging tile
    (kvarn_append_token, which quantises the tile when its 128th token arrives) and decodes
    that token's query over the packed tiles plus staging (kvarn_decode_attention). Each step's
    append and decode are timed with HIP events; steps whose append completes tiles are the
    quantisation bursts."""
    import ctypes
    from workloads import gen
    V = ctypes.c_void_p
    sp = gen.spec("write-stream")
    steps = steps or sp.steps
    st = gen.prefill(sp, max_new_tokens=steps)
    cfg = kv.default_config(sp.hkv)
    n = len(st["dst_blocks"])
    pool = torch.zeros(st["num_blocks"], sp.hkv, TILE, dtype=torch.uint8, device="cuda")
    k0, v0 = dev(st["k"]), dev(st["v"])
    kv.quantize_tiles(cfg, k0.view(n * T, -1), v0.view(n * T, -1), dev(st["dst_blocks"]), pool)
    del k0, v0
    sk = torch.zeros(sp.batch, sp.hkv, T, D, dtype=torch.float16, device="cuda")
    sv = torch.zeros_like(sk)
    toks = [gen.append_tokens(sp, i) for i in range(steps)]
    kn = dev(np.stack([t[0] for t in toks]))
    vn = dev(np.stack([t[1] for t in toks]))
    lens0 = st["seq_lens"].astype(np.int32)
    pos = dev(np.stack([lens0 + i for i in range(steps)]).astype(np.int32))
    lens = dev(np.stack([lens0 + i + 1 for i in range(steps)]).astype(np.int32))
    q = dev(gen.query(sp))
    out = torch.empty(sp.batch, sp.hq, D, dtype=torch.float32, device="cuda")
    bt_np = st["block_table"]
    bt = dev(bt_np)
    ws_bytes = kv.decode_workspace_bytes(cfg, sp.batch, sp.hq, bt_np.shape[1])
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    cp = ctypes.byref(cfg)
    fa, fd = lib.kvarn_append_token, lib.kvarn_decode_attention
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record(stream)
        assert fa(cp, V(kn[i].data_ptr()), V(vn[i].data_ptr()), V(pos[i].data_ptr()),
                  V(bt.data_ptr()), bt_np.shape[1], V(sk.data_ptr()), V(sv.data_ptr()),
                  V(pool.data_ptr()), st["num_blocks"], sp.batch, V(stream.cuda_stream)) == 0
        evs[i][1].record(stream)
        assert fd(cp, V(q.data_ptr()), sp.hq, V(pool.data_ptr()), st["num_blocks"],
                  V(bt.data_ptr()), bt_np.shape[1], V(lens[i].data_ptr()), V(sk.data_ptr()),
                  V(sv.data_ptr()), ctypes.c_float(1.0 / math.sqrt(D)), V(out.data_ptr()),
                  V(ws.data_ptr()), max(ws_bytes, 256), sp.batch, V(stream.cuda_stream)) == 0
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    ta = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    td = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    burst = np.array([int(lens0[0] + i) % T == T - 1 for i in range(steps)])
    dbytes = sum(algorithmic_bytes(lens0 + i + 1, sp.hkv, sp.hq, True) for i in range(steps))
    tile_heads_burst = sp.batch * sp.hkv
    print(f"# write stream: {steps} steps, append {ta.mean() * 1e6:.1f} us "
          f"(bursts {ta[burst].mean() * 1e6:.1f} us), decode {td.mean() * 1e6:.1f} us",
          file=sys.stderr, flush=True)
    return {"workload": "write-stream", "batch": sp.batch, "kv_heads": sp.hkv, "q_heads": sp.hq,
            "start_context": int(lens0[0]), "steps": steps,
            "step_us_mean": round((ta + td).mean() * 1e6, 2),
            "append_us_mean": round(ta[~burst].mean() * 1e6, 2),
            "burst_steps": int(burst.sum()),
            "burst_append_us_mean": round(ta[burst].mean() * 1e6, 2) if burst.any() else None,
            "burst_tile_heads_per_s": (round(tile_heads_burst / ta[burst].mean(), 1)
                                       if burst.any() else None),
            "decode_us_mean": round(td.mean() * 1e6, 2),
            "decode_gbps": round(dbytes / td.sum() / 1e9, 1),
            "decode_frac_of_peak": round(dbytes / td.sum() / 1e9 / HBM_PEAK_GBPS, 4)}


def cpu_baseline(sp, st, q, lens, sm, tile_heads_total, pairs_total, step_bytes,
                 quant_budget_s=12.0, decode_budget_s=8.0):
    """The fp64 oracle, single-threaded, on a time-bounded sample of the same step: tile-head
    quantisations in order until all are done or quant_budget_s has passed, then (sequence,
    KV head) decodes over oracle-built caches until all are done or decode_budget_s has
    passed; the per-item times are extrapolated to the whole step."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    from oracle import attention as oatt
    from oracle import codec
    n_tiles = st["k"].shape[0] // T
    t0 = time.perf_counter()
    n_q = 0
    while n_q < tile_heads_total and time.perf_counter() - t0 < quant_budget_s:
        tile, head = n_q // sp.hkv, n_q % sp.hkv
        rows = slice(T * tile, T * tile + T)
        codec.encode_record(st["k"][rows, head], st["v"][rows, head])
        n_q += 1
    tq = (time.perf_counter() - t0) / n_q
    first = np.concatenate([[0], np.cumsum(st["seq_lens"] // T)])   # first tile of each sequence
    pool = np.zeros((st["num_blocks"], 1, TILE), np.uint8)
    td_total, n_d = 0.0, 0
    while n_d < pairs_total and td_total < decode_budget_s:
        b, g = n_d // sp.hkv, n_d % sp.hkv
        n = int(lens[b]) // T
        for i in range(n):
            rows = slice(T * (first[b] + i), T * (first[b] + i) + T)
            pool[st["block_table"][b, i], 0] = codec.encode_record(st["k"][rows, g],
                                                                   st["v"][rows, g])
        sk = np.zeros((1, 1, T, D), np.float16)
        t1 = time.perf_counter()
        oatt.decode_attention(q[b:b + 1, g * sp.group:(g + 1) * sp.group], pool,
                              st["block_table"][b:b + 1], lens[b:b + 1], sk, sk, sm)
        td_total += time.perf_counter() - t1
        n_d += 1
    td = td_total / n_d
    est = tq * tile_heads_total + td * pairs_total
    if limiter is not None:
        limiter.unregister()
    return {"value": step_bytes / est / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_q} of {tile_heads_total} tile-head quantisations "
                      f"({tq * 1e3:.2f} ms each) and {n_d} of {pairs_total} (sequence, KV head) "
                      f"decodes ({td * 1e3:.1f} ms each) of this step on one host core, "
                      f"extrapolated to the whole step ({est:.2f} s per step)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path is not built for "
              "more than one GPU", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import decode_attention_tok_amd as kv
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    spec_name, over = WORKLOADS[args.workload]
    sp = gen.spec(spec_name, **over)
    st = gen.prefill(sp, max_new_tokens=1)
    q_np = gen.query(sp)
    k_new_np, v_new_np = gen.append_tokens(sp, 0)
    lens_pre = st["seq_lens"].astype(np.int32)
    pos_np = lens_pre.copy()
    lens_np = lens_pre + 1
    bt_np = st["block_table"]
    cfg = kv.default_config(sp.hkv)
    sm = 1.0 / math.sqrt(D)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    n_tiles = int(st["dst_blocks"].shape[0])
    tile_heads = n_tiles * sp.hkv
    q_bytes = tile_heads * (2 * T * D * 2 + TILE)
    a_bytes = sp.batch * sp.hkv * 4 * D * 2
    d_bytes = algorithmic_bytes(lens_np, sp.hkv, sp.hq, True)
    step_bytes = q_bytes + a_bytes + d_bytes

    k0, v0 = dev(st["k"]), dev(st["v"])
    per_replica = k0.numel() * 4 + st["num_blocks"] * sp.hkv * TILE
    reps = args.replicas or max(2, min(16, math.ceil(1.2e9 / per_replica)))
    ws_bytes = kv.decode_workspace_bytes(cfg, sp.batch, sp.hq, bt_np.shape[1])
    R = []
    for _ in range(reps):
        R.append(dict(
            k=k0.clone().view(k0.shape[0], -1), v=v0.clone().view(v0.shape[0], -1),
            pool=torch.zeros(st["num_blocks"], sp.hkv, TILE, dtype=torch.uint8, device="cuda"),
            sk=torch.zeros(sp.batch, sp.hkv, T, D, dtype=torch.float16, device="cuda"),
            sv=torch.zeros(sp.batch, sp.hkv, T, D, dtype=torch.float16, device="cuda"),
            q=dev(q_np), kn=dev(k_new_np), vn=dev(v_new_np),
            out=torch.empty(sp.batch, sp.hq, D, dtype=torch.float32, device="cuda"),
            ws=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")))
    del k0, v0
    dst = dev(st["dst_blocks"])
    bt = dev(bt_np)
    pos = dev(pos_np)
    lens = dev(lens_np)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    import ctypes
    lib = kv.lib()
    cfgp = ctypes.byref(cfg)
    V = ctypes.c_void_p
    calls = []
    for r in R:
        calls.append((
            (cfgp, V(r["k"].data_ptr()), V(r["v"].data_ptr()), r["k"].stride(0), n_tiles,
             V(dst.data_ptr()), V(r["pool"].data_ptr()), st["num_blocks"], V(sptr)),
            (cfgp, V(r["kn"].data_ptr()), V(r["vn"].data_ptr()), V(pos.data_ptr()),
             V(bt.data_ptr()), bt_np.shape[1], V(r["sk"].data_ptr()), V(r["sv"].data_ptr()),
             V(r["pool"].data_ptr()), st["num_blocks"], sp.batch, V(sptr)),
            (cfgp, V(r["q"].data_ptr()), sp.hq, V(r["pool"].data_ptr()), st["num_blocks"],
             V(bt.data_ptr()), bt_np.shape[1], V(lens.data_ptr()), V(r["sk"].data_ptr()),
             V(r["sv"].data_ptr()), ctypes.c_float(sm), V(r["out"].data_ptr()),
             V(r["ws"].data_ptr()), max(ws_bytes, 256), sp.batch, V(sptr))))
    fq, fa, fd = lib.kvarn_quantize_tiles, lib.kvarn_append_token, lib.kvarn_decode_attention

    def step(i, ev=None):
        cq, ca, cd = calls[i % reps]
        if ev is not None:
            ev[0].record(stream)
        assert fq(*cq) == 0
        if ev is not None:
            ev[1].record(stream)
        assert fa(*ca) == 0
        if ev is not None:
            ev[2].record(stream)
        assert fd(*cd) == 0
        if ev is not None:
            ev[3].record(stream)

    print(f"# workload {args.workload}: {tile_heads} tile-heads, batch {sp.batch}, "
          f"{reps} replicas, warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tq = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps * 1e-3
    ta = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps * 1e-3
    td = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps * 1e-3
    ms = elapsed / args.steps * 1e3
    print(f"# step {ms:.4f} ms: quantise {tq * 1e6:.1f} us, append {ta * 1e6:.1f} us, "
          f"decode {td * 1e6:.1f} us", file=sys.stderr, flush=True)

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        b_.copy_(a)
        torch.cuda.synchronize()

    fp16 = None
    if not args.no_fp16_decode:
        fp16 = fp16_decode_comparison(args, kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R,
                                      sm, ws_bytes, td, torch, np, dev)

    multi = None
    if not args.no_multi_decode:
        multi = multi_decode_measure(args, kv, lib, cfg, sp, bt, bt_np, lens, lens_np, R, sm, td,
                                     torch, np, dev)

    k4v4 = None
    if not args.no_k4v4:
        k4v4 = k4v4_measure(args, kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R, sm, torch,
                            dev)

    hbm = layer_stream = wstream = None
    if not args.no_extras:
        hbm = hbm_copy_measure(torch)
        layer_stream = layer_stream_measure(kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R,
                                            sm, torch, dev)
        wstream = write_stream_measure(kv, lib, torch, np, dev)

    decode_gbps = d_bytes / td / 1e9
    quant_gbps = q_bytes / tq / 1e9
    timings = {"quantise": tq, "append": ta, "decode": td}
    dominant = max(timings, key=timings.get)
    ach = {"quantise": quant_gbps, "append": a_bytes / ta / 1e9, "decode": decode_gbps}[dominant]
    # HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by what those
    # counters read for a device copy of known size; null once the kernels have changed
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        tr = json.load(open(tpath)).get(args.workload, {}).get(dominant)
        if tr and tr.get("source_digest") == source_digest(dominant):
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": {"quantise": "kvarn_quantize_tiles (quantize_tiles_kernel<2>)",
                           "append": "kvarn_append_token (append_token_kernel<2>)",
                           "decode": "kvarn_decode_attention (decode_tiles_kernel<false, 2> + "
                                     "decode_merge_kernel<true, false>)"}[dominant],
                "algorithmic_bytes_per_launch": {"quantise": q_bytes, "append": a_bytes,
                                                 "decode": d_bytes}[dominant],
                "avg_launch_us": round(timings[dominant] * 1e6, 2)}
    value = step_bytes / (elapsed / args.steps) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the oracle on a bounded sample", file=sys.stderr, flush=True)
        pairs = sp.batch * sp.hkv
        cpu = cpu_baseline(sp, st, q_np, lens_np, sm, tile_heads, pairs, step_bytes)
    line = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + tiles quantised/s, K4V2 g128",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16-in/fp32-acc, u4/u2 codes",
        "data": "synthetic (seeded generators; no model weights)",
        "config": {"workload": args.workload, "batch": sp.batch, "kv_heads": sp.hkv,
                   "q_heads": sp.hq, "context": int(lens_pre.max()),
                   "tile_heads_quantised_per_step": tile_heads, "replicas": reps},
        "decode_attn": {"gbps": round(decode_gbps, 1),
                        "frac_of_peak": round(decode_gbps / HBM_PEAK_GBPS, 4),
                        "us": round(td * 1e6, 2), "algorithmic_bytes": d_bytes},
        "quantise": {"tiles_per_s": round(tile_heads / tq, 1), "gbps": round(quant_gbps, 1),
                     "frac_of_peak": round(quant_gbps / HBM_PEAK_GBPS, 4),
                     "us": round(tq * 1e6, 2), "algorithmic_bytes": q_bytes},
        "append": {"us": round(ta * 1e6, 2), "algorithmic_bytes": a_bytes},
        "fp16_decode": fp16,
        "multi_decode": multi,
        "preset_k4v4": k4v4,
        "hbm_copy": hbm,
        "decode_layer_stream": layer_stream,
        "write_stream": wstream,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
