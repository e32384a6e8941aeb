"""Benchmark of the KVarN K4V2 g128 hot path on one MI355X.

One step = the whole path on one batch: quantise every full prefill tile of the batch into the
paged block pool (kvarn_quantize_tiles), append one new key/value token per sequence into the
fp16 staging tile (kvarn_append_token), and one decode-attention step over the packed tiles plus
the staging token (kvarn_decode_attention). Default workload: the Phi-4-14B-like ragged batch
(10 KV heads, 40 query heads, batch 32, contexts 1K-32K tokens, randomly permuted blocks), the
largest configuration that fits one GPU.

All inputs are resident in HBM before timing starts. Each step uses the next of several
identical input/cache replicas so that the 256 MB last-level (Infinity) cache cannot serve a
step from the previous one. Host-side work that forks processes (drawing the inputs, timing the
oracle on all host cores) runs before the GPU is first touched.

Printed: one JSON line. value = decode-attention effective HBM GB/s (algorithmic bytes of the
decode call / its time by HIP events on the launch stream); beside it tiles quantised per
second, each call's fraction of the 8 TB/s peak, the roofline of the dominant kernel, the same
figures for the Qwen3-32B-like 16K and Qwen3-4B-like workloads, and the fp64 oracle timed on a
bounded sample on one host core and on all of them.
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

WORKLOADS = ("phi4-ragged", "qwen3-32b-16k", "qwen3-4b")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="phi4-ragged", choices=WORKLOADS)
    p.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 1.2 GB")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run one device copy of this many MiB (counter calibration)")
    p.add_argument("--no-fp16-decode", action="store_true",
                   help="skip the comparison decode over an unquantised fp16 cache")
    p.add_argument("--no-multi-decode", action="store_true",
                   help="skip the several-token (Q = 4) decode measurement")
    p.add_argument("--no-k4v4", action="store_true",
                   help="skip the measurement of the 4-bit value preset")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the quantise + decode figures of the other two workloads")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the bandwidth probes, warm-cache, rounds sweep, layer-stream and "
                        "write-stream measurements")
    p.add_argument("--no-head-dims", action="store_true",
                   help="skip the 16K workload at head dimensions 64 and 256")
    p.add_argument("--host-workers", type=int, default=0,
                   help="processes for the host phase (0 = the usable cores, at most 16); use 1 "
                        "under a profiler that initialises the GPU before the program starts")
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


def algorithmic_bytes(lens, hkv, hq, appended, tile_bytes=TILE, head_dim=D):
    """Bytes the method must move (not what an implementation happens to move); tile_bytes is
    the size of one (block, KV head) record: 13,312 packed, 65,536 for the fp16 cache (head
    dimension 128; the record scales with head_dim)."""
    n_full = [int(l) // T for l in lens]
    n_stage = [int(l) % T for l in lens]
    decode = sum(n * hkv * tile_bytes + s * hkv * 2 * head_dim * 2 + 4 * n + 4
                 for n, s in zip(n_full, n_stage))
    decode += len(lens) * hq * head_dim * (2 + 4)                # q in (fp16), out (fp32)
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
    stream = torch.cuda.current_stream()
    keep = []

    def calls(c, pools):
        cp = ctypes.byref(c)
        # each preset's decode has its own split plan, so its own workspace
        ws_bytes = max(kv.decode_workspace_bytes(c, sp.batch, sp.hq, bt_np.shape[1]), 256)
        wss = [torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") for _ in R]
        keep.append(wss)
        qc = [(cp, V(r["k"].data_ptr()), V(r["v"].data_ptr()), r["k"].stride(0), n_tiles,
               V(dst.data_ptr()), V(p.data_ptr()), st["num_blocks"], V(stream.cuda_stream))
              for r, p in zip(R, pools)]
        dc = [(cp, V(r["q"].data_ptr()), sp.hq, V(p.data_ptr()), st["num_blocks"],
               V(bt.data_ptr()), bt_np.shape[1], V(lens.data_ptr()), V(r["sk"].data_ptr()),
               V(r["sv"].data_ptr()), ctypes.c_float(sm), V(r["out"].data_ptr()),
               V(w.data_ptr()), ws_bytes, sp.batch, V(stream.cuda_stream))
              for r, p, w in zip(R, pools, wss)]
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
    # the same steps captured once into a HIP graph and replayed: no launch or event between
    # the kernels. A replay repeats every write with the same values (the appends rewrite the
    # same staging slots and completed records), so each replay is the whole stream again.
    graph_step = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for i in range(steps):
                assert fa(cp, V(kn[i].data_ptr()), V(vn[i].data_ptr()), V(pos[i].data_ptr()),
                          V(bt.data_ptr()), bt_np.shape[1], V(sk.data_ptr()), V(sv.data_ptr()),
                          V(pool.data_ptr()), st["num_blocks"], sp.batch, V(cs.cuda_stream)) == 0
                assert fd(cp, V(q.data_ptr()), sp.hq, V(pool.data_ptr()), st["num_blocks"],
                          V(bt.data_ptr()), bt_np.shape[1], V(lens[i].data_ptr()),
                          V(sk.data_ptr()), V(sv.data_ptr()), ctypes.c_float(1.0 / math.sqrt(D)),
                          V(out.data_ptr()), V(ws.data_ptr()), max(ws_bytes, 256), sp.batch,
                          V(cs.cuda_stream)) == 0
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_step = e0.elapsed_time(e1) * 1e-3 / (reps * steps)
        del g
    except Exception as exc:                     # reported, never fatal for the bench line
        print(f"# write stream: graph capture failed: {exc}", file=sys.stderr, flush=True)
    burst = np.array([int(lens0[0] + i) % T == T - 1 for i in range(steps)])
    dbytes = sum(algorithmic_bytes(lens0 + i + 1, sp.hkv, sp.hq, True) for i in range(steps))
    tile_heads_burst = sp.batch * sp.hkv
    print(f"# write stream: {steps} steps, append {ta.mean() * 1e6:.1f} us "
          f"(bursts {ta[burst].mean() * 1e6:.1f} us), decode {td.mean() * 1e6:.1f} us"
          + (f"; in one HIP graph {graph_step * 1e6:.1f} us per step" if graph_step else ""),
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
            "graph_step_us": round(graph_step * 1e6, 2) if graph_step else None,
            "decode_gbps": round(dbytes / td.sum() / 1e9, 1),
            "decode_frac_of_peak": round(dbytes / td.sum() / 1e9 / HBM_PEAK_GBPS, 4)}


def read_probe_measure(torch, lib_path, n_bytes=4 << 30, repeats=5):
    """Achievable read bandwidth: a streaming read-only kernel (libkvarn_probe.so) over a
    4 GiB buffer at a few grid sizes, median of repeats at each, the best grid reported.
    Context for the fractions of peak, never their denominator."""
    import ctypes
    if not os.path.exists(lib_path):
        return None
    plib = ctypes.CDLL(lib_path)
    plib.kvarn_probe_read.restype = ctypes.c_int
    plib.kvarn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_int,
                                      ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(3)
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    for per_cu in (2, 4, 8, 16):
        wg = cus * per_cu
        call = (buf.data_ptr(), n_bytes, wg, 0x9E3779B9, out.data_ptr(), stream.cuda_stream)
        assert plib.kvarn_probe_read(*call) == 0
        torch.cuda.synchronize()
        ts = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert plib.kvarn_probe_read(*call) == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(ts)[len(ts) // 2]
        if best is None or t < best[0]:
            best = (t, wg)
    del buf
    t, wg = best
    print(f"# read probe {n_bytes / t / 1e9:.0f} GB/s ({wg} workgroups)", file=sys.stderr,
          flush=True)
    return {"read_bytes": n_bytes, "workgroups": wg, "gbps": round(n_bytes / t / 1e9, 1),
            "frac_of_peak": round(n_bytes / t / 1e9 / HBM_PEAK_GBPS, 4)}


def record_probe_measure(torch, lib_path, rec_sizes=(13312, 65536), n_bytes=2 << 30,
                         read_bytes=640 << 20, repeats=9):
    """Achievable read bandwidth in the decode's access pattern: whole tile records (packed and
    fp16) at random places in a 2 GiB buffer, one wave per record stream, two waves per SIMD,
    about 640 MB per launch (the Phi-4-like decode's size). Launches rotate through three
    disjoint record sets, so none finds its records in the 256 MB last-level cache; median of
    the repeats. Context, never a denominator."""
    import ctypes
    import numpy as np
    if not os.path.exists(lib_path):
        return None
    plib = ctypes.CDLL(lib_path)
    plib.kvarn_probe_records.restype = ctypes.c_int
    plib.kvarn_probe_records.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(5)
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    waves = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    res = []
    for rb in rec_sizes:
        nrec = n_bytes // rb
        per_wave = max(1, read_bytes // rb // waves)
        per_set = waves * per_wave
        if 3 * per_set > nrec:
            continue
        perm = np.random.default_rng(11).permutation(nrec)[:3 * per_set].astype(np.int32)
        sets = [torch.from_numpy(perm[k * per_set:(k + 1) * per_set].copy()).cuda()
                for k in range(3)]
        def launch(k):
            assert plib.kvarn_probe_records(buf.data_ptr(), n_bytes, rb, sets[k % 3].data_ptr(),
                                            waves, per_wave, 0x9E3779B9, out.data_ptr(),
                                            stream.cuda_stream) == 0
        for k in range(3):
            launch(k)
        torch.cuda.synchronize()
        ts = []
        for k in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(k)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(ts)[len(ts) // 2]
        nb = per_set * rb
        res.append({"rec_bytes": rb, "waves": waves, "read_bytes": nb,
                    "gbps": round(nb / t / 1e9, 1), "frac_of_peak": round(nb / t / 1e9 / HBM_PEAK_GBPS, 4)})
        print(f"# record probe: {rb}-byte records at random places, {nb / 1e6:.0f} MB: "
              f"{nb / t / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    del buf
    return res


def warm_decode_measure(lib, calls, torch, steps=50):
    """The decode of the main loop launched back to back on ONE replica: its pool may then be
    served partly from the 256 MB last-level cache (context, not the metric)."""
    stream = torch.cuda.current_stream()
    cd = calls[0][2]
    f = lib.kvarn_decode_attention
    for _ in range(5):
        assert f(*cd) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        assert f(*cd) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def quantise_rounds_measure(kv, lib, sp, st, R, torch, rounds=(1, 2, 4, 8), reps=8):
    """The quantiser at several normalisation round counts (the config's sinkhorn_iters) on the
    main workload's prefill: each round is one column step and one row step, so the time is
    linear in the count and its slope is the cost of one round. A reproducible breakdown of
    the write path: what the normalisation costs next to rotation, rounding and packing."""
    import ctypes
    import numpy as np
    V = ctypes.c_void_p
    stream = torch.cuda.current_stream()
    n_tiles = int(st["dst_blocks"].shape[0])
    dst = torch.from_numpy(np.ascontiguousarray(st["dst_blocks"])).cuda()
    out = {}
    for it in rounds:
        cfg = kv.default_config(sp.hkv, sinkhorn_iters=it)
        cl = [(ctypes.byref(cfg), V(r["k"].data_ptr()), V(r["v"].data_ptr()), r["k"].stride(0),
               n_tiles, V(dst.data_ptr()), V(r["pool"].data_ptr()), st["num_blocks"],
               V(stream.cuda_stream)) for r in R]
        for i in range(2):
            assert lib.kvarn_quantize_tiles(*cl[i % len(cl)]) == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            assert lib.kvarn_quantize_tiles(*cl[i % len(cl)]) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        out[it] = e0.elapsed_time(e1) * 1e-3 / reps
    xs = np.array(rounds, float)
    ys = np.array([out[r] for r in rounds])
    slope, icpt = np.polyfit(xs, ys, 1)
    t4 = out.get(4, float(icpt + 4 * slope))
    print("# quantiser by rounds: " + ", ".join(f"{r}: {out[r] * 1e6:.0f} us" for r in rounds),
          file=sys.stderr, flush=True)
    return {"rounds": list(rounds), "us": [round(out[r] * 1e6, 2) for r in rounds],
            "us_per_round": round(slope * 1e6, 2), "us_at_zero_rounds_fit": round(icpt * 1e6, 2),
            "normalisation_share_at_4": round(4 * slope / t4, 4)}


# ------------------------------------------------------------------ the oracle on the host


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _oracle_pairs_job(args):
    """Encode every tile of the given (sequence, KV head) pairs with the oracle, then decode
    each pair's queries over those records; stop starting new pairs after `budget` seconds.
    Returns (tiles encoded, encode seconds, tiles decoded, decode seconds)."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import codec
    pairs, budget = args
    st, q, sm, group = _ORACLE_STATE
    first = np.concatenate([[0], np.cumsum(st["seq_lens"] // T)])
    n_enc = n_dec = 0
    t_enc = t_dec = 0.0
    start = time.perf_counter()
    for b, g in pairs:
        if time.perf_counter() - start > budget:
            break
        n = int(st["seq_lens"][b]) // T
        if n == 0:
            continue
        pool = np.zeros((n, 1, TILE), np.uint8)          # this pair's records, blocks 0..n-1
        t0 = time.perf_counter()
        for i in range(n):
            rows = slice(T * (first[b] + i), T * (first[b] + i) + T)
            pool[i, 0] = codec.encode_record(st["k"][rows, g], st["v"][rows, g])
        t1 = time.perf_counter()
        sk = np.zeros((1, 1, T, D), np.float16)         # one (zero) staging token, as in a step
        lens = np.array([n * T + 1], np.int32)
        oatt.decode_attention(q[b:b + 1, g * group:(g + 1) * group], pool,
                              np.arange(n + 1, dtype=np.int32)[None], lens, sk, sk, sm)
        t2 = time.perf_counter()
        n_enc += n
        n_dec += n
        t_enc += t1 - t0
        t_dec += t2 - t1
    return n_enc, t_enc, n_dec, t_dec


_ORACLE_STATE = None


def cpu_baseline(sp, st, q, sm, d_bytes, tile_heads_total, workers, budget_s=12.0):
    """The fp64 oracle on a time-bounded sample of the same step, on one host core and then on
    `workers` cores at once (one process each, BLAS threads = 1): (sequence, KV head) pairs in
    an order that walks the length mix, every tile of a pair encoded by the oracle and the
    pair's query heads decoded over those records. Per-tile rates are extrapolated to the whole
    step: decode GB/s (the metric's unit) and tile-heads quantised per second."""
    global _ORACLE_STATE
    import multiprocessing as mp
    _ORACLE_STATE = (st, q, sm, sp.group)
    order = [(b, g) for g in range(sp.hkv) for b in range(sp.batch)]
    _oracle_worker_init()
    e1, te1, d1, td1 = _oracle_pairs_job((order, budget_s))
    single = {"value": round(d_bytes / (td1 / d1 * tile_heads_total) / 1e9, 5), "cores": 1,
              "tiles_per_s": round(e1 / te1, 2), "tiles_encoded": e1, "tiles_decoded": d1}
    res = None
    if workers > 1:
        shares = [order[w::workers] for w in range(workers)]
        with mp.get_context("fork").Pool(workers, initializer=_oracle_worker_init) as pool:
            res = pool.map(_oracle_pairs_job, [(sh, budget_s) for sh in shares])
    if res:
        enc_rate = sum(e / t for e, t, _, _ in res if t > 0)
        dec_rate = sum(d / t for _, _, d, t in res if t > 0)
        n_e = sum(r[0] for r in res)
        value = d_bytes / (tile_heads_total / dec_rate) / 1e9
        cores = workers
    else:
        enc_rate, dec_rate, n_e = e1 / te1, d1 / td1, e1
        value, cores = single["value"], 1
    return {"value": round(value, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "tiles_per_s": round(enc_rate, 2),
            "sample": f"(sequence, KV head) pairs of this step, every tile of a pair encoded and "
                      f"its query heads decoded over them: {n_e} tile-heads on {cores} cores at "
                      f"once ({budget_s:.0f} s budget each), per-tile rates summed over the "
                      f"cores and extrapolated to the step's {tile_heads_total} tile-heads",
            "single_core": single}


# ------------------------------------------------------------------ one workload on the GPU


def setup_workload(kv, lib, sp, st, replicas, torch, np, dev):
    """Device replicas of one workload's step (prefill tiles, pools, staging, queries, new
    tokens, outputs, workspaces) and the three calls of each replica's step."""
    import ctypes
    from workloads import gen
    q_np = gen.query(sp)
    k_new_np, v_new_np = gen.append_tokens(sp, 0)
    lens_pre = st["seq_lens"].astype(np.int32)
    bt_np = st["block_table"]
    hd = sp.head_dim
    cfg = kv.default_config(sp.hkv, head_dim=hd)
    tile = kv.tile_bytes(cfg)
    sm = 1.0 / math.sqrt(hd)
    n_tiles = int(st["dst_blocks"].shape[0])
    k0, v0 = dev(st["k"]), dev(st["v"])
    per_replica = k0.numel() * 4 + st["num_blocks"] * sp.hkv * tile
    reps = replicas or max(2, min(16, math.ceil(1.2e9 / per_replica)))
    ws_bytes = kv.decode_workspace_bytes(cfg, sp.batch, sp.hq, bt_np.shape[1])
    R = []
    for _ in range(reps):
        R.append(dict(
            k=k0.clone().view(k0.shape[0], -1), v=v0.clone().view(v0.shape[0], -1),
            pool=torch.zeros(st["num_blocks"], sp.hkv, tile, dtype=torch.uint8, device="cuda"),
            sk=torch.zeros(sp.batch, sp.hkv, T, hd, dtype=torch.float16, device="cuda"),
            sv=torch.zeros(sp.batch, sp.hkv, T, hd, dtype=torch.float16, device="cuda"),
            q=dev(q_np), kn=dev(k_new_np), vn=dev(v_new_np),
            out=torch.empty(sp.batch, sp.hq, hd, dtype=torch.float32, device="cuda"),
            ws=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")))
    del k0, v0
    W = dict(sp=sp, st=st, cfg=cfg, sm=sm, q_np=q_np, lens_pre=lens_pre, bt_np=bt_np,
             lens_np=lens_pre + 1, n_tiles=n_tiles, reps=reps, ws_bytes=ws_bytes, R=R,
             dst=dev(st["dst_blocks"]), bt=dev(bt_np), pos=dev(lens_pre),
             lens=dev(lens_pre + 1))
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    cfgp = ctypes.byref(cfg)
    Vp = ctypes.c_void_p
    calls = []
    for r in R:
        calls.append((
            (cfgp, Vp(r["k"].data_ptr()), Vp(r["v"].data_ptr()), r["k"].stride(0), n_tiles,
             Vp(W["dst"].data_ptr()), Vp(r["pool"].data_ptr()), st["num_blocks"], Vp(sptr)),
            (cfgp, Vp(r["kn"].data_ptr()), Vp(r["vn"].data_ptr()), Vp(W["pos"].data_ptr()),
             Vp(W["bt"].data_ptr()), bt_np.shape[1], Vp(r["sk"].data_ptr()),
             Vp(r["sv"].data_ptr()), Vp(r["pool"].data_ptr()), st["num_blocks"], sp.batch,
             Vp(sptr)),
            (cfgp, Vp(r["q"].data_ptr()), sp.hq, Vp(r["pool"].data_ptr()), st["num_blocks"],
             Vp(W["bt"].data_ptr()), bt_np.shape[1], Vp(W["lens"].data_ptr()),
             Vp(r["sk"].data_ptr()), Vp(r["sv"].data_ptr()), ctypes.c_float(sm),
             Vp(r["out"].data_ptr()), Vp(r["ws"].data_ptr()), max(ws_bytes, 256), sp.batch,
             Vp(sptr))))
    W["calls"] = calls
    tile_heads = n_tiles * sp.hkv
    W["tile_heads"] = tile_heads
    W["q_bytes"] = tile_heads * (2 * T * hd * 2 + tile)
    W["a_bytes"] = sp.batch * sp.hkv * 4 * hd * 2
    W["d_bytes"] = algorithmic_bytes(W["lens_np"], sp.hkv, sp.hq, True, tile, hd)
    W["tile_bytes"] = tile
    return W


def time_steps(lib, W, steps, warmup, torch, label):
    """Warm-up steps, then `steps` timed steps (quantise, append, decode on the next replica);
    HIP events on the launch stream around each call, the wall clock around the whole loop."""
    stream = torch.cuda.current_stream()
    fq, fa, fd = lib.kvarn_quantize_tiles, lib.kvarn_append_token, lib.kvarn_decode_attention
    calls, reps = W["calls"], W["reps"]

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

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tq = sum(e[0].elapsed_time(e[1]) for e in evs) / steps * 1e-3
    ta = sum(e[1].elapsed_time(e[2]) for e in evs) / steps * 1e-3
    td = sum(e[2].elapsed_time(e[3]) for e in evs) / steps * 1e-3
    print(f"# {label}: step {elapsed / steps * 1e3:.4f} ms: quantise {tq * 1e6:.1f} us, append "
          f"{ta * 1e6:.1f} us, decode {td * 1e6:.1f} us", file=sys.stderr, flush=True)
    return dict(tq=tq, ta=ta, td=td, elapsed=elapsed, steps=steps)


def summary(W, tm):
    sp = W["sp"]
    dg = W["d_bytes"] / tm["td"] / 1e9
    qg = W["q_bytes"] / tm["tq"] / 1e9
    return {"batch": sp.batch, "kv_heads": sp.hkv, "q_heads": sp.hq, "head_dim": sp.head_dim,
            "tile_bytes": W["tile_bytes"], "context_max": int(W["lens_pre"].max()),
            "decode_attn": {"gbps": round(dg, 1), "frac_of_peak": round(dg / HBM_PEAK_GBPS, 4),
                            "us": round(tm["td"] * 1e6, 2), "algorithmic_bytes": W["d_bytes"]},
            "quantise": {"tiles_per_s": round(W["tile_heads"] / tm["tq"], 1),
                         "gbps": round(qg, 1), "frac_of_peak": round(qg / HBM_PEAK_GBPS, 4),
                         "us": round(tm["tq"] * 1e6, 2), "algorithmic_bytes": W["q_bytes"],
                         "tile_heads": W["tile_heads"]},
            "append": {"us": round(tm["ta"] * 1e6, 2), "algorithmic_bytes": W["a_bytes"]},
            "replicas": W["reps"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path is not built for "
              "more than one GPU", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import decode_attention_tok_amd as kv
    from decode_attention_tok_amd import build as kbuild
    from workloads import gen

    assert torch.cuda.device_count() >= 1, "bench.py needs a GPU"   # does not initialise it
    workers = args.host_workers or max(1, min(16, len(os.sched_getaffinity(0))))

    # ---- host phase (forks processes; the GPU is not initialised yet)
    sp = gen.spec(args.workload)
    t0 = time.perf_counter()
    st = gen.prefill(sp, max_new_tokens=1, workers=workers)
    others = {}
    if not args.no_other_workloads:
        for name in WORKLOADS:
            if name != args.workload:
                osp = gen.spec(name)
                others[name] = (osp, gen.prefill(osp, max_new_tokens=1, workers=workers))
    heads = {}
    if not args.no_head_dims:
        # the 16K GQA-8 workload at head dimensions 64 and 256 (reading R29)
        for hd in (64, 256):
            hsp = gen.spec("qwen3-32b-16k", head_dim=hd)
            heads[hd] = (hsp, gen.prefill(hsp, max_new_tokens=1, workers=workers))
    print(f"# inputs drawn in {time.perf_counter() - t0:.1f} s on {workers} host cores",
          file=sys.stderr, flush=True)
    lens_np = st["seq_lens"].astype(np.int32) + 1
    d_bytes = algorithmic_bytes(lens_np, sp.hkv, sp.hq, True)
    tile_heads = int(st["dst_blocks"].shape[0]) * sp.hkv
    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(sp, st, gen.query(sp), 1.0 / math.sqrt(D), d_bytes, tile_heads,
                           workers)

    # ---- GPU phase
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    lib = kv.lib()
    W = setup_workload(kv, lib, sp, st, args.replicas, torch, np, dev)
    print(f"# workload {args.workload}: {W['tile_heads']} tile-heads, batch {sp.batch}, "
          f"{W['reps']} replicas, warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    tm = time_steps(lib, W, args.steps, args.warmup, torch, args.workload)
    tq, ta, td = tm["tq"], tm["ta"], tm["td"]
    ms = tm["elapsed"] / args.steps * 1e3
    main_sum = summary(W, tm)

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        b_.copy_(a)
        torch.cuda.synchronize()
        del a, b_

    cfg, bt, bt_np, lens, R, sm = W["cfg"], W["bt"], W["bt_np"], W["lens"], W["R"], W["sm"]
    fp16 = multi = k4v4 = None
    if not args.no_fp16_decode:
        fp16 = fp16_decode_comparison(args, kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R,
                                      sm, W["ws_bytes"], td, torch, np, dev)
    if not args.no_multi_decode:
        multi = multi_decode_measure(args, kv, lib, cfg, sp, bt, bt_np, lens, lens_np, R, sm, td,
                                     torch, np, dev)
    if not args.no_k4v4:
        k4v4 = k4v4_measure(args, kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R, sm, torch,
                            dev)

    hbm = rprobe = recprobe = warm = rounds = layer_stream = wstream = None
    if not args.no_extras:
        hbm = hbm_copy_measure(torch)
        rprobe = read_probe_measure(torch, kbuild.PROBE_LIB)
        recprobe = record_probe_measure(torch, kbuild.PROBE_LIB)
        tw = warm_decode_measure(lib, W["calls"], torch)
        warm = {"us": round(tw * 1e6, 2), "gbps": round(d_bytes / tw / 1e9, 1),
                "pool_bytes": st["num_blocks"] * sp.hkv * TILE}
        rounds = quantise_rounds_measure(kv, lib, sp, st, R, torch)
        layer_stream = layer_stream_measure(kv, lib, cfg, sp, st, bt, bt_np, lens, lens_np, R,
                                            sm, torch, dev)
        wstream = write_stream_measure(kv, lib, torch, np, dev)
    del W, R

    other_res = {}
    for name, (osp, ost) in others.items():
        OW = setup_workload(kv, lib, osp, ost, 0, torch, np, dev)
        otm = time_steps(lib, OW, max(10, args.steps // 2), max(2, args.warmup), torch, name)
        other_res[name] = summary(OW, otm)
        del OW
        torch.cuda.empty_cache()
    head_res = {}
    for hd, (hsp, hst) in heads.items():
        HW = setup_workload(kv, lib, hsp, hst, 0, torch, np, dev)
        htm = time_steps(lib, HW, max(10, args.steps // 2), max(2, args.warmup), torch,
                         f"qwen3-32b-16k head_dim {hd}")
        head_res[str(hd)] = summary(HW, htm)
        del HW
        torch.cuda.empty_cache()

    timings = {"quantise": tq, "append": ta, "decode": td}
    dominant = max(timings, key=timings.get)
    byts = {"quantise": main_sum["quantise"]["algorithmic_bytes"],
            "append": main_sum["append"]["algorithmic_bytes"], "decode": d_bytes}
    ach = byts[dominant] / timings[dominant] / 1e9
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
                "kernel": {"quantise": "kvarn_quantize_tiles (quantize_tiles_kernel<2, 128>)",
                           "append": "kvarn_append_token (append_token_kernel<2, 128>)",
                           "decode": "kvarn_decode_attention (decode_pairs_kernel<false, 2> on "
                                     "large tables with at most 4 query heads per KV head, else "
                                     "decode_tiles_kernel<false, 2, 128, list schedule on large "
                                     "tables>; then decode_merge_kernel<true, false, 128>)"}[dominant],
                "algorithmic_bytes_per_launch": byts[dominant],
                "avg_launch_us": round(timings[dominant] * 1e6, 2)}
    decode_gbps = d_bytes / td / 1e9
    line = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + tiles quantised/s, K4V2 g128",
        "value": round(decode_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16-in/fp32-acc, u4/u2 codes",
        "data": "synthetic (seeded generators; no model weights)",
        "config": {"workload": args.workload, "batch": sp.batch, "kv_heads": sp.hkv,
                   "q_heads": sp.hq, "context_max": int(W_lens_max(st)),
                   "tile_heads_quantised_per_step": tile_heads, "replicas": main_sum["replicas"]},
        "decode_attn": main_sum["decode_attn"],
        "quantise": main_sum["quantise"],
        "append": main_sum["append"],
        "workloads": other_res or None,
        "head_dims": head_res or None,
        "fp16_decode": fp16,
        "multi_decode": multi,
        "preset_k4v4": k4v4,
        "hbm_copy": hbm,
        "hbm_read_probe": rprobe,
        "hbm_record_probe": recprobe,
        "decode_warm": warm,
        "quantise_rounds": rounds,
        "decode_layer_stream": layer_stream,
        "write_stream": wstream,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)


def W_lens_max(st):
    return max(int(x) for x in st["seq_lens"])


if __name__ == "__main__":
    main()
