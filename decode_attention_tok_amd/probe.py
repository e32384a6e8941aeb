"""Synthetic error-accumulation probe of the packed cache.

The pages' central diagnostic ([GR] "Why KV-cache quantization degrades under autoregressive
decoding"): per-token quantisation errors are skewed, the largest 5% of them carry most of the
end-to-end loss, and in autoregressive decoding they compound because each generated token
feeds the next ([TSM] "Why 2-bit usually breaks"). Without a model, two measurements stand in:

1. per_token_errors(): the library quantises a workload's tiles (for a few normalisation round
   counts) and writes them back out with kvarn_dequantize_tiles; for every token row, the
   relative squared error ||x_t - x^_t||^2 / ||x_t||^2, its distribution, and the share of the
   total squared error held by the largest 5% of rows.
2. autoregressive(): a synthetic loop in which each step's attention output feeds the next
   token's key, value and query through fixed orthogonal maps mixed with fresh noise.
   Queries are at the "dense" scale (scores of standard deviation near 1). Trajectory Q runs
   on the packed cache (kvarn_append_token, kvarn_decode_attention);
   trajectory R is exact fp32 attention over its own unquantised tokens. Per step: the
   one-step error (the packed cache's output over R's own tokens, against R) and the
   divergence of Q from R; divergence above the one-step error is what compounding adds.

Everything on the cache runs through the library's C ABI; torch holds device memory and
computes the reference trajectory's exact attention and the feedback maps (both outside the
path). Both measurements run for each value width asked for (2: kvarn_k4v2_g128, 4:
kvarn_k4v4_g128). Usage: python -m decode_attention_tok_amd.probe [--steps N] [--v-bits 2,4]
[--out FILE]
"""

import argparse
import json
import math

import numpy as np

T = D = 128


def top_share(err_sq, frac=0.05):
    """Share of sum(err_sq) held by the largest ceil(frac * n) entries."""
    e = np.sort(np.asarray(err_sq, np.float64).ravel())[::-1]
    if e.size == 0 or e.sum() == 0:
        return 0.0
    k = max(1, int(math.ceil(frac * e.size)))
    return float(e[:k].sum() / e.sum())


def summarise(rel):
    """Percentiles of relative per-row errors and the top-5% share of their sum."""
    rel = np.asarray(rel, np.float64).ravel()
    p = np.percentile(rel, [50, 90, 95, 99, 100])
    return {"rows": int(rel.size), "p50": float(p[0]), "p90": float(p[1]), "p95": float(p[2]),
            "p99": float(p[3]), "max": float(p[4]), "mean": float(rel.mean()),
            "top5_share": top_share(rel)}


def per_token_errors(name="qwen3-4b", iters=(1, 4, 8), v_bits=2, **over):
    """Relative squared dequantisation error of every token row of a workload's tiles."""
    import torch
    import decode_attention_tok_amd as kv
    from workloads import gen
    sp = gen.spec(name, **over)
    st = gen.prefill(sp)
    k = torch.from_numpy(st["k"]).cuda()
    v = torch.from_numpy(st["v"]).cuda()
    dst = torch.from_numpy(st["dst_blocks"]).cuda()
    n = dst.numel()
    out = {}
    for it in iters:
        cfg = kv.default_config(sp.hkv, sinkhorn_iters=it, v_bits=v_bits)
        pool = torch.zeros(st["num_blocks"], sp.hkv, kv.tile_bytes(cfg), dtype=torch.uint8,
                           device="cuda")
        kv.quantize_tiles(cfg, k.view(n * T, -1), v.view(n * T, -1), dst, pool)
        ko = torch.empty(n * T, sp.hkv, D, dtype=torch.float32, device="cuda")
        vo = torch.empty_like(ko)
        kv.dequantize_tiles(cfg, pool, dst, ko, vo)
        res = {}
        for half, x, xh in (("k", k, ko), ("v", v, vo)):
            xf = x.float()
            rel = ((xf - xh) ** 2).sum(-1) / (xf ** 2).sum(-1).clamp_min(1e-30)
            res[half] = summarise(rel.cpu().numpy())
        out[f"iters={it}"] = res
    return out


def autoregressive(name="qwen3-4b", steps=512, alpha=0.5, v_bits=2, **over):
    """The synthetic autoregressive loop (see the module notes); returns per-step series and
    the dequantisation-error summary of the tiles completed during the loop."""
    import torch
    import decode_attention_tok_amd as kv
    from workloads import gen
    sp = gen.spec(name, **over)
    st = gen.prefill(sp, max_new_tokens=steps)
    cfg = kv.default_config(sp.hkv, v_bits=v_bits)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B, G, Hkv = sp.batch, sp.group, sp.hkv
    ctx = int(st["seq_lens"][0])
    assert np.all(st["seq_lens"] == ctx) and ctx % T == 0, "fixed-length, whole-tile prefill"
    beta = math.sqrt(1.0 - alpha * alpha)
    mult_np = gen.head_params(sp)
    mult = dev(mult_np)                                           # [Hkv, 2, 128]
    # queries at the "dense" scale (reading R21): scores of standard deviation near 1, so the
    # attention spreads over many tokens instead of picking one
    key_rms = np.sqrt(np.sum(mult_np[:, 0, :].astype(np.float64) ** 2, axis=1))
    qscale = dev(np.repeat(np.sqrt(D) / key_rms, sp.group).astype(np.float32))[None, :, None]
    maps = {key: dev(m) for key, m in gen.feedback_maps(sp).items()}
    sm = 1.0 / math.sqrt(D)
    n = len(st["dst_blocks"])
    kpre, vpre = dev(st["k"]), dev(st["v"])
    bt = dev(st["block_table"])

    def packed_cache():
        pool = torch.zeros(st["num_blocks"], Hkv, kv.tile_bytes(cfg), dtype=torch.uint8,
                           device="cuda")
        if n:
            kv.quantize_tiles(cfg, kpre.view(n * T, -1), vpre.view(n * T, -1),
                              dev(st["dst_blocks"]), pool)
        sk = torch.zeros(B, Hkv, T, D, dtype=torch.float16, device="cuda")
        return dict(pool=pool, sk=sk, sv=torch.zeros_like(sk))

    cq, cqr = packed_cache(), packed_cache()        # Q's own cache; R's tokens, packed
    Lmax = ctx + steps
    kr = torch.zeros(B, Hkv, Lmax, D, dtype=torch.float16, device="cuda")
    vr = torch.zeros_like(kr)
    for b in range(B):                               # prefill, sequence by sequence
        rows = slice(b * ctx, (b + 1) * ctx)
        kr[b, :, :ctx] = kpre[rows].permute(1, 0, 2)
        vr[b, :, :ctx] = vpre[rows].permute(1, 0, 2)
    ws = torch.empty(max(kv.decode_workspace_bytes(cfg, B, sp.hq, st["block_table"].shape[1]),
                         256), dtype=torch.uint8, device="cuda")

    def packed_decode(cache, q16, length):
        out = torch.empty(B, sp.hq, D, dtype=torch.float32, device="cuda")
        lens = torch.full((B,), length, dtype=torch.int32, device="cuda")
        kv.decode_attention(cfg, q16, cache["pool"], bt, lens, cache["sk"], cache["sv"], sm,
                            out, ws)
        return out

    def exact(q32, length):
        qg = q32.view(B, Hkv, G, D)
        kk = kr[:, :, :length].float()
        s = torch.matmul(qg, kk.transpose(-1, -2).contiguous()) * sm
        p = torch.softmax(s, dim=-1)
        return torch.matmul(p, vr[:, :, :length].float()).view(B, sp.hq, D)

    def unit_rms(x):
        return x / x.pow(2).mean(-1, keepdim=True).sqrt().clamp_min(1e-30)

    def next_token(o, noise):
        """Keys, values (fp16 [B, Hkv, 128]) and queries (fp16 [B, Hq, 128]) fed by output o."""
        u = unit_rms(o.view(B, Hkv, G, D).mean(2))                       # [B, Hkv, 128]
        rot = lambda m, x: torch.matmul(m[None], x[..., None]).squeeze(-1)   # per-head map
        k = mult[None, :, 0] * (alpha * rot(maps["k"], u) + beta * noise["k"])
        v = mult[None, :, 1] * (alpha * rot(maps["v"], u) + beta * noise["v"])
        q = (alpha * rot(maps["q"], unit_rms(o)) + beta * noise["q"]) * qscale
        return k.half(), v.half(), q.half()

    def rel(a, b_):
        return ((a - b_).norm(dim=-1) / b_.norm(dim=-1).clamp_min(1e-30)).mean().item()

    q_q = q_r = dev(gen.query(sp, dense=True))
    one_step, diverge = [], []
    for t in range(steps):
        L = ctx + t
        o_q = packed_decode(cq, q_q, L)
        o_r = exact(q_r.float(), L)
        o_qr = packed_decode(cqr, q_r, L)
        one_step.append(rel(o_qr, o_r))
        diverge.append(rel(o_q, o_r))
        noise = {key: dev(x) for key, x in gen.feedback_noise(sp, t).items()}
        kq, vq, q_q = next_token(o_q, noise)
        kr_new, vr_new, q_r = next_token(o_r, noise)
        pos = torch.full((B,), L, dtype=torch.int32, device="cuda")
        kv.append_token(cfg, kq, vq, pos, bt, cq["sk"], cq["sv"], cq["pool"])
        kv.append_token(cfg, kr_new, vr_new, pos, bt, cqr["sk"], cqr["sv"], cqr["pool"])
        kr[:, :, L] = kr_new
        vr[:, :, L] = vr_new
    torch.cuda.synchronize()
    # dequantisation error of the tiles completed during the loop (R's tokens, packed)
    done = (ctx + steps) // T - ctx // T
    tiles = {}
    if done > 0:
        ids = st["block_table"][:, ctx // T:ctx // T + done].reshape(-1)
        ko = torch.empty(len(ids) * T, Hkv, D, dtype=torch.float32, device="cuda")
        vo = torch.empty_like(ko)
        kv.dequantize_tiles(cfg, cqr["pool"], dev(ids.astype(np.int32)), ko, vo)
        for half, hist, xh in (("k", kr, ko), ("v", vr, vo)):
            x = hist[:, :, ctx:ctx + done * T].float()                  # [B, Hkv, done*T, D]
            x = x.view(B, Hkv, done, T, D).permute(0, 2, 3, 1, 4).reshape(-1, Hkv, D)
            r = ((x - xh) ** 2).sum(-1) / (x ** 2).sum(-1).clamp_min(1e-30)
            tiles[half] = summarise(r.cpu().numpy())
    marks = [t for t in (0, 1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048) if t < steps]
    return {"workload": name, "batch": B, "kv_heads": Hkv, "q_heads": sp.hq, "prefill": ctx,
            "steps": steps, "alpha": alpha, "v_bits": v_bits,
            "one_step_rel_err": {"mean": float(np.mean(one_step)),
                                 "p95": float(np.percentile(one_step, 95)),
                                 "max": float(np.max(one_step))},
            "divergence_at_step": {str(t): diverge[t] for t in marks},
            "one_step_at_step": {str(t): one_step[t] for t in marks},
            "tiles_written_in_loop": tiles}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--ctx", type=int, default=1024)
    ap.add_argument("--alpha", type=float, default=0.5)
    ap.add_argument("--v-bits", default="2", help="comma-separated value widths, e.g. 2,4")
    ap.add_argument("--out", default="")
    a = ap.parse_args()
    res = {}
    for vb in (int(x) for x in a.v_bits.split(",")):
        res[f"v_bits={vb}"] = {
            "per_token_dequant_error": per_token_errors("qwen3-4b", v_bits=vb, batch=2, ctx=1024),
            "autoregressive": autoregressive("qwen3-4b", steps=a.steps, alpha=a.alpha, v_bits=vb,
                                             batch=a.batch, ctx=a.ctx)}
    text = json.dumps(res, indent=1)
    print(text)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
