"""Exact decode attention over a paged KVarN cache, and the three cache-level operations.

[GR] "The four-stage pipeline", stage 4: the stored scales meet the codes again only inside
attention, at read time; writing a token involves no dequantisation.
[GR] "What KVarN changes in vLLM's serving path": the cache lives in fixed-size paged blocks,
one 128-token tile per block. [GR] stage 1: the rotation is orthonormal and does not change
attention scores, which is what lets the folded form below equal the plain one.

Cache model (the library's, reading R16/R17): a sequence of L tokens holds floor(L/128)
packed tiles at block_table[b][0 .. floor(L/128) - 1] followed by L mod 128 raw fp16 tokens
in its staging tile staging[b][kv_head][0 .. L mod 128 - 1]. Query head h reads KV head
h // (Hq / Hkv) (reading R19). Softmax scale sm_scale (reading R18). Outputs are float64 here
(the library writes fp32, reading R20).

Test infrastructure only (see the package header).
"""

import numpy as np

from . import codec
from .hadamard import H_OF

T = codec.T
D = codec.D   # the pages' head dimension; every function takes D from its arguments


# ------------------------------------------------------------------ cache-level operations


def quantize_tiles(k, v, dst_blocks, pool, iters: int = codec.DEFAULT_ITERS, signs=None):
    """Quantise whole prefill tiles into the block pool, in place.

    k, v: [n_tiles * 128, Hkv, D] fp16 values (D = 64, 128 or 256); tile i holds tokens
    128 i .. 128 i + 127 and goes to block dst_blocks[i]; pool: uint8 [num_blocks, Hkv, record
    bytes] (with D = 128: 13312 for 2-bit values, 17408 for 4-bit; the pool's record size
    selects the preset and must match D)."""
    k = np.asarray(k)
    v = np.asarray(v)
    n_tiles = len(dst_blocks)
    hkv = k.shape[1]
    d, vb = codec.geometry_of_record(pool.shape[-1])
    if k.shape[2] != d or v.shape[2] != d:
        raise ValueError("record size does not match the head dimension")
    for i in range(n_tiles):
        rows = slice(T * i, T * i + T)
        for h in range(hkv):
            pool[dst_blocks[i], h] = codec.encode_record(k[rows, h, :], v[rows, h, :], iters,
                                                         signs, vb)


def append_token(k_new, v_new, positions, block_table, staging_k, staging_v, pool,
                 iters: int = codec.DEFAULT_ITERS, signs=None):
    """Write one new token per sequence into its staging tile; when the token is the 128th of
    its tile, quantise the staging tile into block_table[b][position // 128]. In place.

    k_new, v_new: [B, Hkv, D]; positions: [B] 0-based index of the new token, negative =
    skip this row; staging_k, staging_v: [B, Hkv, 128, D]. The pool's record size selects
    the preset and must match D, as in quantize_tiles()."""
    d, vb = codec.geometry_of_record(pool.shape[-1])
    if staging_k.shape[-1] != d:
        raise ValueError("record size does not match the head dimension")
    for b, pos in enumerate(np.asarray(positions)):
        if pos < 0:
            continue
        slot = int(pos) % T
        staging_k[b, :, slot, :] = k_new[b]
        staging_v[b, :, slot, :] = v_new[b]
        if slot == T - 1:
            blk = block_table[b, int(pos) // T]
            for h in range(staging_k.shape[1]):
                pool[blk, h] = codec.encode_record(staging_k[b, h], staging_v[b, h], iters,
                                                   signs, vb)


def _sequence_kv(pool, block_table, staging_k, staging_v, b, g, length, signs=None):
    """Dequantised keys and values (original space) of sequence b, KV head g, length tokens."""
    n_full = length // T
    ks, vs = [], []
    for i in range(n_full):
        kh, vh = codec.decode_record(pool[block_table[b, i], g], signs)
        ks.append(kh)
        vs.append(vh)
    tail = length % T
    ks.append(np.asarray(staging_k[b, g, :tail], dtype=np.float64))
    vs.append(np.asarray(staging_v[b, g, :tail], dtype=np.float64))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def softmax_attend(q, keys, values, sm_scale):
    """Exact softmax attention of one query vector over keys/values rows (float64)."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1])
    s = sm_scale * (keys @ np.asarray(q, dtype=np.float64))
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


def decode_attention(q, pool, block_table, seq_lens, staging_k, staging_v, sm_scale,
                     signs=None):
    """Plain form: dequantise every packed tile, then exact softmax attention.

    q: [B, Hq, D]; returns [B, Hq, D] float64. A sequence of length 0 gives zeros."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = staging_k.shape[1]
    group = hq // hkv
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        for g in range(hkv):
            keys, values = _sequence_kv(pool, block_table, staging_k, staging_v, b, g,
                                        int(seq_lens[b]), signs)
            for h in range(g * group, (g + 1) * group):
                out[b, h] = softmax_attend(q[b, h], keys, values, sm_scale)
    return out


def decode_attention_multi(q, pool, block_table, seq_lens, staging_k, staging_v, sm_scale,
                           signs=None):
    """Several query tokens per sequence (reading R25): q [B, Q, Hq, D] holds the last Q of
    each sequence's L tokens; query token i sits at position L - Q + i and attends to
    positions 0 .. L - Q + i of the same cache (causal; an empty range gives zeros).
    Returns [B, Q, Hq, D] float64; Q = 1 is decode_attention()."""
    q = np.asarray(q, dtype=np.float64)
    bsz, nq, hq, d = q.shape
    hkv = staging_k.shape[1]
    group = hq // hkv
    out = np.zeros((bsz, nq, hq, d))
    for b in range(bsz):
        length = int(seq_lens[b])
        for g in range(hkv):
            keys, values = _sequence_kv(pool, block_table, staging_k, staging_v, b, g, length,
                                        signs)
            for i in range(nq):
                n_vis = max(0, length - nq + i + 1)
                for h in range(g * group, (g + 1) * group):
                    out[b, i, h] = softmax_attend(q[b, i, h], keys[:n_vis], values[:n_vis],
                                                  sm_scale)
    return out


def decode_attention_folded(q, pool, block_table, seq_lens, staging_k, staging_v, sm_scale,
                            signs=None):
    """Folded form: the per-channel key scales and the rotation go into the query, the
    per-token key scale and zero-point into the score, the per-token value scale and
    zero-point into the probabilities, the per-channel value scale into the per-tile partial
    output, and the rotation back onto the summed output. Must equal decode_attention()."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = staging_k.shape[1]
    group = hq // hkv
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        length = int(seq_lens[b])
        n_full, tail = length // T, length % T
        for g in range(hkv):
            recs = [codec.unpack_record(pool[block_table[b, i], g]) for i in range(n_full)]
            sk = np.asarray(staging_k[b, g, :tail], dtype=np.float64)
            sv = np.asarray(staging_v[b, g, :tail], dtype=np.float64)
            for h in range(g * group, (g + 1) * group):
                if length == 0:
                    continue
                q_rot = (q[b, h] if signs is None else q[b, h] * signs) @ H_OF[d]
                scores = []
                for r in recs:
                    qt = q_rot * r["k"]["c_hat"]
                    scores.append(sm_scale * (r["k"]["s_hat"] * (r["k"]["codes"] @ qt)
                                              + r["k"]["z_hat"] * qt.sum()))
                scores.append(sm_scale * (sk @ q[b, h]))
                s = np.concatenate(scores)
                p = np.exp(s - s.max())
                o_rot = np.zeros(d)
                for i, r in enumerate(recs):
                    pt = p[T * i:T * i + T]
                    o_rot += r["v"]["c_hat"] * ((pt * r["v"]["s_hat"]) @ r["v"]["codes"]
                                                + np.dot(pt, r["v"]["z_hat"]))
                o_back = o_rot @ H_OF[d]
                if signs is not None:
                    o_back = o_back * signs
                o = o_back + p[T * n_full:] @ sv
                out[b, h] = o / p.sum()
    return out


# ------------------------------------------------------------------ fp16 cache (comparison path)


def decode_attention_fp16(q, k_tiles, v_tiles, block_table, seq_lens, staging_k, staging_v,
                          sm_scale):
    """Exact softmax attention over an unquantised paged fp16 cache: the comparison point for
    the packed cache ([GR] "Reported benchmarks and the verification gap" compares KVarN with
    FP16 serving on the same model).

    k_tiles, v_tiles: [num_blocks, Hkv, 128, 128] fp16, logical content of each block (token,
    channel); block_table, seq_lens, staging and q as in decode_attention(). The same cache
    model: floor(L/128) blocks, then L mod 128 staging tokens. Returns [B, Hq, 128] float64."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = staging_k.shape[1]
    group = hq // hkv
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        length = int(seq_lens[b])
        n_full, tail = length // T, length % T
        for g in range(hkv):
            blocks = [block_table[b, i] for i in range(n_full)]
            keys = np.concatenate([np.asarray(k_tiles[blk, g], dtype=np.float64) for blk in blocks]
                                  + [np.asarray(staging_k[b, g, :tail], dtype=np.float64)], axis=0)
            values = np.concatenate([np.asarray(v_tiles[blk, g], dtype=np.float64) for blk in blocks]
                                    + [np.asarray(staging_v[b, g, :tail], dtype=np.float64)], axis=0)
            for h in range(g * group, (g + 1) * group):
                out[b, h] = softmax_attend(q[b, h], keys, values, sm_scale)
    return out

