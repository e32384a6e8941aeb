"""Seeded synthetic KV-cache workloads shaped like the attention layers the KVarN pages discuss.

The pages evaluate on Qwen3-4B, Qwen3-32B (16K context) and Phi-4-14B with reasoning and
retrieval datasets; neither weights nor data are used here. These generators stand in for the
head layouts and context lengths only, with keys and values that have the per-channel outlier
structure the pages describe (tools.thesoundmethod.me, "KVarN: 2-Bit KV-Cache That Beats FP16
Throughput, and Where the Catch Lives", section "Why 2-bit usually breaks": a few channels far
larger than the rest).

Every stream of random numbers is keyed by (seed, purpose[, index]) so that one sequence, one
step or the queries can be regenerated alone, in any order:

  (seed, 0)           per-(KV head, K|V) channel multipliers, then outlier channel picks
  (seed, 1)           per-sequence context lengths (ragged workload)
  (seed, 2)           block permutation
  (seed, 3)           queries
  (seed, 6, i)        queries of the earlier tokens of a several-token query (token i)
  (seed, 7)           fixed orthogonal maps of the autoregressive error probe
  (seed, 8, s)        fresh noise of probe step s
  (seed, 9)           per-channel rotation sign words (optional sign flips)
  (seed, 100 + b)     keys, then values, then per-token drift of sequence b
  (seed, 10**6 + s)   keys then values of append step s

Values are drawn in float32 and rounded to fp16 (the cache's input precision).
"""

from dataclasses import dataclass, field

import numpy as np

T = 128
D = 128


@dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    hkv: int
    hq: int
    batch: int
    ctx: int                      # context of every sequence (fixed-length workloads)
    lognormal: bool               # per-channel log-normal(0, 1) multipliers
    outlier_channels: tuple = ()  # fixed outlier channels (tiny workload)
    outlier_count: int = 0        # seeded outlier picks per (KV head, K|V)
    outlier_gain: float = 1.0
    drift_sigma: float = 0.0      # per-token magnitude drift log-normal(0, sigma)
    shuffle_blocks: bool = False
    ragged: tuple = ()            # (lo, hi) context range, rounded to a multiple of 128
    steps: int = 0                # append steps (write-stream workload)
    extra: dict = field(default_factory=dict)
    head_dim: int = D             # channels per head: 128 (the pages' preset), 64 or 256

    @property
    def group(self) -> int:
        return self.hq // self.hkv


SPECS = {
    # one KV head, one tile, channels {3, 17, 64, 101} x20
    "tiny": Spec("tiny", 1, 1, 1, 1, 128, False, (3, 17, 64, 101), 0, 20.0),
    # Qwen3-4B-like layer: GQA 4, batch 8, 4K context, 2% of channels x15
    "qwen3-4b": Spec("qwen3-4b", 2, 8, 32, 8, 4096, True, (), 3, 15.0),
    # Qwen3-32B-like layer: GQA 8, batch 16, 16K context, drift, shuffled blocks
    "qwen3-32b-16k": Spec("qwen3-32b-16k", 3, 8, 64, 16, 16384, True, (), 3, 15.0, 0.5, True),
    # write stream: batch 64, start at 1024 tokens, 512 append steps
    "write-stream": Spec("write-stream", 4, 8, 32, 64, 1024, True, (), 3, 15.0, steps=512),
    # Phi-4-14B-like ragged batch: GQA 4, 10 KV heads, contexts U[1024, 32768], 1% x20
    "phi4-ragged": Spec("phi4-ragged", 5, 10, 40, 32, 0, True, (), 1, 20.0,
                        shuffle_blocks=True, ragged=(1024, 32768)),
}


def spec(name: str, **overrides) -> Spec:
    """A workload spec by name, optionally with fields overridden (for smaller test cases)."""
    base = SPECS[name]
    if not overrides:
        return base
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(overrides)
    return Spec(**d)


def _rng(sp: Spec, *key) -> np.random.Generator:
    return np.random.default_rng([sp.seed, *key])


def head_params(sp: Spec) -> np.ndarray:
    """Per-(KV head, K|V, channel) multipliers, float32 [Hkv, 2, head_dim]."""
    rng = _rng(sp, 0)
    d = sp.head_dim
    mult = np.ones((sp.hkv, 2, d), np.float32)
    if sp.lognormal:
        mult *= np.exp(rng.standard_normal((sp.hkv, 2, d))).astype(np.float32)
    for h in range(sp.hkv):
        for kv in range(2):
            if sp.outlier_channels:
                picks = np.array(sp.outlier_channels)
            elif sp.outlier_count:
                picks = rng.choice(d, size=sp.outlier_count, replace=False)
            else:
                picks = np.array([], dtype=np.int64)
            mult[h, kv, picks] *= sp.outlier_gain
    return mult


def seq_lens(sp: Spec) -> np.ndarray:
    """Context length of every sequence at prefill (int32 [B])."""
    if sp.ragged:
        lo, hi = sp.ragged
        raw = _rng(sp, 1).uniform(lo, hi, size=sp.batch)
        return (np.rint(raw / T) * T).astype(np.int32)
    return np.full(sp.batch, sp.ctx, np.int32)


def _sequence_kv(sp: Spec, b: int, length: int, mult: np.ndarray):
    rng = _rng(sp, 100 + b)
    k = rng.standard_normal((length, sp.hkv, sp.head_dim), dtype=np.float32) * mult[None, :, 0, :]
    v = rng.standard_normal((length, sp.hkv, sp.head_dim), dtype=np.float32) * mult[None, :, 1, :]
    if sp.drift_sigma:
        k *= np.exp(sp.drift_sigma * rng.standard_normal((length, sp.hkv, 1), dtype=np.float32))
        v *= np.exp(sp.drift_sigma * rng.standard_normal((length, sp.hkv, 1), dtype=np.float32))
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    if not (np.isfinite(k16).all() and np.isfinite(v16).all()):
        raise ValueError("generated values overflow fp16")
    return k16, v16


def _sequence_job(args):
    sp, b, length = args
    return _sequence_kv(sp, b, length, head_params(sp))


def prefill(sp: Spec, max_new_tokens: int = 0, sequences=None, workers: int = 1) -> dict:
    """Prefill state of the workload.

    Returns a dict with
      k, v          fp16 [n_tiles * 128, Hkv, head_dim]: the full tiles of the chosen sequences,
                    concatenated sequence after sequence (what kvarn_quantize_tiles reads)
      dst_blocks    int32 [n_tiles]: destination block of each of those tiles
      tail_k/tail_v list (per chosen sequence) of fp16 [len % 128, Hkv, head_dim] staging tokens
      block_table   int32 [B, max_blocks] (room for max_new_tokens more tokens per sequence)
      seq_lens      int32 [B]
      num_blocks    int
      sequences     the sequence indices included in k/v (default: all).
    workers > 1 draws the sequences in that many forked processes (same values: every
    sequence has its own stream); call it before the process initialises a GPU."""
    lens = seq_lens(sp)
    max_blocks = int(max((int(l) + max_new_tokens + T - 1) // T for l in lens))
    max_blocks = max(max_blocks, 1)
    num_blocks = sp.batch * max_blocks
    ids = np.arange(num_blocks, dtype=np.int32)
    if sp.shuffle_blocks:
        ids = _rng(sp, 2).permutation(num_blocks).astype(np.int32)
    block_table = ids.reshape(sp.batch, max_blocks)
    mult = head_params(sp)
    chosen = range(sp.batch) if sequences is None else list(sequences)
    ks, vs, dst, tk, tv = [], [], [], [], []
    if workers > 1 and len(chosen) > 1:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(min(workers, len(chosen))) as pool:
            drawn = pool.map(_sequence_job, [(sp, b, int(lens[b])) for b in chosen])
    else:
        drawn = [_sequence_kv(sp, b, int(lens[b]), mult) for b in chosen]
    for b, (k, v) in zip(chosen, drawn):
        length = int(lens[b])
        n_full = length // T
        ks.append(k[:n_full * T])
        vs.append(v[:n_full * T])
        dst.append(block_table[b, :n_full])
        tk.append(k[n_full * T:])
        tv.append(v[n_full * T:])
    empty = np.zeros((0, sp.hkv, sp.head_dim), np.float16)
    return dict(k=np.concatenate(ks) if ks else empty, v=np.concatenate(vs) if vs else empty,
                dst_blocks=np.concatenate(dst).astype(np.int32) if dst else np.zeros(0, np.int32),
                tail_k=tk, tail_v=tv, block_table=block_table, seq_lens=lens,
                num_blocks=num_blocks, sequences=list(chosen))


def tiles_by_block(st: dict, hkv: int) -> tuple:
    """The prefill tiles of a prefill() state as block-indexed arrays [num_blocks, Hkv, 128,
    head_dim] fp16 (K and V; blocks that hold no prefill tile are zero): the logical content
    of an unquantised paged cache."""
    kt = np.zeros((st["num_blocks"], hkv, T, st["k"].shape[2]), np.float16)
    vt = np.zeros_like(kt)
    for i, blk in enumerate(st["dst_blocks"]):
        kt[blk] = np.transpose(st["k"][T * i:T * (i + 1)], (1, 0, 2))
        vt[blk] = np.transpose(st["v"][T * i:T * (i + 1)], (1, 0, 2))
    return kt, vt


def query(sp: Spec, dense: bool = False) -> np.ndarray:
    """Decode queries fp16 [B, Hq, head_dim], N(0, 1) (reading R21).

    dense=True scales each query head so that its scores against a typical key have a
    standard deviation near 1 under the default 1/sqrt(head_dim) softmax scale."""
    q = _rng(sp, 3).standard_normal((sp.batch, sp.hq, sp.head_dim), dtype=np.float32)
    if dense:
        mult = head_params(sp)
        key_rms = np.sqrt(np.sum(mult[:, 0, :].astype(np.float64) ** 2, axis=1))  # [Hkv]
        scale = np.sqrt(sp.head_dim) / key_rms
        q *= np.repeat(scale, sp.group)[None, :, None].astype(np.float32)
    return q.astype(np.float16)


def query_tokens(sp: Spec, n_query: int, dense: bool = False) -> np.ndarray:
    """Queries of n_query tokens per sequence, fp16 [B, n_query, Hq, head_dim] (R25): the
    last token's queries are query(sp, dense); the earlier ones are drawn the same way from
    their own stream."""
    q = np.empty((sp.batch, n_query, sp.hq, sp.head_dim), np.float16)
    q[:, -1] = query(sp, dense)
    for i in range(n_query - 1):
        x = _rng(sp, 6, i).standard_normal((sp.batch, sp.hq, sp.head_dim), dtype=np.float32)
        if dense:
            mult = head_params(sp)
            key_rms = np.sqrt(np.sum(mult[:, 0, :].astype(np.float64) ** 2, axis=1))
            x *= np.repeat(np.sqrt(sp.head_dim) / key_rms, sp.group)[None, :, None].astype(np.float32)
        q[:, i] = x.astype(np.float16)
    return q


def feedback_maps(sp: Spec) -> dict:
    """Fixed random orthogonal head_dim x head_dim maps (float32) of the autoregressive error probe: one
    per KV head for keys and for values, one per query head for queries."""
    rng = _rng(sp, 7)

    def orth(n):
        a = rng.standard_normal((n, sp.head_dim, sp.head_dim))
        qm, r = np.linalg.qr(a)
        return (qm * np.sign(np.diagonal(r, axis1=1, axis2=2))[:, None, :]).astype(np.float32)
    return dict(k=orth(sp.hkv), v=orth(sp.hkv), q=orth(sp.hq))


def feedback_noise(sp: Spec, step: int) -> dict:
    """Fresh N(0, 1) noise of probe step `step` (float32): k, v [B, Hkv, head_dim], q [B, Hq,
    head_dim]."""
    rng = _rng(sp, 8, step)
    d = sp.head_dim
    return dict(k=rng.standard_normal((sp.batch, sp.hkv, d), dtype=np.float32),
                v=rng.standard_normal((sp.batch, sp.hkv, d), dtype=np.float32),
                q=rng.standard_normal((sp.batch, sp.hq, d), dtype=np.float32))


def rotation_sign_words(sp: Spec) -> np.ndarray:
    """head_dim / 32 random 32-bit words (uint32): the optional per-channel sign flips before
    the rotation, channel j negated when bit j % 32 of word j // 32 is set (reading R27)."""
    return _rng(sp, 9).integers(0, 2 ** 32, size=sp.head_dim // 32,
                                dtype=np.uint64).astype(np.uint32)


def append_tokens(sp: Spec, step: int):
    """New keys and values of append step `step`: fp16 [B, Hkv, head_dim] each."""
    mult = head_params(sp)
    rng = _rng(sp, 10 ** 6 + step)
    d = sp.head_dim
    k = rng.standard_normal((sp.batch, sp.hkv, d), dtype=np.float32) * mult[None, :, 0, :]
    v = rng.standard_normal((sp.batch, sp.hkv, d), dtype=np.float32) * mult[None, :, 1, :]
    return k.astype(np.float16), v.astype(np.float16)
