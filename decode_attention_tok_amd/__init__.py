"""Python binding of libkvarn (the KVarN K4V2 g128 codec, a K4V4 variant, and paged decode
attention on MI355X). Argument marshalling only: every step runs in the HIP kernels of libkvarn.so.

The entry points carry the C names of include/kvarn.h without the ``kvarn_`` prefix and take
torch tensors (device memory) plus plain integers; torch is used only to own device memory and
to supply the current stream. There is no fallback: if libkvarn.so is missing the import of a
function raises, and a non-OK status raises KvarnError.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvarn.so")

TILE_TOKENS = 128
HEAD_DIM = 128            # the preset's head dimension; 64 and 256 are accepted too
HEAD_DIMS = (64, 128, 256)
SIGN_WORDS = 8
TILE_BYTES = 13312        # record of the default preset kvarn_k4v2_g128
TILE_BYTES_V4 = 17408     # record with 4-bit values (kvarn_k4v4_g128)

STATUS = {0: "OK", 1: "ERR_NULL_ARG", 2: "ERR_BAD_SHAPE", 3: "ERR_UNSUPPORTED",
          4: "ERR_WORKSPACE", 5: "ERR_HIP", 6: "ERR_SCRATCH_LIMIT"}


class KvarnError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({text})")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("k_bits", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32),
                ("rotation_signs", ctypes.c_uint32 * SIGN_WORDS)]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_CFG = ctypes.POINTER(Config)

_SIGNATURES = {
    "kvarn_default_config": (None, [_CFG, _I32]),
    "kvarn_tile_bytes": (ctypes.c_size_t, [_CFG]),
    "kvarn_block_bytes": (ctypes.c_size_t, [_CFG]),
    "kvarn_quantize_tiles": (ctypes.c_int, [_CFG, _P, _P, _I64, _I32, _P, _P, _I64, _P]),
    "kvarn_append_token": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _I32,
                                          _P]),
    "kvarn_decode_workspace_bytes": (ctypes.c_int, [_CFG, _I32, _I32, _I32,
                                                    ctypes.POINTER(ctypes.c_size_t)]),
    "kvarn_decode_attention": (ctypes.c_int, [_CFG, _P, _I32, _P, _I64, _P, _I32, _P, _P, _P,
                                              ctypes.c_float, _P, _P, ctypes.c_size_t, _I32,
                                              _P]),
    "kvarn_decode_attention_noalloc": (ctypes.c_int, [_CFG, _P, _I32, _P, _I64, _P, _I32, _P,
                                                      _P, _P, ctypes.c_float, _P, _I32, _P]),
    "kvarn_decode_multi_workspace_bytes": (ctypes.c_int, [_CFG, _I32, _I32, _I32, _I32,
                                                          ctypes.POINTER(ctypes.c_size_t)]),
    "kvarn_decode_attention_multi": (ctypes.c_int, [_CFG, _P, _I32, _I32, _P, _I64, _P, _I32, _P,
                                                    _P, _P, ctypes.c_float, _P, _P,
                                                    ctypes.c_size_t, _I32, _P]),
    "kvarn_dequantize_tiles": (ctypes.c_int, [_CFG, _P, _I64, _P, _I32, _P, _P, _P]),
    "kvarn_fp16_block_bytes": (ctypes.c_size_t, [_CFG]),
    "kvarn_fp16_write_tiles": (ctypes.c_int, [_CFG, _P, _P, _I64, _I32, _P, _P, _I64, _P]),
    "kvarn_decode_attention_fp16": (ctypes.c_int, [_CFG, _P, _I32, _P, _I64, _P, _I32, _P, _P,
                                                   _P, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                                   _I32, _P]),
    "kvarn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvarn_abi_version": (ctypes.c_int32, []),
}

EXPORTS = tuple(_SIGNATURES)


def lib():
    """The loaded libkvarn.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with decode_attention_tok_amd/build.py "
                          "(or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn, code):
    if code != 0:
        raise KvarnError(fn, code, lib().kvarn_status_string(code).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def default_config(num_kv_heads: int, sinkhorn_iters: int = 4, rotation_signs=None,
                   v_bits: int = 2, head_dim: int = HEAD_DIM) -> Config:
    """The preset for num_kv_heads heads; rotation_signs: optional head_dim / 32 32-bit words
    of per-channel sign flips before the rotation (None: the plain Hadamard); v_bits 2
    (kvarn_k4v2_g128) or 4 (kvarn_k4v4_g128); head_dim 64, 128 or 256."""
    cfg = Config()
    lib().kvarn_default_config(ctypes.byref(cfg), num_kv_heads)
    cfg.sinkhorn_iters = sinkhorn_iters
    cfg.v_bits = v_bits
    cfg.head_dim = head_dim
    if rotation_signs is not None:
        words = list(rotation_signs)
        if len(words) > SIGN_WORDS:
            raise ValueError("at most 8 sign words")
        for i, w in enumerate(words):
            cfg.rotation_signs[i] = int(w) & 0xFFFFFFFF
    return cfg


def tile_bytes(cfg: Config) -> int:
    return lib().kvarn_tile_bytes(ctypes.byref(cfg))


def block_bytes(cfg: Config) -> int:
    return lib().kvarn_block_bytes(ctypes.byref(cfg))


def abi_version() -> int:
    return lib().kvarn_abi_version()


def decode_workspace_bytes(cfg: Config, batch: int, num_q_heads: int,
                           max_blocks_per_seq: int) -> int:
    out = ctypes.c_size_t(0)
    _check("kvarn_decode_workspace_bytes",
           lib().kvarn_decode_workspace_bytes(ctypes.byref(cfg), batch, num_q_heads,
                                              max_blocks_per_seq, ctypes.byref(out)))
    return out.value


def quantize_tiles(cfg: Config, k, v, dst_blocks, block_pool, token_stride=None, stream=None):
    """k, v: fp16 [n_tiles*128, ...] with stride(0) = token_stride; dst_blocks int32 [n_tiles];
    block_pool uint8 [num_blocks, Hkv, tile_bytes(cfg)] (or any tensor of num_blocks blocks)."""
    n_tiles = dst_blocks.numel()
    stride = k.stride(0) if token_stride is None else token_stride
    num_blocks = block_pool.numel() // block_bytes(cfg)
    _check("kvarn_quantize_tiles",
           lib().kvarn_quantize_tiles(ctypes.byref(cfg), _ptr(k), _ptr(v), stride, n_tiles,
                                      _ptr(dst_blocks), _ptr(block_pool), num_blocks,
                                      _stream(stream)))


def append_token(cfg: Config, k_new, v_new, positions, block_table, staging_k, staging_v,
                 block_pool, stream=None):
    """k_new, v_new fp16 [B, Hkv, D]; positions int32 [B]; block_table int32 [B, max_blocks];
    staging_k/v fp16 [B, Hkv, 128, D]; block_pool uint8 blocks (D = cfg.head_dim)."""
    batch, max_blocks = block_table.shape
    num_blocks = block_pool.numel() // block_bytes(cfg)
    _check("kvarn_append_token",
           lib().kvarn_append_token(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(positions),
                                    _ptr(block_table), max_blocks, _ptr(staging_k),
                                    _ptr(staging_v), _ptr(block_pool), num_blocks, batch,
                                    _stream(stream)))


def decode_attention(cfg: Config, q, block_pool, block_table, seq_lens, staging_k, staging_v,
                     sm_scale, out, workspace, stream=None):
    """q fp16 [B, Hq, D]; out fp32 [B, Hq, D]; workspace: a device tensor of at least
    decode_workspace_bytes(...) bytes."""
    batch, hq, _ = q.shape
    max_blocks = block_table.shape[1]
    num_blocks = block_pool.numel() // block_bytes(cfg)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("kvarn_decode_attention",
           lib().kvarn_decode_attention(ctypes.byref(cfg), _ptr(q), hq, _ptr(block_pool),
                                        num_blocks, _ptr(block_table), max_blocks,
                                        _ptr(seq_lens), _ptr(staging_k), _ptr(staging_v),
                                        float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes,
                                        batch, _stream(stream)))


STATIC_SCRATCH_BYTES = 16 << 20


def decode_attention_noalloc(cfg: Config, q, block_pool, block_table, seq_lens, staging_k,
                             staging_v, sm_scale, out, stream=None):
    """decode_attention() with the library's static per-device scratch instead of a workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    batch, hq, _ = q.shape
    max_blocks = block_table.shape[1]
    num_blocks = block_pool.numel() // block_bytes(cfg)
    _check("kvarn_decode_attention_noalloc",
           lib().kvarn_decode_attention_noalloc(ctypes.byref(cfg), _ptr(q), hq, _ptr(block_pool),
                                                num_blocks, _ptr(block_table), max_blocks,
                                                _ptr(seq_lens), _ptr(staging_k),
                                                _ptr(staging_v), float(sm_scale), _ptr(out),
                                                batch, _stream(stream)))


def dequantize_tiles(cfg: Config, block_pool, src_blocks, k_out, v_out, stream=None):
    """Records of blocks src_blocks (int32 [n_tiles]) back to fp32 tiles in the original
    space: k_out, v_out fp32 [n_tiles * 128, Hkv, D]."""
    num_blocks = block_pool.numel() // block_bytes(cfg)
    _check("kvarn_dequantize_tiles",
           lib().kvarn_dequantize_tiles(ctypes.byref(cfg), _ptr(block_pool), num_blocks,
                                        _ptr(src_blocks), src_blocks.numel(), _ptr(k_out),
                                        _ptr(v_out), _stream(stream)))


MAX_QUERY_TOKENS = 16


def decode_multi_workspace_bytes(cfg: Config, batch: int, num_q_heads: int, n_query: int,
                                 max_blocks_per_seq: int) -> int:
    out = ctypes.c_size_t(0)
    _check("kvarn_decode_multi_workspace_bytes",
           lib().kvarn_decode_multi_workspace_bytes(ctypes.byref(cfg), batch, num_q_heads,
                                                    n_query, max_blocks_per_seq,
                                                    ctypes.byref(out)))
    return out.value


def decode_attention_multi(cfg: Config, q, block_pool, block_table, seq_lens, staging_k,
                           staging_v, sm_scale, out, workspace, stream=None):
    """q fp16 [B, Q, Hq, D]: the last Q tokens of each sequence, query token i at position
    seq_lens[b] - Q + i, attending causally; out fp32 [B, Q, Hq, D]; workspace of at least
    decode_multi_workspace_bytes(...) bytes."""
    batch, n_query, hq, _ = q.shape
    max_blocks = block_table.shape[1]
    num_blocks = block_pool.numel() // block_bytes(cfg)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("kvarn_decode_attention_multi",
           lib().kvarn_decode_attention_multi(ctypes.byref(cfg), _ptr(q), hq, n_query,
                                              _ptr(block_pool), num_blocks, _ptr(block_table),
                                              max_blocks, _ptr(seq_lens), _ptr(staging_k),
                                              _ptr(staging_v), float(sm_scale), _ptr(out),
                                              _ptr(workspace), ws_bytes, batch,
                                              _stream(stream)))


# ------------------------------------------------------------------ fp16 cache (comparison path)

FP16_RECORD_BYTES = 65536


def fp16_block_bytes(cfg: Config) -> int:
    return int(lib().kvarn_fp16_block_bytes(ctypes.byref(cfg)))


def fp16_write_tiles(cfg: Config, k, v, dst_blocks, block_pool, token_stride=None, stream=None):
    """k, v fp16 [n_tiles * 128, ...] with stride(0) = token_stride; tile i goes to fp16 block
    dst_blocks[i] of block_pool (uint8 device tensor of num_blocks fp16 blocks)."""
    n_tiles = dst_blocks.numel()
    stride = k.stride(0) if token_stride is None else token_stride
    num_blocks = block_pool.numel() // fp16_block_bytes(cfg)
    _check("kvarn_fp16_write_tiles",
           lib().kvarn_fp16_write_tiles(ctypes.byref(cfg), _ptr(k), _ptr(v), stride, n_tiles,
                                        _ptr(dst_blocks), _ptr(block_pool), num_blocks,
                                        _stream(stream)))


def decode_attention_fp16(cfg: Config, q, block_pool, block_table, seq_lens, staging_k,
                          staging_v, sm_scale, out, workspace, stream=None):
    """decode_attention() over an fp16 pool (block_pool: fp16 blocks of fp16_block_bytes)."""
    batch, hq, _ = q.shape
    max_blocks = block_table.shape[1]
    num_blocks = block_pool.numel() // fp16_block_bytes(cfg)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("kvarn_decode_attention_fp16",
           lib().kvarn_decode_attention_fp16(ctypes.byref(cfg), _ptr(q), hq, _ptr(block_pool),
                                             num_blocks, _ptr(block_table), max_blocks,
                                             _ptr(seq_lens), _ptr(staging_k), _ptr(staging_v),
                                             float(sm_scale), _ptr(out), _ptr(workspace),
                                             ws_bytes, batch, _stream(stream)))

