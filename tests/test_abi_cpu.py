"""The C-ABI library without a GPU: it loads, exports every entry point include/kvarn.h
declares, and its host-side validation returns the documented status codes before any HIP
call (every call below fails validation, so nothing is launched)."""

import ctypes
import os
import re

import pytest

import decode_attention_tok_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvarn.h")

OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kv.LIB_PATH):
        pytest.skip("libkvarn.so not built")
    return kv.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KVARN_API\s+[\w\s\*]+?\b(kvarn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(kv.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.kvarn_abi_version() == 5


def test_sizes(lib):
    cfg = kv.default_config(8)
    assert kv.tile_bytes(cfg) == 13312
    assert kv.block_bytes(cfg) == 8 * 13312
    for d in (32, 96, 512):
        bad = kv.default_config(8)
        bad.head_dim = d
        assert kv.tile_bytes(bad) == 0 and kv.block_bytes(bad) == 0


@pytest.mark.parametrize("d,vb,size", [(64, 2, 7040), (64, 4, 9088), (128, 2, 13312),
                                       (128, 4, 17408), (256, 2, 25856), (256, 4, 34048)])
def test_head_dim_record_sizes_match_the_layout(lib, d, vb, size):
    cfg = kv.default_config(4, v_bits=vb, head_dim=d)
    assert kv.tile_bytes(cfg) == size == 64 * d + 16 * d * vb + 2 * (d + 384)
    assert kv.block_bytes(cfg) == 4 * size


def test_head_dim_rules(lib):
    # token_stride must cover num_kv_heads * head_dim
    c64 = kv.default_config(8, head_dim=64)
    assert lib.kvarn_quantize_tiles(ctypes.byref(c64), FAKE, FAKE, 8 * 64 - 8, 1, FAKE, FAKE, 1,
                                    None) == SHAPE
    c256 = kv.default_config(8, head_dim=256)
    assert lib.kvarn_quantize_tiles(ctypes.byref(c256), FAKE, FAKE, 8 * 128, 1, FAKE, FAKE, 1,
                                    None) == SHAPE
    # sign words past head_dim / 32 must be zero: word 2 is channel 64.. at head_dim 64
    assert kv.tile_bytes(kv.default_config(8, head_dim=64, rotation_signs=[1, 1])) == 7040
    assert kv.tile_bytes(kv.default_config(8, head_dim=64, rotation_signs=[0, 0, 1])) == 0
    assert kv.tile_bytes(kv.default_config(8, rotation_signs=[0, 0, 0, 0, 1])) == 0
    assert kv.tile_bytes(kv.default_config(8, head_dim=256, rotation_signs=[0] * 7 + [1])) > 0
    # the fp16 comparison cache exists at head_dim 128 only
    assert kv.fp16_block_bytes(c64) == 0 and kv.fp16_block_bytes(c256) == 0
    assert lib.kvarn_fp16_write_tiles(ctypes.byref(c64), FAKE, FAKE, 1024, 1, FAKE, FAKE, 1,
                                      None) == UNSUP
    # the workspace holds one partial of 2 + head_dim floats per query head and split; these
    # sizes take the four-wave tile kernel at every head dimension (eight query heads per KV
    # head), so the split plan is the same
    ws = {d: kv.decode_workspace_bytes(kv.default_config(8, head_dim=d), 16, 64, 128)
          for d in (64, 128, 256)}
    assert ws[64] * 130 == ws[128] * 66 and ws[256] * 130 == ws[128] * 258


def test_value_bit_presets(lib):
    c4 = kv.default_config(8, v_bits=4)
    assert kv.tile_bytes(c4) == kv.TILE_BYTES_V4 == 17408
    assert kv.block_bytes(c4) == 8 * 17408
    for vb in (0, 1, 3, 8):
        bad = kv.default_config(8)
        bad.v_bits = vb
        assert kv.tile_bytes(bad) == 0
        assert lib.kvarn_quantize_tiles(ctypes.byref(bad), FAKE, FAKE, 1024, 1, FAKE, FAKE, 1,
                                        None) == UNSUP
    bad = kv.default_config(8, v_bits=4)
    bad.k_bits = 2
    assert kv.tile_bytes(bad) == 0
    # with more than four virtual heads per KV head the workspace does not depend on the
    # preset (both use the four-wave tile kernel)
    assert (kv.decode_workspace_bytes(c4, 16, 64, 128)
            == kv.decode_workspace_bytes(kv.default_config(8), 16, 64, 128))


def test_workspace_bytes_depends_only_on_sizes_and_device(lib):
    cfg = kv.default_config(8)
    a = kv.decode_workspace_bytes(cfg, 16, 64, 128)
    b = kv.decode_workspace_bytes(cfg, 16, 64, 128)
    assert a == b and a > 0 and a % 4 == 0
    assert kv.decode_workspace_bytes(cfg, 0, 64, 128) == 0


def test_workspace_follows_the_split_plan(lib):
    """The workspace holds 130 floats per (sequence, query head, partial slot). This host has
    no GPU: the plan assumes 256 compute units.
    List schedules, for tables of at least 64 entries x KV heads x sequences per compute unit:
    the sequences' full tiles (four-wave tile kernel, at most 8 virtual heads per KV head; at
    head dimension 128 the 16-head kernel for more, one list unit per head group of 16) or
    tile pairs (paired-tile kernel: at most four virtual heads, 2-bit values, head dimension
    128) form one list that the resident workers share evenly, at least m positions each: tiles,
    m = max(4, (entries - 1) // 62 + 1); pairs, m = (p - 1) // 62 + 1 for p = ceil(entries / 2).
    A (sequence, KV head) of up to n positions (entries or p) then meets at most
    (n - 1) // m + 2 workers, each writing its own partial slot.
    (At head dimensions 64 and 256 the tile kernel's list likewise makes one unit per head
    group of 8.) Split grid (a smaller table; also the fp16
    comparison decode, whose need the size always covers): two workgroups per compute unit, at
    least two tiles per wave
    unless that leaves fewer than two workgroups per compute unit (then one), at most 32 full
    tiles per split for the longest table (its last entry is the staging tile)."""
    per = 130 * 4
    # 16K context, batch 16, 8 KV heads, group 8: tile list, m = 4, 128 // 4 + 2 = 34 slots
    # (the split grid of the same sizes needs 4)
    assert kv.decode_workspace_bytes(kv.default_config(8), 16, 64, 129) == 16 * 64 * 34 * per
    # the same with group 16: the 16-head kernel on the tile list, 34 slots
    assert kv.decode_workspace_bytes(kv.default_config(8), 16, 128, 129) == 16 * 128 * 34 * per
    # group 16 x 2 query tokens (two groups of 16): the 16-head kernel on the tile list, one
    # unit per head group, 34 slots for 2 x the rows
    assert (kv.decode_multi_workspace_bytes(kv.default_config(8), 16, 128, 2, 129)
            == 16 * 2 * 128 * 34 * per)
    # 4K context, batch 8 (33 entries; 2,112 < 16,384): split grid, 8 splits wanted; two tiles
    # per wave would allow 4, or 256 workgroups, so one tile per wave is allowed: 8
    assert kv.decode_workspace_bytes(kv.default_config(8), 8, 32, 33) == 8 * 32 * 8 * per
    # 4K context, batch 64 (16,896 entries), group 4: paired tiles, p = 17, m = 1,
    # 16 // 1 + 2 = 18 slots
    assert kv.decode_workspace_bytes(kv.default_config(8), 64, 32, 33) == 64 * 32 * 18 * per
    # the same with 4-bit values: tile list, 10 slots
    assert kv.decode_workspace_bytes(kv.default_config(8, v_bits=4), 64, 32, 33) == 64 * 32 * 10 * per
    # ragged batch up to 32K tokens, batch 32, 10 KV heads, group 4 (82,240 entries): paired
    # tiles, p = 129, m = 128 // 62 + 1 = 3, 128 // 3 + 2 = 44 slots
    assert kv.decode_workspace_bytes(kv.default_config(10), 32, 40, 257) == 32 * 40 * 44 * per
    # the same batch with group 8: tile list, m = 256 // 62 + 1 = 5, 256 // 5 + 2 = 53 slots
    assert kv.decode_workspace_bytes(kv.default_config(10), 32, 80, 257) == 32 * 80 * 53 * per
    # 128K context, batch 64, 8 KV heads, group 4 (524,800 entries): paired tiles, p = 513,
    # m = 9, 512 // 9 + 2 = 58 slots; the split grid of the same sizes needs 32
    assert kv.decode_workspace_bytes(kv.default_config(8), 64, 32, 1025) == 64 * 32 * 58 * per


def test_multi_workspace_and_query_token_limits(lib):
    cfg = kv.default_config(8)
    one = kv.decode_workspace_bytes(cfg, 16, 64, 128)
    assert kv.decode_multi_workspace_bytes(cfg, 16, 64, 1, 128) == one
    # four query tokens x group 8 = 32 virtual heads: two head groups of 16 on the tile list
    # (16,384 entries), m = 4, 127 // 4 + 2 = 33 slots for 4x the rows
    assert kv.decode_multi_workspace_bytes(cfg, 16, 64, 4, 128) == 16 * 4 * 64 * 33 * 130 * 4
    assert kv.decode_multi_workspace_bytes(cfg, 16, 64, kv.MAX_QUERY_TOKENS, 128) > 0
    for bad in (0, -1, kv.MAX_QUERY_TOKENS + 1):
        with pytest.raises(RuntimeError):
            kv.decode_multi_workspace_bytes(cfg, 16, 64, bad, 128)


def _call(lib, name, *args):
    return getattr(lib, name)(*args)


def _cfg(**kw):
    c = kv.default_config(kw.pop("hkv", 2))
    for k, v in kw.items():
        setattr(c, k, v)
    return ctypes.byref(c)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("head_dim", 32), ("block_tokens", 64),
                                         ("k_bits", 2), ("v_bits", 3), ("v_bits", 8),
                                         ("sinkhorn_iters", 0), ("sinkhorn_iters", 17)])
def test_unsupported_configs(lib, field, value):
    st = _call(lib, "kvarn_quantize_tiles", _cfg(**{field: value}), FAKE, FAKE, 256, 1, FAKE,
               FAKE, 1, None)
    assert st == UNSUP


def test_null_config(lib):
    assert _call(lib, "kvarn_quantize_tiles", None, FAKE, FAKE, 256, 1, FAKE, FAKE, 1, None) == NULL
    out = ctypes.c_size_t()
    assert _call(lib, "kvarn_decode_workspace_bytes", None, 1, 2, 1, ctypes.byref(out)) == NULL


def test_quantize_validation(lib):
    f = "kvarn_quantize_tiles"
    assert _call(lib, f, _cfg(), FAKE, FAKE, 256, 0, None, None, 0, None) == OK   # no-op
    assert _call(lib, f, _cfg(), None, FAKE, 256, 1, FAKE, FAKE, 1, None) == NULL
    assert _call(lib, f, _cfg(), FAKE, FAKE, 256, -1, FAKE, FAKE, 1, None) == SHAPE
    assert _call(lib, f, _cfg(), FAKE, FAKE, 128, 1, FAKE, FAKE, 1, None) == SHAPE  # < Hkv*128
    assert _call(lib, f, _cfg(), FAKE, FAKE, 260, 1, FAKE, FAKE, 1, None) == SHAPE  # % 8
    assert _call(lib, f, _cfg(), ctypes.c_void_p(0x1002), FAKE, 256, 1, FAKE, FAKE, 1,
                 None) == SHAPE                                                  # misaligned
    assert _call(lib, f, _cfg(hkv=0), FAKE, FAKE, 256, 1, FAKE, FAKE, 1, None) == SHAPE
    assert _call(lib, f, _cfg(), FAKE, FAKE, 256, 1, FAKE, ctypes.c_void_p(0x1004), 1,
                 None) == SHAPE                                                  # pool


def test_append_validation(lib):
    f = "kvarn_append_token"
    args = [FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 10]
    assert _call(lib, f, _cfg(), *args, 0, None) == OK                           # no-op
    assert _call(lib, f, _cfg(), None, *args[1:], 2, None) == NULL
    bad = list(args)
    bad[4] = 0
    assert _call(lib, f, _cfg(), *bad, 2, None) == SHAPE                         # max_blocks
    assert _call(lib, f, _cfg(), *args, -1, None) == SHAPE
    bad = list(args)
    bad[5] = ctypes.c_void_p(0x1008)
    assert _call(lib, f, _cfg(), *bad, 2, None) == SHAPE                         # misaligned
    bad = list(args)
    bad[7] = ctypes.c_void_p(0x1001)
    assert _call(lib, f, _cfg(), *bad, 2, None) == SHAPE                         # pool


def test_decode_validation(lib):
    f = "kvarn_decode_attention"
    cfg = kv.default_config(2)
    need = kv.decode_workspace_bytes(cfg, 2, 8, 4)
    good = [FAKE, 8, FAKE, 10, FAKE, 4, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
            ctypes.c_void_p(0x10000), need, 2, None]
    def call(**over):
        a = list(good)
        names = ["q", "hq", "pool", "nblk", "bt", "maxb", "lens", "sk", "sv", "sm", "out", "ws",
                 "wsb", "batch", "stream"]
        for k, v in over.items():
            a[names.index(k)] = v
        return _call(lib, f, _cfg(), *a)
    assert call(batch=0) == OK
    assert call(q=None) == NULL
    assert call(out=None) == NULL
    assert call(hq=7) == SHAPE                      # not a multiple of Hkv
    assert call(hq=2 * 17) == SHAPE                 # group > 16
    assert call(maxb=0) == SHAPE
    assert call(ws=None) == WS
    assert call(wsb=need - 4) == WS
    assert call(ws=ctypes.c_void_p(0x10010)) == WS  # not 256-byte aligned
    assert call(sm=ctypes.c_float(float("nan"))) == SHAPE
    assert call(q=ctypes.c_void_p(0x1004)) == SHAPE
    assert call(pool=ctypes.c_void_p(0x1008)) == SHAPE


def test_decode_multi_validation(lib):
    f = "kvarn_decode_attention_multi"
    cfg = kv.default_config(2)
    need = kv.decode_multi_workspace_bytes(cfg, 2, 8, 4, 4)
    names = ["q", "hq", "nq", "pool", "nblk", "bt", "maxb", "lens", "sk", "sv", "sm", "out", "ws",
             "wsb", "batch", "stream"]
    good = [FAKE, 8, 4, FAKE, 10, FAKE, 4, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
            ctypes.c_void_p(0x10000), need, 2, None]
    def call(**over):
        a = list(good)
        for k, v in over.items():
            a[names.index(k)] = v
        return _call(lib, f, _cfg(), *a)
    assert call(batch=0) == OK
    assert call(nq=0) == SHAPE
    assert call(nq=17) == SHAPE
    assert call(wsb=need - 4) == WS                  # sized for Q = 4
    assert call(nq=5) == WS                          # needs more than the Q = 4 workspace
    assert call(q=None) == NULL
    assert call(hq=2 * 17) == SHAPE
    assert call(pool=ctypes.c_void_p(0x1002)) == SHAPE


def test_decode_noalloc_validation(lib):
    f = "kvarn_decode_attention_noalloc"
    names = ["q", "hq", "pool", "nblk", "bt", "maxb", "lens", "sk", "sv", "sm", "out", "batch",
             "stream"]
    good = [FAKE, 8, FAKE, 10, FAKE, 4, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, 2, None]
    def call(hkv=2, **over):
        a = list(good)
        for k, v in over.items():
            a[names.index(k)] = v
        return _call(lib, f, _cfg(hkv=hkv), *a)
    assert call(batch=0) == OK
    assert call(q=None) == NULL
    assert call(hq=7) == SHAPE
    assert call(maxb=0) == SHAPE
    # sizes whose workspace would exceed the static scratch are rejected before any HIP call
    assert kv.decode_workspace_bytes(kv.default_config(8), 4096, 64, 8) > kv.STATIC_SCRATCH_BYTES
    assert call(hkv=8, hq=64, maxb=8, batch=4096) == 6
    assert b"scratch" in lib.kvarn_status_string(6)


def test_dequantize_validation(lib):
    f = "kvarn_dequantize_tiles"
    assert _call(lib, f, _cfg(), FAKE, 4, FAKE, 0, None, None, None) == OK          # no-op
    assert _call(lib, f, _cfg(), None, 4, FAKE, 1, FAKE, FAKE, None) == NULL
    assert _call(lib, f, _cfg(), FAKE, 4, FAKE, 1, FAKE, None, None) == NULL
    assert _call(lib, f, _cfg(), FAKE, 4, FAKE, -1, FAKE, FAKE, None) == SHAPE
    assert _call(lib, f, _cfg(), FAKE, -4, FAKE, 1, FAKE, FAKE, None) == SHAPE
    assert _call(lib, f, _cfg(), FAKE, 4, FAKE, 1, ctypes.c_void_p(0x1004), FAKE,
                 None) == SHAPE                                                   # misaligned
    assert _call(lib, f, _cfg(), ctypes.c_void_p(0x1004), 4, FAKE, 1, FAKE, FAKE,
                 None) == SHAPE                                                   # pool


def test_fp16_path_validation(lib):
    cfg = kv.default_config(8)
    assert kv.fp16_block_bytes(cfg) == 8 * 65536
    assert kv.fp16_block_bytes(kv.default_config(8, v_bits=4)) == 8 * 65536   # any preset
    bad = kv.default_config(8)
    bad.v_bits = 3
    assert kv.fp16_block_bytes(bad) == 0
    f = "kvarn_fp16_write_tiles"
    assert _call(lib, f, _cfg(), FAKE, FAKE, 256, 0, None, None, 0, None) == OK   # no-op
    assert _call(lib, f, _cfg(), FAKE, None, 256, 1, FAKE, FAKE, 1, None) == NULL
    assert _call(lib, f, _cfg(), FAKE, FAKE, 128, 1, FAKE, FAKE, 1, None) == SHAPE  # < Hkv*128
    assert _call(lib, f, _cfg(), FAKE, FAKE, 256, 1, FAKE, ctypes.c_void_p(0x1008), 1,
                 None) == SHAPE                                                  # misaligned pool
    f = "kvarn_decode_attention_fp16"
    cfgd = kv.default_config(2)
    need = kv.decode_workspace_bytes(cfgd, 2, 8, 4)
    good = [FAKE, 8, FAKE, 10, FAKE, 4, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE,
            ctypes.c_void_p(0x10000), need, 2, None]
    def call(**over):
        a = list(good)
        names = ["q", "hq", "pool", "nblk", "bt", "maxb", "lens", "sk", "sv", "sm", "out", "ws",
                 "wsb", "batch", "stream"]
        for k, v in over.items():
            a[names.index(k)] = v
        return _call(lib, f, _cfg(), *a)
    assert call(batch=0) == OK
    assert call(pool=None) == NULL
    assert call(hq=7) == SHAPE
    assert call(wsb=need - 4) == WS
    assert call(pool=ctypes.c_void_p(0x1008)) == SHAPE
    assert call(sm=ctypes.c_float(float("nan"))) == SHAPE


def test_status_strings(lib):
    for code in range(6):
        assert lib.kvarn_status_string(code)
    assert lib.kvarn_status_string(99) == b"unknown status"


def test_binding_raises_on_error(lib):
    cfg = kv.default_config(2)
    cfg.head_dim = 96
    with pytest.raises(kv.KvarnError) as e:
        kv.decode_workspace_bytes(cfg, 1, 2, 1)
    assert e.value.code == UNSUP
