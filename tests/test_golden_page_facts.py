"""The packed record against the format figures the pages state (tests/golden/page_facts.json).

Reading R10: the quoted ~2.3 bits per element cannot be the key+value mean of a 4-bit/2-bit
code (the codes alone average 3 bits); it matches the value half of the record (2.25 bits with
its scales and zero-points). The whole record stores 3.25 bits per element, 4.92x fewer bytes
than fp16, which sits inside every capacity range the pages quote."""

import json
import os

import numpy as np

from oracle import codec

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _record_for(kbits_code, vbits_code):
    kq = dict(codes=np.full((128, 128), kbits_code), c_code=np.zeros(128, np.uint8),
              s_code=np.zeros(128, np.uint8), z_bits=np.zeros(128, np.uint16))
    vq = dict(kq, codes=np.full((128, 128), vbits_code))
    return codec.pack_record(kq, vq)


def test_code_widths_fill_their_sections_exactly():
    # the largest code of each width fills its section; one more bit would not fit
    kmax = 2 ** GOLD["key_bits"]["value"] - 1
    vmax = 2 ** GOLD["value_bits"]["value"] - 1
    rec = _record_for(kmax, vmax)
    assert np.all(rec[codec.K_CODES_OFF:codec.V_CODES_OFF] == 0xFF)
    assert np.all(rec[codec.V_CODES_OFF:codec.K_META_OFF] == 0xFF)
    u = codec.unpack_record(rec)
    assert u["k"]["codes"].max() == kmax and u["v"]["codes"].max() == vmax


def test_rates_against_page_figures():
    t = GOLD["tile_tokens"]["value"]
    elems = t * 128
    assert codec.TILE_BYTES == 13312
    k_bytes = (codec.V_CODES_OFF - codec.K_CODES_OFF) + (codec.V_META_OFF - codec.K_META_OFF)
    v_bytes = (codec.K_META_OFF - codec.V_CODES_OFF) + (codec.TILE_BYTES - codec.V_META_OFF)
    assert k_bytes + v_bytes == codec.TILE_BYTES
    k_rate = 8 * k_bytes / elems
    v_rate = 8 * v_bytes / elems
    assert k_rate == 4.25 and v_rate == 2.25
    assert abs(v_rate - GOLD["approx_bits_per_element"]["value"]) < 0.1
    ratio = 2 * elems * 2 / codec.TILE_BYTES          # fp16 K+V bytes over packed bytes
    lo, hi = GOLD["capacity_vs_fp16_range"]["value"]
    assert lo <= ratio <= hi
    lo, hi = GOLD["capacity_vs_fp16_compression_range"]["value"]
    assert lo <= ratio <= hi
    assert ratio >= GOLD["capacity_vs_fp16_headline"]["value"]
