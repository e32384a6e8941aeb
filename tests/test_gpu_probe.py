"""The error-accumulation probe on a small case: invariants of its two measurements."""

import numpy as np
import pytest
import torch

from decode_attention_tok_amd import probe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_per_token_errors_small():
    r = probe.per_token_errors("qwen3-4b", iters=(1, 4), batch=1, ctx=256, hkv=2, hq=4)
    for it in ("iters=1", "iters=4"):
        for half in ("k", "v"):
            s = r[it][half]
            assert s["rows"] == 2 * 128 * 2
            assert 0 < s["p50"] <= s["p95"] <= s["max"] < 1
            assert 0.05 <= s["top5_share"] <= 1


def test_autoregressive_small():
    r = probe.autoregressive("qwen3-4b", steps=130, batch=1, ctx=128, hkv=2, hq=4)
    # both caches hold the same tokens before the first step: identical outputs
    assert r["divergence_at_step"]["0"] == r["one_step_at_step"]["0"]
    assert 0 < r["one_step_rel_err"]["mean"] < 1
    assert all(np.isfinite(v) for v in r["divergence_at_step"].values())
    assert r["tiles_written_in_loop"]["k"]["rows"] == 128 * 2          # one tile, 2 heads


def test_four_bit_values_lower_the_value_error():
    r2 = probe.per_token_errors("qwen3-4b", iters=(4,), v_bits=2, batch=1, ctx=256, hkv=2, hq=4)
    r4 = probe.per_token_errors("qwen3-4b", iters=(4,), v_bits=4, batch=1, ctx=256, hkv=2, hq=4)
    k2, k4 = r2["iters=4"]["k"], r4["iters=4"]["k"]
    v2, v4 = r2["iters=4"]["v"], r4["iters=4"]["v"]
    # the key path is the same code in both presets: identical errors
    assert k2 == k4
    # 16 value levels instead of 4: the per-row squared error falls by roughly (15 / 3)^2
    assert v4["p50"] < v2["p50"] / 10
    a = probe.autoregressive("qwen3-4b", steps=130, v_bits=4, batch=1, ctx=128, hkv=2, hq=4)
    assert a["v_bits"] == 4 and 0 < a["one_step_rel_err"]["mean"] < 1
