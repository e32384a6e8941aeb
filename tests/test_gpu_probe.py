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
