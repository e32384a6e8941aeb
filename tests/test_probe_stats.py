"""Statistics of the error-accumulation probe (host side): closed-form cases."""

import numpy as np

from decode_attention_tok_amd import probe


def test_top_share_closed_forms():
    assert probe.top_share(np.ones(100)) == 0.05                  # equal errors: 5 of 100
    assert probe.top_share(np.ones(101)) == 6 / 101               # ceil(0.05 * 101) = 6 rows
    e = np.zeros(1000)
    e[7] = 3.0
    assert probe.top_share(e) == 1.0                              # one row holds everything
    e = np.arange(1, 21, dtype=float)                             # 20 rows: top 1 = 20 of 210
    assert probe.top_share(e) == 20 / 210
    assert probe.top_share(np.zeros(5)) == 0.0


def test_summarise_fields():
    r = probe.summarise(np.linspace(0, 1, 101))
    assert r["rows"] == 101 and abs(r["p50"] - 0.5) < 1e-12 and r["max"] == 1.0
    assert abs(r["mean"] - 0.5) < 1e-12 and abs(r["top5_share"] - 5.85 / 50.5) < 1e-12
