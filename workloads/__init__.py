"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

Holds no part of the codec's arithmetic: only random draws, shapes and block tables.
"""

from .gen import SPECS, spec, prefill, query, append_tokens, head_params  # noqa: F401
