"""Plain, slow fp64 CPU oracle for the KVarN K4V2 g128 codec and the decode attention that reads it.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code, table or constant generator with the HIP library
under ``decode_attention_tok_amd/``; the two meet only through the seeded inputs of
``workloads/`` and through byte buffers.

Page abbreviations used in the citations of this package (all four pages are about KVarN):

* [TSM] tools.thesoundmethod.me, "KVarN: 2-Bit KV-Cache That Beats FP16 Throughput, and
  Where the Catch Lives".
* [GR]  groundy.com, "Huawei's KVarN puts KV-cache quantization inside vLLM's backend"
  (sections "What KVarN changes in vLLM's serving path", "The four-stage pipeline",
  "Frequently Asked Questions").
* [BH]  beyondheadline.xyz, "Huawei's KV-cache trick claims FP16 accuracy, 4x the capacity,
  and faster throughput at once".
* [SI]  stuffinsider.com, "KVarN: KV-Cache Quantization with 3-5x Compression from Huawei".

What the oracle computes is stated per function. Where the pages leave a step open the
function names the reading it takes (R-numbers, listed with reasons in the repository's
design notes). Parity against the real KVarN release is unpinned: the pages carry no code,
no tensors and no printed intermediate values; every function here is pinned instead by
closed forms, invariants, library routines and brute force (``tests/test_oracle_*.py``).

Modules
-------
formats    FP8 E4M3 (OCP) and FP16 rounding by exhaustive, sorted value tables.
hadamard   the 128-point orthonormal Sylvester Hadamard matrix.
codec      one-tile quantisation (rotation, log-space normalisation, asymmetric RTN),
           the packed tile record, dequantisation.
attention  exact softmax attention over a paged packed cache plus the fp16 staging tile,
           in the plain (dequantise, then attend) and the folded form, and the three
           cache-level operations the library exposes.
"""

from . import formats, hadamard, codec, attention  # noqa: F401

__all__ = ["formats", "hadamard", "codec", "attention"]
