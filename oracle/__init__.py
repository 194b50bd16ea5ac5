"""CPU oracle for MLA latent-cache decode -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the GPU
path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``mla_latent_cache_decode_amd``) never imports, links or calls anything here,
and nothing here imports the product path: the two share no code.

Every floating-point step runs in float64.  Sources, by page:

* "DeepSeek R1 Architecture & Deployment Guide", section 1 (low-rank KV
  projections, the MHA footprint equation) and section 1.1 (matrix
  absorption, decoupled RoPE, the 576-element cache row and its footprint).
* "DeepSeek-R1" model record (inference-research), intro (61 x 576 x 2 bytes
  per token) and engine kernel constraints (1) (page-block size 64) and (2)
  (FP8 latent row: e4m3 codes over every dimension, RoPE dimensions included,
  plus one e8m0 scale per 32 codes).
* Same guide, section 4: E4M3 max normal 448.
* "DeepSeek-V3.2" model record: the same latent cache, read through a
  top-k selector (index_topk = 2048) -- the sparse decode.

Modules
-------
formats     bf16 / e4m3fn / e8m0 decoding and cache-row decoding
mla         the absorbed MLA decode definition (scores, softmax, latent output)
sparse      the same decode over each query's selected tokens only (top-k)
unabsorbed  the explicit per-head MHA form (up-projected keys and values)
brute       pure-Python triple loop for tiny inputs
footprint   closed-form cache sizes

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(printed page figures, library routines, closed forms, invariants, brute
force); none is "parity unpinned".
"""

from . import formats, mla, sparse, unabsorbed, brute, footprint  # noqa: F401
from .mla import mla_decode_ref  # noqa: F401
from .sparse import mla_sparse_decode_ref  # noqa: F401
