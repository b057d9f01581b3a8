"""Plain, slow, fp64 CPU oracle for position-free paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library under
``position_independent_kv_amd/`` and its Python binding) may import, call,
link or execute anything in this package.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code, tables or constants with the HIP path; the only thing
both sides consume is the seeded input data built by ``workloads/``.

What it follows: "MiniPIC: Flexible Position-Independent Caching in <100LOC"
(gist.science summary of arXiv 2606.13126), §2.1 "Position-free KV
implementation": keys are cached unrotated, the score of query t against
cached key j is (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d), where pi(j) is the
logical position of stored key j in the current request, and doing the
rotation inside attention is algebraically the same as re-rotating the cache
hit.  Every step the page leaves open is a documented reading (rotate-half
pairing, standard RoPE frequencies, bottom-right causal mask over slot index,
GQA head mapping h -> h // G, unrotated V); see the module docstrings.

The span-hashing reference (``pic_spans``) follows §2.2 (the SSEP / PDEP
block-hash primitives) and is pinned by ``tests/test_spans_oracle.py``
(published FNV-1a test vectors, closed-form hash chains, mutation checks).

Parity status: every attention function here is pinned by ``tests/test_oracle_pins.py``
(brute force with explicit rotation matrices, pre-rotated equality with a
library attention routine, shift invariance, closed forms and special cases).
"""

from .pic_oracle import (  # noqa: F401
    rope_frequencies,
    rope_table,
    rotate_half,
    place_tokens,
    gather_request,
    attention_request,
    attention,
    bf16_bits_to_f64,
)
from .pic_spans import (  # noqa: F401
    fnv1a64,
    block_hashes,
    build_block_tables,
)
