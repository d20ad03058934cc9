"""CPU oracle for packed ternary weight-streaming decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this package.  The GPU path never
calls it and shares no code with it.

Everything here is plain numpy in float64, written from the page "The Neutrino
Engine" (fermionresearch.com), and from the build's own packed-format
specification for the packed-byte decoder/encoder:

* ``reference``       - ternary GEMV with row scales, int8 vocabulary GEMV,
                        greedy argmax, embedding-row gather, the decode-step
                        composition;
* ``attention``       - grouped-query decode attention over a bfloat16
                        key/value cache;
* ``verify``          - the speculative verify step's acceptance rule;
* ``chain``           - the chained decode step: RMSNorm, one-position
                        grouped-query attention, SwiGLU and residual adds
                        between the projections;
* ``packed_format``   - encoder/decoder of the 2-bit packed ternary format;
* ``base3_format``    - encoder/decoder and device arrangement of the
                        base-3 format (five weights per byte);
* ``blob_header``     - the packed-blob header and its FNV-1a checksum of
                        the logical values;
* ``accounting``      - byte accounting of the 8B shape and the KV cache.

Parity status of each function is stated in its module.  One part is
"parity unpinned": the internals of the pages' own packed format (the pages
name it but never specify it), so the library's 2-bit and base-3 formats are
pinned only by their own specifications, hand-derived bytes and round trips,
not by the pages.
"""
from . import accounting, attention, base3_format, blob_header, chain, packed_format, reference, verify  # noqa: F401
