"""MI355X-native DeepSeek Sparse Attention (DSA) forward path.

The path is: pool the indexer keys in groups of 4, give each query a score
for each pool before it (a chunk of queries at a time), select the top-k pools per query as int32
ids, and run softmax attention over only the selected tokens.  All four steps
are hand-written HIP kernels for gfx950 behind the C ABI declared in
``include/dsa.h`` (library ``libdsa.so``); ``long_context_sparse_dsa_amd.dsa``
is the thin Python binding with the same entry-point names.  Importing this
package loads nothing; the binding loads the library on first use and raises
if it is missing.
"""

__all__ = ["dsa", "inputs"]
