"""fp64 CPU oracle for exact scaled-dot-product attention (TEST INFRASTRUCTURE).

This package is the reference the GPU path is checked against.  It is plain,
slow NumPy in float64 that materialises whole score rows; it shares no code,
table or helper with the HIP library and imports nothing from it.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it; the
product path never calls it.

Modules
-------
``oracle.dense``      the definition: RoPE (with the rounding model), dense
                      scores, stable softmax, O and logsumexp; decode over a
                      contiguous KV cache.
``oracle.online``     the blocked online-softmax recurrence and the merge of
                      partial (m, l, O) states, as the pages state them; used
                      to pin the algebra the kernels rely on.

Pins (``tests/test_oracle.py``, ``tests/test_online.py``): the printed softmax
example of "coding-interview attention from scratch" (section 三.1), brute-force
scalar loops on tiny inputs, the fp64 ``torch.nn.functional.scaled_dot_product_attention``
routine, and the invariants the pages fix (rows sum to one, shift invariance,
masked weight exactly zero, causal row 0 equals V[0], uniform scores give the
mean of V, GQA equals MHA with repeated KV heads, RoPE scores depend only on the
position difference, convex hull, decode equals the last causal row).

Parity unpinned: the pages print no attention output values at any shape, so
absolute O / logsumexp values are pinned only through the checks above; the
rounding of rotated Q/K to the input dtype before the product is a reading of
the pages, not a fact they state.
"""

from .dense import (  # noqa: F401
    attention,
    attention_rows,
    decode,
    logsumexp,
    round_to_dtype,
    rope,
    rope_cos_sin,
    scores_and_weights,
    softmax,
)
