"""CPU oracle for PISA hierarchical block selection and block-sparse attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
statement of what the GPU path computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the library and
its Python binding never do, and nothing here imports them.

Source of every rule: the paper-summary page "Block Sparse Attention with
Log-Linear Complexity" (Tang, Qin, Pan, Li, Liu), sections Prerequisites,
Core method and Method steps.  Each function names the passage it follows.

Modules
-------
``pisa``           level-by-level vectorised oracle (pyramid, routing, leaf
                   LSE, top-K, attention, decode).
``per_query``      an independently written per-query routine (pure-Python
                   loops, its own pyramid, its own LSE) used to pin ``pisa``
                   on tiny inputs; also a brute-force flat top-K over exact
                   leaf LSE.

``score="mean"`` / ``"mean_var"`` (both routines) are the PISA-1 / PISA-2
score variants (mean, and mean + half the population variance, of the
children's logits), pinned by the second-order Taylor expansion of the LSE,
by agreement of the two routines, and by equality of PISA-1 without cuts
with the flat mean-key selection.

``pisa.flat_mean_select`` is the single-level baseline of the block-sparse
framework (every valid leaf scored by its mean-key dot product, head sum,
top K); it is pinned to the exact-LSE brute force through the closed forms
of constant-key blocks and of the small-logit limit.

``pisa.attention_backward`` gives the gradients of the block-sparse attention
with the selections held fixed (the page calls the method trainable but
states no gradient); it is pinned by central finite differences of the
forward oracle, by float64 autograd of dense causal attention when every
leaf is selected, and by the softmax-gradient invariants (sum of dk = 0,
sum of dv = sum of dO).

Parity status
-------------
Pinned: pyramid (closed form over full spans, hand-derived partial-node
fixture), LSE (high-precision Decimal brute force, bounds, Taylor
expansion), flat equivalence when every level keeps all candidates (brute
force), K >= number of leaves (textbook dense causal attention), attention
weights summing to one, selection-set invariants (size formula, causal
validity, lower-index tie rule), decode (incremental update == rebuild,
decode step == prefill of the last token), and the boundary record that the
acceptance rule reads (K-th minus (K+1)-th score, smallest over the scored
levels): hand-derived values in tests/golden/route_tiny.json whose minimum
sits at the top, middle and leaf level, plus agreement with the per-query
routine's own record on random tiny inputs.
The general hierarchical case (K smaller than half the leaves) has no worked
example on the pages: it is pinned only by agreement of the two
independently written routines plus the invariants above ("parity
unpinned" beyond that).
"""
