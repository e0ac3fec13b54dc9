"""CPU float64 oracle for block-sparse streaming attention (SSA) and its variants.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test-suite, the smoke check of the graft entry point and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or helper with the HIP library; the two meet only through the seeded
input generators in ``synth``.

Every function computes the plain definition of its operation in float64 with
numpy, one query block (or one sequence) at a time, so a reader can check it
against the sources by eye:

* ``window_blocks`` / ``block_index`` / ``block_index_seq`` -- which 128-token
  blocks a query may read: the global block 0 plus the 7 most recent blocks,
  the query's own block included (QbitAI report on LongCat LoZA, the paragraph
  on the 1024-token sparse window: 1 global + 7 local blocks of 128 tokens).
* ``ssa_rows`` / ``ssa_attention`` -- softmax attention restricted to that
  window and to causally earlier keys ("LoZA: ZigZag sparse attention" page,
  section 2.1, equations (1) and (2); section 2.2.1 for the causal rule j <= i),
  computed with the row maximum subtracted before exp (CSA/HCA tutorial page,
  section 7.1, stable softmax).
* ``ssa_backward`` -- gradients of ``ssa_attention`` with respect to q, k and v,
  written out by the chain rule through o = P v and the softmax (the sparse
  operator has a custom deterministic backward in training: LongCat sparse
  attention article, section 4).
* ``dense_causal_rows`` / ``dense_causal`` -- the full causal attention used as
  the comparison layer; written on its own, without the window code, so that
  "SSA equals dense when L <= 1024" is a real check.
* ``decode`` -- one new query per sequence over a paged cache.
* ``dense_decode`` -- one new query per sequence over every cached key (the
  decode step of the dense layers, for the layer-stack comparison).
* ``chunk_prefill`` -- a chunk of T new queries per sequence over a paged
  cache, each with the window of its own block (the step between prefill and
  decode: a long prompt prefilled in pieces).
* ``block_sums`` / ``page_select`` / ``block_list_rows`` -- the page-selection
  variant (LongCat sparse attention article, section 3: streaming-aware
  indexing keeps sink + local window, hierarchical indexing scores 128-token
  pages and keeps the top-M).
* ``page_scores_exact`` / ``token_scores_exact`` -- one row's selection scores
  as exact rationals with the rounding band the selections are certified
  against, so that a list decided differently inside that band can be judged.
* ``token_select`` / ``token_list_attention`` -- the second stage of
  hierarchical indexing (same section: inside the recalled pages every token is
  scored and the top K are kept) and attention over window blocks plus those
  tokens.

Parity status: every function here is pinned by the CPU tests (brute force on
tiny inputs, the dense special case against torch's own attention routine,
closed-form key counts, structural one-hot outputs, decode == last prefill row,
chunked prefill == brute force over the cached sequence, dense decode == the
last row of the (torch-pinned) dense causal attention, gradients == central
finite differences of the forward and == torch autograd with an explicit mask,
exact rational re-scoring of page and token selections, token lists that
keep every candidate == the page-list attention, planted and duplicated
tokens).  No function is "parity
unpinned".
"""
from .ssa import (  # noqa: F401
    Window,
    DEFAULT_WINDOW,
    window_blocks,
    block_index,
    block_index_seq,
    ssa_rows,
    ssa_attention,
    ssa_backward,
    dense_causal_rows,
    dense_causal,
    decode,
    dense_decode,
    chunk_prefill,
    block_sums,
    page_select,
    page_scores_exact,
    token_scores_exact,
    block_list_rows,
    block_list_attention,
    token_select,
    token_list_attention,
)
