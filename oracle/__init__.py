"""CPU oracle for paged-attention decode — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding in ``decode_attention_pa_amd``) never
imports, calls or links it, and the oracle imports nothing from the product
path: the two share no code.  The only thing both sides consume is the seeded
input generator in ``workloads.py``, which holds none of the method's
arithmetic.

What is computed, and where it comes from:

* ``paged_attention.decode`` — the plain definition, float64 throughout.
  Window semantics follow gllm "feat(backend): sliding-window PagedAttention"
  (#116), summary and "What changes — CPU reference": with window w > 0 the
  token at position p sees positions p-w+1 .. p; w = 0 keeps unlimited causal
  attention; the visible range starts at max(0, end - w).  Multi-token
  queries are the trailing tokens of the context (aiter PR #2914 "Pa gluon
  swa mtp opt", summary: sliding-window MTP decode), causal among themselves.
  GQA maps query head h_q to KV head h_q // (H_q // H_kv) (executorch PR
  #18759, review of ``sdpa_decode_splitk``: grouped-query attention handled
  inside the kernel by integer division of the head index).
* ``paged_attention.decode_split`` — the split-K / flash-decoding algorithm
  (executorch PR #18759, Copilot overview and review suggestion 5; aiter PR
  #2914, workspace buffers ``max_logits`` / ``exp_sums`` /
  ``temporary_output``): each context partition produces a max logit, an
  exp-sum and a partial output, and a second pass merges the partitions by
  log-sum-exp.  In float64 it must agree with ``decode``.
* ``paged_attention.spans`` — the integer index facts (row positions, window
  starts, logical and physical blocks visited) that the GPU must reproduce
  bit-exactly.
* ``brute.brute_decode`` — pure-Python scalar loops over every position with
  the visibility predicate tested per position; written independently of the
  range arithmetic in ``paged_attention``.

* ``paged_attention.decode_e4m3`` / ``dequantize`` — FP8 (OCP E4M3) cache
  codes to values, times the per-tensor key / value scale (aiter PR #2914,
  review of ``pa_decode_gluon``: FP8 caches come with key_scale /
  value_scale); ``brute.e4m3_value`` decodes one code bit field by bit field.

Readings of points the pages leave open are restated where they are used.
Every function here is pinned by ``tests/test_oracle*.py``
to something other than itself (brute force, a textbook library routine,
closed forms, invariants, hand-derived fixtures under ``tests/golden/``).
"""
