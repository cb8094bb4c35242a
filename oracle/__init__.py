"""CPU float64 oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The GPU library never
calls it and shares no code with it (no kernels, headers, helpers, tables or
constants), and this package imports nothing from the GPU library.

What it computes, and where the pages say so:

* ``codecs``: exact real values of the stored bf16 and OCP e4m3fn codes.
* ``attention``: gathered-index MLA decode by its plain definition -- each
  request row attends over the latent rows its page-size-1 index list names
  (vLLM pull request 53001, "Purpose": one row per request, one flat index
  list), with a causal mask on global positions for the verify pass (ATOM pull
  request 2760, "Problem") or no mask for a draft block (vLLM pull request
  53001, "Purpose"), and emits O plus the natural-log LSE per (token, head).
* ``plan``: the split-plan heuristic (ATOM pull request 2462, "Summary": a
  caller-built split count plus split_indptr per row, uniform or planned per
  call from the real lengths), step by step.
* ``merge``: the log-sum-exp merge of split partials (ATOM pull request 2462,
  "Dependencies": split and merge).
* ``cache_write``: the latent cache write -- a token's 512 compressed dims and
  64 RoPE dims into its slot, each source value taken at its own dtype and
  rounded to the cache format (vLLM pull request 57942, "Details" and its
  review thread).
* ``brute``: pure-Python loops, for tiny cases only.

Readings where the pages are silent are listed in the repository's design
notes and repeated at each function.
"""
from .codecs import bf16_to_f64, e4m3fn_to_f64, decode  # noqa: F401
from .attention import attend_row, attend  # noqa: F401
from .plan import plan_ref, unpack_plan  # noqa: F401
from .merge import merge_partials, split_attend  # noqa: F401
