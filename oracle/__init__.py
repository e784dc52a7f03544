"""CPU oracle for decode context parallelism (DCP) over absorbed-MLA latent KV.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, float64 reference
that the GPU library is checked against.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The GPU library never imports, links or calls anything here, and nothing
here imports the GPU library: the two share no code.

What it computes, and where the pages define it:

* ``layout``    -- which rank owns a global token position, the compact local
  row it is stored at, the per-rank token counts of an interval, and the
  paged physical slot, the prefill-to-decode token relayout plan and a rank's
  share of a global sparse selection.  The striping is produced by *simulating* the
  round-robin hand-out of tokens (page "DCP", section "core abstraction",
  idea one; page "PCP/DCP", sections 5 and 6), not by the closed forms; the
  closed forms are what the tests pin the simulation against.
* ``attention`` -- full-context softmax attention of 576-dim query rows
  against the shared 576-dim latent rows with the value taken as the first
  512 dims (page "MLA 的 Decode Context Parallelism", sections 1 and 2),
  attention restricted to one stripe returning a locally normalised output and
  its log-sum-exp (page "DCP", idea two), and the exact LSE merge (page "DCP",
  "theory": merge identity and max-shifted form; SGLang DCP docs, "MLA decode
  dataflow"); the variants that keep the merge exact (sliding window, logit
  softcap, attention sink, position bias, sparse attention over a global
  top-k; page "DCP", conditions for merging) and the packed head-return
  exchange (page "DCP", "merge: All-to-All").

Every function is pinned by a CPU test against something other than itself:
values the pages print (``tests/golden``), closed forms, brute force on tiny
inputs, a library routine on a special case, or an invariant.  No function
here is "parity unpinned".
"""

from . import layout, attention  # noqa: F401

__all__ = ["layout", "attention"]
