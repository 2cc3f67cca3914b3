"""CPU fp64 oracle for SepLLM separator-sparse attention and the SepCache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``sparse_attention_sepattn_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.

What it computes, and where the pages say so
--------------------------------------------
* ``sepmask``    -- which keys a query may see: the first ``a`` initial tokens,
  every preceding separator token and a local window of ``n`` neighbours
  (SepLLM summary on atlas.scime.ai, "Approach"; the binary mask ``M_b`` of the
  formula O = M(A, V, M_b) in "How SepLLM Reorchestrates the Language Model for
  Speed and Efficiency", section "SepLLM's Architecture: Composing Efficiency").
  It also defines the per-tile index metadata the GPU schedule is built from.
* ``attention``  -- masked softmax attention, forward and backward, in fp64 on a
  materialised mask (same two pages; the backward is the plain derivative of
  the forward, used by the training-from-scratch setting: beiduofen page,
  "The Mechanics of Compression: Why Separators Work").
* ``sepcache``   -- the four-block streaming KV cache (Initial, Local Window,
  Past Window, Separator) as a literal list simulation, positional-encoding
  shifting by cache slot (project card on sourcepulse.org, "Limitations &
  Caveats"; atlas.scime.ai, "Measured effects reported in the paper"), and
  decode attention over the cache.

Readings of points the pages leave open are listed in each function's
docstring and collected in the design doc.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
brute force, closed forms, library routines (torch SDPA / autograd on the CPU),
finite differences and hand-derived worked examples under ``tests/golden/``.
The exact SepCache policy details beyond those readings are "parity unpinned"
against the authors (the pages print no trace).
"""

from . import sepmask, attention, sepcache  # noqa: F401
