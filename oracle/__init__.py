"""fp64 CPU oracle for causal attention with the per-RoPE-wavelength distance window.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``rope_frequency_pair_amd``) and imports nothing from it.

Sources (the web pages this method is described on):

* "ATFlash — Per-RoPE-Wavelength Attention Windows", the kernel repository's
  README: sections "The idea" and "Porting to something else".
* "ATFlash: Per-RoPE-Wavelength Attention Windows for Compute/Memory-Efficient
  LLM Inference", the arXiv abstract (arXiv:2608.02947).

Everything here is the plain definition of the method written out in float64
(the window defines the result; pruned pair-terms are exactly zero), so no
blocking, fusion or reordering is done beyond what the definition states.

Modules:

* :mod:`oracle.window`    -- per-pair frequencies, wavelengths, integer windows,
  the first retained pair at a distance, tile plans.
* :mod:`oracle.counts`    -- pruned / total pair-term counts: brute force and
  the per-row closed form; the large-N logarithmic approximation; the same
  counts restricted to a block-sparse key selection.
* :mod:`oracle.attention` -- RoPE, pair terms, windowed prefill and decode.

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
closed forms, an independent complex-number RoPE route, brute force, a
high-precision (mpmath) evaluation of the windows and the shares the pages
print.  The attention *output* has no printed worked example on the pages, so
it is pinned only by invariants and closed-form special cases (see the tests).
"""

from .window import (  # noqa: F401
    UNBOUNDED,
    pair_frequencies,
    pair_wavelengths,
    window_widths,
    first_retained_pair,
    tile_plan,
)
from .counts import (  # noqa: F401
    pruned_terms,
    pruned_terms_blocks,
    pruned_terms_blocks_bruteforce,
    pruned_terms_bruteforce,
    pruned_terms_square_closed_form,
    pruned_share_log_approx,
)
from .attention import (  # noqa: F401
    rope,
    pair_terms,
    windowed_scores,
    prefill,
    decode,
    decode_multi,
)
