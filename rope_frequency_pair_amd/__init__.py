"""rope_frequency_pair_amd -- per-RoPE-wavelength attention windows on MI355X.

Causal softmax attention in which RoPE frequency pair r contributes to a
query-key score only while the query-key distance is within k wavelengths of
that pair ("ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The
idea").  The work runs in hand-written HIP kernels for gfx950 behind the C
ABI of ``libatw.so`` (``include/atw.h``); this package is the thin Python
binding (argument marshalling only) plus the build script.

    from rope_frequency_pair_amd import prefill, decode, pruned_terms
"""

from .binding import (  # noqa: F401
    ATW_BF16,
    ATW_F32,
    EXPORTED,
    SPARSE_BLOCK,
    LIB_PATH,
    UNBOUNDED,
    AtwError,
    block_mask_words,
    decode,
    decode_banded,
    decode_multi,
    decode_multi_workspace_bytes,
    decode_noalloc,
    decode_noalloc_max_bytes,
    decode_sparse,
    kcache_band,
    pack_block_mask,
    decode_workspace_bytes,
    default_scale,
    load_library,
    prefill,
    prefill_sparse,
    prefill_workspace_bytes,
    pruned_terms,
    pruned_terms_sparse,
    rope_descriptor,
    rope_theta,
    version,
    window_plan,
    window_plan_device,
    window_widths,
)
