"""Flash-attention forward for AMD Instinct MI355X (gfx950).

The compute lives in libattn.so (hand-written HIP kernels behind a C ABI,
declared in include/attn.h); this package holds the ctypes binding with the
same entry-point names, the build script and the seeded workload generators.
"""

from ._lib import (  # noqa: F401
    attn_fwd,
    attn_fwd_split,
    attn_fwd_split_workspace_size,
    attn_fwd_fp8,
    attn_fwd_fp8_full,
    attn_quant_fp8_block,
    attn_quant_fp8_block_pow2,
    attn_decode_paged_workspace_size,
    attn_decode_paged,
    attn_gather_paged,
    attn_prefill_paged,
    attn_cross_paged,
    attn_tile_class,
    attn_k_tile_range,
    attn_full_tile_range,
    attn_status_str,
    attn_abi_version,
    load,
)
