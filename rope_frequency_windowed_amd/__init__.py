"""Windowed-RoPE attention (the ATFlash idea) for AMD Instinct MI355X (gfx950).

Causal attention in which rotary pair p keeps its share of the query-key
product only within a distance window proportional to its wavelength (source
page "ATFlash: RoPE-Frequenzen kuerzen Attention-Arbeit um bis zu 57 Prozent",
sudo-ai.de, section "Was ATFlash anders macht"), followed by the unchanged
online softmax times V (same page, section "Die Zahlen - und ihre Grenze").

The computation lives in librfw_atf.so (HIP kernels for gfx950 behind the C
ABI in include/atf.h); this package is a thin ctypes binding with the same
function names.
"""
from ._binding import (  # noqa: F401
    ALPHA_INF, ATF_BF16, ATF_F32, EXPORTED, LIB_PATH, W_INF, AtfError, atf_decode, atf_decode_kcache,
    atf_decode_kcache_bytes, atf_decode_pack_k, atf_decode_append_kv, atf_decode_paged, atf_decode_paged_noalloc,
    atf_decode_paged_workspace_bytes, NOALLOC_SCRATCH_BYTES,
    atf_decode_workspace_bytes, atf_paged_page_bytes,
    atf_paged_write, atf_prefill, atf_prefill_attend, atf_prefill_chunk, atf_prefill_chunk_workspace_bytes,
    atf_prefill_cache_append, atf_prefill_cache_bytes, atf_prefill_cached_scratch_bytes, atf_prefill_chunk_cached,
    atf_prefill_prepare_kv,
    atf_prefill_workspace_bytes, atf_skipped_pair_products, atf_version, atf_window_table,
    library, workspace,
)
