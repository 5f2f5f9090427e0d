"""TurboQuant KV-cache decode path for AMD Instinct MI355X (gfx950).

The work happens in libtq.so (hand-written HIP, C ABI in include/tq.h); this
package is its thin ctypes binding. See binding.py for the entry points:
tq_rht, tq_encode_kv, tq_qjl_sketch, tq_attend_decode, tq_append_attend_decode,
tq_append_chunk_attend_decode,
tq_attend_decode_noalloc (no workspace: a static per-GPU scratch buffer),
tq_attend_prefill, the group-affine variant tq_affine_encode_kv /
tq_affine_attend_decode (+ host helpers).
"""

from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, TQ_BF16, TQ_ERR_ALIGN, TQ_ERR_ARG, TQ_ERR_CAPACITY,
    TQ_ERR_HIP, TQ_ERR_NO_DEVICE, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_F16,
    TQ_F32, TQ_OK, Config, PackedCache, TqError, lib, tq_append_attend_decode,
    tq_append_chunk_attend_decode,
    tq_attend_decode, tq_attend_decode_noalloc, tq_attend_prefill,
    tq_bits_split, tq_cache_bytes, tq_codebook, tq_codebook_ex, tq_config, tq_cache,
    TQ_CODEBOOK_GAUSS, TQ_CODEBOOK_SPHERE,
    tq_dense_decode_bf16, tq_dense_workspace_bytes, tq_encode_kv, tq_num_splits,
    tq_qjl_sketch, tq_read_probe, tq_rht, tq_signs, tq_strerror, tq_workspace_bytes,
    workspace, AffineCache, AffineConfig, tq_affine_attend_decode, tq_affine_cache_bytes,
    tq_affine_config, tq_affine_cache, tq_affine_encode_kv, tq_affine_num_splits,
    tq_affine_workspace_bytes,
)
