"""Decode-time attention on an int4 (or int8) group-affine KV cache for MI355X
(gfx950).

Thin Python binding over ``libkvq.so`` (the C ABI declared in
``include/kvq.h``). It only marshals arguments: PyTorch provides device memory
and the current HIP stream, every step of the computation runs in the HIP
kernels of ``csrc/``. There is no CPU fallback: if the library is missing the
import of the functions raises.
"""

from ._binding import (  # noqa: F401
    KVQ_F16,
    KVQ_F32,
    KERNEL_AUTO,
    KERNEL_MFMA,
    KERNEL_MFMA_SPLIT,
    KERNEL_MFMA_WAVE,
    KERNEL_VALU,
    Int4KVCache,
    KvqError,
    QuantKVCache,
    cache_bytes,
    decode_step,
    decode_step_noalloc,
    decode_step_single_launch,
    decode_workspace,
    decode_workspace_bytes,
    decode_step_rotated,
    hadamard_rotate,
    hbm_read,
    lib,
    lib_path,
    num_chunks,
    partials_buffers,
    quantize_kv_append,
    quantize_kv_append_rotated,
    sdpa_int4,
    sdpa_int4_partial,
    sdpa_int4_partial_timed,
    sdpa_int4_prefill,
    sdpa_int4_reduce,
    status_str,
    version,
)
