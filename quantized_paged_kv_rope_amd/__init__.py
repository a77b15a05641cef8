"""MI355X (gfx950) paged KV-record codec: fused RoPE + MXFP8 quantise +
paged insert (also into plain bf16 and per-tensor-scaled fp8 caches), and the
paged dequantise-and-gather, for 512-dim MLA latent KV.

The compute lives in ``libkvrec.so`` (HIP kernels behind the C ABI of
``include/kvrec.h``); :mod:`.binding` marshals torch tensors into it. The
library is loaded on first use, so importing this package (for instance for
:mod:`.workloads`) needs neither a GPU nor a built library, while every
compute call fails loudly without them.
"""
from .binding import (  # noqa: F401
    HEAD_DIM,
    RECORD_BF16,
    RECORD_FP8,
    RECORD_LEGACY,
    RECORD_MXFP8,
    ROPE_DIM,
    KvrecError,
    alloc_cache,
    cache_descriptor,
    kvrec_expand_candidates,
    kvrec_gather,
    insert_options,
    kvrec_insert,
    kvrec_insert_ex,
    kvrec_insert_full,
    kvrec_insert_options,
    kvrec_page_stride,
    kvrec_qnorm_rope_insert,
    kvrec_status_str,
    load_library,
)
