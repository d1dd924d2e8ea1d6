"""split_kv_attention_amd: split-KV attention (forward and backward) for AMD Instinct MI355X.

The computation lives in libsplitkv.so (hand-written HIP kernels for gfx950,
C ABI in include/splitkv.h).  This package is its thin Python binding:
`_lib` mirrors the C entry points one to one, `attention` builds problems from
torch tensors and allocates outputs, `workloads` draws seeded synthetic inputs.
There is no CPU or PyTorch fallback: without the built library every call
raises.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    SK_BF16,
    SK_ERR_HIP,
    SK_ERR_INVALID_ARG,
    SK_ERR_UNSUPPORTED,
    SK_F16,
    SK_F32,
    SK_MASK_CAUSAL,
    SK_MASK_NONE,
    SK_MASK_PREFIX_CAUSAL,
    SK_OK,
    SkProblem,
    SplitKVError,
    load,
    sk_abi_version,
    sk_attn_backward,
    sk_attn_combine,
    sk_attn_partial,
    sk_attn_partial_noalloc,
    sk_backward_workspace_bytes,
    sk_last_error,
    sk_partial_m_per_block,
    sk_rows,
    sk_status_string,
    sk_valid_split_counts,
    sk_workspace_bytes,
)
