"""ctypes binding of libsplitkv (include/splitkv.h): argument marshalling only.

Each sk_* function here has the name and the arguments of the C entry point;
tensors may be passed as torch tensors (their data_ptr() is used) or as raw
integer device addresses.  A non-OK status raises SplitKVError carrying the
library's message.  Nothing here computes any part of the method.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPLITKV_LIBRARY names another build of the same library (the host-side
# AddressSanitizer build of split_kv_attention_amd.build.build_asan).
LIB_PATH = os.environ.get("SPLITKV_LIBRARY") or os.path.join(_PKG, "libsplitkv.so")

SK_OK, SK_ERR_INVALID_ARG, SK_ERR_UNSUPPORTED, SK_ERR_HIP = 0, 1, 2, 3
SK_MASK_NONE, SK_MASK_CAUSAL, SK_MASK_PREFIX_CAUSAL = 0, 1, 2
SK_F32, SK_BF16, SK_F16 = 0, 1, 2

# Every function include/splitkv.h declares.
EXPORTS = (
    "sk_abi_version",
    "sk_last_error",
    "sk_status_string",
    "sk_rows",
    "sk_split_kv",
    "sk_workspace_bytes",
    "sk_partial_scratch_bytes",
    "sk_partial_m_per_block",
    "sk_valid_split_counts",
    "sk_attn_partial",
    "sk_attn_partial_noalloc",
    "sk_attn_combine",
    "sk_attn_backward",
    "sk_backward_workspace_bytes",
    "sk_check_violations",
)


class SkProblem(ctypes.Structure):
    """Mirror of `sk_problem` (field order and types as in the header)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("split_kv", ctypes.c_int32),
        ("n_per_block", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("prefix_offset", ctypes.c_int64),
        ("last_valid_kv_index", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("reserved0", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("split_kv_per_seq", ctypes.c_void_p),
        ("prefix_offset_per_seq", ctypes.c_void_p),
        ("last_valid_per_seq", ctypes.c_void_p),
        ("q_stride_row", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("q_stride_batch", ctypes.c_int64),
        ("k_stride_row", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("k_stride_batch", ctypes.c_int64),
        ("v_stride_row", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("v_stride_batch", ctypes.c_int64),
        ("o_stride_row", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
        ("o_stride_batch", ctypes.c_int64),
        ("partial_scratch", ctypes.c_void_p),
        ("partial_scratch_bytes", ctypes.c_int64),
        ("window_left", ctypes.c_int64),
    ]


class SplitKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libsplitkv.so (built in-tree by split_kv_attention_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it first (python -m split_kv_attention_amd.build); "
            "there is no fallback implementation"
        )
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(SkProblem)
    vp = ctypes.c_void_p
    lib.sk_abi_version.restype = ctypes.c_int32
    lib.sk_abi_version.argtypes = []
    lib.sk_last_error.restype = ctypes.c_char_p
    lib.sk_last_error.argtypes = []
    lib.sk_status_string.restype = ctypes.c_char_p
    lib.sk_status_string.argtypes = [ctypes.c_int]
    lib.sk_rows.restype = ctypes.c_int64
    lib.sk_rows.argtypes = [P]
    lib.sk_split_kv.restype = ctypes.c_int32
    lib.sk_split_kv.argtypes = [P]
    lib.sk_workspace_bytes.restype = ctypes.c_int
    lib.sk_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.sk_partial_scratch_bytes.restype = ctypes.c_int64
    lib.sk_partial_scratch_bytes.argtypes = [P]
    lib.sk_partial_m_per_block.restype = ctypes.c_int32
    lib.sk_partial_m_per_block.argtypes = [P]
    lib.sk_valid_split_counts.restype = ctypes.c_int
    lib.sk_valid_split_counts.argtypes = [P, vp, vp]
    lib.sk_attn_partial.restype = ctypes.c_int
    lib.sk_attn_partial.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sk_attn_partial_noalloc.restype = ctypes.c_int
    lib.sk_attn_partial_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sk_attn_combine.restype = ctypes.c_int
    lib.sk_attn_combine.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sk_attn_backward.restype = ctypes.c_int
    lib.sk_attn_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp]
    lib.sk_backward_workspace_bytes.restype = ctypes.c_int64
    lib.sk_backward_workspace_bytes.argtypes = [P]
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.sk_check_violations.restype = ctypes.c_int64
    lib.sk_check_violations.argtypes = [i64p, i64p, i64p]
    if path is None:
        _lib = lib
    return lib


def _status_name(status: int) -> str:
    return {0: "SK_OK", 1: "SK_ERR_INVALID_ARG", 2: "SK_ERR_UNSUPPORTED", 3: "SK_ERR_HIP"}.get(status, str(status))


def _ptr(x) -> int | None:
    """Device address of a tensor (data_ptr) or an int; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != SK_OK:
        raise SplitKVError(status, load().sk_last_error().decode())


def sk_abi_version() -> int:
    return load().sk_abi_version()


def sk_status_string(status: int) -> str:
    return load().sk_status_string(status).decode()


def sk_last_error() -> str:
    return load().sk_last_error().decode()


def sk_rows(problem: SkProblem) -> int:
    r = load().sk_rows(ctypes.byref(problem))
    if r < 0:
        raise SplitKVError(SK_ERR_INVALID_ARG, sk_last_error())
    return r


def sk_workspace_bytes(problem: SkProblem) -> tuple[int, int]:
    o = ctypes.c_size_t(0)
    l = ctypes.c_size_t(0)
    _check(load().sk_workspace_bytes(ctypes.byref(problem), ctypes.byref(o), ctypes.byref(l)))
    return o.value, l.value


def sk_split_kv(problem: SkProblem) -> int:
    n = load().sk_split_kv(ctypes.byref(problem))
    if n < 0:
        raise SplitKVError(SK_ERR_INVALID_ARG, sk_last_error())
    return n


def sk_partial_scratch_bytes(problem: SkProblem) -> int:
    n = load().sk_partial_scratch_bytes(ctypes.byref(problem))
    if n < 0:
        raise SplitKVError(SK_ERR_INVALID_ARG, sk_last_error())
    return n


def sk_partial_m_per_block(problem: SkProblem) -> int:
    m = load().sk_partial_m_per_block(ctypes.byref(problem))
    if m < 0:
        raise SplitKVError(SK_ERR_UNSUPPORTED, sk_last_error())
    return m


def sk_valid_split_counts(problem: SkProblem, counts, stream=None) -> None:
    _check(load().sk_valid_split_counts(ctypes.byref(problem), _ptr(counts), _stream(stream)))


def sk_attn_partial(problem: SkProblem, q, k, v, o_part, lse_part, stream=None) -> None:
    _check(
        load().sk_attn_partial(
            ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), _stream(stream)
        )
    )


def sk_attn_partial_noalloc(problem: SkProblem, q, k, v, o_part, lse_part, stream=None) -> None:
    _check(
        load().sk_attn_partial_noalloc(
            ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), _stream(stream)
        )
    )


def sk_attn_combine(problem: SkProblem, o_part, lse_part, counts, out, lse_out, stream=None) -> None:
    _check(
        load().sk_attn_combine(
            ctypes.byref(problem), _ptr(o_part), _ptr(lse_part), _ptr(counts), _ptr(out), _ptr(lse_out),
            _stream(stream),
        )
    )


def sk_backward_workspace_bytes(problem: SkProblem) -> int:
    n = load().sk_backward_workspace_bytes(ctypes.byref(problem))
    if n < 0:
        raise SplitKVError(SK_ERR_INVALID_ARG, sk_last_error())
    return n


def sk_check_violations(lib: ctypes.CDLL | None = None):
    """(count, first site, first index, first limit) of a bounds-checked
    build (`lib`, default the loaded library); raises for a normal build."""
    lib = lib or load()
    site, index, limit = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    n = lib.sk_check_violations(ctypes.byref(site), ctypes.byref(index), ctypes.byref(limit))
    if n < 0:
        raise SplitKVError(SK_ERR_UNSUPPORTED, lib.sk_last_error().decode())
    return n, site.value, index.value, limit.value


def sk_attn_backward(problem: SkProblem, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes: int,
                     stream=None) -> None:
    _check(
        load().sk_attn_backward(
            ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace_bytes, _stream(stream),
        )
    )
