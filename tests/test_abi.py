"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function include/splitkv.h declares, its struct layout matches the Python
mirror, and every argument error is reported before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

import split_kv_attention_amd as sk
from split_kv_attention_amd import _lib, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splitkv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(sk_\w+)\s*\(", text, flags=re.M)))


def test_library_builds_and_loads():
    lib = _lib.load()
    version = int(re.search(r"#define SK_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.sk_abi_version() == version


def test_every_declared_function_is_exported():
    decl = _declared_functions()
    assert len(decl) >= 9, decl
    lib = _lib.load()
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTS) == decl


def test_struct_layout_matches_header(tmp_path):
    fields = [f for f, _ in _lib.SkProblem._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "splitkv.h"', "int main(void){",
             'printf("size %zu\\n", sizeof(sk_problem));']
    for f in fields:
        lines.append(f'printf("{f} %zu\\n", offsetof(sk_problem, {f}));')
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.split() for l in out if l)
    assert int(got["size"]) == ctypes.sizeof(_lib.SkProblem)
    for f in fields:
        assert int(got[f]) == getattr(_lib.SkProblem, f).offset, f


def _good():
    p = _lib.SkProblem()
    p.batch, p.num_heads, p.max_seqlen_q, p.max_seqlen_k = 2, 4, 100, 300
    p.head_dim_qk, p.head_dim_v = 128, 128
    p.split_kv, p.n_per_block = 4, 64
    p.mask, p.dtype, p.out_dtype = sk.SK_MASK_CAUSAL, sk.SK_BF16, sk.SK_BF16
    p.last_valid_kv_index = -1
    p.window_left = -1
    p.softmax_scale = 128 ** -0.5
    p.q_stride_row, p.q_stride_head, p.q_stride_batch = 128, 100 * 128, 4 * 100 * 128
    p.k_stride_row, p.k_stride_head, p.k_stride_batch = 128, 300 * 128, 4 * 300 * 128
    p.v_stride_row, p.v_stride_head, p.v_stride_batch = 128, 300 * 128, 4 * 300 * 128
    p.o_stride_row, p.o_stride_head, p.o_stride_batch = 128, 100 * 128, 4 * 100 * 128
    return p


def test_rows_workspace_and_block_size():
    p = _good()
    assert sk.sk_rows(p) == 200
    o, l = sk.sk_workspace_bytes(p)
    assert o == 4 * 4 * 200 * 128 * 4 and l == 4 * 4 * 200 * 4
    assert sk.sk_partial_m_per_block(p) >= 1
    p.cu_seqlens_q = 0x1000
    p.total_q = 77
    assert sk.sk_rows(p) == 77


def test_one_row_problems_take_the_decode_kernel():
    """A problem whose sequences hold one query row at most runs on the
    decode kernel (block of one row, no key pieces) where it exists: 16-bit
    storage with head dims 64/64 or 128/128."""
    for dtype in (sk.SK_BF16, sk.SK_F16):
        for d in (64, 128):
            p = _good()
            p.max_seqlen_q, p.dtype, p.out_dtype = 1, dtype, dtype
            p.head_dim_qk = p.head_dim_v = d
            assert sk.sk_partial_m_per_block(p) == 1
            assert _lib.sk_partial_scratch_bytes(p) == 0
    p = _good()
    p.max_seqlen_q = 1
    p.head_dim_qk, p.head_dim_v = 192, 128
    assert sk.sk_partial_m_per_block(p) == 128  # the MFMA kernel
    p = _good()
    p.max_seqlen_q, p.dtype, p.out_dtype = 1, sk.SK_F32, sk.SK_F32
    assert sk.sk_partial_m_per_block(p) == 64  # the f32 kernel
    p = _good()
    p.max_seqlen_q = 2
    assert sk.sk_partial_m_per_block(p) == 128


# A non-NULL, aligned address that is never dereferenced: every call below
# must fail validation on the host first.
FAKE = 1 << 20


def _all_calls(p):
    lib = _lib.load()
    pp = ctypes.byref(p)
    return [
        lib.sk_valid_split_counts(pp, FAKE, None),
        lib.sk_attn_partial(pp, FAKE, FAKE, FAKE, FAKE, FAKE, None),
        lib.sk_attn_combine(pp, FAKE, FAKE, FAKE, FAKE, FAKE, None),
        lib.sk_attn_backward(pp, *([FAKE] * 10), 1 << 40, None),
    ]


BAD = [
    ("num_heads", 0, sk.SK_ERR_INVALID_ARG),
    ("batch", -1, sk.SK_ERR_INVALID_ARG),
    ("batch", 65536, sk.SK_ERR_UNSUPPORTED),
    ("max_seqlen_q", -5, sk.SK_ERR_INVALID_ARG),
    ("split_kv", -1, sk.SK_ERR_INVALID_ARG),
    ("split_kv", 1000, sk.SK_ERR_UNSUPPORTED),
    ("n_per_block", 0, sk.SK_ERR_INVALID_ARG),
    ("mask", 7, sk.SK_ERR_INVALID_ARG),
    ("dtype", 9, sk.SK_ERR_INVALID_ARG),
    ("out_dtype", 9, sk.SK_ERR_INVALID_ARG),
    ("softmax_scale", 0.0, sk.SK_ERR_INVALID_ARG),
    ("softmax_scale", float("inf"), sk.SK_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), sk.SK_ERR_INVALID_ARG),
    ("head_dim_qk", 0, sk.SK_ERR_INVALID_ARG),
    ("head_dim_v", 512, sk.SK_ERR_UNSUPPORTED),
    ("reserved0", 1, sk.SK_ERR_INVALID_ARG),
    ("k_stride_row", -8, sk.SK_ERR_INVALID_ARG),
    ("partial_scratch_bytes", -1, sk.SK_ERR_INVALID_ARG),
    ("window_left", -2, sk.SK_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("field,value,status", BAD, ids=[f"{f}={v}" for f, v, _ in BAD])
def test_invalid_arguments_are_rejected_on_the_host(field, value, status):
    p = _good()
    setattr(p, field, value)
    for st in _all_calls(p):
        assert st == status
        assert sk.sk_last_error() != ""


def test_null_problem_and_null_tensors():
    lib = _lib.load()
    assert lib.sk_valid_split_counts(None, FAKE, None) == sk.SK_ERR_INVALID_ARG
    p = _good()
    pp = ctypes.byref(p)
    assert lib.sk_valid_split_counts(pp, None, None) == sk.SK_ERR_INVALID_ARG
    assert lib.sk_attn_partial(pp, None, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_INVALID_ARG
    assert lib.sk_attn_partial(pp, FAKE, FAKE, FAKE, None, FAKE, None) == sk.SK_ERR_INVALID_ARG
    assert lib.sk_attn_combine(pp, FAKE, FAKE, None, None, None, None) == sk.SK_ERR_INVALID_ARG


def test_unsupported_layouts_are_rejected():
    lib = _lib.load()
    p = _good()
    p.q_stride_row = 130  # not a multiple of 8 bf16 elements
    assert lib.sk_attn_partial(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_UNSUPPORTED
    p = _good()
    assert lib.sk_attn_partial(ctypes.byref(p), FAKE + 2, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_UNSUPPORTED
    p = _good()
    p.head_dim_qk, p.head_dim_v = 96, 96  # valid, but no kernel instantiated
    assert lib.sk_attn_partial(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_UNSUPPORTED
    assert lib.sk_partial_m_per_block(ctypes.byref(p)) == -1
    p = _good()
    p.head_dim_v = 126
    assert lib.sk_attn_combine(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_UNSUPPORTED


def test_automatic_split_count_on_the_host():
    lib = _lib.load()
    p = _good()
    assert lib.sk_split_kv(ctypes.byref(p)) == p.split_kv  # explicit counts pass through
    p.split_kv = 0
    n = lib.sk_split_kv(ctypes.byref(p))
    assert 1 <= n <= 8  # 1 without a GPU (no CU count to fill)
    p.max_seqlen_k = 8191  # below the key threshold: unsplit on any device
    assert lib.sk_split_kv(ctypes.byref(p)) == 1
    p.split_kv_per_seq = FAKE  # per-sequence counts need an explicit maximum
    assert lib.sk_split_kv(ctypes.byref(p)) == -1
    assert lib.sk_attn_partial(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_INVALID_ARG
    assert "split_kv_per_seq" in sk.sk_last_error()


def test_partial_scratch_checks():
    lib = _lib.load()
    p = _good()
    assert lib.sk_partial_scratch_bytes(ctypes.byref(p)) >= 0  # 0 without a GPU
    p.num_heads = 0
    assert lib.sk_partial_scratch_bytes(ctypes.byref(p)) == -1
    p = _good()
    p.partial_scratch = FAKE + 4  # not 16-byte aligned
    p.partial_scratch_bytes = 1 << 20
    assert lib.sk_attn_partial(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None) == sk.SK_ERR_INVALID_ARG
    assert "aligned" in sk.sk_last_error()


def test_empty_problems_are_no_ops():
    """Nothing to do (no sequence, or no query row) is success, with no launch."""
    p = _good()
    p.batch = 0
    assert _all_calls(p) == [sk.SK_OK] * 4
    p = _good()
    p.max_seqlen_q = 0
    assert _all_calls(p)[:3] == [sk.SK_OK] * 3  # the backward still zeroes dK, dV
    p.max_seqlen_k = 0
    assert _all_calls(p)[3] == sk.SK_OK


def _backward(p, ws=FAKE, ws_bytes=1 << 40, **ptrs):
    args = {n: FAKE for n in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv")}
    args.update(ptrs)
    return _lib.load().sk_attn_backward(ctypes.byref(p), *args.values(), ws, ws_bytes, None)


def test_backward_workspace_and_host_checks():
    p = _good()  # H = 4, S = 4, 200 rows, D_qk = 128
    assert sk.sk_backward_workspace_bytes(p) == 3328 + 4 * 4 * 200 * 128 * 4  # D (256-aligned), then dQ sums
    p.num_heads = 0
    with pytest.raises(sk.SplitKVError):
        sk.sk_backward_workspace_bytes(p)
    for field, value in (("dtype", sk.SK_F32), ("out_dtype", _lib.SK_F16), ("head_dim_qk", 96),
                         ("q_stride_row", 132)):
        p = _good()
        setattr(p, field, value)
        if field == "dtype":
            p.out_dtype = sk.SK_F32
        assert _backward(p) == sk.SK_ERR_UNSUPPORTED, field
    p = _good()
    need = sk.sk_backward_workspace_bytes(p)
    assert _backward(p, ws_bytes=need - 1) == sk.SK_ERR_INVALID_ARG
    assert "workspace" in sk.sk_last_error()
    assert _backward(p, ws=None, ws_bytes=need) == sk.SK_ERR_INVALID_ARG
    assert _backward(p, ws_bytes=-1) == sk.SK_ERR_INVALID_ARG
    assert _backward(p, dq=None) == sk.SK_ERR_INVALID_ARG
    assert _backward(p, dk=FAKE + 8) == sk.SK_ERR_UNSUPPORTED
    assert _backward(p, ws=FAKE + 8) == sk.SK_ERR_UNSUPPORTED
    assert _backward(p, lse=FAKE + 2) == sk.SK_ERR_INVALID_ARG


def test_status_strings():
    assert sk.sk_status_string(0) == "SK_OK"
    assert sk.sk_status_string(1) == "SK_ERR_INVALID_ARG"
    assert sk.sk_status_string(2) == "SK_ERR_UNSUPPORTED"
    assert sk.sk_status_string(3) == "SK_ERR_HIP"


def test_binding_raises_without_the_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "libsplitkv.so"))


def test_split_kv_error_carries_the_message():
    p = _good()
    p.split_kv = -2
    with pytest.raises(sk.SplitKVError, match="split_kv"):
        sk.sk_valid_split_counts(p, FAKE, 0)


def test_normal_build_has_no_bounds_check_record():
    lib = _lib.load()
    assert lib.sk_check_violations(None, None, None) == -1
    assert "SK_CHECKED" in lib.sk_last_error().decode()
    with pytest.raises(sk.SplitKVError, match="bounds-checked"):
        _lib.sk_check_violations()


def test_checked_build_links_and_exports_every_function():
    lib = _lib.load(build.build_checked())
    assert lib.sk_abi_version() == _lib.load().sk_abi_version()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # host-side argument checks are the same code in both builds
    p = _good()
    p.split_kv = -2
    assert lib.sk_valid_split_counts(ctypes.byref(p), FAKE, 0) == sk.SK_ERR_INVALID_ARG
