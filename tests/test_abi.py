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


# ---------------------------------------------------------------------------
# Fuzzed problems: every entry point, with NULL tensors, must return a status
# (nothing can be enqueued without tensors) and the pure host queries must
# return without crashing, whatever the fields hold.  Under the sanitizer
# build (test_asan_host.py runs this file) any out-of-bounds host access in
# argument checking or planning aborts the run.
# ---------------------------------------------------------------------------
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

_I32 = st.one_of(st.integers(-3, 3), st.sampled_from([0, 1, 8, 63, 64, 65, 127, 128, 129, 192, 255, 256, 257,
                                                       4096, 65535, 65536, 2**31 - 1, -2**31]),
                 st.integers(-2**31, 2**31 - 1))
_I64 = st.one_of(st.integers(-3, 3), st.sampled_from([2**31, -2**31 - 1, 2**40, -2**40, 2**63 - 1, -2**63]),
                 st.integers(-2**63, 2**63 - 1))
_PTR = st.sampled_from([None, FAKE])
_SMALL_DIM = st.sampled_from([-1, 0, 1, 16, 32, 64, 96, 128, 192, 256, 257])
_FIELDS = st.fixed_dictionaries({
    "batch": _I32, "num_heads": _I32, "max_seqlen_q": _I32, "max_seqlen_k": _I32, "total_q": _I32,
    "head_dim_qk": _SMALL_DIM, "head_dim_v": _SMALL_DIM, "split_kv": _I32, "n_per_block": _I32,
    "mask": st.integers(-1, 3), "dtype": st.integers(-1, 3), "out_dtype": st.integers(-1, 3),
    "prefix_offset": _I64, "last_valid_kv_index": _I64,
    "softmax_scale": st.sampled_from([0.0, -1.0, 0.125, 1e-30, 1e30, float("inf"), float("nan")]),
    "reserved0": st.sampled_from([0, 0, 0, 1]),
    "cu_seqlens_q": _PTR, "cu_seqlens_k": _PTR, "split_kv_per_seq": _PTR, "prefix_offset_per_seq": _PTR,
    "last_valid_per_seq": _PTR,
    "q_stride_row": _I64, "q_stride_head": _I64, "q_stride_batch": _I64,
    "k_stride_row": _I64, "k_stride_head": _I64, "k_stride_batch": _I64,
    "v_stride_row": _I64, "v_stride_head": _I64, "v_stride_batch": _I64,
    "o_stride_row": _I64, "o_stride_head": _I64, "o_stride_batch": _I64,
    "partial_scratch": _PTR, "partial_scratch_bytes": _I64, "window_left": _I64,
})


@settings(max_examples=400, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(fields=_FIELDS)
def test_fuzzed_problems_are_answered_on_the_host(fields):
    p = _lib.SkProblem()
    for name, value in fields.items():
        setattr(p, name, value)
    lib = _lib.load()
    bp = ctypes.byref(p)
    # pure host queries
    lib.sk_rows(bp)
    lib.sk_split_kv(bp)
    o, l = ctypes.c_size_t(), ctypes.c_size_t()
    lib.sk_workspace_bytes(bp, ctypes.byref(o), ctypes.byref(l))
    lib.sk_partial_scratch_bytes(bp)
    lib.sk_partial_m_per_block(bp)
    lib.sk_backward_workspace_bytes(bp)
    # entry points without tensors: rejected, or a no-op for an empty problem
    statuses = [
        lib.sk_valid_split_counts(bp, None, None),
        lib.sk_attn_partial(bp, None, None, None, None, None, None),
        lib.sk_attn_partial_noalloc(bp, None, None, None, None, None, None),
        lib.sk_attn_combine(bp, None, None, None, None, None, None),
        lib.sk_attn_backward(bp, None, None, None, None, None, None, None, None, None, None, 0, None),
    ]
    for s in statuses:
        assert s in (sk.SK_OK, sk.SK_ERR_INVALID_ARG, sk.SK_ERR_UNSUPPORTED), s
        if s != sk.SK_OK:
            assert lib.sk_last_error().decode()
    if any(s == sk.SK_OK for s in statuses[:4]):
        # only a problem with no rows may succeed without tensors
        assert p.batch == 0 or p.max_seqlen_q == 0 or lib.sk_rows(bp) == 0


_NEAR = st.fixed_dictionaries({
    "batch": st.integers(0, 70000), "num_heads": st.integers(1, 70000), "max_seqlen_q": st.integers(0, 300000),
    "max_seqlen_k": st.integers(0, 2**31 - 1), "head_dim_qk": st.sampled_from([64, 128, 192, 256]),
    "head_dim_v": st.sampled_from([64, 128]), "split_kv": st.integers(0, 130), "n_per_block": st.integers(1, 4096),
    "mask": st.integers(0, 2), "dtype": st.integers(0, 2), "prefix_offset": _I64, "last_valid_kv_index": _I64,
    "window_left": st.one_of(st.just(-1), st.integers(0, 2**40)), "packed": st.booleans(),
    "total_q": st.integers(0, 2**31 - 1), "per_seq": st.booleans(),
})


@settings(max_examples=400, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(f=_NEAR)
def test_fuzzed_valid_looking_problems_are_answered_on_the_host(f):
    """Problems that pass most checks, so that work planning, the automatic
    split count and the workspace sizes are reached: the same contract."""
    p = _good()
    for name in ("batch", "num_heads", "max_seqlen_q", "max_seqlen_k", "head_dim_qk", "head_dim_v", "split_kv",
                 "n_per_block", "mask", "dtype", "prefix_offset", "last_valid_kv_index", "window_left"):
        setattr(p, name, f[name])
    p.out_dtype = f["dtype"]
    if f["packed"]:
        p.cu_seqlens_q, p.cu_seqlens_k, p.total_q = FAKE, FAKE, f["total_q"]
    if f["per_seq"] and f["split_kv"] > 0:
        p.split_kv_per_seq = p.prefix_offset_per_seq = p.last_valid_per_seq = FAKE
    lib = _lib.load()
    bp = ctypes.byref(p)
    rows = lib.sk_rows(bp)
    lib.sk_split_kv(bp)
    lib.sk_workspace_bytes(bp, None, None)
    lib.sk_partial_scratch_bytes(bp)
    lib.sk_partial_m_per_block(bp)
    lib.sk_backward_workspace_bytes(bp)
    for s in (lib.sk_valid_split_counts(bp, None, None),
              lib.sk_attn_partial(bp, None, None, None, None, None, None),
              lib.sk_attn_partial_noalloc(bp, None, None, None, None, None, None),
              lib.sk_attn_combine(bp, None, None, None, None, None, None)):
        assert s in (sk.SK_OK, sk.SK_ERR_INVALID_ARG, sk.SK_ERR_UNSUPPORTED), s
        if s == sk.SK_OK:
            assert p.batch == 0 or p.max_seqlen_q == 0 or rows == 0
    s = lib.sk_attn_backward(bp, None, None, None, None, None, None, None, None, None, None, 0, None)
    assert s in (sk.SK_OK, sk.SK_ERR_INVALID_ARG, sk.SK_ERR_UNSUPPORTED), s


def test_plain_c_client_compiles_against_the_header():
    """tests/c_client/sk_client.c (a C99 program that includes only the
    header and the HIP runtime API) builds with -Wall -Wextra -Werror and
    links libsplitkv.so by name."""
    exe = build.build_c_client()
    assert os.access(exe, os.X_OK)
    deps = subprocess.run(["ldd", exe], capture_output=True, text=True).stdout
    assert "libsplitkv.so" in deps
