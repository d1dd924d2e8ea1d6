"""The bounds-checked build of the library on the GPU, through the C ABI.

libsplitkv_checked.so is the same source compiled with SK_CHECKED=1: each
kernel tests every global index it derives (work item, Q row, key range,
partial / piece / counts slots, combine row and split, the backward's rows,
keys and dQ split sums) against the extent it addresses, skips an access
that falls outside and counts it in a device record that
sk_check_violations reads and resets.

* Every workload of the parity suite, at full size, and small cases of each
  feature (f16, sliding window, key pieces, causal) run through both builds
  in one process: the checked one reports no violation and writes the same
  bits as the normal one in every buffer.
* The backward on three cases likewise: no violation, the same gradients.
* A packed batch whose cu_seqlens_k decreases (sequence 0 claims 8000 keys,
  the table's total is 4000) is reported at the key-range site with the
  table's total as the limit.  K and V hold all 8000 claimed rows, so every
  access either build could make stays inside the buffers.
"""
import ctypes
import dataclasses

import pytest
import torch

from parity import DEV, log
from split_kv_attention_amd import _lib, attention, build, workloads

pytestmark = pytest.mark.gpu

SITE_KEYS = 3  # last key row of a partial kernel's key range

CASES = list(workloads.CONFIGS) + [
    dataclasses.replace(workloads.LONG_PREFILL, name="checked_pieces_H12_Sq512_Sk6000_S3", sq=(512,), sk=(6000,)),
    dataclasses.replace(workloads.LONG_PREFILL, name="checked_f16_Sq300_Sk2000_S3", sq=(300,), sk=(2000,),
                        dtype="f16"),
    dataclasses.replace(workloads.VARLEN_BATCH_PREFIX, name="checked_window_varlen_prefix", sq=(130, 1, 257, 64),
                        sk=(500, 70, 1500, 3000), split_kv_per_seq=(2, 4, 6, 8),
                        prefix_offset_per_seq=(370, 69, 1243, 2936), last_valid_per_seq=(499, 69, 1499, 2999),
                        window_left=300),
    dataclasses.replace(workloads.CAUSAL_BF16, name="checked_causal_ragged", sq=(200, 200), sk=(333, 333),
                        split_kv=3),
]


@pytest.fixture(scope="module")
def checked_lib():
    return _lib.load(build.CHECKED_LIB_PATH)


def _forward(lib, prob, inputs):
    """counts -> partial -> combine through `lib` on poisoned buffers."""
    counts, o_part, lse_part, out, lse_out = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
    counts.fill_(-7)
    for t in (o_part, lse_part, out, lse_out):
        t.fill_(float("nan"))
    c = ctypes.byref(prob.c)
    s = torch.cuda.current_stream().cuda_stream
    q, k, v = (inputs[n].data_ptr() for n in "qkv")
    assert lib.sk_valid_split_counts(c, counts.data_ptr(), s) == 0, lib.sk_last_error()
    assert lib.sk_attn_partial(c, q, k, v, o_part.data_ptr(), lse_part.data_ptr(), s) == 0, lib.sk_last_error()
    assert lib.sk_attn_combine(c, o_part.data_ptr(), lse_part.data_ptr(), counts.data_ptr(), out.data_ptr(),
                               lse_out.data_ptr(), s) == 0, lib.sk_last_error()
    torch.cuda.synchronize()
    return dict(counts=counts, o_part=o_part, lse_part=lse_part, out=out, lse_out=lse_out)


def _same_bits(a, b):
    if a.dtype.is_floating_point:
        a, b = a.view(torch.int16 if a.element_size() == 2 else torch.int32), \
            b.view(torch.int16 if b.element_size() == 2 else torch.int32)
    return torch.equal(a, b)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_checked_build_reports_nothing_and_matches(w, checked_lib):
    log(f"checked {w.name}")
    assert _lib.sk_check_violations(checked_lib)[0] == 0  # nothing left over
    inputs = workloads.make_inputs(w, DEV, seed=5)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    ref = _forward(_lib.load(), prob, inputs)
    got = _forward(checked_lib, prob, inputs)
    n, site, index, limit = _lib.sk_check_violations(checked_lib)
    assert n == 0, f"{n} violations, first at site {site}: index {index} >= limit {limit}"
    for name in ref:
        assert _same_bits(ref[name], got[name]), name
    assert not torch.isnan(got["lse_out"]).all()


def test_checked_build_reports_keys_past_the_table_total(checked_lib):
    log("checked decreasing cu_seqlens_k")
    H, D, claimed, total = 2, 128, 8000, 4000
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    q = torch.randn((512, H, D), generator=g, device=DEV).to(torch.bfloat16)
    # K and V hold every row sequence 0 claims
    k = torch.randn((claimed, H, D), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((claimed, H, D), generator=g, device=DEV).to(torch.bfloat16)
    cu_q = torch.tensor([0, 256, 512], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, claimed, total], dtype=torch.int32, device=DEV)
    prob = attention.build_problem(q, k, v, split_kv=3, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=256,
                                   max_seqlen_k=claimed)
    assert _lib.sk_check_violations(checked_lib)[0] == 0
    _forward(checked_lib, prob, dict(q=q, k=k, v=v))
    n, site, index, limit = _lib.sk_check_violations(checked_lib)
    assert n > 0
    assert site == SITE_KEYS and limit == total and total <= index < claimed, (site, index, limit)
    # the record was reset by the read
    assert _lib.sk_check_violations(checked_lib)[0] == 0


BWD_CASES = [
    dataclasses.replace(workloads.LONG_PREFILL, name="checked_bwd_prefill_Sq300_Sk2000", sq=(300,), sk=(2000,)),
    dataclasses.replace(workloads.VARLEN_BATCH_PREFIX, name="checked_bwd_varlen_prefix", sq=(130, 1, 257, 64),
                        sk=(500, 70, 1500, 3000), heads=2, split_kv_per_seq=(2, 4, 6, 8),
                        prefix_offset_per_seq=(370, 69, 1243, 2936), last_valid_per_seq=(499, 69, 1499, 2999),
                        window_left=300),
    dataclasses.replace(workloads.DECODE_BF16, name="checked_bwd_decode_B4_H4_Sk3000", sq=(1,) * 4,
                        sk=(3000,) * 4, heads=4),
]


def _backward(lib, prob, inputs, out, lse, dout):
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    grads = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    nbytes = _lib.sk_backward_workspace_bytes(prob.c)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    st = lib.sk_attn_backward(ctypes.byref(prob.c), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), *(g.data_ptr() for g in grads), ws.data_ptr(),
                              nbytes, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.sk_last_error()
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_checked_backward_reports_nothing_and_matches(w, checked_lib):
    log(f"checked backward {w.name}")
    assert _lib.sk_check_violations(checked_lib)[0] == 0
    inputs = workloads.make_inputs(w, DEV, seed=8)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    fwd = _forward(_lib.load(), prob, inputs)
    dout = workloads.make_dout(w, DEV, 8)
    ref = _backward(_lib.load(), prob, inputs, fwd["out"], fwd["lse_out"], dout)
    got = _backward(checked_lib, prob, inputs, fwd["out"], fwd["lse_out"], dout)
    n, site, index, limit = _lib.sk_check_violations(checked_lib)
    assert n == 0, f"{n} violations, first at site {site}: index {index} >= limit {limit}"
    for name, r, g in zip(("dq", "dk", "dv"), ref, got):
        assert _same_bits(r, g), name
        assert not torch.isnan(g).any(), name
