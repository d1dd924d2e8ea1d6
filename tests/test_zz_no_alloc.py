"""sk_attn_partial_noalloc against sk_attn_partial (GPU, through the C ABI).

The no-alloc variant runs the same kernels with the library's own static
scratch for the last round's key pieces instead of the caller's buffer, so
its partials must equal sk_attn_partial's with a caller-allocated scratch
bit for bit.  Calls in a row, each on a smaller problem than the last, all
of which use the key pieces (each differs from a run without scratch, where
every item runs whole); the merged output of each is also checked against
the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity import DEV, compare, log
from split_kv_attention_amd import _lib, attention, workloads

pytestmark = pytest.mark.gpu

# Every shape leaves a partial last round of workgroups whose items are cut
# into key pieces (16+ key tiles per split).  The first has 16 x 17 = 272
# items of 256 rows, enough for the 256-row kernel on a 256-CU device (the
# last 16 run as pieces); the others run the 128-row kernel.
CASES = [
    dataclasses.replace(workloads.LONG_PREFILL, name="noalloc_H16_Sq200_Sk17408_S17", heads=16, sq=(200,),
                        sk=(17 * 1024,), split_kv=17),
    dataclasses.replace(workloads.LONG_PREFILL, name="noalloc_H12_Sq512_Sk6000_S3", sq=(512,), sk=(6000,)),
    dataclasses.replace(workloads.LONG_PREFILL, name="noalloc_H8_Sq256_Sk4000_S3", heads=8, sq=(256,), sk=(4000,)),
]


def _partials(prob, inputs, fn, scratch: bool):
    c = prob.c
    saved = (c.partial_scratch, c.partial_scratch_bytes)
    if not scratch:
        c.partial_scratch, c.partial_scratch_bytes = None, 0
    counts, o_part, lse_part, out, lse_out = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
    o_part.fill_(float("nan"))
    lse_part.fill_(float("nan"))
    fn(c, inputs["q"], inputs["k"], inputs["v"], o_part, lse_part)
    c.partial_scratch, c.partial_scratch_bytes = saved
    _lib.sk_valid_split_counts(c, counts)
    _lib.sk_attn_combine(c, o_part, lse_part, counts, out, lse_out)
    torch.cuda.synchronize()
    return dict(counts=counts, o_part=o_part, lse_part=lse_part, out=out, lse_out=lse_out, poisoned=True)


def _same(a, b):
    return torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0)) and \
        torch.equal(torch.isnan(a), torch.isnan(b))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_partial_on_two_calls(order):
    for w in CASES:
        log(f"noalloc {w.name}")
        inputs = workloads.make_inputs(w, DEV, seed=11)
        prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
        assert prob.c.partial_scratch and _lib.sk_partial_scratch_bytes(prob.c) > 0
        log(f"  {prob.m_per_block}-row blocks")
        ref = _partials(prob, inputs, _lib.sk_attn_partial, scratch=True)
        got = _partials(prob, inputs, _lib.sk_attn_partial_noalloc, scratch=True)
        whole = _partials(prob, inputs, _lib.sk_attn_partial, scratch=False)
        assert _same(got["o_part"], ref["o_part"]) and _same(got["lse_part"], ref["lse_part"]), w.name
        assert torch.equal(got["out"], ref["out"]) and torch.equal(got["lse_out"], ref["lse_out"]), w.name
        # the key pieces ran: whole items round their weights elsewhere
        assert not _same(whole["o_part"], ref["o_part"]), f"{w.name}: no key pieces were used"
        st = compare(w, inputs, prob, got, label=f"{w.name} noalloc")
        log(f"  {st}")
        del inputs, prob, ref, got, whole
        torch.cuda.empty_cache()


def test_noalloc_ignores_the_callers_scratch_and_rejects_bad_arguments():
    w = CASES[-1]
    inputs = workloads.make_inputs(w, DEV, seed=12)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    ref = _partials(prob, inputs, _lib.sk_attn_partial, scratch=True)
    got = _partials(prob, inputs, _lib.sk_attn_partial_noalloc, scratch=False)  # NULL caller scratch
    assert _same(got["o_part"], ref["o_part"]) and _same(got["lse_part"], ref["lse_part"])
    with pytest.raises(_lib.SplitKVError):
        _lib.sk_attn_partial_noalloc(prob.c, None, inputs["k"], inputs["v"], got["o_part"], got["lse_part"])
    torch.cuda.synchronize()
    assert np.isfinite(got["out"].float().cpu().numpy()).all()


def test_noalloc_on_the_decode_kernel_needs_no_scratch():
    """One-row sequences run on the decode kernel, which uses no piece
    scratch: the no-alloc call gives the same bits and needs none."""
    w = dataclasses.replace(workloads.DECODE_BF16, name="noalloc_decode_B8_H4_Sk3000", sq=(1,) * 8, sk=(3000,) * 8,
                            heads=4)
    inputs = workloads.make_inputs(w, DEV, seed=13)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    assert prob.m_per_block == 1 and _lib.sk_partial_scratch_bytes(prob.c) == 0
    ref = _partials(prob, inputs, _lib.sk_attn_partial, scratch=True)
    got = _partials(prob, inputs, _lib.sk_attn_partial_noalloc, scratch=True)
    assert _same(got["o_part"], ref["o_part"]) and _same(got["lse_part"], ref["lse_part"])
    assert torch.equal(got["out"], ref["out"]) and torch.equal(got["lse_out"], ref["lse_out"])
    st = compare(w, inputs, prob, got, label=f"{w.name} noalloc")
    log(f"  {st}")
