"""GPU parity: libsplitkv (through its C ABI) against the float64 oracle.

Small cases are compared on every row; the full-size workloads, in the launch
configuration the benchmark times, on every row and head (long-context
prefill in bf16 and f16 storage, both packed batches) or on every
(sequence, head) pair (decode, the oracle fed one sequence at a time).
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import adapter
from parity import DEV, compare, log, run_gpu, sample_rows
from split_kv_attention_amd import _lib, attention, workloads
from split_kv_attention_amd.workloads import Workload

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "split_counts_worked_examples.json")


def _shrink(w: Workload, **kw) -> Workload:
    return dataclasses.replace(w, **kw)


# ---------------------------------------------------------------------------
# counts: bit-exact
# ---------------------------------------------------------------------------

def _gpu_counts(w: Workload):
    inputs = workloads.make_inputs(_shrink(w, d_qk=16, d_v=16, dtype="f32"), DEV) if w.packed else None
    if inputs is None:
        # dense: counts only need the problem description, tiny tensors suffice
        q = torch.zeros(1, device=DEV).expand(w.batch, w.heads, w.sq[0], 16)
        k = torch.zeros(1, device=DEV).expand(w.batch, w.heads, w.sk[0], 16)
        inputs = {"q": q, "k": k, "v": k}
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    counts = torch.full((prob.rows,), -7, dtype=torch.int32, device=DEV)
    _lib.sk_valid_split_counts(prob.c, counts)
    torch.cuda.synchronize()
    return counts.cpu().numpy()


@pytest.mark.parametrize("w", workloads.CONFIGS, ids=lambda w: w.name)
def test_counts_bit_exact_on_every_workload(w):
    log(f"counts {w.name}")
    np.testing.assert_array_equal(_gpu_counts(w), adapter.counts(w))


def test_counts_worked_examples_on_gpu():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        w = Workload(c["name"], heads=1, sq=(c["sq"],), sk=(c["sk"],), d_qk=16, d_v=16, split_kv=c["split_kv"],
                     n_per_block=c["n_per_block"], mask=c["mask"], prefix_offset=c["prefix_offset"],
                     last_valid_kv_index=c["last_valid"], dtype="f32")
        exp = c["expected"] if "expected" in c else sum(([v] * n for v, n in c["expected_runs"]), [])
        np.testing.assert_array_equal(_gpu_counts(w), np.array(exp), err_msg=c["name"])


def test_counts_random_varlen_sweep():
    rng = np.random.default_rng(11)
    for it in range(40):
        B = int(rng.integers(1, 6))
        sq = tuple(int(x) for x in rng.integers(0, 300, B))
        sk = tuple(int(x) for x in rng.integers(0, 2000, B))
        mask = ["none", "causal", "prefix_causal"][it % 3]
        S = int(rng.integers(1, 12))
        w = Workload(f"sweep{it}", heads=2, sq=sq, sk=sk, d_qk=16, d_v=16, split_kv=S,
                     split_kv_per_seq=tuple(int(x) for x in rng.integers(1, S + 1, B)),
                     n_per_block=int(rng.choice([1, 16, 32, 64, 100])), mask=mask, packed=True, dtype="f32",
                     prefix_offset_per_seq=tuple(int(x) for x in rng.integers(-200, 2000, B)),
                     last_valid_per_seq=tuple(int(x) for x in rng.integers(-1, 2500, B)))
        np.testing.assert_array_equal(_gpu_counts(w), adapter.counts(w), err_msg=str(w))


# ---------------------------------------------------------------------------
# end to end on every row (small cases)
# ---------------------------------------------------------------------------

def test_tiny_f32_all_rows():
    w = workloads.TINY_F32
    log(f"e2e {w.name}")
    inputs, prob, res = run_gpu(w)
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


def test_causal_bf16_all_rows_and_empty_splits():
    w = workloads.CAUSAL_BF16
    log(f"e2e {w.name}")
    inputs, prob, res = run_gpu(w)
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")
    # Early rows have empty splits of two kinds.  A split holding keys for
    # the block but none the row sees is written as exactly 0 / -inf; a split
    # with no key for the whole block is skipped (real early exit) and keeps
    # the NaN the buffers were poisoned with.  Which slots are skipped
    # follows from the block partition at the kernel's own query block, so
    # the expected set comes from the oracle at prob.m_per_block.
    lp = res["lse_part"].cpu().numpy()
    op = res["o_part"].cpu().numpy()
    mpb = prob.m_per_block
    expect_skipped = np.zeros(lp.shape, dtype=bool)  # [H][S][rows]
    for b, (spec, r0) in enumerate(zip(adapter.seq_specs(w), adapter.row_starts(w))):
        for r in range(spec.sq):
            expect_skipped[:, oracle.block_populated_splits(spec, mpb, r):, r0 + r] = True
    row_empty = np.isneginf(lp)
    skipped = np.isnan(lp)
    np.testing.assert_array_equal(skipped, expect_skipped)
    assert row_empty.any()  # rows near a block's start see none of its later splits' keys
    assert (op[np.broadcast_to(row_empty[..., None], op.shape)] == 0).all()
    assert np.isnan(op[np.broadcast_to(skipped[..., None], op.shape)]).all()


SMALL = [
    _shrink(workloads.LONG_PREFILL, name="prefill_small_Sq300_Sk2000_S3", sq=(300,), sk=(2000,)),
    _shrink(workloads.VARLEN_BATCH, name="varlen_small", sq=(130, 1, 257, 64), sk=(500, 70, 1500, 3000),
            split_kv_per_seq=(2, 4, 6, 8)),
    _shrink(workloads.VARLEN_BATCH_PREFIX, name="varlen_prefix_small", sq=(130, 1, 257, 64), sk=(500, 70, 1500, 3000),
            split_kv_per_seq=(2, 4, 6, 8), prefix_offset_per_seq=(370, 69, 1243, 2936),
            last_valid_per_seq=(499, 69, 1499, 2999)),
    # 63 (sequence, split) pairs: ranked longest first; 189 groups, not a multiple of the 8 XCDs
    _shrink(workloads.VARLEN_BATCH, name="varlen_63_pairs_ranked", heads=3, split_kv=7, split_kv_per_seq=None,
            sq=(33, 1, 70, 5, 128, 129, 2, 64, 17), sk=(900, 64, 1200, 31, 700, 2500, 5, 333, 1024)),
    # 77 pairs: beyond the ranked range, identity order
    _shrink(workloads.VARLEN_BATCH, name="varlen_77_pairs_unranked", heads=2, split_kv=7,
            split_kv_per_seq=(7, 1, 3, 7, 5, 2, 7, 6, 4, 7, 1),
            sq=(33, 1, 70, 5, 128, 129, 2, 64, 17, 200, 9), sk=(900, 64, 1200, 31, 700, 2500, 5, 333, 1024, 222, 4000)),
    # dense rows flattened across sequences in the combine: one block spans
    # several sequences with their own split counts, offsets and last keys
    _shrink(workloads.DECODE_BF16, name="dense_B7_Sq3_per_seq_params", sq=(3,) * 7, sk=(700,) * 7, heads=3,
            split_kv=6, split_kv_per_seq=(1, 2, 3, 6, 5, 4, 6), mask="prefix_causal",
            prefix_offset_per_seq=(697, 0, 300, -2, 696, 150, 650), last_valid_per_seq=(699, 699, 500, 699, -1, 99, 680)),
    _shrink(workloads.DECODE_BF16, name="decode_small_B4_H4_Sk3000", sq=(1,) * 4, sk=(3000,) * 4, heads=4),
    _shrink(workloads.CAUSAL_BF16, name="causal_d64_Sq200", d_qk=64, d_v=64, sq=(200, 200), sk=(333, 333)),
    _shrink(workloads.CAUSAL_BF16, name="prefix_negative_fully_masked", mask="prefix_causal", prefix_offset=-70,
            sq=(300, 300), sk=(250, 250), n_per_block=16, split_kv=5),
    _shrink(workloads.CAUSAL_BF16, name="last_valid_short", mask="none", last_valid_kv_index=100, sq=(150, 150),
            sk=(400, 400), n_per_block=32, split_kv=3),
    _shrink(workloads.CAUSAL_BF16, name="npb1_many_splits", n_per_block=1, split_kv=37, sq=(129, 129), sk=(129, 129)),
    _shrink(workloads.CAUSAL_BF16, name="unsplit_S1", split_kv=1, sq=(200, 200), sk=(640, 640), mask="none"),
    _shrink(workloads.TINY_F32, name="f32_causal_ragged", mask="causal", sq=(100,), sk=(77,), split_kv=3,
            n_per_block=8),
    _shrink(workloads.TINY_F32, name="f32_d128_prefix", d_qk=128, d_v=128, mask="prefix_causal", prefix_offset=40,
            sq=(70,), sk=(200,), split_kv=6, n_per_block=16),
]


# Few work items against many resident workgroups with long splits: the
# partial kernel runs these items as several key pieces and merges them
# (load balance of the last round).  Masks leave whole pieces empty for some
# rows, and short sequences get fewer key tiles than pieces.
TAIL = [
    _shrink(workloads.LONG_PREFILL, name="tail_split_H2_Sq256_Sk8192_S2", heads=2, sq=(256,), sk=(8192,), split_kv=2),
    _shrink(workloads.LONG_PREFILL, name="tail_split_prefix_H3_Sq300_Sk9000_S3", heads=3, sq=(300,), sk=(9000,),
            split_kv=3, mask="prefix_causal", prefix_offset_per_seq=(8100,), last_valid_per_seq=(8899,)),
    _shrink(workloads.VARLEN_BATCH, name="tail_split_varlen_short_seqs", heads=2, sq=(130, 1, 64, 0, 200),
            sk=(12000, 100, 7000, 50, 3), split_kv=4, split_kv_per_seq=(4, 1, 3, 2, 4)),
    _shrink(workloads.CAUSAL_BF16, name="tail_split_dense_bottom_right_d128", heads=2, sq=(200, 200),
            sk=(6000, 6000), split_kv=2, mask="prefix_causal", prefix_offset=5800),
]


@pytest.mark.parametrize("w", TAIL, ids=lambda w: w.name)
def test_tail_split_all_rows(w):
    log(f"tail {w.name}")
    inputs, prob, res = run_gpu(w, seed=5)
    assert prob.c.partial_scratch and prob.c.partial_scratch_bytes > 0
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")
    # the same problem without scratch runs every item whole
    from split_kv_attention_amd import attention
    prob2 = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], partial_scratch=False,
                                    **workloads.problem_kwargs(w, inputs))
    o2 = torch.full_like(res["o_part"], float("nan"))
    l2 = torch.full_like(res["lse_part"], float("nan"))
    from split_kv_attention_amd import _lib
    _lib.sk_attn_partial(prob2.c, inputs["q"], inputs["k"], inputs["v"], o2, l2)
    torch.cuda.synchronize()
    written = ~torch.isnan(res["o_part"])
    assert torch.equal(written, ~torch.isnan(o2))
    assert torch.equal(torch.isneginf(res["lse_part"]), torch.isneginf(l2))
    # pieces round their weights to bf16 against their own running max, so
    # the two runs differ by the weights' rounding, far inside the tolerance
    assert (res["o_part"][written] - o2[written]).abs().max().item() < 2e-3
    fin = torch.isfinite(l2)
    assert (res["lse_part"][fin] - l2[fin]).abs().max().item() < 2e-3


def test_automatic_split_count_both_sides_of_the_thresholds():
    """split_kv = 0: unsplit below 8192 keys; above, the fewest splits (up to
    8) that give the 256-row kernel one item per CU, which then runs it."""
    from split_kv_attention_amd import attention

    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def auto(sq, sk, dtype="bf16", d=(192, 128)):
        w = _shrink(workloads.LONG_PREFILL, sq=(sq,), sk=(sk,), split_kv=0, dtype=dtype, d_qk=d[0], d_v=d[1])
        inputs = workloads.make_inputs(w, DEV, seed=0)
        prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
        return prob.split_kv, prob.m_per_block

    def rule(sq, heads=12):
        per_split = -(-sq // 256) * heads  # 256-row items per split
        return next((s for s in range(1, 8) if per_split * s >= cus), 8)

    assert auto(1024, 8191) == (1, 128)  # one key below the threshold (the page's tile-rounded form split here)
    assert auto(1024, 8192) == (rule(1024), 256) and rule(1024) > 1
    assert auto(2048, 42700) == (rule(2048), 256)
    assert auto(4096, 42700) == (rule(4096), 256)
    assert auto(8192, 16384) == (rule(8192), 256)
    assert auto(256, 8192) == (8, 128)  # too few rows to fill the CUs even at 8 splits
    assert auto(1024, 8192, dtype="f32", d=(64, 64)) == (1, 64)  # the f32 kernel: unsplit


def test_automatic_split_end_to_end():
    """The resolved count drives every entry point; results match the oracle
    run with that count."""
    w = _shrink(workloads.LONG_PREFILL, name="auto_split_Sq1024_Sk8192", sq=(1024,), sk=(8192,), split_kv=0)
    log(f"auto {w.name}")
    inputs, prob, res = run_gpu(w, seed=7)
    S = prob.split_kv
    assert S > 1 and res["o_part"].shape[1] == S
    rows = {0: sample_rows(1024, 48, seed=0, tile=prob.m_per_block)}
    st = compare(_shrink(w, split_kv=S), inputs, prob, res, rows_per_seq=rows, label=w.name)
    log(f"  S={S} {st}")


# f16 storage (scores, softmax and merge in f32; rocmlirTriton page, "f32
# merge for f16/bf16"): the same kernels on IEEE half operands
SMALL_F16 = [
    _shrink(workloads.LONG_PREFILL, name="f16_prefill_Sq300_Sk2000_S3", sq=(300,), sk=(2000,), dtype="f16"),
    _shrink(workloads.CAUSAL_BF16, name="f16_causal_d64", d_qk=64, d_v=64, sq=(200, 200), sk=(333, 333),
            dtype="f16"),
    _shrink(workloads.VARLEN_BATCH_PREFIX, name="f16_varlen_prefix", sq=(130, 1, 257, 64), sk=(500, 70, 1500, 3000),
            split_kv_per_seq=(2, 4, 6, 8), prefix_offset_per_seq=(370, 69, 1243, 2936),
            last_valid_per_seq=(499, 69, 1499, 2999), dtype="f16"),
    _shrink(workloads.DECODE_BF16, name="f16_decode_B4_H4_Sk3000", sq=(1,) * 4, sk=(3000,) * 4, heads=4, dtype="f16"),
    _shrink(workloads.LONG_PREFILL, name="f16_tail_split_H2_Sq256_Sk8192_S2", heads=2, sq=(256,), sk=(8192,),
            split_kv=2, dtype="f16"),
]


@pytest.mark.parametrize("w", SMALL_F16, ids=lambda w: w.name)
def test_f16_storage_all_rows(w):
    log(f"f16 {w.name}")
    inputs, prob, res = run_gpu(w, seed=9)
    assert res["out"].dtype == torch.float16
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")
    # f32 output from f16 inputs: one rounding less
    inputs, prob, res = run_gpu(w, seed=9, out_dtype=torch.float32)
    compare(w, inputs, prob, res, label=w.name + "/f32out")


def test_f16_scores_far_above_the_reference():
    """Weights against a stale reference can exceed the f16 range; the range
    check then takes the max update and recomputes them."""
    w = _shrink(workloads.LONG_PREFILL, name="f16_growing_scores", sq=(150,), sk=(3000,), split_kv=2, dtype="f16")
    inputs = workloads.make_inputs(w, DEV, 12)
    inputs["k"][200:] *= 6  # later keys score up to ~6x higher than the first tile's
    inputs, prob, res = run_gpu(w, inputs=inputs)
    compare(w, inputs, prob, res, label=w.name)


# Sliding window (reading: keys k >= q + off - window_left, on top of the
# other rules; the count formula is unchanged).  Whole tiles below a block's
# window are skipped, tiles the window cuts are masked per element.
WINDOW = [
    _shrink(workloads.CAUSAL_BF16, name="window_causal_100", sq=(300, 300), sk=(300, 300), split_kv=3,
            window_left=100),
    _shrink(workloads.CAUSAL_BF16, name="window_causal_0_diagonal_only", sq=(200, 200), sk=(200, 200), split_kv=2,
            window_left=0),
    _shrink(workloads.LONG_PREFILL, name="window_bottom_right_Sq300_Sk2000", sq=(300,), sk=(2000,),
            mask="prefix_causal", prefix_offset=1700, window_left=500),
    _shrink(workloads.LONG_PREFILL, name="window_no_mask_64", sq=(257,), sk=(900,), mask="none", window_left=64),
    _shrink(workloads.VARLEN_BATCH_PREFIX, name="window_varlen_prefix", sq=(130, 1, 257, 64), sk=(500, 70, 1500, 3000),
            split_kv_per_seq=(2, 4, 6, 8), prefix_offset_per_seq=(370, 69, 1243, 2936),
            last_valid_per_seq=(499, 69, 1499, 2999), window_left=300),
    _shrink(workloads.TINY_F32, name="window_f32_causal", mask="causal", sq=(100,), sk=(100,), split_kv=3,
            window_left=20),
    _shrink(workloads.CAUSAL_BF16, name="window_wider_than_all", sq=(200, 200), sk=(333, 333), window_left=100000),
    _shrink(workloads.LONG_PREFILL, name="window_tail_split_H2_Sq256_Sk8192", heads=2, sq=(256,), sk=(8192,),
            split_kv=2, mask="prefix_causal", prefix_offset=7936, window_left=1000),
]


# Prefix offsets far outside 32 bits (the offset is a 64-bit field): no row
# sees a key, every row sees every key, or every row's window starts past
# the last key.
EXTREME_OFFSETS = [
    _shrink(workloads.LONG_PREFILL, name="offset_far_below", sq=(200,), sk=(700,), mask="prefix_causal",
            prefix_offset=-(1 << 40)),
    _shrink(workloads.LONG_PREFILL, name="offset_far_above", sq=(200,), sk=(700,), mask="prefix_causal",
            prefix_offset=1 << 40),
    _shrink(workloads.LONG_PREFILL, name="offset_far_above_window", sq=(200,), sk=(700,), mask="prefix_causal",
            prefix_offset=1 << 40, window_left=50),
    _shrink(workloads.TINY_F32, name="offset_far_above_f32", mask="prefix_causal", prefix_offset=1 << 40),
]


@pytest.mark.parametrize("w", EXTREME_OFFSETS, ids=lambda w: w.name)
def test_extreme_prefix_offsets_all_rows(w):
    log(f"offsets {w.name}")
    inputs, prob, res = run_gpu(w, seed=14)
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


@pytest.mark.parametrize("w", WINDOW, ids=lambda w: w.name)
def test_sliding_window_all_rows(w):
    log(f"window {w.name}")
    inputs, prob, res = run_gpu(w, seed=13)
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_cases_all_rows(w):
    log(f"e2e {w.name}")
    inputs, prob, res = run_gpu(w, seed=3)
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


def test_maximum_split_count():
    """split_kv = 128, the most the library takes, at a key tile of 1: the
    combine merges each row in four chunks of 32 splits, and most splits of
    the early rows are empty."""
    w = _shrink(workloads.CAUSAL_BF16, name="max_splits_S128", heads=2, n_per_block=1, split_kv=128, sq=(150, 150),
                sk=(300, 300), mask="prefix_causal", prefix_offset=150)
    log(f"e2e {w.name}")
    inputs, prob, res = run_gpu(w, seed=6)
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")
    assert int(res["counts"].max()) == 128


def test_maximum_batch_packed():
    """65535 packed sequences, the most the library takes (one grid row of
    the combine per sequence), with ragged lengths of 0..3 rows and 0..40
    keys, bottom-right prefix-causal offsets and two splits; compared on a
    sample of sequences, and the output is finite everywhere."""
    B = 65535
    rng = np.random.default_rng(65535)
    sq = tuple(int(x) for x in rng.integers(0, 4, B))
    sk = tuple(int(x) for x in rng.integers(0, 41, B))
    w = Workload("max_batch_B65535", heads=1, sq=sq, sk=sk, d_qk=64, d_v=64, split_kv=2, n_per_block=8,
                 mask="prefix_causal", packed=True, prefix_offset_per_seq=tuple(k - q for q, k in zip(sq, sk)))
    log(f"e2e {w.name}")
    inputs, prob, res = run_gpu(w, seed=7)
    picked = set([0, 1, B - 2, B - 1] + [int(x) for x in rng.choice(B, 300, replace=False)])
    rows_per_seq = {b: (np.arange(sq[b]) if b in picked else np.array([], dtype=np.int64)) for b in range(B)}
    st = compare(w, inputs, prob, res, rows_per_seq=rows_per_seq, label=w.name)
    log(f"  {st}")
    assert torch.isfinite(res["out"]).all()
    del inputs, res
    torch.cuda.empty_cache()


def test_empty_sequences_in_a_packed_batch():
    """Sk = 0 gives zero output / -inf LSE without error; Sq = 0 is skipped."""
    w = _shrink(workloads.VARLEN_BATCH, name="empties", sq=(5, 0, 40, 3), sk=(0, 100, 0, 90),
                split_kv_per_seq=(2, 4, 6, 8))
    inputs, prob, res = run_gpu(w, seed=4)
    compare(w, inputs, prob, res, label=w.name)
    out = res["out"].float().cpu().numpy()
    assert (out[:5] == 0).all() and (out[5:45] == 0).all()
    assert np.isneginf(res["lse_out"][:, :45].cpu().numpy()).all()


def test_f32_output_and_no_lse_and_inline_counts():
    w = _shrink(workloads.LONG_PREFILL, name="prefill_small", sq=(200,), sk=(1500,))
    inputs, prob, res = run_gpu(w, seed=5, out_dtype=torch.float32)
    st = compare(w, inputs, prob, res, label="f32 out")
    log(f"  f32 out {st}")
    # counts computed inline by the combine: identical output
    _, _, res2 = run_gpu(w, inputs=inputs, counts_in_combine=False)
    _, prob3, res3 = run_gpu(w, inputs=inputs)
    assert torch.equal(res2["out"], res3["out"])
    assert torch.equal(res2["lse_out"], res3["lse_out"])
    # lse_out = NULL leaves out unchanged
    out = torch.empty_like(res3["out"])
    _lib.sk_attn_combine(prob3.c, res3["o_part"], res3["lse_part"], res3["counts"], out, None)
    torch.cuda.synchronize()
    assert torch.equal(out, res3["out"])


def test_deterministic():
    w = _shrink(workloads.VARLEN_BATCH_PREFIX, name="det", sq=(130, 257), sk=(500, 1500), split_kv_per_seq=(3, 5),
                prefix_offset_per_seq=(370, 1243), last_valid_per_seq=(499, 1499))
    inputs, _, a = run_gpu(w)
    _, _, b = run_gpu(w, inputs=inputs)
    for key in ("counts", "out", "lse_out"):
        assert torch.equal(a[key], b[key]), key


def test_combine_alone_on_oracle_partials():
    """The combine kernel fed with the oracle's own partials (uploaded as f32),
    including -inf splits and garbage in the splits s >= count it must not read."""
    w = _shrink(workloads.CAUSAL_BF16, name="combine_only", sq=(96, 96), sk=(96, 96), heads=3, split_kv=2,
                n_per_block=32)
    inputs = workloads.make_inputs(w, DEV, 6)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    mpb = prob.m_per_block  # the block partition the combine assumes the partials follow
    exp = adapter.expected(w, inputs, mpb)
    rows = prob.rows
    o_part = torch.full((w.heads, w.split_kv, rows, w.d_v), float("nan"), dtype=torch.float32)
    lse_part = torch.full((w.heads, w.split_kv, rows), float("nan"), dtype=torch.float32)
    counts = torch.zeros(rows, dtype=torch.int32)
    for (b, h), e in exp.items():
        r0 = b * w.sq[0]
        c = e["counts"]
        counts[r0 : r0 + w.sq[0]] = torch.from_numpy(c.astype(np.int32))
        for s in range(w.split_kv):
            valid = s < c
            o_part[h, s, r0 : r0 + w.sq[0]][torch.from_numpy(valid)] = torch.from_numpy(e["O_s"][s][valid]).float()
            lse_part[h, s, r0 : r0 + w.sq[0]][torch.from_numpy(valid)] = torch.from_numpy(e["L_s"][s][valid]).float()
    out = torch.empty((2, w.heads, w.sq[0], w.d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.heads, rows), dtype=torch.float32, device=DEV)
    prob.c.out_dtype = _lib.SK_F32
    _lib.sk_attn_combine(prob.c, o_part.to(DEV), lse_part.to(DEV), counts.to(DEV), out, lse)
    torch.cuda.synchronize()
    for (b, h), e in exp.items():
        O, l = oracle.combine(e["O_s"].astype(np.float32), e["L_s"].astype(np.float32), e["counts"])
        g = out[b, h].double().cpu().numpy()
        assert np.abs(g - O).max() <= 1e-6
        gl = lse[h, b * w.sq[0] : (b + 1) * w.sq[0]].double().cpu().numpy()
        np.testing.assert_array_equal(np.isneginf(gl), np.isneginf(l))
        fin = np.isfinite(l)
        assert np.abs(gl[fin] - l[fin]).max() <= 1e-5


# ---------------------------------------------------------------------------
# full-size workloads, sampled
# ---------------------------------------------------------------------------

def test_full_decode_every_head():
    """Batched decode at full size (B = 64, H = 32, Sq = 1, Sk = 32768,
    split 16) in the benchmark's launch configuration: every (sequence, head)
    pair against the oracle, one sequence at a time (its 32 heads' keys and
    values copied to the host, then each head's slice converted)."""
    w = workloads.DECODE_BF16
    log(f"full {w.name}, every (b, h)")
    inputs, prob, res = run_gpu(w)
    for b in range(w.batch):
        host = {k: (v[b : b + 1].cpu() if torch.is_tensor(v) else v) for k, v in inputs.items()}
        wb = _shrink(w, sq=(w.sq[b],), sk=(w.sk[b],))
        exp = adapter.expected(wb, host, prob.m_per_block)
        # the one-sequence oracle's rows are this sequence's packed rows
        exp = {(b, h): e for (_, h), e in exp.items()}
        rows_per_seq = {i: (np.arange(w.sq[b]) if i == b else np.array([], dtype=np.int64)) for i in range(w.batch)}
        st = compare(w, inputs, prob, res, rows_per_seq=rows_per_seq, label=f"{w.name} b={b}", exp=exp)
        if b % 8 == 0 or b == w.batch - 1:
            log(f"  b={b}: {st}")
    del inputs, res
    torch.cuda.empty_cache()


LONG_PREFILL_F16 = _shrink(workloads.LONG_PREFILL, name="varlen_prefill_f16_H12_Sq4096_Sk42700_D192x128_S3",
                           dtype="f16")


@pytest.mark.parametrize("w", [workloads.LONG_PREFILL, LONG_PREFILL_F16, workloads.VARLEN_BATCH,
                               workloads.VARLEN_BATCH_PREFIX], ids=lambda w: w.name)
def test_full_prefill_every_row_and_head(w):
    """The long-context prefill (H = 12, Sq = 4096, Sk = 42700, split 3), in
    bf16 and in f16 storage, and the packed batch (4 x Sq = 4096, Sk
    8K..128K, splits 2..8), without mask and prefix-causal, at full size on
    every row of every head: counts, partials and the merged output and LSE
    against the oracle (about 1 s of host time per head for the prefill,
    five times that for the batches)."""
    log(f"full {w.name}, every row and head")
    inputs, prob, res = run_gpu(w)
    assert res["out"].dtype == w.torch_dtype
    host = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inputs.items()}
    stats = []
    for h in range(w.heads):
        exp = adapter.expected(w, host, prob.m_per_block, heads=[h])
        stats.append(compare(w, inputs, prob, res, heads=[h], label=f"{w.name} h={h}", exp=exp))
        log(f"  head {h}: {stats[-1]}")
    del inputs, res, host
    torch.cuda.empty_cache()


def test_scores_growing_far_beyond_the_first_tile():
    """Keys after the first tile with ~50x larger scores: unmasked tiles that
    skip the running-max update must fall back to it (their weights would
    overflow), and the result still matches the oracle."""
    for mask in ("none", "causal"):
        w = _shrink(workloads.CAUSAL_BF16, name=f"growth_{mask}", mask=mask, sq=(300, 300), sk=(700, 700),
                    split_kv=2, heads=2)
        inputs = workloads.make_inputs(w, DEV, 9)
        k = inputs["k"].float()
        k[:, :, 200:] *= 40.0
        inputs["k"] = k.to(torch.bfloat16)
        log(f"e2e {w.name}")
        _, prob, res = run_gpu(w, inputs=inputs)
        st = compare(w, inputs, prob, res, label=w.name)
        log(f"  {st}")
