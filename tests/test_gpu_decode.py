"""The decode kernel (sequences of at most one query row) against the oracle
(GPU, through the C ABI), every row and head.

Problems whose longest sequence has one query row run on a streaming kernel
of their own for head dims 64/64 and 128/128 (bf16, f16), whose block is the
single row.  These cases cover what it decides for itself: the row's key
range under every mask (causal row 0, prefix offsets on both sides of the
keys, the last valid key, a sliding window), splits with no key, per-sequence
split counts, sequences with no key or no row in a packed batch, key tiles of
1 and 128, 128 splits, ragged key counts against its 32- and 64-key steps,
and seeded random draws.
"""
import dataclasses

import numpy as np
import pytest

from parity import compare, log, run_gpu
from split_kv_attention_amd import workloads
from split_kv_attention_amd.workloads import Workload

pytestmark = pytest.mark.gpu

D = workloads.DECODE_BF16


def _dec(name, **kw):
    return dataclasses.replace(D, name=name, **kw)


CASES = [
    _dec("dec_B8_H4_Sk3001_S16", sq=(1,) * 8, sk=(3001,) * 8, heads=4),
    _dec("dec_f16_B8_H4_Sk3001_S5", sq=(1,) * 8, sk=(3001,) * 8, heads=4, split_kv=5, dtype="f16"),
    _dec("dec_d64_B6_H3_Sk777_S3", sq=(1,) * 6, sk=(777,) * 6, heads=3, d_qk=64, d_v=64, split_kv=3),
    _dec("dec_d64_f16_B6_H3_Sk777_S4", sq=(1,) * 6, sk=(777,) * 6, heads=3, d_qk=64, d_v=64, split_kv=4,
         dtype="f16"),
    # causal row 0 sees key 0 only: one populated split
    _dec("dec_causal_B4_H2_Sk500", sq=(1,) * 4, sk=(500,) * 4, heads=2, split_kv=4, mask="causal"),
    # bottom-right aligned (off = Sk - 1): every key
    _dec("dec_prefix_bottom_right_B4_H2_Sk1500", sq=(1,) * 4, sk=(1500,) * 4, heads=2, split_kv=6,
         mask="prefix_causal", prefix_offset=1499),
    # per-sequence offsets, one negative (no visible key), lastValid per sequence
    _dec("dec_packed_prefix_offsets", packed=True, sq=(1, 1, 1, 1, 1), sk=(900, 64, 2049, 300, 10), heads=3,
         split_kv=8, split_kv_per_seq=(8, 2, 5, 1, 3), mask="prefix_causal",
         prefix_offset_per_seq=(899, -1, 1000, 299, 4), last_valid_per_seq=(899, 63, 1500, 120, 9)),
    # sequences with no key and with no row in one packed batch
    _dec("dec_packed_empty_sequences", packed=True, sq=(1, 0, 1, 1, 0, 1), sk=(700, 300, 0, 1, 0, 129), heads=2,
         split_kv=4),
    # sliding window: the row sees the last keys of its range only
    _dec("dec_window_B3_H2_Sk2000", sq=(1,) * 3, sk=(2000,) * 3, heads=2, split_kv=8, mask="prefix_causal",
         prefix_offset=1999, window_left=100),
    _dec("dec_window_no_mask_B2_H2_Sk600", sq=(1,) * 2, sk=(600,) * 2, heads=2, split_kv=3, window_left=0),
    # split counts above the key tiles: empty splits, and key tiles of 1
    _dec("dec_more_splits_than_tiles", sq=(1,) * 3, sk=(200,) * 3, heads=2, split_kv=16, n_per_block=64),
    _dec("dec_S128_nPB1", sq=(1,) * 2, sk=(300,) * 2, heads=2, split_kv=128, n_per_block=1),
    _dec("dec_nPB128_ragged", sq=(1,) * 4, sk=(1031,) * 4, heads=2, split_kv=7, n_per_block=128),
    _dec("dec_single_key", sq=(1,) * 4, sk=(1,) * 4, heads=2, split_kv=4),
    _dec("dec_last_valid_short", sq=(1,) * 4, sk=(1000,) * 4, heads=2, split_kv=4, last_valid_kv_index=37),
    # offsets far outside 32 bits: nothing visible, everything visible, or a
    # window that starts past the last key
    _dec("dec_offset_far_below", sq=(1,) * 2, sk=(500,) * 2, heads=2, split_kv=4, mask="prefix_causal",
         prefix_offset=-(1 << 40)),
    _dec("dec_offset_far_above", sq=(1,) * 2, sk=(500,) * 2, heads=2, split_kv=4, mask="prefix_causal",
         prefix_offset=1 << 40),
    _dec("dec_offset_far_above_window", sq=(1,) * 2, sk=(500,) * 2, heads=2, split_kv=4, mask="prefix_causal",
         prefix_offset=1 << 40, window_left=10),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_decode_kernel_all_rows(w):
    log(f"decode {w.name}")
    inputs, prob, res = run_gpu(w, seed=17)
    assert prob.m_per_block == 1, "a one-row problem with these head dims runs on the decode kernel"
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


def test_decode_kernel_not_used_for_two_rows_or_other_dims():
    two_rows = _dec("dec_two_rows", sq=(2,) * 2, sk=(300,) * 2, heads=2)
    inputs, prob, _ = run_gpu(two_rows, seed=1)
    assert prob.m_per_block == 128
    wide = _dec("dec_d192", packed=True, sq=(1, 1), sk=(500, 700), heads=2, d_qk=192, d_v=128)
    inputs, prob, res = run_gpu(wide, seed=2)
    assert prob.m_per_block == 128
    compare(wide, inputs, prob, res, label=wide.name)


def _draw(seed: int) -> Workload:
    rng = np.random.default_rng(9100 + seed)
    B = int(rng.integers(1, 7))
    packed = bool(rng.random() < 0.5)
    sk = [int(x) for x in rng.integers(0, 4000, B)] if packed else [int(rng.integers(1, 4000))] * B
    sq = [1] * B
    if packed:
        for b in range(B):
            if rng.random() < 0.15:
                sq[b] = 0
        if max(sq) == 0:
            sq[0] = 1
    d = int(rng.choice([64, 128]))
    split_kv = int(rng.integers(1, 17))
    mask = str(rng.choice(["none", "causal", "prefix_causal"]))
    offsets = tuple(int(sk[b] - 1 + rng.integers(-300, 5)) for b in range(B)) if mask == "prefix_causal" else None
    last_valid = tuple(int(rng.integers(-1, max(sk[b], 1))) for b in range(B)) if rng.random() < 0.3 else None
    per_seq = tuple(int(x) for x in rng.integers(1, split_kv + 1, B)) if rng.random() < 0.3 else None
    window = int(rng.integers(0, 800)) if rng.random() < 0.3 else -1
    return Workload(f"dec_rand{seed}", heads=int(rng.integers(1, 5)), sq=tuple(sq), sk=tuple(sk), d_qk=d, d_v=d,
                    split_kv=split_kv, n_per_block=int(rng.choice([1, 16, 64, 128])), mask=mask, packed=packed,
                    dtype=str(rng.choice(["bf16", "f16"])), split_kv_per_seq=per_seq, prefix_offset_per_seq=offsets,
                    last_valid_per_seq=last_valid, window_left=window)


@pytest.mark.parametrize("seed", range(16))
def test_decode_kernel_random(seed):
    w = _draw(seed)
    log(f"decode random {w} ")
    inputs, prob, res = run_gpu(w, seed=seed)
    assert prob.m_per_block == 1
    compare(w, inputs, prob, res, label=w.name)

