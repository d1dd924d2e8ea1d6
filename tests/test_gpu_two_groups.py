"""The 256-row MFMA partial kernel (two groups of 4 waves per workgroup)
against the oracle (GPU, through the C ABI), every row and head.

The library takes that kernel for 16-bit problems with at least one
256-row work item per CU, and the 128-row kernel below that, so the small
cases of the other tests run on the 128-row one.  Each case here is sized
to cross the threshold (and asserts that it did): a ragged last block
whose later waves see no row, causal and prefix-causal masks with
per-sequence offsets, a sliding window, a last valid key, f16 storage,
every head-dimension pair, and a tail of items cut into key pieces.  The
partials are compared at the kernel's block of 256 rows, so the block's
key partition and its empty-split slots are checked too.
"""
import dataclasses

import numpy as np
import pytest

from parity import compare, log, run_gpu
from split_kv_attention_amd import workloads
from split_kv_attention_amd.workloads import Workload

pytestmark = pytest.mark.gpu

CUS = 256  # MI355X compute units: one 256-row item per CU or more


def _blocks(sq, packed: bool) -> int:
    """256-row query blocks as the library counts them from the sizes the
    host knows: B x blocks of the longest sequence, for a packed batch at
    most ceil(total rows / 256) + B - 1."""
    dense = -(-max(sq) // 256) * len(sq)
    return min(dense, -(-sum(sq) // 256) + len(sq) - 1) if packed else dense


def _items(w: Workload) -> int:
    return _blocks(w.sq, w.packed) * w.heads * w.split_kv


CASES = [
    # 300 rows: the second block holds 44 rows, so waves 2-7 of it see no row
    dataclasses.replace(workloads.CAUSAL_BF16, name="two_groups_causal_B2_H16_Sq300_Sk2500_S4", sq=(300, 300),
                        sk=(2500, 2500), heads=16, split_kv=4),
    # 257 rows: the second block holds one row
    Workload("two_groups_d64_B4_H16_Sq257_Sk1000_S2", heads=16, sq=(257,) * 4, sk=(1000,) * 4, d_qk=64, d_v=64,
             split_kv=2, n_per_block=64),
    # packed, f16, prefix-causal with offsets below zero, a window, last valid keys, an empty sequence
    Workload("two_groups_f16_packed_prefix_window_H8_S8", heads=8, sq=(300, 130, 0, 257), sk=(1800, 900, 40, 2600),
             d_qk=128, d_v=128, split_kv=8, split_kv_per_seq=(8, 3, 2, 6), n_per_block=32, mask="prefix_causal",
             packed=True, dtype="f16", prefix_offset_per_seq=(1500, -40, 0, 2343),
             last_valid_per_seq=(1700, 899, -1, 2599), window_left=700),
    # 260 items on 256 CUs: the last 4 run as key pieces (16 key tiles per
    # split, so 2 pieces each), merged before the combine
    Workload("two_groups_tail_pieces_H4_Sq200_Sk66560_S65", heads=4, sq=(200,), sk=(65 * 1024,), d_qk=192,
             d_v=128, split_kv=65, n_per_block=64, packed=True),
]


def _draw(seed: int) -> Workload:
    """A seeded random configuration with at least one 256-row item per CU."""
    rng = np.random.default_rng(8800 + seed)
    dtype = str(rng.choice(["bf16", "bf16", "f16"]))
    d_qk, d_v = [(64, 64), (128, 128), (192, 128)][rng.integers(3)]
    B = int(rng.integers(2, 5))
    packed = bool(rng.random() < 0.6)
    if packed:
        sq = [int(x) for x in rng.integers(1, 521, B)]
        sk = [int(x) for x in rng.integers(0, 1501, B)]
    else:
        sq = [int(rng.integers(1, 521))] * B
        sk = [int(rng.integers(1, 1501))] * B
    split_kv = int(rng.integers(4, 17))
    per_seq = tuple(int(x) for x in rng.integers(1, split_kv + 1, B)) if rng.random() < 0.3 else None
    mask = str(rng.choice(["none", "causal", "prefix_causal"]))
    offsets = tuple(int(sk[b] - sq[b] + rng.integers(-64, 65)) for b in range(B)) if mask == "prefix_causal" else None
    last_valid = tuple(int(rng.integers(-1, max(sk[b], 1))) for b in range(B)) if rng.random() < 0.3 else None
    window = int(rng.integers(0, 600)) if rng.random() < 0.3 else -1
    heads = max(1, -(-CUS // (_blocks(sq, packed) * split_kv)))
    name = (f"two_groups_rand{seed}_{dtype}_{'packed' if packed else 'dense'}_B{B}_H{heads}_D{d_qk}x{d_v}_"
            f"S{split_kv}_{mask}{'_lv' if last_valid else ''}{f'_w{window}' if window >= 0 else ''}")
    return Workload(name, heads=heads, sq=tuple(sq), sk=tuple(sk), d_qk=d_qk, d_v=d_v, split_kv=split_kv,
                    n_per_block=int(rng.choice([16, 32, 64, 128])), mask=mask, packed=packed, dtype=dtype,
                    split_kv_per_seq=per_seq, prefix_offset_per_seq=offsets, last_valid_per_seq=last_valid,
                    window_left=window)


N_RANDOM = 12


@pytest.mark.parametrize("w", CASES + [_draw(s) for s in range(N_RANDOM)], ids=lambda w: w.name)
def test_two_group_kernel_all_rows(w):
    assert _items(w) >= CUS, "sized to take the 256-row kernel"
    log(f"two groups {w.name} sq={w.sq} sk={w.sk} items={_items(w)}")
    inputs, prob, res = run_gpu(w, seed=61)
    assert prob.m_per_block == 256, "the library picked the 128-row kernel"
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


def _choice(w: Workload) -> int:
    from split_kv_attention_amd import attention

    inputs = workloads.make_inputs(w, "cuda", seed=0)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    return prob.m_per_block


def test_kernel_choice_at_one_item_per_cu():
    """The 256-row kernel from exactly one 256-row item per CU, the 128-row
    one below; a packed batch counts at most ceil(total rows / 256) + B - 1
    blocks (here 3 where the longest sequence alone would give 4)."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dense = Workload("choice_dense", heads=cus, sq=(100,), sk=(300,), d_qk=64, d_v=64, split_kv=1, n_per_block=64)
    assert _choice(dense) == 256
    assert _choice(dataclasses.replace(dense, heads=cus - 1)) == 128
    packed = Workload("choice_packed", heads=-(-cus // 3), sq=(300, 1), sk=(300, 300), d_qk=64, d_v=64, split_kv=1,
                      n_per_block=64, packed=True)
    assert _blocks(packed.sq, True) == 3 and _items(packed) >= cus
    assert _choice(packed) == 256
    assert _choice(dataclasses.replace(packed, heads=(cus - 1) // 3)) == 128
    for w in (dense, dataclasses.replace(dense, heads=cus - 1), packed):
        inputs, prob, res = run_gpu(w, seed=62)
        compare(w, inputs, prob, res, label=w.name)


def test_block_size_and_automatic_split_follow_the_documented_rules():
    """Host queries only (no kernel runs), over seeded random shapes: the
    block size is 256 exactly when the 256-row item count reaches the CU
    count, and split_kv = 0 resolves to the fewest splits (at most 8) that
    reach it, for problems with at least 8192 keys and more than one row."""
    import torch

    from split_kv_attention_amd import _lib

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(8900)
    for _ in range(400):
        packed = bool(rng.random() < 0.5)
        B = int(rng.integers(1, 9))
        sq = [int(x) for x in rng.integers(2, 2049, B)]
        if not packed:
            sq = [max(sq)] * B
        sk = int(rng.choice([4096, 8191, 8192, 20000, 42700]))
        heads = int(rng.integers(1, 33))
        split = int(rng.integers(0, 13))
        dtype = "bf16" if rng.random() < 0.7 else "f16"
        w = Workload("rules", heads=heads, sq=tuple(sq), sk=(sk,) * B, d_qk=128, d_v=128, split_kv=split,
                     n_per_block=64, packed=packed, dtype=dtype)
        c = _lib.SkProblem()
        c.batch, c.num_heads, c.max_seqlen_q, c.max_seqlen_k = B, heads, max(sq), sk
        c.head_dim_qk = c.head_dim_v = 128
        c.split_kv, c.n_per_block = split, 64
        c.dtype = c.out_dtype = _lib.SK_BF16 if dtype == "bf16" else _lib.SK_F16
        c.softmax_scale = 0.1
        c.window_left = -1
        c.last_valid_kv_index = -1
        if packed:
            c.cu_seqlens_q = 1 << 20  # never dereferenced by these host queries
            c.total_q = sum(sq)
        per_split = _blocks(sq, packed) * heads
        s_exp = split
        if split == 0:
            s_exp = 1 if sk < 8192 else next((s for s in range(1, 8) if per_split * s >= cus), 8)
        assert _lib.sk_split_kv(c) == s_exp, (w, s_exp)
        assert _lib.sk_partial_m_per_block(c) == (256 if per_split * s_exp >= cus else 128), (w, s_exp)
