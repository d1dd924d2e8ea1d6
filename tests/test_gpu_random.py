"""Seeded random configurations of the forward path against the oracle (GPU,
through the C ABI), every row and head.

Each case draws, from its own seed: the storage type (bf16, f16, f32) and a
head-dimension pair the kernels take for it; a dense batch or a packed one
of 1-4 sequences with 0-300 query rows and 0-2500 keys each; 1-4 heads;
split_kv 1-12, sometimes per sequence; the key tile n_per_block; the mask
(none, causal, prefix-causal with per-sequence offsets that may be
negative); sometimes a last valid key per sequence and a sliding window;
and the output type (mostly the input's, else f32 or the other 16-bit one).
The oracle follows the pages' steps for whatever the draw gives, so the
draws reach combinations no hand-written case names: ragged row blocks
against small key tiles, empty sequences beside long ones, per-sequence
split counts above a sequence's key count, windows narrower than a tile.
"""
import numpy as np
import pytest
import torch

from parity import compare, log, run_gpu
from split_kv_attention_amd.workloads import Workload

pytestmark = pytest.mark.gpu

N_CASES = 32
DIMS = {"bf16": [(64, 64), (128, 128), (192, 128)], "f16": [(64, 64), (128, 128), (192, 128)],
        "f32": [(16, 16), (32, 32), (64, 64), (128, 128)]}


def draw(seed: int) -> Workload:
    rng = np.random.default_rng(7000 + seed)
    dtype = str(rng.choice(["bf16", "bf16", "f16", "f32"]))
    d_qk, d_v = DIMS[dtype][rng.integers(len(DIMS[dtype]))]
    B = int(rng.integers(1, 5))
    packed = bool(rng.random() < 0.6)
    if packed:
        sq = [int(x) for x in rng.integers(1, 301, B)]
        sk = [int(x) for x in rng.integers(0, 2501, B)]
        for b in range(B):
            if rng.random() < 0.1:
                sq[b] = 0
    else:
        sq = [int(rng.integers(1, 301))] * B
        sk = [int(rng.integers(1, 2501))] * B
    split_kv = int(rng.integers(1, 13))
    per_seq_splits = tuple(int(x) for x in rng.integers(1, split_kv + 1, B)) if rng.random() < 0.3 else None
    mask = str(rng.choice(["none", "causal", "prefix_causal"]))
    offsets = None
    if mask == "prefix_causal":
        offsets = tuple(int(sk[b] - sq[b] + rng.integers(-64, 65)) for b in range(B))
    last_valid = None
    if rng.random() < 0.3:
        last_valid = tuple(int(rng.integers(-1, max(sk[b], 1))) for b in range(B))
    window = int(rng.integers(0, 600)) if rng.random() < 0.3 else -1
    n_per_block = int(rng.choice([1, 16, 32, 64, 128]))
    name = (f"rand{seed}_{dtype}_{'packed' if packed else 'dense'}_B{B}_D{d_qk}x{d_v}_S{split_kv}_"
            f"N{n_per_block}_{mask}{'_lv' if last_valid else ''}{f'_w{window}' if window >= 0 else ''}")
    return Workload(name, heads=int(rng.integers(1, 5)), sq=tuple(sq), sk=tuple(sk), d_qk=d_qk, d_v=d_v,
                    split_kv=split_kv, n_per_block=n_per_block, mask=mask, packed=packed, dtype=dtype,
                    split_kv_per_seq=per_seq_splits, prefix_offset_per_seq=offsets, last_valid_per_seq=last_valid,
                    window_left=window)


def draw_out_dtype(seed: int, w: Workload):
    """The output type, from a generator of its own (so the draws above stay
    as they are): mostly the input type, else f32 or the other 16-bit type."""
    rng = np.random.default_rng(57000 + seed)
    pick = rng.random()
    if pick < 0.6:
        return None
    if pick < 0.8 or w.dtype == "f32":
        return torch.float32
    return torch.float16 if w.dtype == "bf16" else torch.bfloat16


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration_all_rows(seed):
    w = draw(seed)
    out_dtype = draw_out_dtype(seed, w)
    log(f"random {w.name} sq={w.sq} sk={w.sk} splits={w.split_kv_per_seq} off={w.prefix_offset_per_seq} "
        f"lv={w.last_valid_per_seq} out={out_dtype}")
    inputs, prob, res = run_gpu(w, seed=seed, out_dtype=out_dtype)
    if out_dtype is not None:
        assert res["out"].dtype == out_dtype
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")
