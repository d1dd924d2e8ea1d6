"""Axes long enough that 32-bit byte offsets overflow (GPU, through the C
ABI), against the oracle.

Keys: a key axis longer than 2^24 keys.

One head's K and V then span more than 4 GiB, so every key offset past the
first 2^24 rows (at 256 bytes per row) exceeds 32 bits: the kernels must
address key tiles from 64-bit bases.  Decode (the streaming kernel) is
checked on its row; the prefill (the MFMA kernel, two query blocks) on
rows at both block edges.  Each case copies one head's K and V to the host
(tens of GB in float64 for the oracle).

Rows: a dense batch of 2^21 + 5 query rows, 2 heads and 4 splits, whose
partial buffers (8.6 GB) put most slots beyond 4 GiB; prefix-causal
aligned to the bottom right, so the first rows see no key.  Rows near both
ends and around the first visible one are compared.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity import compare, log, run_gpu
from split_kv_attention_amd import workloads

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SK = (1 << 24) + 123

CASES = [
    dataclasses.replace(workloads.DECODE_BF16, name="long_keys_decode_Sk2^24+123_S16", sq=(1,), sk=(SK,), heads=1),
    dataclasses.replace(workloads.LONG_PREFILL, name="long_keys_prefill_Sq130_Sk2^24+123_S8", sq=(130,), sk=(SK,),
                        heads=1, split_kv=8),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_key_axis_beyond_32_bit_byte_offsets(w):
    log(f"long keys {w.name}")
    inputs, prob, res = run_gpu(w, seed=31)
    rows = np.array([0, 1, 63, 64, 127, 128, 129]) if w.sq[0] > 1 else np.array([0])
    st = compare(w, inputs, prob, res, rows_per_seq={0: rows}, label=w.name)
    log(f"  {st}")
    del inputs, res
    torch.cuda.empty_cache()


SQ = (1 << 21) + 5


def test_query_axis_beyond_32_bit_partial_offsets():
    w = dataclasses.replace(workloads.CAUSAL_BF16, name="long_rows_Sq2^21+5_Sk700_S4", sq=(SQ,), sk=(700,), heads=2,
                            split_kv=4, mask="prefix_causal", prefix_offset=700 - SQ)
    log(f"long rows {w.name}")
    inputs, prob, res = run_gpu(w, seed=32)
    first = SQ - 700  # first row that sees a key
    rows = np.array(sorted({0, 1, 127, 128, first - 1, first, first + 1, first + 130, SQ - 129, SQ - 128,
                            SQ - 2, SQ - 1}))
    st = compare(w, inputs, prob, res, rows_per_seq={0: rows}, label=w.name)
    log(f"  {st}")
    assert not torch.isnan(res["out"]).any()
    del inputs, res
    torch.cuda.empty_cache()
