"""The C ABI from a plain C99 program (GPU) against the oracle.

tests/c_client/sk_client.c includes only include/splitkv.h and the HIP
runtime API, links libsplitkv.so by name, and runs counts -> partial ->
combine on its own stream from input files; it also checks that an invalid
call is refused with a message.  This test writes the inputs, runs the
client as a child process, and compares what it wrote (counts, output, LSE)
with the oracle on every row and head.
"""
import dataclasses
import os
import subprocess

import numpy as np
import pytest
import torch

from parity import compare, log
from split_kv_attention_amd import attention, build, workloads

pytestmark = pytest.mark.gpu

MASK_CODE = {"none": 0, "causal": 1, "prefix_causal": 2}

CASES = [
    dataclasses.replace(workloads.CAUSAL_BF16, name="c_client_causal_B2_H4_Sq200_Sk333", sq=(200, 200),
                        sk=(333, 333), heads=4, split_kv=3),
    dataclasses.replace(workloads.CAUSAL_BF16, name="c_client_prefix_D192x128", sq=(130, 130), sk=(1500, 1500),
                        heads=2, d_qk=192, d_v=128, split_kv=5, mask="prefix_causal", prefix_offset=1370,
                        last_valid_kv_index=1400),
    dataclasses.replace(workloads.DECODE_BF16, name="c_client_decode_B8_H4_Sk3000", sq=(1,) * 8, sk=(3000,) * 8,
                        heads=4),
    # 256 items of 256 rows: the 256-row kernel on a 256-CU device
    dataclasses.replace(workloads.CAUSAL_BF16, name="c_client_causal_256rows_B2_H16_Sq300_Sk2500", sq=(300, 300),
                        sk=(2500, 2500), heads=16),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_c_client_forward_all_rows(w, tmp_path):
    assert os.path.exists(build.C_CLIENT_PATH), "build the client first (__graft_entry__.build())"
    log(f"C client {w.name}")
    inputs = workloads.make_inputs(w, "cpu", seed=41)
    for n in "qkv":
        inputs[n].contiguous().view(torch.int16).numpy().tofile(str(tmp_path / f"{n}.bin"))
    B, H, Sq, Sk = w.batch, w.heads, w.sq[0], w.sk[0]
    (tmp_path / "problem.txt").write_text(
        f"batch {B}\nheads {H}\nsq {Sq}\nsk {Sk}\ndqk {w.d_qk}\ndv {w.d_v}\nsplit {w.split_kv}\n"
        f"npb {w.n_per_block}\nmask {MASK_CODE[w.mask]}\nprefix_offset {w.prefix_offset}\n"
        f"last_valid {w.last_valid_kv_index}\nscale {w.softmax_scale!r}\n")
    run = subprocess.run([build.C_CLIENT_PATH, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    log(f"  {run.stdout.strip()}")
    rows = B * Sq
    out = torch.from_numpy(np.fromfile(str(tmp_path / "out.bin"), dtype=np.int16)).view(torch.bfloat16)
    res = dict(out=out.reshape(B, H, Sq, w.d_v),
               lse_out=torch.from_numpy(np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32).reshape(H, rows)),
               counts=torch.from_numpy(np.fromfile(str(tmp_path / "counts.bin"), dtype=np.int32)))
    # the problem as the client built it, for its block size (host-only queries)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    st = compare(w, inputs, prob, res, check_partials=False, label=w.name)
    log(f"  {st}")
