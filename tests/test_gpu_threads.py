"""Concurrent calls from several host threads, each on its own stream (GPU,
through the C ABI).

The library keeps no per-call state outside the arguments: its per-device
caches are atomics and its error message is per thread.  Five threads run
different workloads, each on its own stream, several times over, while a
sixth thread makes calls that fail argument checks.  Every thread's last
results must equal, bit for bit, a run of the same workload alone, and each
thread must read its own error message.
"""
import ctypes
import dataclasses
import threading

import pytest
import torch

from parity import DEV, log
from split_kv_attention_amd import _lib, attention, workloads

pytestmark = pytest.mark.gpu

CASES = [
    dataclasses.replace(workloads.LONG_PREFILL, name="threads_prefill_Sq300_Sk2000_S3", sq=(300,), sk=(2000,)),
    dataclasses.replace(workloads.VARLEN_BATCH_PREFIX, name="threads_varlen_prefix", sq=(130, 1, 257, 64),
                        sk=(500, 70, 1500, 3000), heads=2, split_kv_per_seq=(2, 4, 6, 8),
                        prefix_offset_per_seq=(370, 69, 1243, 2936), last_valid_per_seq=(499, 69, 1499, 2999)),
    dataclasses.replace(workloads.CAUSAL_BF16, name="threads_causal_f16", sq=(200, 200), sk=(333, 333),
                        dtype="f16"),
    dataclasses.replace(workloads.DECODE_BF16, name="threads_decode_B8_H4_Sk3000", sq=(1,) * 8, sk=(3000,) * 8,
                        heads=4),
    # the 256-row kernel, its last round as key pieces
    dataclasses.replace(workloads.LONG_PREFILL, name="threads_256rows_pieces_H16_Sq300_Sk9216_S9", heads=16,
                        sq=(300,), sk=(9216,), split_kv=9),
]
ROUNDS = 6


def _setup(w, seed):
    inputs = workloads.make_inputs(w, DEV, seed)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    return inputs, prob


def _poison(bufs):
    bufs[0].fill_(-7)
    for b in bufs[1:]:
        b.fill_(float("nan"))


def test_concurrent_threads_on_their_own_streams():
    setups = [_setup(w, 30 + i) for i, w in enumerate(CASES)]
    # each workload alone, on the current stream
    alone = []
    for inputs, prob in setups:
        bufs = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
        _poison(bufs)
        attention.run(prob, inputs["q"], inputs["k"], inputs["v"], *bufs)
        torch.cuda.synchronize()
        alone.append([bufs[0], bufs[3], bufs[4]])  # counts, out, lse_out

    results = [None] * len(CASES)
    errors = []
    start = threading.Barrier(len(CASES) + 1)

    def worker(i):
        try:
            inputs, prob = setups[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                bufs = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
                start.wait(timeout=60)
                for _ in range(ROUNDS):
                    _poison(bufs)
                    attention.run(prob, inputs["q"], inputs["k"], inputs["v"], *bufs, stream=stream)
                stream.synchronize()
            assert _lib.sk_last_error() == "", f"thread {i} sees an error it did not cause"
            results[i] = [bufs[0], bufs[3], bufs[4]]
        except BaseException as e:  # reported by the main thread
            errors.append((i, e))

    def failing():
        try:
            p = _lib.SkProblem()
            ctypes.memmove(ctypes.byref(p), ctypes.byref(setups[0][1].c), ctypes.sizeof(p))
            p.split_kv = -2
            start.wait(timeout=60)
            for _ in range(ROUNDS * 4):
                st = _lib.load().sk_valid_split_counts(ctypes.byref(p), None, None)
                assert st == _lib.SK_ERR_INVALID_ARG
                assert "split_kv" in _lib.sk_last_error()
        except BaseException as e:
            errors.append(("failing", e))

    # daemon threads and a barrier timeout: a thread that fails early cannot
    # leave the others (or the interpreter's exit) waiting
    threads = [threading.Thread(target=worker, args=(i,), daemon=True) for i in range(len(CASES))]
    threads.append(threading.Thread(target=failing, daemon=True))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for w, got, exp in zip(CASES, results, alone):
        for name, g, e in zip(("counts", "out", "lse_out"), got, exp):
            assert torch.equal(g, e), f"{w.name}: {name} differs from the workload run alone"
        log(f"  {w.name}: {ROUNDS} concurrent runs match the run alone")
