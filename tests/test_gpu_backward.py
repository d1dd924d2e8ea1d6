"""GPU parity of the backward (sk_attn_backward, through the C ABI) against
the float64 oracle gradients.

The forward runs through the library first (its out and LSE are the
backward's inputs, as in training); the oracle differentiates the exact
attention of the same bf16/f16 inputs.  Small cases are compared on every
row and key; the long-context prefill at full size on sampled rows and keys.

Tolerance (16-bit storage): per gradient tensor, max |error| <= 1e-2 of the
tensor's largest |value| and cosine similarity >= 0.99999, the forward's bar
scaled to the gradient's magnitude.  The final rounding of each gradient to
bf16 alone costs up to 2^-9 (0.2 %) of that magnitude; the kernel also rounds
P and dS to the storage type before their products (2^-9 relative each,
summed with mixed signs) and takes D from the stored 16-bit output, so a few
2^-9 in all: 1e-2 is about five.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import adapter
from parity import DEV, log, run_gpu, sample_rows
from split_kv_attention_amd import _lib, attention, workloads

pytestmark = pytest.mark.gpu

TOL_REL = 1e-2
COS_MIN = 0.99999


def _shrink(w, **kw):
    return dataclasses.replace(w, **kw)


def run_backward(w, seed=0, inputs=None):
    """Forward then backward through the library; every gradient and the
    workspace start as NaN so that unwritten elements show."""
    inputs, prob, res = run_gpu(w, seed=seed, inputs=inputs)
    dout = workloads.make_dout(w, DEV, seed)
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    nbytes = _lib.sk_backward_workspace_bytes(prob.c)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    _lib.sk_attn_backward(prob.c, q, k, v, res["out"], dout, res["lse_out"], dq, dk, dv, ws, nbytes)
    torch.cuda.synchronize()
    return inputs, dout, dq, dk, dv


def _rows(w, x, b, h, n):
    """Rows of sequence b (query rows if n == 'q', else key rows), head h."""
    if w.packed:
        lens = w.sq if n == "q" else w.sk
        r0 = int(sum(lens[:b]))
        return x[r0 : r0 + lens[b], h]
    return x[b, h]


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _check(name, got, ref):
    assert np.isfinite(got).all(), f"{name}: non-finite values (unwritten or overflow)"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    if scale == 0.0:
        assert err == 0.0, f"{name}: expected all zeros, max |got| = {err}"
        return dict(err=err, scale=0.0, cos=1.0)
    cos = float((got * ref).sum() / (np.linalg.norm(got) * np.linalg.norm(ref)))
    assert err <= TOL_REL * scale, f"{name}: max err {err:.3g} > {TOL_REL} * {scale:.3g}"
    assert cos >= COS_MIN, f"{name}: cosine {cos:.7f}"
    return dict(err=err / scale, cos=cos)


def compare_all(w, inputs, dout, dq, dk, dv):
    if w.split_kv == 0:  # the gradients do not depend on the split count
        w = _shrink(w, split_kv=1)
    ref = adapter.backward(w, inputs, dout)
    out = {}
    for i, (name, g, n) in enumerate((("dQ", dq, "q"), ("dK", dk, "k"), ("dV", dv, "k"))):
        gs, rs = [], []
        for (b, h), grads in ref.items():
            gs.append(_f64(_rows(w, g, b, h, n)).ravel())
            rs.append(grads[i].ravel())
        out[name] = _check(name, np.concatenate(gs), np.concatenate(rs))
    return out


BWD = [
    _shrink(workloads.LONG_PREFILL, name="bwd_prefill_Sq300_Sk2000_S3_D192x128", sq=(300,), sk=(2000,)),
    _shrink(workloads.CAUSAL_BF16, name="bwd_causal_d128_Sq200_Sk333", sq=(200, 200), sk=(333, 333)),
    _shrink(workloads.CAUSAL_BF16, name="bwd_causal_d64_Sq257", d_qk=64, d_v=64, sq=(257, 257), sk=(257, 257),
            heads=3),
    _shrink(workloads.VARLEN_BATCH_PREFIX, name="bwd_varlen_prefix", sq=(130, 1, 257, 64), sk=(500, 70, 1500, 3000),
            heads=2, split_kv_per_seq=(2, 4, 6, 8), prefix_offset_per_seq=(370, 69, 1243, 2936),
            last_valid_per_seq=(499, 69, 1499, 2999)),
    _shrink(workloads.VARLEN_BATCH, name="bwd_varlen_none_ragged", sq=(33, 1, 70, 129), sk=(900, 64, 1200, 31),
            heads=2, split_kv=3, split_kv_per_seq=None),
    _shrink(workloads.DECODE_BF16, name="bwd_decode_B4_H4_Sk3000", sq=(1,) * 4, sk=(3000,) * 4, heads=4),
    _shrink(workloads.DECODE_BF16, name="bwd_dense_B5_Sq3_per_seq", sq=(3,) * 5, sk=(700,) * 5, heads=2, split_kv=6,
            split_kv_per_seq=(1, 2, 3, 6, 5), mask="prefix_causal", prefix_offset_per_seq=(697, 0, 300, -2, 696),
            last_valid_per_seq=(699, 699, 500, 699, -1)),
    _shrink(workloads.CAUSAL_BF16, name="bwd_prefix_negative_fully_masked", mask="prefix_causal", prefix_offset=-70,
            sq=(300, 300), sk=(250, 250), n_per_block=16, split_kv=5, heads=2),
    _shrink(workloads.CAUSAL_BF16, name="bwd_last_valid_short", mask="none", last_valid_kv_index=100, sq=(150, 150),
            sk=(400, 400), n_per_block=32, split_kv=3, heads=2),
    _shrink(workloads.CAUSAL_BF16, name="bwd_window_causal_100", sq=(300, 300), sk=(300, 300), split_kv=3,
            window_left=100, heads=2),
    _shrink(workloads.LONG_PREFILL, name="bwd_window_no_mask_64", sq=(257,), sk=(900,), mask="none", window_left=64),
    _shrink(workloads.VARLEN_BATCH_PREFIX, name="bwd_window_varlen_prefix", sq=(130, 1, 257, 64),
            sk=(500, 70, 1500, 3000), heads=2, split_kv_per_seq=(2, 4, 6, 8),
            prefix_offset_per_seq=(370, 69, 1243, 2936), last_valid_per_seq=(499, 69, 1499, 2999), window_left=300),
    _shrink(workloads.LONG_PREFILL, name="bwd_f16_prefill_Sq300_Sk2000", sq=(300,), sk=(2000,), dtype="f16"),
    _shrink(workloads.CAUSAL_BF16, name="bwd_f16_causal_d64", d_qk=64, d_v=64, sq=(130, 130), sk=(200, 200),
            dtype="f16", heads=2),
    _shrink(workloads.CAUSAL_BF16, name="bwd_unsplit_S1", split_kv=1, sq=(200, 200), sk=(640, 640), mask="none",
            heads=2),
    _shrink(workloads.LONG_PREFILL, name="bwd_auto_split_Sq128_Sk9000", heads=2, sq=(128,), sk=(9000,), split_kv=0),
    # prefix offsets far outside 32 bits (a 64-bit field): no row sees a key,
    # every row sees every key, or every window starts past the last key
    _shrink(workloads.CAUSAL_BF16, name="bwd_offset_far_below", mask="prefix_causal", prefix_offset=-(1 << 40),
            sq=(130, 130), sk=(200, 200), heads=2),
    _shrink(workloads.CAUSAL_BF16, name="bwd_offset_far_above", mask="prefix_causal", prefix_offset=1 << 40,
            sq=(130, 130), sk=(200, 200), heads=2),
    _shrink(workloads.CAUSAL_BF16, name="bwd_offset_far_above_window", mask="prefix_causal", prefix_offset=1 << 40,
            window_left=50, sq=(130, 130), sk=(200, 200), heads=2),
]


@pytest.mark.parametrize("w", BWD, ids=lambda w: w.name)
def test_backward_all_rows_and_keys(w):
    log(f"backward {w.name}")
    inputs, dout, dq, dk, dv = run_backward(w, seed=5)
    log(f"  {compare_all(w, inputs, dout, dq, dk, dv)}")


def test_backward_empty_sequences():
    """Sk = 0: dQ = 0; Sq = 0: dK = dV = 0; both in one packed batch."""
    w = _shrink(workloads.VARLEN_BATCH, name="bwd_empties", sq=(5, 0, 40, 3), sk=(0, 100, 0, 90), heads=2,
                split_kv_per_seq=(2, 4, 6, 8))
    log(f"backward {w.name}")
    inputs, dout, dq, dk, dv = run_backward(w, seed=6)
    compare_all(w, inputs, dout, dq, dk, dv)
    assert (_f64(_rows(w, dq, 0, 0, "q")) == 0).all()
    assert (_f64(_rows(w, dk, 1, 1, "k")) == 0).all() and (_f64(_rows(w, dv, 1, 1, "k")) == 0).all()


def _dq_splits(w, inputs):
    """S_dq the library chose, read back from the workspace size."""
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], partial_scratch=False,
                                   **workloads.problem_kwargs(w, inputs))
    rows, H, D = prob.rows, w.heads, w.d_qk
    first = (H * rows * 4 + 255) // 256 * 256
    per_split = H * rows * D * 4
    nbytes = _lib.sk_backward_workspace_bytes(prob.c)
    assert (nbytes - first) % 256 == 0
    return -(-(nbytes - first) // per_split) if per_split else 0


def test_backward_dq_split_count_follows_the_device():
    """dQ is a plain sum over key splits, so the library picks S_dq to fill
    the GPU: several splits for one short query block with long keys, one
    for short keys; both agree with the oracle."""
    many = _shrink(workloads.LONG_PREFILL, name="bwd_dq_many_splits", sq=(200,), sk=(3000,), heads=2)
    one = _shrink(workloads.CAUSAL_BF16, name="bwd_dq_one_split", sq=(300, 300), sk=(500, 500), heads=2)
    for w, expect_many in ((many, True), (one, False)):
        inputs = workloads.make_inputs(w, DEV, 8)
        s_dq = _dq_splits(w, inputs)
        log(f"backward {w.name}: S_dq = {s_dq}")
        assert (s_dq > 1) if expect_many else (s_dq == 1)
        _, dout, dq, dk, dv = run_backward(w, seed=8, inputs=inputs)
        compare_all(w, inputs, dout, dq, dk, dv)


def test_backward_full_size_prefill_sampled():
    """The long-context prefill (H = 12, Sq = 4096, Sk = 42700, D 192/128,
    S = 3) at full size: dQ at sampled rows and dK, dV at sampled keys of two
    heads against the oracle's chunked gradients."""
    w = workloads.LONG_PREFILL
    log(f"backward full {w.name}")
    inputs, dout, dq, dk, dv = run_backward(w, seed=0)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    rows = sample_rows(w.sq[0], 24, 1, 128)
    keys = sample_rows(w.sk[0], 24, 2, 128)
    keys = np.unique(np.concatenate([keys, [14233, 14234, 28466, 28467, 42688, 42699]]))
    for h in (0, 7):
        rq, rk, rv = adapter.backward_sampled(w, inputs, dout, 0, h, rows, keys)
        st = [
            _check("dQ", _f64(dq[torch.as_tensor(rows, device=DEV), h]), rq),
            _check("dK", _f64(dk[torch.as_tensor(keys, device=DEV), h]), rk),
            _check("dV", _f64(dv[torch.as_tensor(keys, device=DEV), h]), rv),
        ]
        log(f"  head {h}: {st}")


def test_backward_full_size_prefill_every_row_and_key():
    """The long-context prefill at full size: dQ at every row and dK, dV at
    every key of every head against the oracle's chunked gradients (about
    3 s of host time per head)."""
    w = workloads.LONG_PREFILL
    log(f"backward full {w.name}, every row, key and head")
    inputs, dout, dq, dk, dv = run_backward(w, seed=5)
    host = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inputs.items()}
    dout_h = dout.cpu()
    rows, keys = np.arange(w.sq[0]), np.arange(w.sk[0])
    for h in range(w.heads):
        rq, rk, rv = adapter.backward_sampled(w, host, dout_h, 0, h, rows, keys)
        st = [
            _check("dQ", _f64(dq[:, h]), rq),
            _check("dK", _f64(dk[:, h]), rk),
            _check("dV", _f64(dv[:, h]), rv),
        ]
        log(f"  head {h}: {st}")


def test_backward_full_size_packed_batch_sampled():
    """The packed 4-sequence batch (Sq = 4096 each, Sk = 8K / 32K / 64K /
    128K, prefix-causal with the query rows at the end of the keys) at full
    size: dQ at sampled rows and dK, dV at sampled keys of the shortest and
    the longest sequence against the oracle's chunked gradients."""
    w = workloads.VARLEN_BATCH_PREFIX
    log(f"backward full {w.name}")
    inputs, dout, dq, dk, dv = run_backward(w, seed=4)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    q0 = [0] + list(np.cumsum(w.sq)[:-1])
    k0 = [0] + list(np.cumsum(w.sk)[:-1])
    for b, h in ((0, 0), (3, 5)):
        rows = sample_rows(w.sq[b], 12, 10 + b, 128)
        keys = sample_rows(w.sk[b], 12, 20 + b, 128)
        # keys that only the last rows see, and the very last ones
        keys = np.unique(np.concatenate([keys, [w.sk[b] - 4096, w.sk[b] - 4095, w.sk[b] - 2, w.sk[b] - 1]]))
        rq, rk, rv = adapter.backward_sampled(w, inputs, dout, b, h, rows, keys)
        st = [
            _check("dQ", _f64(dq[torch.as_tensor(q0[b] + rows, device=DEV), h]), rq),
            _check("dK", _f64(dk[torch.as_tensor(k0[b] + keys, device=DEV), h]), rk),
            _check("dV", _f64(dv[torch.as_tensor(k0[b] + keys, device=DEV), h]), rv),
        ]
        log(f"  sequence {b} head {h}: {st}")


def test_backward_maximum_batch_packed():
    """65535 packed sequences (the most the library takes) of 0..3 rows and
    0..40 keys, bottom-right prefix-causal: every gradient finite, and the
    gradients of 300 sampled sequences (all their rows and keys) against the
    oracle."""
    B = 65535
    rng = np.random.default_rng(65536)
    sq = tuple(int(x) for x in rng.integers(0, 4, B))
    sk = tuple(int(x) for x in rng.integers(0, 41, B))
    w = workloads.Workload("bwd_max_batch_B65535", heads=1, sq=sq, sk=sk, d_qk=64, d_v=64, split_kv=2,
                           n_per_block=8, mask="prefix_causal", packed=True,
                           prefix_offset_per_seq=tuple(k - q for q, k in zip(sq, sk)))
    log(f"backward {w.name}")
    inputs, dout, dq, dk, dv = run_backward(w, seed=8)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    q0 = np.concatenate([[0], np.cumsum(sq)[:-1]])
    k0 = np.concatenate([[0], np.cumsum(sk)[:-1]])
    got = {"dQ": [], "dK": [], "dV": []}
    ref = {"dQ": [], "dK": [], "dV": []}
    dq_c, dk_c, dv_c = _f64(dq[:, 0]), _f64(dk[:, 0]), _f64(dv[:, 0])
    for b in sorted(set([0, 1, B - 2, B - 1] + [int(x) for x in rng.choice(B, 300, replace=False)])):
        rq, rk, rv = adapter.backward_sampled(w, inputs, dout, b, 0, np.arange(sq[b]), np.arange(sk[b]))
        got["dQ"].append(dq_c[q0[b] : q0[b] + sq[b]].ravel())
        got["dK"].append(dk_c[k0[b] : k0[b] + sk[b]].ravel())
        got["dV"].append(dv_c[k0[b] : k0[b] + sk[b]].ravel())
        ref["dQ"].append(rq.ravel())
        ref["dK"].append(rk.ravel())
        ref["dV"].append(rv.ravel())
    st = {n: _check(n, np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    log(f"  {st}")


def test_backward_rejects_f32_and_mismatched_out_dtype():
    w = _shrink(workloads.TINY_F32, name="bwd_f32")
    inputs = workloads.make_inputs(w, DEV, 0)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    q = inputs["q"]
    with pytest.raises(_lib.SplitKVError, match="SK_ERR_UNSUPPORTED"):
        _lib.sk_attn_backward(prob.c, q, q, q, q, q, q, q, q, q, q, 1 << 20)


def _draw_backward(seed: int):
    """A seeded random backward case: storage type, head dims, dense or
    packed (sequences may have no row or no key), mask, per-sequence offsets,
    last valid keys and a window."""
    rng = np.random.default_rng(8100 + seed)
    dtype = str(rng.choice(["bf16", "f16"]))
    d_qk, d_v = [(64, 64), (128, 128), (192, 128)][rng.integers(3)]
    B = int(rng.integers(1, 4))
    packed = bool(rng.random() < 0.6)
    if packed:
        sq = [int(x) for x in rng.integers(0, 201, B)]
        sk = [int(x) for x in rng.integers(0, 1501, B)]
        if max(sq) == 0:
            sq[0] = 1
    else:
        sq, sk = [int(rng.integers(1, 201))] * B, [int(rng.integers(1, 1501))] * B
    mask = str(rng.choice(["none", "causal", "prefix_causal"]))
    offsets = tuple(int(sk[b] - sq[b] + rng.integers(-40, 41)) for b in range(B)) if mask == "prefix_causal" else None
    last_valid = tuple(int(rng.integers(-1, max(sk[b], 1))) for b in range(B)) if rng.random() < 0.3 else None
    window = int(rng.integers(0, 400)) if rng.random() < 0.3 else -1
    return workloads.Workload(f"bwd_rand{seed}_{dtype}_D{d_qk}x{d_v}_{'packed' if packed else 'dense'}_{mask}",
                              heads=int(rng.integers(1, 4)), sq=tuple(sq), sk=tuple(sk), d_qk=d_qk, d_v=d_v,
                              split_kv=int(rng.integers(1, 9)), n_per_block=int(rng.choice([16, 64, 128])),
                              mask=mask, packed=packed, dtype=dtype, prefix_offset_per_seq=offsets,
                              last_valid_per_seq=last_valid, window_left=window)


@pytest.mark.parametrize("seed", range(12))
def test_backward_random_configurations(seed):
    w = _draw_backward(seed)
    log(f"backward random {w.name} sq={w.sq} sk={w.sk} off={w.prefix_offset_per_seq} lv={w.last_valid_per_seq} "
        f"win={w.window_left}")
    inputs, dout, dq, dk, dv = run_backward(w, seed=seed)
    log(f"  {compare_all(w, inputs, dout, dq, dk, dv)}")
