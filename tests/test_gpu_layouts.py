"""Strided layouts through the C ABI against the oracle (GPU), every row and
head.

The ABI takes element strides for Q, K, V and the output (and the backward's
gradients follow the strides of the tensor they belong to).  The other GPU
tests pass contiguous tensors; these pass the same values stored in other
layouts, as callers hold them:
  * dense batches stored [B, S, H, D] and seen as [B, H, S, D] (row stride
    H * D, head stride D), with the output in the same layout;
  * packed batches whose head dims are padded (Q in a [tokens, H, D + 64]
    buffer) and whose K and V sit side by side in one [tokens, H, D_qk +
    D_v] buffer, with the output padded too;
for the MFMA, decode and f32 kernels, and for the backward.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import adapter
from parity import DEV, compare, log
from split_kv_attention_amd import _lib, attention, workloads

pytestmark = pytest.mark.gpu


def _bshd(x):
    """Same values, stored [B, S, H, D], viewed [B, H, S, D]."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def _inputs(w, seed, layout):
    inputs = workloads.make_inputs(w, DEV, seed)
    if layout == "bshd":
        for n in "qkv":
            inputs[n] = _bshd(inputs[n])
            x = inputs[n]
            # rows H * D apart (a one-row sequence has no row stride to speak of)
            assert x.shape[2] == 1 or x.stride(2) == x.shape[1] * x.shape[3]
    else:  # packed, padded Q, K and V in one buffer
        q, k, v = inputs["q"], inputs["k"], inputs["v"]
        qbuf = torch.zeros(q.shape[0], q.shape[1], q.shape[2] + 64, dtype=q.dtype, device=DEV)
        qbuf[..., : q.shape[2]] = q
        kv = torch.zeros(k.shape[0], k.shape[1], k.shape[2] + v.shape[2], dtype=k.dtype, device=DEV)
        kv[..., : k.shape[2]] = k
        kv[..., k.shape[2]:] = v
        inputs["q"], inputs["k"], inputs["v"] = qbuf[..., : q.shape[2]], kv[..., : k.shape[2]], kv[..., k.shape[2]:]
    return inputs


def _out(prob, q, v, layout):
    """The output tensor in the layout under test and its (row, head, batch)
    element strides."""
    c = prob.c
    dt = {_lib.SK_BF16: torch.bfloat16, _lib.SK_F16: torch.float16, _lib.SK_F32: torch.float32}[c.out_dtype]
    if layout == "bshd":
        out = _bshd(torch.empty((c.batch, c.num_heads, c.max_seqlen_q, c.head_dim_v), dtype=dt, device=DEV))
        return out, (out.stride(2), out.stride(1), out.stride(0))
    buf = torch.empty((q.shape[0], c.num_heads, c.head_dim_v + 32), dtype=dt, device=DEV)
    out = buf[..., : c.head_dim_v]
    return out, (out.stride(0), out.stride(1), 0)


def _run(w, layout, seed):
    inputs = _inputs(w, seed, layout)
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    prob0 = attention.build_problem(q, k, v, **workloads.problem_kwargs(w, inputs))
    out, strides = _out(prob0, q, v, layout)
    prob = attention.build_problem(q, k, v, out_strides=strides, **workloads.problem_kwargs(w, inputs))
    counts, o_part, lse_part, _, lse_out = attention.alloc_outputs(prob, q, v)
    counts.fill_(-7)
    for t in (o_part, lse_part, out, lse_out):
        t.fill_(float("nan"))
    attention.run(prob, q, k, v, counts, o_part, lse_part, out, lse_out)
    torch.cuda.synchronize()
    return inputs, prob, dict(counts=counts, o_part=o_part, lse_part=lse_part, out=out, lse_out=lse_out,
                              poisoned=True)


CASES = [
    ("bshd", dataclasses.replace(workloads.CAUSAL_BF16, name="layout_bshd_causal", sq=(200, 200), sk=(333, 333))),
    ("bshd", dataclasses.replace(workloads.DECODE_BF16, name="layout_bshd_decode", sq=(1,) * 6, sk=(3000,) * 6,
                                 heads=4)),
    ("bshd", dataclasses.replace(workloads.TINY_F32, name="layout_bshd_f32", mask="causal", sq=(100,), sk=(130,))),
    ("padded", dataclasses.replace(workloads.LONG_PREFILL, name="layout_padded_prefill", sq=(300,), sk=(2000,))),
    ("padded", dataclasses.replace(workloads.VARLEN_BATCH_PREFIX, name="layout_padded_varlen_prefix",
                                   sq=(130, 1, 257, 64), sk=(500, 70, 1500, 3000), heads=2,
                                   split_kv_per_seq=(2, 4, 6, 8), prefix_offset_per_seq=(370, 69, 1243, 2936),
                                   last_valid_per_seq=(499, 69, 1499, 2999))),
    ("padded", dataclasses.replace(workloads.DECODE_BF16, name="layout_padded_decode_packed", packed=True,
                                   sq=(1, 1, 0, 1), sk=(900, 2049, 10, 0), heads=3, d_qk=64, d_v=64, split_kv=5)),
    # sized for the 256-row kernel (at least one 256-row item per CU on MI355X)
    ("bshd", dataclasses.replace(workloads.CAUSAL_BF16, name="layout_bshd_causal_256rows", sq=(300, 300),
                                 sk=(2500, 2500), heads=16, split_kv=4)),
    ("padded", dataclasses.replace(workloads.LONG_PREFILL, name="layout_padded_prefill_256rows", sq=(300,),
                                   sk=(3000,), heads=16, split_kv=8)),
]


@pytest.mark.parametrize("layout,w", CASES, ids=lambda x: x if isinstance(x, str) else x.name)
def test_strided_layouts_forward_all_rows(layout, w):
    log(f"layout {w.name}")
    inputs, prob, res = _run(w, layout, seed=23)
    if w.name.endswith("_256rows"):
        assert prob.m_per_block == 256
    st = compare(w, inputs, prob, res, label=w.name)
    log(f"  {st}")


BWD = [c for c in CASES if c[1].dtype != "f32" and c[1].name != "layout_padded_decode_packed"]


@pytest.mark.parametrize("layout,w", BWD, ids=lambda x: x if isinstance(x, str) else x.name)
def test_strided_layouts_backward(layout, w):
    """Gradients in the layout of the tensor they belong to; dO in the
    output's layout."""
    from test_gpu_backward import _check, _f64, _rows

    log(f"layout backward {w.name}")
    inputs, prob, res = _run(w, layout, seed=24)
    q, k, v, out = inputs["q"], inputs["k"], inputs["v"], res["out"]
    dout = torch.empty_strided(out.shape, out.stride(), dtype=out.dtype, device=DEV)
    dout.copy_(workloads.make_dout(w, DEV, 24))
    grads = [torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=DEV).fill_(float("nan"))
             for x in (q, k, v)]
    nbytes = _lib.sk_backward_workspace_bytes(prob.c)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    _lib.sk_attn_backward(prob.c, q, k, v, out, dout, res["lse_out"], *grads, ws, nbytes)
    torch.cuda.synchronize()
    ref = adapter.backward(w, inputs, dout)
    for i, (name, g, n) in enumerate((("dQ", grads[0], "q"), ("dK", grads[1], "k"), ("dV", grads[2], "k"))):
        got = np.concatenate([_f64(_rows(w, g, b, h, n)).ravel() for (b, h) in ref])
        exp = np.concatenate([grads_ref[i].ravel() for grads_ref in ref.values()])
        log(f"  {name}: {_check(name, got, exp)}")
