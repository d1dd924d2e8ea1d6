"""Run the oracle over a whole batch laid out like the library's tensors.

TEST INFRASTRUCTURE ONLY (tests/, smoke check, benchmark CPU baseline).
It imports nothing from the library: a workload is any object with the
attributes sq, sk, heads, split_kv, split_kv_per_seq, n_per_block, mask,
prefix_offset(_per_seq), last_valid_kv_index, last_valid_per_seq, packed and
softmax_scale, and tensors are torch tensors or numpy arrays on the host.

Layouts handled: dense [B, H, S, D] and packed [tokens, H, D] with the
sequences one after another (packed row of (b, r) = sum of earlier Sq + r).
"""
from __future__ import annotations

import numpy as np

from .splitkv import (
    MASK_CAUSAL,
    MASK_NONE,
    MASK_PREFIX_CAUSAL,
    SeqSpec,
    combine,
    partials,
    sampled_backward,
    unsplit,
    unsplit_backward,
    valid_split_counts,
)

_MASKS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "prefix_causal": MASK_PREFIX_CAUSAL}


def seq_specs(w) -> list:
    specs = []
    for b in range(len(w.sq)):
        specs.append(
            SeqSpec(
                sq=w.sq[b],
                sk=w.sk[b],
                split_kv=w.split_kv_per_seq[b] if w.split_kv_per_seq else w.split_kv,
                n_per_block=w.n_per_block,
                mask=_MASKS[w.mask],
                prefix_offset=w.prefix_offset_per_seq[b] if w.prefix_offset_per_seq else w.prefix_offset,
                last_valid=w.last_valid_per_seq[b] if w.last_valid_per_seq else w.last_valid_kv_index,
                window_left=getattr(w, "window_left", -1),
            )
        )
    return specs


def row_starts(w) -> np.ndarray:
    """Packed row index of each sequence's first query."""
    if w.packed:
        return np.concatenate([[0], np.cumsum(w.sq)[:-1]]).astype(np.int64)
    return np.arange(len(w.sq), dtype=np.int64) * w.sq[0]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def head_slices(w, inputs, b: int, h: int, rows=None):
    """Q rows (default all), K and V of sequence b, head h, as float64 arrays."""
    sq, sk = w.sq[b], w.sk[b]
    rows = np.arange(sq) if rows is None else np.asarray(rows)
    if w.packed:
        q0 = int(sum(w.sq[:b]))
        k0 = int(sum(w.sk[:b]))
        Q = _f64(inputs["q"][q0 + rows, h]) if len(rows) else np.zeros((0, inputs["q"].shape[-1]))
        K = _f64(inputs["k"][k0 : k0 + sk, h])
        V = _f64(inputs["v"][k0 : k0 + sk, h])
    else:
        Q = _f64(inputs["q"][b, h][rows]) if len(rows) else np.zeros((0, inputs["q"].shape[-1]))
        K = _f64(inputs["k"][b, h, :sk])
        V = _f64(inputs["v"][b, h, :sk])
    return Q, K, V


def counts(w) -> np.ndarray:
    """Valid-split counts for every packed row."""
    return np.concatenate([valid_split_counts(s) for s in seq_specs(w)]).astype(np.int64)


def expected(w, inputs, m_per_block: int, rows_per_seq=None, heads=None, with_unsplit=False):
    """Oracle results for the listed rows of each sequence (default all).

    Returns a dict keyed by (b, h) with entries
      rows, counts, O, lse (merged), O_s, L_s (partials at m_per_block)
    and, when with_unsplit, O_ref / lse_ref from the unsplit definition."""
    specs = seq_specs(w)
    heads = range(w.heads) if heads is None else heads
    res = {}
    for b, spec in enumerate(specs):
        rows = np.arange(spec.sq) if rows_per_seq is None else np.asarray(rows_per_seq[b], dtype=np.int64)
        if len(rows) == 0:
            continue
        cnt = valid_split_counts(spec, rows)
        for h in heads:
            Q, K, V = head_slices(w, inputs, b, h, rows)
            O_s, L_s = partials(Q, K, V, w.softmax_scale, spec, m_per_block, rows)
            O, lse = combine(O_s, L_s, cnt)
            d = {"rows": rows, "counts": cnt, "O": O, "lse": lse, "O_s": O_s, "L_s": L_s}
            if with_unsplit:
                d["O_ref"], d["lse_ref"] = unsplit(Q, K, V, w.softmax_scale, spec, rows)
            res[(b, h)] = d
    return res


def _dout_slice(w, dout, b: int, h: int):
    if w.packed:
        q0 = int(sum(w.sq[:b]))
        return _f64(dout[q0 : q0 + w.sq[b], h])
    return _f64(dout[b, h])


def backward(w, inputs, dout, heads=None):
    """Oracle gradients of every sequence and head, keyed by (b, h):
    dQ [sq, Dqk], dK [sk, Dqk], dV [sk, Dv] from `unsplit_backward`."""
    heads = range(w.heads) if heads is None else heads
    res = {}
    for b, spec in enumerate(seq_specs(w)):
        for h in heads:
            Q, K, V = head_slices(w, inputs, b, h)
            res[(b, h)] = unsplit_backward(Q, K, V, _dout_slice(w, dout, b, h), w.softmax_scale, spec)
    return res


def backward_sampled(w, inputs, dout, b: int, h: int, rows, keys):
    """Oracle dQ at `rows` and dK, dV at `keys` of sequence b, head h
    (`sampled_backward`, for sizes whose whole score matrix is too large)."""
    spec = seq_specs(w)[b]
    Q, K, V = head_slices(w, inputs, b, h)
    return sampled_backward(Q, K, V, _dout_slice(w, dout, b, h), w.softmax_scale, spec, rows, keys)
