"""Torch-facing helpers over the libsplitkv C ABI (marshalling only).

`build_problem` fills an sk_problem from tensors; `split_kv_attention` allocates
the outputs and the partial buffers with torch on the inputs' device and
enqueues the three entry points on the current stream:

    sk_valid_split_counts -> sk_attn_partial -> sk_attn_combine

and `split_kv_attention_backward` enqueues sk_attn_backward for the gradients.

Layouts: a dense batch is [B, H, S, D]; a packed variable-length batch is
[tokens, H, D] with int32 cu_seqlens (aiter page, flash_attn_varlen_func).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _lib
from ._lib import SK_BF16, SK_F16, SK_F32, SK_MASK_CAUSAL, SK_MASK_NONE, SK_MASK_PREFIX_CAUSAL, SkProblem

_MASKS = {"none": SK_MASK_NONE, "causal": SK_MASK_CAUSAL, "prefix_causal": SK_MASK_PREFIX_CAUSAL}
_DTYPES = {torch.float32: SK_F32, torch.bfloat16: SK_BF16, torch.float16: SK_F16}


@dataclass
class Problem:
    """An sk_problem plus the tensors its pointers refer to (kept alive)."""

    c: SkProblem
    keep: list = field(default_factory=list)

    @property
    def rows(self) -> int:
        return _lib.sk_rows(self.c)

    @property
    def split_kv(self) -> int:
        """Splits the library uses (the automatic count when split_kv = 0)."""
        return _lib.sk_split_kv(self.c)

    @property
    def m_per_block(self) -> int:
        return _lib.sk_partial_m_per_block(self.c)

    def workspace_bytes(self) -> tuple[int, int]:
        return _lib.sk_workspace_bytes(self.c)


def _i32(x, device):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        t = x.to(device=device, dtype=torch.int32).contiguous()
    else:
        t = torch.tensor(list(x), dtype=torch.int32, device=device)
    return t


def build_problem(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    *,
    split_kv: int,
    n_per_block: int = 64,
    mask: str = "none",
    prefix_offset: int = 0,
    last_valid_kv_index: int = -1,
    softmax_scale: float | None = None,
    cu_seqlens_q=None,
    cu_seqlens_k=None,
    max_seqlen_q: int | None = None,
    max_seqlen_k: int | None = None,
    split_kv_per_seq=None,
    prefix_offset_per_seq=None,
    last_valid_per_seq=None,
    out_dtype: torch.dtype | None = None,
    out_strides: tuple[int, int, int] | None = None,
    partial_scratch: bool = True,
    window_left: int = -1,
) -> Problem:
    """Describe one forward call; tensors stay where they are.  With
    `partial_scratch` (and tensors on a GPU) the problem carries the scratch
    buffer sk_attn_partial balances its last round of workgroups with."""
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype: float32, bfloat16 or float16")
    dev = q.device
    keep = []
    p = SkProblem()
    d_qk, d_v = q.shape[-1], v.shape[-1]
    if q.dim() == 4:  # dense [B, H, S, D]
        if cu_seqlens_q is not None:
            raise ValueError("a 4-D q is a dense batch; cu_seqlens_q must be None")
        B, H, Sq, _ = q.shape
        p.q_stride_batch, p.q_stride_head, p.q_stride_row = q.stride(0), q.stride(1), q.stride(2)
        mq = Sq
        total_q = B * Sq
    elif q.dim() == 3:  # packed [tokens, H, D]
        if cu_seqlens_q is None or max_seqlen_q is None:
            raise ValueError("a 3-D q is packed: cu_seqlens_q and max_seqlen_q are required")
        H = q.shape[1]
        B = len(cu_seqlens_q) - 1
        p.q_stride_row, p.q_stride_head, p.q_stride_batch = q.stride(0), q.stride(1), 0
        mq = max_seqlen_q
        total_q = q.shape[0]
    else:
        raise ValueError("q must be [B, H, S, D] or [tokens, H, D]")
    if k.dim() == 4:
        if cu_seqlens_k is not None:
            raise ValueError("a 4-D k is a dense batch; cu_seqlens_k must be None")
        mk = k.shape[2]
        p.k_stride_batch, p.k_stride_head, p.k_stride_row = k.stride(0), k.stride(1), k.stride(2)
        p.v_stride_batch, p.v_stride_head, p.v_stride_row = v.stride(0), v.stride(1), v.stride(2)
    else:
        if cu_seqlens_k is None or max_seqlen_k is None:
            raise ValueError("a 3-D k is packed: cu_seqlens_k and max_seqlen_k are required")
        mk = max_seqlen_k
        p.k_stride_row, p.k_stride_head, p.k_stride_batch = k.stride(0), k.stride(1), 0
        p.v_stride_row, p.v_stride_head, p.v_stride_batch = v.stride(0), v.stride(1), 0
    if out_strides is None:
        if q.dim() == 4:
            out_strides = (d_v, mq * d_v, H * mq * d_v)  # [B, H, S, Dv] contiguous
        else:
            out_strides = (H * d_v, d_v, 0)  # [tokens, H, Dv] contiguous
    p.o_stride_row, p.o_stride_head, p.o_stride_batch = out_strides

    p.batch = B
    p.num_heads = H
    p.max_seqlen_q = mq
    p.max_seqlen_k = mk
    p.total_q = total_q
    p.head_dim_qk = d_qk
    p.head_dim_v = d_v
    p.split_kv = split_kv
    p.n_per_block = n_per_block
    p.mask = _MASKS[mask]
    p.dtype = _DTYPES[q.dtype]
    p.out_dtype = _DTYPES[out_dtype or q.dtype]
    p.prefix_offset = prefix_offset
    p.last_valid_kv_index = last_valid_kv_index
    p.softmax_scale = softmax_scale if softmax_scale is not None else d_qk ** -0.5
    p.reserved0 = 0
    p.window_left = window_left
    for name, val in (
        ("cu_seqlens_q", cu_seqlens_q),
        ("cu_seqlens_k", cu_seqlens_k),
        ("split_kv_per_seq", split_kv_per_seq),
        ("prefix_offset_per_seq", prefix_offset_per_seq),
        ("last_valid_per_seq", last_valid_per_seq),
    ):
        t = _i32(val, dev)
        if t is not None:
            keep.append(t)
            setattr(p, name, t.data_ptr())
    if partial_scratch and q.is_cuda:
        nbytes = _lib.sk_partial_scratch_bytes(p)
        if nbytes > 0:
            scratch = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            keep.append(scratch)
            p.partial_scratch = scratch.data_ptr()
            p.partial_scratch_bytes = nbytes
    return Problem(p, keep)


def alloc_outputs(prob: Problem, q: torch.Tensor, v: torch.Tensor, out_dtype: torch.dtype | None = None):
    """Allocate counts, o_part, lse_part, out and lse_out for `prob`."""
    c = prob.c
    dev = q.device
    rows = prob.rows
    counts = torch.empty(rows, dtype=torch.int32, device=dev)
    s_max = prob.split_kv
    o_part = torch.empty((c.num_heads, s_max, rows, c.head_dim_v), dtype=torch.float32, device=dev)
    lse_part = torch.empty((c.num_heads, s_max, rows), dtype=torch.float32, device=dev)
    od = out_dtype or q.dtype
    if q.dim() == 4:
        out = torch.empty((c.batch, c.num_heads, c.max_seqlen_q, c.head_dim_v), dtype=od, device=dev)
    else:
        out = torch.empty((q.shape[0], c.num_heads, c.head_dim_v), dtype=od, device=dev)
    lse_out = torch.empty((c.num_heads, rows), dtype=torch.float32, device=dev)
    return counts, o_part, lse_part, out, lse_out


def run(prob: Problem, q, k, v, counts, o_part, lse_part, out, lse_out, stream=None, counts_in_combine=True):
    """Enqueue counts -> partial -> combine on `stream` (default: current)."""
    _lib.sk_valid_split_counts(prob.c, counts, stream)
    _lib.sk_attn_partial(prob.c, q, k, v, o_part, lse_part, stream)
    _lib.sk_attn_combine(prob.c, o_part, lse_part, counts if counts_in_combine else None, out, lse_out, stream)


def split_kv_attention(q, k, v, *, return_lse: bool = True, return_partials: bool = False,
                       out_dtype: torch.dtype | None = None, **kw):
    """Split-KV attention forward through libsplitkv; see build_problem for arguments.

    Returns out (and lse [H, rows] when return_lse; and the dict of counts and
    partials when return_partials)."""
    prob = build_problem(q, k, v, out_dtype=out_dtype, **kw)
    counts, o_part, lse_part, out, lse_out = alloc_outputs(prob, q, v, out_dtype)
    run(prob, q, k, v, counts, o_part, lse_part, out, lse_out if return_lse else None)
    res = [out]
    if return_lse:
        res.append(lse_out)
    if return_partials:
        res.append({"counts": counts, "o_part": o_part, "lse_part": lse_part, "m_per_block": prob.m_per_block,
                    "problem": prob})
    return res[0] if len(res) == 1 else tuple(res)


def split_kv_attention_backward(q, k, v, out, lse, dout, **kw):
    """dQ, dK, dV of split_kv_attention through sk_attn_backward.

    `out` and `lse` are the forward's results for the same arguments (`kw` as
    for build_problem; out_dtype must be q's dtype).  The gradients have the
    shapes of q, k, v; a packed K/V's rows that belong to no sequence come
    back as zeros.  The workspace is allocated with torch."""
    prob = build_problem(q, k, v, partial_scratch=False, **kw)
    dq = torch.empty_like(q)
    dk = torch.zeros_like(k) if k.dim() == 3 else torch.empty_like(k)
    dv = torch.zeros_like(v) if v.dim() == 3 else torch.empty_like(v)
    nbytes = _lib.sk_backward_workspace_bytes(prob.c)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _lib.sk_attn_backward(prob.c, q, k, v, out, dout, lse, dq, dk, dv, ws, nbytes)
    return dq, dk, dv
