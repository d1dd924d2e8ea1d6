"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

The five workload shapes follow the pages: a tiny f32 case, causal prefill
with more query rows than a key tile, batched decode, and the long-context
packed-varlen prefill of the aiter page "[ASM][HIP][JIT][gfx942] Optimize
long-context FMHA with split-KV" (H = 12, D_qk = 192, D_v = 128, Sq = 4096,
Sk from 8K to 128K; Motivation and Test Result), which synthetic N(0, 1)
tensors stand in for.  Q, K and V are drawn as float32 N(0, 1) from a torch
generator seeded per (seed, tensor), then rounded to bf16 or f16 (round to
nearest even) for 16-bit workloads.  Both the HIP path and the oracle read the same
generated tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    sq: tuple            # per-sequence query rows
    sk: tuple            # per-sequence keys
    d_qk: int
    d_v: int
    split_kv: int        # S_max
    n_per_block: int
    mask: str = "none"
    packed: bool = False
    dtype: str = "bf16"
    split_kv_per_seq: tuple | None = None
    prefix_offset: int = 0
    prefix_offset_per_seq: tuple | None = None
    last_valid_kv_index: int = -1
    last_valid_per_seq: tuple | None = None
    scale: float | None = None
    window_left: int = -1  # sliding window (keys behind q + offset), -1 = none
    notes: str = field(default="", compare=False)

    @property
    def batch(self) -> int:
        return len(self.sq)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d_qk)

    @property
    def torch_dtype(self):
        return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[self.dtype]


TINY_F32 = Workload(
    "tiny_f32_B1_H2_Sq64_Sk256_D64_S4", heads=2, sq=(64,), sk=(256,), d_qk=64, d_v=64, split_kv=4,
    n_per_block=32, dtype="f32", scale=1.0 / 8.0,
)
CAUSAL_BF16 = Workload(
    "causal_bf16_B2_H8_Sq512_Sk512_D128_S4", heads=8, sq=(512, 512), sk=(512, 512), d_qk=128, d_v=128,
    split_kv=4, n_per_block=64, mask="causal",
)
DECODE_BF16 = Workload(
    "decode_bf16_B64_H32_Sq1_Sk32768_D128_S16", heads=32, sq=(1,) * 64, sk=(32768,) * 64, d_qk=128, d_v=128,
    split_kv=16, n_per_block=64,
)
LONG_PREFILL = Workload(
    "varlen_prefill_bf16_H12_Sq4096_Sk42700_D192x128_S3", heads=12, sq=(4096,), sk=(42700,), d_qk=192, d_v=128,
    split_kv=3, n_per_block=64, packed=True,
)
VARLEN_BATCH = Workload(
    "varlen_batch_bf16_H12_Sq4096_Sk8K-128K_D192x128_S2-8", heads=12, sq=(4096,) * 4,
    sk=(8192, 32768, 65536, 131072), d_qk=192, d_v=128, split_kv=8, split_kv_per_seq=(2, 4, 6, 8),
    n_per_block=64, packed=True,
)
VARLEN_BATCH_PREFIX = Workload(
    "varlen_batch_prefix_causal_bf16_H12_Sq4096_Sk8K-128K_D192x128_S2-8", heads=12, sq=(4096,) * 4,
    sk=(8192, 32768, 65536, 131072), d_qk=192, d_v=128, split_kv=8, split_kv_per_seq=(2, 4, 6, 8),
    n_per_block=64, packed=True, mask="prefix_causal",
    prefix_offset_per_seq=(8192 - 4096, 32768 - 4096, 65536 - 4096, 131072 - 4096),
    last_valid_per_seq=(8191, 32767, 65535, 131071),
)

CONFIGS = [TINY_F32, CAUSAL_BF16, DECODE_BF16, LONG_PREFILL, VARLEN_BATCH, VARLEN_BATCH_PREFIX]


def _gen(device, seed: int, tensor_id: int):
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + tensor_id)
    return g


def make_inputs(w: Workload, device, seed: int = 0) -> dict:
    """Q, K, V (and cu_seqlens for packed workloads) on `device`.

    Dense workloads: [B, H, S, D]; packed: [tokens, H, D] with int32
    cu_seqlens.  Drawn in float32 then cast to the workload dtype."""
    dt = w.torch_dtype
    H = w.heads

    def draw(shape, tid):
        x = torch.randn(shape, generator=_gen(device, seed, tid), device=device, dtype=torch.float32)
        return x.to(dt) if dt != torch.float32 else x

    out = {}
    if w.packed:
        tq, tk = sum(w.sq), sum(w.sk)
        out["q"] = draw((tq, H, w.d_qk), 0)
        out["k"] = draw((tk, H, w.d_qk), 1)
        out["v"] = draw((tk, H, w.d_v), 2)
        cq = [0]
        ck = [0]
        for a, b in zip(w.sq, w.sk):
            cq.append(cq[-1] + a)
            ck.append(ck[-1] + b)
        out["cu_seqlens_q"] = torch.tensor(cq, dtype=torch.int32, device=device)
        out["cu_seqlens_k"] = torch.tensor(ck, dtype=torch.int32, device=device)
    else:
        if len(set(w.sq)) != 1 or len(set(w.sk)) != 1:
            raise ValueError("a dense workload has equal lengths")
        B = w.batch
        out["q"] = draw((B, H, w.sq[0], w.d_qk), 0)
        out["k"] = draw((B, H, w.sk[0], w.d_qk), 1)
        out["v"] = draw((B, H, w.sk[0], w.d_v), 2)
    return out


def make_dout(w: Workload, device, seed: int = 0):
    """Output gradient dO, N(0, 1) in the workload dtype, shaped like the
    output: [B, H, Sq, D_v] dense, [tokens, H, D_v] packed."""
    shape = (sum(w.sq), w.heads, w.d_v) if w.packed else (w.batch, w.heads, w.sq[0], w.d_v)
    x = torch.randn(shape, generator=_gen(device, seed, 3), device=device, dtype=torch.float32)
    return x.to(w.torch_dtype) if w.torch_dtype != torch.float32 else x


def problem_kwargs(w: Workload, inputs: dict) -> dict:
    """Keyword arguments of attention.build_problem for workload `w`."""
    kw = dict(
        split_kv=w.split_kv, n_per_block=w.n_per_block, mask=w.mask, prefix_offset=w.prefix_offset,
        last_valid_kv_index=w.last_valid_kv_index, softmax_scale=w.softmax_scale,
        split_kv_per_seq=w.split_kv_per_seq, prefix_offset_per_seq=w.prefix_offset_per_seq,
        last_valid_per_seq=w.last_valid_per_seq, window_left=w.window_left,
    )
    if w.packed:
        kw.update(cu_seqlens_q=inputs["cu_seqlens_q"], cu_seqlens_k=inputs["cu_seqlens_k"],
                  max_seqlen_q=max(w.sq), max_seqlen_k=max(w.sk))
    return kw
