"""Shared helpers of the GPU parity tests: run a workload through libsplitkv,
run the oracle on the same inputs, and compare.

Tolerances (bf16 inputs): max |error| <= 1e-2 on f32 results (partials, LSE,
f32 output) and cosine similarity >= 0.99999; a bf16 output may additionally
differ by half a bf16 ulp of the exact value, the rounding the final cast
itself adds.  f32 inputs: max |error| <= 1e-5.  Valid-split counts and the
-inf pattern of every LSE are compared exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import adapter
from split_kv_attention_amd import attention, workloads

DEV = "cuda"
TOL_BF16 = 1e-2
TOL_F32 = 1e-5
COS_MIN = 0.99999


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, seed=0, out_dtype=None, counts_in_combine=True, inputs=None, poison=True):
    """Inputs, problem and every buffer of one forward pass (synchronised)."""
    if inputs is None:
        inputs = workloads.make_inputs(w, DEV, seed)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], out_dtype=out_dtype,
                                   **workloads.problem_kwargs(w, inputs))
    counts, o_part, lse_part, out, lse_out = attention.alloc_outputs(prob, inputs["q"], inputs["v"], out_dtype)
    if poison:  # every slot the library must write starts as NaN / -7
        counts.fill_(-7)
        o_part.fill_(float("nan"))
        lse_part.fill_(float("nan"))
        out.fill_(float("nan"))
        lse_out.fill_(float("nan"))
    attention.run(prob, inputs["q"], inputs["k"], inputs["v"], counts, o_part, lse_part, out, lse_out,
                  counts_in_combine=counts_in_combine)
    torch.cuda.synchronize()
    return inputs, prob, dict(counts=counts, o_part=o_part, lse_part=lse_part, out=out, lse_out=lse_out,
                              poisoned=poison)


def sample_rows(sq: int, n: int, seed: int, tile: int) -> np.ndarray:
    """Rows to check at full size: tile edges, both ends, and random rows."""
    fixed = {0, 1, sq - 1, sq - 2, tile - 1, tile, tile + 1, sq // 2, sq // 2 - 1}
    rng = np.random.default_rng(seed)
    extra = rng.choice(sq, size=min(n, sq), replace=False)
    rows = sorted(r for r in fixed.union(int(x) for x in extra) if 0 <= r < sq)
    return np.array(rows, dtype=np.int64)


def _out_rows(w, out, b, h, rows, row0):
    if w.packed:
        return out[torch.as_tensor(row0 + rows, device=out.device), h]
    return out[b, h][torch.as_tensor(rows, device=out.device)]


def _half_ulp(x: np.ndarray, mantissa_bits: int) -> np.ndarray:
    """Half a unit in the last place of x in a format with that many stored
    mantissa bits (bf16: 7, f16: 10; f16 subnormals below 2^-14)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if mantissa_bits == 10:
        e = np.maximum(e, -14.0)
    return np.where(ax > 0, np.exp2(e - mantissa_bits - 1), 0.0)


def compare(w, inputs, prob, res, rows_per_seq=None, heads=None, check_partials=True, label="", exp=None):
    """Compare GPU results with the oracle on the listed rows; returns stats.
    `exp`: the oracle's results (adapter.expected) when already computed."""
    f32_in = w.dtype == "f32"
    tol = TOL_F32 if f32_in else TOL_BF16
    mpb = prob.m_per_block
    if exp is None:
        exp = adapter.expected(w, inputs, mpb, rows_per_seq=rows_per_seq, heads=heads)
    starts = adapter.row_starts(w)
    specs = adapter.seq_specs(w)
    gc = res["counts"].cpu().numpy()
    out_bits = {torch.bfloat16: 7, torch.float16: 10}.get(res["out"].dtype)
    num = den_g = den_r = 0.0
    stats = dict(max_err_out=0.0, max_err_lse=0.0, max_err_part=0.0, max_err_out_vs_rounded=0.0)
    for (b, h), e in exp.items():
        rows = e["rows"]
        row0 = int(starts[b])
        prow = row0 + rows
        # counts: bit-exact
        np.testing.assert_array_equal(gc[prow], e["counts"], err_msg=f"{label} counts b={b}")
        # partials
        if check_partials:
            S_b = specs[b].split_kv
            idx = torch.as_tensor(prow, device=res["o_part"].device)
            gL = res["lse_part"][h][:S_b][:, idx].double().cpu().numpy()
            gO = res["o_part"][h][:S_b][:, idx].double().cpu().numpy()
            rL, rO = e["L_s"].copy(), e["O_s"].copy()
            # splits past the block's populated ones are not written (early exit);
            # in the oracle they are (0, -inf) for every row of the block
            pop = np.array([oracle.block_populated_splits(specs[b], mpb, int(q)) for q in rows])
            skipped = np.arange(S_b)[:, None] >= pop[None, :]
            assert np.isneginf(rL[skipped]).all() and (rO[skipped] == 0).all(), f"{label} oracle b={b}"
            if res.get("poisoned"):
                assert np.isnan(gL[skipped]).all() and np.isnan(gO[skipped]).all(), \
                    f"{label} a block-empty split was written b={b} h={h}"
            gL[skipped], gO[skipped] = rL[skipped], rO[skipped]
            assert not np.isnan(gL).any() and not np.isnan(gO).any(), f"{label} unwritten partial slot b={b} h={h}"
            np.testing.assert_array_equal(np.isneginf(gL), np.isneginf(rL), err_msg=f"{label} -inf pattern b={b} h={h}")
            fin = np.isfinite(rL)
            if fin.any():
                stats["max_err_lse"] = max(stats["max_err_lse"], float(np.abs(gL[fin] - rL[fin]).max()))
            err = float(np.abs(gO - rO).max()) if gO.size else 0.0
            stats["max_err_part"] = max(stats["max_err_part"], err)
            assert err <= tol, f"{label} partial O error {err} b={b} h={h}"
        # merged output
        g = _out_rows(w, res["out"], b, h, rows, row0).double().cpu().numpy()
        r = e["O"]
        assert np.isfinite(g).all(), f"{label} non-finite output b={b} h={h}"
        err = np.abs(g - r)
        if out_bits:
            allow = tol + _half_ulp(r, out_bits)
            rr = torch.from_numpy(r).to(res["out"].dtype).double().numpy()
            stats["max_err_out_vs_rounded"] = max(stats["max_err_out_vs_rounded"], float(np.abs(g - rr).max()))
        else:
            allow = tol
        bad = err > allow
        assert not bad.any(), f"{label} output error {float(err[bad].max())} b={b} h={h}"
        stats["max_err_out"] = max(stats["max_err_out"], float(err.max()) if err.size else 0.0)
        num += float((g * r).sum())
        den_g += float((g * g).sum())
        den_r += float((r * r).sum())
        # merged LSE
        gl = res["lse_out"][h][torch.as_tensor(prow, device=res["lse_out"].device)].double().cpu().numpy()
        rl = e["lse"]
        np.testing.assert_array_equal(np.isneginf(gl), np.isneginf(rl), err_msg=f"{label} lse -inf b={b} h={h}")
        fin = np.isfinite(rl)
        if fin.any():
            le = float(np.abs(gl[fin] - rl[fin]).max())
            stats["max_err_lse"] = max(stats["max_err_lse"], le)
            assert le <= tol, f"{label} lse error {le} b={b} h={h}"
    if den_g > 0 and den_r > 0:
        cos = num / np.sqrt(den_g * den_r)
        stats["cos"] = cos
        assert cos >= COS_MIN, f"{label} cosine {cos}"
    else:
        assert den_g == 0 and den_r == 0, f"{label} one output is zero, the other not"
    stats["max_err_lse_ok"] = stats["max_err_lse"] <= tol
    assert stats["max_err_lse_ok"], f"{label} partial lse error {stats['max_err_lse']}"
    return stats
