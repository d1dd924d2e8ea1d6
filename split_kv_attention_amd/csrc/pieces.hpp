// Merge of the key pieces of the partial kernels' last round (shared by the
// 16-bit partial kernels; BM = the kernel's query rows per workgroup).
#pragma once

#include <float.h>

#include "sk_common.hpp"

namespace sk {

// Merge of the pieces of each tail item into its o_part /
// lse_part slot: the pieces are a partition of the split's keys, so this is
// the same log-sum-exp merge as the combine (rocmlirTriton page, "NaN-safe
// merge"): m = max(max_p L_p, lowest finite), w_p = exp(L_p - m),
// O_s = sum_p w_p O_p / max(sum_p w_p, 1), L_s = m + log(sum_p w_p), and a
// row no piece saw any key of keeps (0, -inf).
// One thread per (row, 4 values) of a tail item; a block covers
// 256 / (DV / 4) rows of one item.  All pieces of a row are loaded
// before any is used.
template <int BM, int DV>
__global__ __launch_bounds__(256) void merge_pieces_kernel(PartialArgs a) {
    constexpr int kParts = DV / 4;
    constexpr int kRows = 256 / kParts;  // rows per block
    constexpr int kBlocks = BM / kRows;  // blocks per item
    const uint32_t tail_i = blockIdx.x / kBlocks;
    const int r = (int)(blockIdx.x % kBlocks) * kRows + (int)threadIdx.x / kParts;
    const int part = (int)threadIdx.x % kParts;
    const WorkItem it = decode_work(a, a.n_main + tail_i);
    const Seq sq = load_seq(a.seqs, it.batch);
    if (it.split >= sq.splits) return;
    const int r0 = it.tile * BM;
    if (r0 + r >= sq.sq) return;
    int ks, ke;  // a block-empty split: no piece ran, nothing is written
    block_split_range(sq, a.seqs.mask, a.seqs.n_per_block, min(r0 + BM, sq.sq) - 1, it.split, ks, ke);
    if (ks >= ke) return;
    const int64_t prow = sq.row0 + r0 + r;
    if (prow >= a.rows) return;
    const int P = a.pieces;
    const int64_t base = (int64_t)tail_i * P * BM + r;  // piece p: row base + p * BM
    if (!in_bounds(a.check, kSitePieceSlot, base + (int64_t)(P - 1) * BM, (int64_t)(a.n_work - a.n_main) * P * BM))
        return;
    float L[kMaxPieces];
    float4 O[kMaxPieces];
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p) {
        if (p < P) {
            L[p] = a.piece_l[base + (int64_t)p * BM];
            O[p] = *reinterpret_cast<const float4*>(a.piece_o + (base + (int64_t)p * BM) * DV + part * 4);
        }
    }
    float m = -FLT_MAX;
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p)
        if (p < P) m = fmaxf(m, L[p]);
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p) {
        if (p < P) {
            const float w = expf(L[p] - m);
            den += w;
            acc.x = fmaf(w, O[p].x, acc.x);
            acc.y = fmaf(w, O[p].y, acc.y);
            acc.z = fmaf(w, O[p].z, acc.z);
            acc.w = fmaf(w, O[p].w, acc.w);
        }
    }
    const float inv = 1.0f / fmaxf(den, 1.0f);
    const int64_t slot = ((int64_t)it.head * a.seqs.s_max + it.split) * a.rows + prow;
    if (!in_bounds(a.check, kSitePartialSlot, slot, (int64_t)a.heads * a.seqs.s_max * a.rows)) return;
    *reinterpret_cast<float4*>(a.o_part + slot * DV + part * 4) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (part == 0) a.lse_part[slot] = den > 0.f ? m + logf(den) : -INFINITY;
}

// One launch of the merge for n_tail tail items.
template <int BM, int DV>
void launch_merge_pieces(const PartialArgs& a, uint32_t n_tail, hipStream_t stream) {
    constexpr int kBlocks = BM / (256 / (DV / 4));
    hipLaunchKernelGGL((merge_pieces_kernel<BM, DV>), dim3(n_tail * kBlocks), dim3(256), 0, stream, a);
}

}  // namespace sk
