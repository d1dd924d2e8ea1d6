// NaN-safe f32 merge of split partials (rocmlirTriton page "Recombine fully
// masked split-KV attention partials on the host", sections "NaN-safe merge",
// "f32 merge for f16/bf16" and "Per-row mask layout").
//
// HBM-bound: every (row, head) reads its valid partial rows once and writes
// one output row.  One thread owns four consecutive elements of one
// (row, head); consecutive threads walk the value dimension, then the rows of
// one head, so the reads of o_part[h][s][rows][D_v] are contiguous.  All
// loads of a row are independent of each other and of the count, so they are
// in flight together.
#include <float.h>

#include "sk_common.hpp"

namespace sk {

__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

__device__ __forceinline__ void store4(__bf16* p, float4 v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 r;
    r[0] = (__bf16)v.x;  // round to nearest even
    r[1] = (__bf16)v.y;
    r[2] = (__bf16)v.z;
    r[3] = (__bf16)v.w;
    *reinterpret_cast<bf16x4*>(p) = r;
}

// Splits held in registers at once; rows with more splits take a second
// pass over their LSEs first.
constexpr int kRegSplits = 8;

template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int b = blockIdx.y;
    const Seq s = load_seq(a.seqs, b);
    // blockIdx.x = head * row_blocks + row_block; a block covers
    // rows_per_block consecutive rows of one head, parts threads per row.
    const int parts = a.dv >> 2;
    const int rows_per_block = blockDim.x / parts;
    const int row_blocks = (a.seqs.max_sq + rows_per_block - 1) / rows_per_block;
    const int h = blockIdx.x / row_blocks;
    const int rloc = threadIdx.x / parts;
    const int part = threadIdx.x - rloc * parts;
    const int r = (blockIdx.x - h * row_blocks) * rows_per_block + rloc;
    if (rloc >= rows_per_block || r >= s.sq) return;
    const int64_t row = s.row0 + r;
    if (row >= a.rows) return;

    // Every slot s < S_b was written by the partial kernel, so these loads
    // are issued together, before the count is known; splits s >= count are
    // then left out of the merge.
    const int S_b = s.splits;
    const int64_t split_stride = a.rows;  // lse_part[h][s][row]
    const float* L = a.lse_part + (int64_t)h * a.seqs.s_max * a.rows + row;
    const float* O = a.o_part + ((int64_t)h * a.seqs.s_max * a.rows + row) * a.dv + part * 4;
    int c = a.counts ? a.counts[row] : valid_split_count(s, a.seqs.mask, a.seqs.n_per_block, r);

    float Ls[kRegSplits];
    float4 Os[kRegSplits];
#pragma unroll
    for (int i = 0; i < kRegSplits; ++i) {
        if (i < S_b) {
            Ls[i] = L[i * split_stride];
            Os[i] = *reinterpret_cast<const float4*>(O + i * split_stride * a.dv);
        }
    }
    c = min(max(c, 0), S_b);  // never read a split the partial kernel did not write

    // m = max(max_s L_s, lowest finite)
    float m = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < kRegSplits; ++i)
        if (i < c) m = fmaxf(m, Ls[i]);
    for (int i = kRegSplits; i < c; ++i) m = fmaxf(m, L[i * split_stride]);

    // w_s = exp(L_s - m); O = sum w_s O_s / max(sum w_s, 1).  Empty splits
    // (L_s = -inf) have w_s = 0 and O_s = 0.
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < kRegSplits; ++i) {
        if (i < c) {
            const float w = expf(Ls[i] - m);
            den += w;
            acc.x = fmaf(w, Os[i].x, acc.x);
            acc.y = fmaf(w, Os[i].y, acc.y);
            acc.z = fmaf(w, Os[i].z, acc.z);
            acc.w = fmaf(w, Os[i].w, acc.w);
        }
    }
    for (int i = kRegSplits; i < c; ++i) {
        const float w = expf(L[i * split_stride] - m);
        den += w;
        if (w > 0.f) {
            const float4 o = *reinterpret_cast<const float4*>(O + i * split_stride * a.dv);
            acc.x = fmaf(w, o.x, acc.x);
            acc.y = fmaf(w, o.y, acc.y);
            acc.z = fmaf(w, o.z, acc.z);
            acc.w = fmaf(w, o.w, acc.w);
        }
    }
    const float inv = 1.0f / fmaxf(den, 1.0f);
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;

    const int64_t obase = (a.seqs.cu_q ? row * a.o_row : (int64_t)b * a.o_batch + (int64_t)r * a.o_row) +
                          (int64_t)h * a.o_head + part * 4;
    store4(reinterpret_cast<OutT*>(a.out) + obase, acc);
    if (a.lse_out && part == 0) a.lse_out[(int64_t)h * a.rows + row] = (den > 0.f) ? m + logf(den) : -INFINITY;
}

hipError_t launch_combine(const CombineArgs& a, int batch, int out_dtype, hipStream_t stream) {
    const int parts = a.dv / 4;
    const int threads = parts <= 256 ? (256 / parts) * parts : parts;
    const int rows_per_block = threads / parts;
    const int row_blocks = (a.seqs.max_sq + rows_per_block - 1) / rows_per_block;
    const dim3 grid((unsigned)(row_blocks * a.heads), batch);
    if (out_dtype == SK_BF16)
        hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sk
