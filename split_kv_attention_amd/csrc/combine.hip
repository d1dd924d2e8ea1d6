// NaN-safe f32 merge of split partials (rocmlirTriton page "Recombine fully
// masked split-KV attention partials on the host", sections "NaN-safe merge",
// "f32 merge for f16/bf16" and "Per-row mask layout").
//
// HBM-bound: every (row, head) reads its valid partial rows once and writes
// one output row.  One thread owns four consecutive elements of one
// (row, head); consecutive threads walk the value dimension, then the rows of
// one head, so the reads of o_part[h][s][rows][D_v] are contiguous.  The
// loads of a row (up to NSR splits) are independent of each other and of the
// count, so they are in flight together.
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

__device__ __forceinline__ void store4(_Float16* p, float4 v) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 r;
    r[0] = (_Float16)v.x;  // round to nearest even
    r[1] = (_Float16)v.y;
    r[2] = (_Float16)v.z;
    r[3] = (_Float16)v.w;
    *reinterpret_cast<f16x4*>(p) = r;
}

// Buffer loads from a base that is uniform over the block, with a 32-bit
// per-lane byte offset and a range of `bytes` (reads beyond it return 0):
// no 64-bit address per lane and split.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}

// Partials are read once: non-temporal loads (cache policy 2, nt) keep them
// from evicting other data.
__device__ __forceinline__ float4 load_o(const float* base, uint32_t bytes, uint32_t off) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rsrc(base, bytes), off, 0, 2);
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
}

__device__ __forceinline__ float load_l(const float* base, uint32_t bytes, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(base, bytes), off, 0, 0));
}

// Merges n (<= NSR) more splits into the running (m, den, acc): the new
// maximum rescales what was summed before.  For the first chunk m starts at
// the lowest finite value and den = acc = 0, so a row with at most NSR
// splits is exactly m = max(max_s L_s, lowest finite), w_s = exp(L_s - m).
template <int NSR>
__device__ __forceinline__ void merge_chunk(const float (&Ls)[NSR], const float4 (&Os)[NSR], int n, float& m,
                                            float& den, float4& acc) {
    float mc = m;
#pragma unroll
    for (int i = 0; i < NSR; ++i)
        if (i < n) mc = fmaxf(mc, Ls[i]);
    const float f = expf(m - mc);
    den *= f;
    acc.x *= f;
    acc.y *= f;
    acc.z *= f;
    acc.w *= f;
#pragma unroll
    for (int i = 0; i < NSR; ++i) {
        if (i < n) {
            // empty splits (L_s = -inf) get w_s = 0 and hold O_s = 0
            const float w = expf(Ls[i] - mc);
            den += w;
            acc.x = fmaf(w, Os[i].x, acc.x);
            acc.y = fmaf(w, Os[i].y, acc.y);
            acc.z = fmaf(w, Os[i].z, acc.z);
            acc.w = fmaf(w, Os[i].w, acc.w);
        }
    }
    m = mc;
}

// NSR splits are loaded into registers at once (rows with more take further
// chunks).
template <typename OutT, int NSR, bool kPacked>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    // A block covers rows_per_block consecutive rows of one head, parts
    // threads per row.  Blocks are dealt round-robin over the 8 XCDs; the
    // remap gives each XCD one contiguous range of rows, so the partial LSE
    // and output lines a block shares with its neighbours stay in one L2.
    const int parts = a.dv >> 2;
    const int rows_per_block = blockDim.x / parts;
    const int rloc = threadIdx.x / parts;
    const int part = threadIdx.x - rloc * parts;
    if (rloc >= rows_per_block) return;
    constexpr uint32_t kXcds = 8;
    const uint32_t nb = gridDim.x, xcd = blockIdx.x % kXcds;
    const uint32_t bx = xcd * (nb / kXcds) + min(xcd, nb % kXcds) + blockIdx.x / kXcds;
    const int h = bx / a.row_blocks;
    const int64_t blk = (int64_t)(bx - h * a.row_blocks) * rows_per_block;  // first row of the block
    const int64_t rr = blk + rloc;
    // packed: one grid row per sequence; dense: the rows of all sequences
    // are flattened, so that short sequences (decode) fill whole blocks
    int b, r;
    if constexpr (kPacked) {
        b = blockIdx.y;
        r = (int)rr;
    } else {
        if (rr >= (int64_t)a.batch * a.seqs.max_sq) return;
        b = (int)(rr / a.seqs.max_sq);
        r = (int)(rr - (int64_t)b * a.seqs.max_sq);
    }
    if (!in_bounds(a.check, kSiteCombineRow, h, a.heads) || !in_bounds(a.check, kSiteCombineRow, b, a.batch)) return;
    const Seq s = load_seq(a.seqs, b);
    if (r >= s.sq) return;
    const int64_t row = s.row0 + r;
    if (row >= a.rows) return;
    if (!in_bounds(a.check, kSiteCombineSplit, s.splits - 1, a.seqs.s_max)) return;

    // Every slot s < S_b was written by the partial kernel, so the first
    // chunk's loads are issued together, before the count is known; splits
    // s >= count are then left out of the merge.  Addresses are a base that
    // is uniform over the block (row `row_blk`, the block's first row) plus
    // a small per-lane offset.
    const int S_b = s.splits;
    const int64_t row_blk = (kPacked ? s.row0 : 0) + blk;
    const uint32_t lane_l = (uint32_t)rloc * 4;
    const uint32_t lane_o = (uint32_t)(rloc * a.dv + part * 4) * 4;
    const uint32_t l_bytes = rows_per_block * 4, o_bytes = rows_per_block * a.dv * 4;
    const float* L0 = a.lse_part + (int64_t)h * a.seqs.s_max * a.rows + row_blk;  // lse_part[h][s][row]
    const float* O0 = a.o_part + ((int64_t)h * a.seqs.s_max * a.rows + row_blk) * a.dv;
    const int64_t l_split = a.rows, o_split = a.rows * a.dv;

    float Ls[NSR];
    float4 Os[NSR];
#pragma unroll
    for (int i = 0; i < NSR; ++i) {
        if (i < S_b) {
            Ls[i] = load_l(L0 + i * l_split, l_bytes, lane_l);
            Os[i] = load_o(O0 + i * o_split, o_bytes, lane_o);
        }
    }
    int c = a.counts ? a.counts[row] : valid_split_count(s, a.seqs.mask, a.seqs.n_per_block, r);
    c = min(max(c, 0), S_b);
    // Splits past the ones the row's M block populates were not written
    // (they hold no key for the block, so their weight would be 0).  Without
    // a mask every row of a sequence has the same last visible key, so the
    // populated count equals the count, except for a sequence with no key
    // (count 1, nothing populated).  A packed block's rows lie in one M block
    // (rows_per_block divides the M block), so the cap is computed once,
    // from the block's first row.
    if (a.m_per_block > 0) {
        if (a.seqs.mask == SK_MASK_NONE) {
            if (s.lv < 0) c = 0;
        } else {
            c = min(c, block_populated_splits(s, a.seqs.mask, a.seqs.n_per_block, a.m_per_block,
                                              kPacked && a.m_per_block % rows_per_block == 0 ? (int)blk : r));
        }
    }

    // m = max(max_s L_s, lowest finite); w_s = exp(L_s - m);
    // O = sum_s w_s O_s / max(sum_s w_s, 1)
    float m = -FLT_MAX, den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    merge_chunk<NSR>(Ls, Os, min(c, NSR), m, den, acc);
    for (int base = NSR; base < c; base += NSR) {
        const int n = min(c - base, NSR);
#pragma unroll
        for (int i = 0; i < NSR; ++i) {
            if (i < n) {
                Ls[i] = load_l(L0 + (base + i) * l_split, l_bytes, lane_l);
                Os[i] = load_o(O0 + (base + i) * o_split, o_bytes, lane_o);
            }
        }
        merge_chunk<NSR>(Ls, Os, n, m, den, acc);
    }
    const float inv = 1.0f / fmaxf(den, 1.0f);
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;

    const int64_t obase = (kPacked ? row * a.o_row : (int64_t)b * a.o_batch + (int64_t)r * a.o_row) +
                          (int64_t)h * a.o_head + part * 4;
    store4(reinterpret_cast<OutT*>(a.out) + obase, acc);
    if (a.lse_out && part == 0) a.lse_out[(int64_t)h * a.rows + row] = (den > 0.f) ? m + logf(den) : -INFINITY;
}

template <typename OutT, int NSR>
hipError_t launch_nsr(const CombineArgs& a, dim3 grid, int threads, hipStream_t stream) {
    if (a.seqs.cu_q)
        hipLaunchKernelGGL((combine_kernel<OutT, NSR, true>), grid, dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL((combine_kernel<OutT, NSR, false>), grid, dim3(threads), 0, stream, a);
    return hipGetLastError();
}

template <typename OutT>
hipError_t launch_out(const CombineArgs& a, dim3 grid, int threads, hipStream_t stream) {
    const int s = a.seqs.s_max;
    if (s <= 4) return launch_nsr<OutT, 4>(a, grid, threads, stream);
    if (s <= 8) return launch_nsr<OutT, 8>(a, grid, threads, stream);
    if (s <= 16) return launch_nsr<OutT, 16>(a, grid, threads, stream);
    return launch_nsr<OutT, 32>(a, grid, threads, stream);
}

int64_t combine_row_blocks(int64_t batch, int64_t max_sq, int dv, bool packed) {
    const int64_t rows_per_block = 256 / (dv / 4);
    return ((packed ? max_sq : batch * max_sq) + rows_per_block - 1) / rows_per_block;
}

hipError_t launch_combine(CombineArgs a, int out_dtype, hipStream_t stream) {
    const int parts = a.dv / 4;
    const int threads = (256 / parts) * parts;
    const bool packed = a.seqs.cu_q != nullptr;
    a.row_blocks = (int32_t)combine_row_blocks(a.batch, a.seqs.max_sq, a.dv, packed);
    const dim3 grid((unsigned)(a.row_blocks * a.heads), packed ? a.batch : 1);
    if (out_dtype == SK_BF16) return launch_out<__bf16>(a, grid, threads, stream);
    if (out_dtype == SK_F16) return launch_out<_Float16>(a, grid, threads, stream);
    return launch_out<float>(a, grid, threads, stream);
}

}  // namespace sk
