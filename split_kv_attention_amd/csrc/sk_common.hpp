// Internal definitions shared by the libsplitkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv.h"

namespace sk {

// Per-sequence data as the kernels see it.  Scalars are copied from
// sk_problem; the pointers are the caller's optional device arrays.
struct SeqTable {
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* splits;
    const int32_t* offsets;
    const int32_t* last_valid;
    int32_t max_sq;
    int32_t max_sk;
    int32_t s_max;
    int32_t mask;
    int32_t n_per_block;
    int32_t pad_;
    int64_t prefix_offset;
    int64_t last_valid_kv_index;
};

// One sequence, resolved.
struct Seq {
    int64_t row0;  // packed row index of query 0 (counts, partials, out, lse)
    int64_t krow0; // packed key row of key 0, or -1 for a dense K/V batch
    int32_t sq;
    int32_t sk;
    int32_t splits; // S_b
    int64_t off;    // prefix offset of the visibility rule (0 unless prefix-causal)
    int64_t lv;     // last valid key index, already clamped to sk - 1 (-1 if sk == 0)
};

__device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ Seq load_seq(const SeqTable& t, int b) {
    Seq s;
    if (t.cu_q) {
        const int32_t a = t.cu_q[b], e = t.cu_q[b + 1];
        s.row0 = a;
        s.sq = min(max(e - a, 0), t.max_sq);
    } else {
        s.row0 = (int64_t)b * t.max_sq;
        s.sq = t.max_sq;
    }
    if (t.cu_k) {
        const int32_t a = t.cu_k[b], e = t.cu_k[b + 1];
        s.krow0 = a;
        s.sk = min(max(e - a, 0), t.max_sk);
    } else {
        s.krow0 = -1;
        s.sk = t.max_sk;
    }
    const int32_t sb = t.splits ? t.splits[b] : t.s_max;
    s.splits = min(max(sb, 1), t.s_max);
    s.off = (t.mask == SK_MASK_PREFIX_CAUSAL) ? (t.offsets ? (int64_t)t.offsets[b] : t.prefix_offset) : 0;
    const int64_t lv = t.last_valid ? (int64_t)t.last_valid[b] : t.last_valid_kv_index;
    s.lv = (lv < 0) ? (int64_t)s.sk - 1 : min(lv, (int64_t)s.sk - 1);
    return s;
}

// Last key index query row q may see (keys 0..vis are visible; vis < 0: none).
// Causal is prefix-causal with offset 0, top-left aligned; every mode stops
// at the last valid key (rocmlirTriton page, "Per-row valid-split counts").
__device__ __forceinline__ int64_t vis_last(const Seq& s, int mask, int64_t q) {
    return (mask == SK_MASK_NONE) ? s.lv : min(q + s.off, s.lv);
}

// rowLast = clamp(q + prefix_offset, 0, lastValid), lower clamp last, so an
// empty key range still gives rowLast = 0 (and a count of 1).
__device__ __forceinline__ int64_t row_last(const Seq& s, int mask, int64_t q) {
    return max((int64_t)0, vis_last(s, mask, q));
}

// keysPerSplit = nPerBlock * ceil(ceil((rowLast + 1) / nPerBlock) / S).
__device__ __forceinline__ int64_t keys_per_split(int64_t rl, int n_per_block, int splits) {
    return (int64_t)n_per_block * ceil_div64(ceil_div64(rl + 1, n_per_block), splits);
}

// count = ceil((rowLast + 1) / keysPerSplit).
__device__ __forceinline__ int32_t valid_split_count(const Seq& s, int mask, int n_per_block, int64_t q) {
    const int64_t rl = row_last(s, mask, q);
    return (int32_t)ceil_div64(rl + 1, keys_per_split(rl, n_per_block, s.splits));
}

// Workgroups are dealt round-robin over the 8 XCDs of an MI355X.  Remap the
// hardware block index so that each XCD receives one contiguous range of work
// items: neighbouring items (the query tiles of one head and split, which read
// the same keys and values) then share that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
    constexpr uint32_t kXcds = 8;
    const uint32_t q = n / kXcds, r = n % kXcds;
    const uint32_t x = bid % kXcds, i = bid / kXcds;
    return x * q + min(x, r) + i;
}

// Arguments of every partial-attention kernel.
struct PartialArgs {
    const void* q;
    const void* k;
    const void* v;
    float* o_part;
    float* lse_part;
    SeqTable seqs;
    int64_t q_row, q_head, q_batch;
    int64_t k_row, k_head, k_batch;
    int64_t v_row, v_head, v_batch;
    int64_t rows;      // packed query rows (o_part / lse_part row count)
    int32_t heads;
    int32_t n_tiles;   // query tiles of the longest sequence
    uint32_t n_work;   // n_tiles * heads * split_kv * batch
    float scale;       // softmax scale
    float scale_log2;  // softmax scale * log2(e)
};

// Decoded work item of a partial kernel.
struct WorkItem {
    int tile, head, split, batch;
};

__device__ __forceinline__ WorkItem decode_work(const PartialArgs& a) {
    uint32_t w = xcd_remap(blockIdx.x, a.n_work);
    WorkItem it;
    it.tile = w % a.n_tiles;
    w /= a.n_tiles;
    it.head = w % a.heads;
    w /= a.heads;
    it.split = w % a.seqs.s_max;
    it.batch = w / a.seqs.s_max;
    return it;
}

struct CountsArgs {
    int32_t* counts;
    SeqTable seqs;
};

struct CombineArgs {
    const float* o_part;
    const float* lse_part;
    const int32_t* counts;
    void* out;
    float* lse_out;
    SeqTable seqs;
    int64_t o_row, o_head, o_batch;
    int64_t rows;
    int32_t heads;
    int32_t dv;
};

// Launchers (one translation unit each).
hipError_t launch_counts(const CountsArgs& a, int batch, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int batch, int out_dtype, hipStream_t stream);

typedef hipError_t (*PartialLauncher)(const PartialArgs& a, hipStream_t stream);
struct PartialKernel {
    PartialLauncher launch;
    int m_per_block;
};
// Kernel for (dtype, d_qk, d_v), or {nullptr, 0} when not built.
PartialKernel find_partial_bf16(int d_qk, int d_v);
PartialKernel find_partial_f32(int d_qk, int d_v);

}  // namespace sk
