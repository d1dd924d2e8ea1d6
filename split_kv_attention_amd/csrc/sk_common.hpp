// Internal definitions shared by the libsplitkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv.h"

#ifndef SK_CHECKED
#define SK_CHECKED 0
#endif

namespace sk {

// Bounds-checked build (compiled with -DSK_CHECKED=1, see
// split_kv_attention_amd/build.py): every global index the forward kernels
// derive is checked against the logical extent of the buffer it addresses
// (rows, heads, splits, slots, keys of cu_seqlens_k).  A violation is counted,
// the first one is recorded, and the access is skipped.  In a normal build
// the checks compile away.
struct CheckRecord {
    unsigned int count;  // violations since the last report
    unsigned int site;   // the first violation's check site (CheckSite)
    long long index;     // its index
    long long limit;     // the extent the index had to stay below
};
enum CheckSite : int {
    kSiteWorkItem = 1,     // decoded (tile, head, split, batch) of a work item
    kSiteQRow = 2,         // query row read by a partial kernel
    kSiteKeys = 3,         // last key row of a partial kernel's key range
    kSitePartialSlot = 4,  // o_part / lse_part slot written
    kSitePieceSlot = 5,    // piece scratch slot written or read
    kSiteCountsRow = 6,    // counts entry written
    kSiteCombineRow = 7,   // row merged by the combine (o_part / lse_part / out / lse_out)
    kSiteCombineSplit = 8, // split slot read by the combine
    kSiteBwdItem = 9,      // decoded (sequence, head, split) of a backward workgroup
    kSiteBwdRow = 10,      // query row of the backward (Q, dO, out, LSE, D, dQ)
    kSiteBwdKey = 11,      // key row of the backward (K, V, dK, dV)
    kSiteBwdPart = 12,     // dQ split-sum slot of the workspace
};
__device__ __forceinline__ bool in_bounds(CheckRecord* rec, int site, int64_t i, int64_t limit) {
#if SK_CHECKED
    if (i >= 0 && i < limit) return true;
    if (rec && atomicAdd(&rec->count, 1u) == 0u) {
        rec->site = (unsigned int)site;
        rec->index = i;
        rec->limit = limit;
    }
    return false;
#else
    (void)rec;
    (void)site;
    (void)i;
    (void)limit;
    return true;
#endif
}

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
    int64_t window_left;  // < 0: no sliding window
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

// First key index row q may see: q + off - window_left under a sliding
// window (0 and below: from the first key), else 0.
__device__ __forceinline__ int64_t vis_first(const Seq& s, int64_t window_left, int64_t q) {
    return window_left < 0 ? 0 : max((int64_t)0, q + s.off - window_left);
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

// Most key pieces one tail item of the partial kernel is split into.
constexpr int kMaxPieces = 16;

// The library's own device scratch (static_scratch.hip), which
// sk_attn_partial_noalloc uses for the last round's key pieces: its size,
// and its address on the current device (looked up once per device).
constexpr int64_t kStaticScratchBytes = (int64_t)36 << 20;
hipError_t static_scratch(void** out);
// The bounds-check record on the current device (NULL in a normal build).
hipError_t check_record(CheckRecord** out);
// Number of keys of a packed K/V (cu_seqlens_k[batch]) or of one dense sequence.
__device__ __forceinline__ int64_t total_keys(const SeqTable& t, int batch) {
    return t.cu_k ? (int64_t)t.cu_k[batch] : (int64_t)t.max_sk;
}

// Key range [ks, ke) of split `split` for the query block whose last row is
// last_row: the count formula at that row gives keys per split, split s
// covers [s*kps, (s+1)*kps) of the keys 0..rowLast, and keys past lastValid
// are never visible (rocmlirTriton page, "Per-row valid-split counts", the
// paragraph on conservative counts).  ks >= ke: the split is empty for the
// whole block.
__device__ __forceinline__ void block_split_range(const Seq& sq, int mask, int n_per_block, int last_row, int split,
                                                  int& ks, int& ke) {
    const int64_t rl = row_last(sq, mask, last_row);
    const int64_t kps = keys_per_split(rl, n_per_block, sq.splits);
    const int64_t kend = min(rl + 1, sq.lv + 1);
    ks = (int)min((int64_t)split * kps, kend);
    ke = (int)min((int64_t)(split + 1) * kps, kend);
}

// Splits that hold a key for the query block (of m_per_block rows) that row
// r belongs to: the only ones the partial kernel writes for that block.
__device__ __forceinline__ int block_populated_splits(const Seq& sq, int mask, int n_per_block, int m_per_block,
                                                      int r) {
    const int last_row = min((r / m_per_block + 1) * m_per_block, sq.sq) - 1;
    const int64_t rl = row_last(sq, mask, last_row);
    const int64_t kps = keys_per_split(rl, n_per_block, sq.splits);
    const int64_t kend = min(rl + 1, sq.lv + 1);
    return kend > 0 ? (int)min(ceil_div64(kend, kps), (int64_t)sq.splits) : 0;
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
    // Tail split (load balance of the last round): work items n_main ..
    // n_work - 1 are each run as `pieces` workgroups over consecutive parts
    // of their key range, which write to the scratch arrays
    //   piece_o [n_work - n_main][pieces][m_per_block][D_v]
    //   piece_l [n_work - n_main][pieces][m_per_block]
    // and a merge kernel folds the pieces into o_part / lse_part.  With
    // n_main = n_work (pieces = 1) every item runs whole.
    uint32_t n_main;
    int32_t pieces;    // 2 .. kMaxPieces when n_main < n_work
    float* piece_o;
    float* piece_l;
    int32_t batch;       // sequences
    int32_t pad_;
    CheckRecord* check;  // bounds-checked build only (else NULL)
};

// Decoded work item of a partial kernel.
struct WorkItem {
    int tile, head, split, batch;
};

// Keys of split s of sequence `sq` under the partition of its last query
// block (the block with the most keys under causal masking): used only to
// order work, never to compute.
__device__ __forceinline__ int64_t split_keys(const Seq& sq, int mask, int n_per_block, int s) {
    if (sq.sq <= 0 || s >= sq.splits) return 0;
    const int64_t rl = row_last(sq, mask, sq.sq - 1);
    const int64_t kps = keys_per_split(rl, n_per_block, sq.splits);
    const int64_t kend = min(rl + 1, sq.lv + 1);
    return max((int64_t)0, min((int64_t)(s + 1) * kps, kend) - min((int64_t)s * kps, kend));
}

// Rank r (0 = most keys) of the (sequence, split) pairs -> pair index.  For
// at most 64 pairs every wave ranks them all, one pair per lane (ties keep
// index order); otherwise the order is the identity.
__device__ __forceinline__ uint32_t pair_by_rank(const PartialArgs& a, uint32_t r) {
    const int npairs = (int)(a.n_work / ((uint32_t)a.n_tiles * a.heads));
    if (npairs <= 1 || npairs > 64) return r;
    const int lane = threadIdx.x & 63;
    int64_t cost = -1;
    if (lane < npairs) {
        const Seq sq = load_seq(a.seqs, lane / a.seqs.s_max);
        cost = split_keys(sq, a.seqs.mask, a.seqs.n_per_block, lane % a.seqs.s_max);
    }
    const int cost32 = (int)min(cost, (int64_t)0x7fffffff);
    int rank = 0;
    for (int j = 0; j < npairs; ++j) {
        const int cj = __builtin_amdgcn_readlane(cost32, j);
        rank += (cj > cost32) || (cj == cost32 && j < lane);
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < npairs && rank == (int)r);
    return hit ? (uint32_t)__builtin_ctzll(hit) : r;
}

// Work item b in [0, n_work): groups (pair, head) of n_tiles query tiles each; groups are
// ordered longest pair first.  Workgroups are dealt round-robin over the 8
// XCDs of an MI355X (XCD = blockIdx.x % 8), so block b is mapped to give XCD x
// the groups x, x + 8, x + 16, ... in that order: every XCD gets an equal
// share of long and short groups, runs its longest first, and the tiles of
// one group (which read the same keys and values) share its L2.  Groups past
// the last multiple of 8 are spread tile by tile.  A bijection on [0, n_work).
__device__ __forceinline__ WorkItem decode_work(const PartialArgs& a, uint32_t b) {
    constexpr uint32_t kXcds = 8;
    const uint32_t T = a.n_tiles, G = a.n_work / T;
    uint32_t u = b;
    if (b < (G / kXcds) * kXcds * T) {
        const uint32_t x = b % kXcds, i = b / kXcds;
        u = ((i / T) * kXcds + x) * T + i % T;
    }
    WorkItem it;
    it.tile = u % T;
    u /= T;
    it.head = u % a.heads;
    const uint32_t pair = pair_by_rank(a, u / a.heads);
    it.split = pair % a.seqs.s_max;
    it.batch = pair / a.seqs.s_max;
    return it;
}

// Arguments of the backward kernels.  Gradients use the strides of the
// tensor they belong to (dq: q's, dk: k's, dv: v's); out and dout share o's.
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;  // [H][rows], natural log, from the merge
    void* dq;
    void* dk;
    void* dv;
    float* dvec;     // workspace: D = rowsum(dO * O), [H][rows]
    float* dq_part;  // workspace: per-split dQ sums, [H][S_max][rows][D_qk]
    SeqTable seqs;
    int64_t q_row, q_head, q_batch;
    int64_t k_row, k_head, k_batch;
    int64_t v_row, v_head, v_batch;
    int64_t o_row, o_head, o_batch;
    int64_t rows;
    int32_t heads;
    int32_t n_qtiles;  // query blocks of the dQ kernel in the longest sequence
    int32_t n_ktiles;  // key blocks of the dK/dV kernel in the longest sequence
    int32_t batch;
    float scale;
    float scale_log2;
    CheckRecord* check;  // bounds-checked build only (else NULL)
};

typedef hipError_t (*BackwardLauncher)(const BackwardArgs& a, hipStream_t stream);
struct BackwardKernel {
    BackwardLauncher launch;
    int q_block;  // query rows per dQ block (its split partition)
    int k_block;  // keys per dK/dV block
};
// Backward for (dtype, d_qk, d_v), or {nullptr, 0, 0} when not built.
BackwardKernel find_backward(int dtype, int d_qk, int d_v);

struct CountsArgs {
    int32_t* counts;
    SeqTable seqs;
    int64_t rows;  // length of counts: rows past it (inconsistent cu_seqlens) are not written
    CheckRecord* check;  // bounds-checked build only (else NULL)
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
    int32_t batch;
    int32_t row_blocks;  // blocks per head (set by the launcher)
    int32_t m_per_block; // query block of the partial kernel (0: unknown, no block clamp)
    int32_t pad_;
    CheckRecord* check;  // bounds-checked build only (else NULL)
};

// Launchers (one translation unit each).
hipError_t launch_counts(const CountsArgs& a, int batch, hipStream_t stream);
hipError_t launch_combine(CombineArgs a, int out_dtype, hipStream_t stream);
// Blocks per head of the combine grid (rows_per_block = 256 / (dv / 4)).
int64_t combine_row_blocks(int64_t batch, int64_t max_sq, int dv, bool packed);

typedef hipError_t (*PartialLauncher)(const PartialArgs& a, hipStream_t stream);
struct PartialKernel {
    PartialLauncher launch;
    int m_per_block;
    // Workgroups of the kernel resident per CU (the automatic split count
    // and the tail split), or nullptr when unknown.
    int (*blocks_per_cu)();
    // The kernel can run the last round's items as key pieces (tail split).
    bool tail_pieces;
};
// Kernel for (dtype, d_qk, d_v), or {nullptr, 0, nullptr, false} when not built.
// The 16-bit MFMA kernels come with one group of 4 waves (128 query rows per
// workgroup) or two (256 rows, one workgroup per CU).
PartialKernel find_partial_bf16(int d_qk, int d_v, bool two_groups);
PartialKernel find_partial_f16(int d_qk, int d_v, bool two_groups);
PartialKernel find_partial_f32(int d_qk, int d_v);
// Decode kernel (sequences of at most one query row) for a 16-bit dtype.
PartialKernel find_partial_decode(int dtype, int d_qk, int d_v);

}  // namespace sk
