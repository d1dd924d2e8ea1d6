// libsplitkv C ABI: argument checking and kernel dispatch.  Every check runs
// on the host before anything is enqueued; the library never allocates,
// frees or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "sk_common.hpp"
#include "splitkv.h"

namespace {

thread_local std::string g_last_error;

constexpr int kMaxSplits = 128;
constexpr int kMaxHeadDim = 256;

sk_status fail(sk_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sk_status fail(sk_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sk_status ok() {
    g_last_error.clear();
    return SK_OK;
}

int64_t rows_of(const sk_problem& p) {
    return p.cu_seqlens_q ? (int64_t)p.total_q : (int64_t)p.batch * p.max_seqlen_q;
}

int elem_bytes(int dtype) { return dtype == SK_F32 ? 4 : 2; }

bool known_dtype(int dtype) { return dtype == SK_F32 || dtype == SK_BF16 || dtype == SK_F16; }

const char* dtype_name(int dtype) { return dtype == SK_BF16 ? "bf16" : dtype == SK_F16 ? "f16" : "f32"; }

// Checks every scalar field.  Pointer checks depend on the entry point.
sk_status check_problem(const sk_problem* p) {
    if (!p) return fail(SK_ERR_INVALID_ARG, "problem is NULL");
    if (p->batch < 0) return fail(SK_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", p->batch);
    // counts (and the packed combine) take one grid row per sequence
    if (p->batch > 65535) return fail(SK_ERR_UNSUPPORTED, "batch above 65535 is not supported (got %d)", p->batch);
    if (p->num_heads < 1) return fail(SK_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", p->num_heads);
    if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0)
        return fail(SK_ERR_INVALID_ARG, "max_seqlen_q/k must be >= 0 (got %d, %d)", p->max_seqlen_q, p->max_seqlen_k);
    if (p->cu_seqlens_q && p->total_q < 0) return fail(SK_ERR_INVALID_ARG, "total_q must be >= 0 (got %d)", p->total_q);
    if (p->head_dim_qk < 1 || p->head_dim_v < 1)
        return fail(SK_ERR_INVALID_ARG, "head dims must be >= 1 (got %d, %d)", p->head_dim_qk, p->head_dim_v);
    if (p->head_dim_qk > kMaxHeadDim || p->head_dim_v > kMaxHeadDim)
        return fail(SK_ERR_UNSUPPORTED, "head dims above %d are not supported (got %d, %d)", kMaxHeadDim,
                    p->head_dim_qk, p->head_dim_v);
    if (p->split_kv < 0) return fail(SK_ERR_INVALID_ARG, "split_kv must be >= 0 (got %d)", p->split_kv);
    if (p->split_kv == 0 && p->split_kv_per_seq)
        return fail(SK_ERR_INVALID_ARG, "split_kv_per_seq needs an explicit split_kv (got 0 = automatic)");
    if (p->split_kv > kMaxSplits)
        return fail(SK_ERR_UNSUPPORTED, "split_kv above %d is not supported (got %d)", kMaxSplits, p->split_kv);
    if (p->n_per_block < 1) return fail(SK_ERR_INVALID_ARG, "n_per_block must be >= 1 (got %d)", p->n_per_block);
    if (p->mask != SK_MASK_NONE && p->mask != SK_MASK_CAUSAL && p->mask != SK_MASK_PREFIX_CAUSAL)
        return fail(SK_ERR_INVALID_ARG, "unknown mask mode %d", p->mask);
    if (!known_dtype(p->dtype)) return fail(SK_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
    if (!known_dtype(p->out_dtype))
        return fail(SK_ERR_INVALID_ARG, "unknown out_dtype %d", p->out_dtype);
    if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f))
        return fail(SK_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
    if (p->reserved0 != 0) return fail(SK_ERR_INVALID_ARG, "reserved0 must be 0");
    if (p->partial_scratch_bytes < 0) return fail(SK_ERR_INVALID_ARG, "partial_scratch_bytes must be >= 0");
    if (p->window_left < -1) return fail(SK_ERR_INVALID_ARG, "window_left must be >= 0, or -1 for none");
    const int64_t strides[] = {p->q_stride_row, p->q_stride_head, p->q_stride_batch, p->k_stride_row,
                               p->k_stride_head, p->k_stride_batch, p->v_stride_row, p->v_stride_head,
                               p->v_stride_batch, p->o_stride_row, p->o_stride_head, p->o_stride_batch};
    for (int64_t s : strides)
        if (s < 0) return fail(SK_ERR_INVALID_ARG, "strides must be >= 0");
    if ((int64_t)p->max_seqlen_q * p->num_heads > (int64_t)1 << 40 || rows_of(*p) > (int64_t)1 << 31)
        return fail(SK_ERR_UNSUPPORTED, "problem too large");
    return SK_OK;
}

sk::SeqTable seq_table(const sk_problem& p) {
    sk::SeqTable t;
    t.cu_q = p.cu_seqlens_q;
    t.cu_k = p.cu_seqlens_k;
    t.splits = p.split_kv_per_seq;
    t.offsets = p.prefix_offset_per_seq;
    t.last_valid = p.last_valid_per_seq;
    t.max_sq = p.max_seqlen_q;
    t.max_sk = p.max_seqlen_k;
    t.s_max = p.split_kv;
    t.mask = p.mask;
    t.n_per_block = p.n_per_block;
    t.pad_ = 0;
    t.prefix_offset = p.prefix_offset;
    t.last_valid_kv_index = p.last_valid_kv_index;
    t.window_left = p.window_left;
    return t;
}

bool aligned(const void* ptr, size_t bytes) { return ((uintptr_t)ptr % bytes) == 0; }

int cu_count();
int32_t auto_split_kv(const sk_problem& p);

// Work items (query blocks x heads x splits x sequences) of the partial
// grid at query blocks of m_per_block rows.
int64_t partial_work_items(const sk_problem& p, int64_t m_per_block) {
    return (p.max_seqlen_q + m_per_block - 1) / m_per_block * p.num_heads * p.split_kv * (int64_t)p.batch;
}

// Query blocks of m_per_block rows that hold rows: batch x blocks of the
// longest sequence, and for a packed batch at most ceil(total_q / block) +
// B - 1 (the host knows only these sizes; the lengths live on the device).
int64_t query_blocks(const sk_problem& p, int64_t m_per_block) {
    int64_t t = (int64_t)p.batch * ((p.max_seqlen_q + m_per_block - 1) / m_per_block);
    if (p.cu_seqlens_q) t = std::min(t, ((int64_t)p.total_q + m_per_block - 1) / m_per_block + p.batch - 1);
    return t;
}

// The partial kernel of a problem: a function of the problem (its split
// count resolved) and the device's CU count, so every entry point that
// depends on the query block (partial, combine, scratch size, the block
// size query) sees the same one.
sk::PartialKernel pick_partial(const sk_problem& p_in) {
    sk_problem p = p_in;
    if (p.split_kv == 0) p.split_kv = auto_split_kv(p_in);
    // Decode (every sequence at most one query row): the streaming kernel
    // where it exists for the head dims.
    if (p.max_seqlen_q == 1) {
        const sk::PartialKernel d = sk::find_partial_decode(p.dtype, p.head_dim_qk, p.head_dim_v);
        if (d.launch) return d;
    }
    if (p.dtype == SK_BF16 || p.dtype == SK_F16) {
        // 256-row workgroups (one per CU, every tile loaded once for twice
        // the rows) once there is at least one such item per CU; below that
        // the 128-row kernel spreads the work over twice as many workgroups.
        // Without a device (CU count unknown) the 128-row kernel.
        const int cus = cu_count();
        const bool two = cus > 0 && query_blocks(p, 256) * p.num_heads * p.split_kv >= cus;
        return p.dtype == SK_BF16 ? sk::find_partial_bf16(p.head_dim_qk, p.head_dim_v, two)
                                  : sk::find_partial_f16(p.head_dim_qk, p.head_dim_v, two);
    }
    return sk::find_partial_f32(p.head_dim_qk, p.head_dim_v);
}

// Compute units of the current device (0 if unknown), cached per device.
int cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) return 0;
    if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of the partial kernel resident on the device at once (0 when
// unknown or when the kernel runs every item whole).
int64_t partial_slots(const sk::PartialKernel& k) {
    if (!k.blocks_per_cu) return 0;
    return (int64_t)k.blocks_per_cu() * cu_count();
}

// Slots of the tail split: the resident workgroups of a kernel that can run
// key pieces, else 0 (every item runs whole, no scratch).
int64_t piece_slots(const sk::PartialKernel& k) { return k.tail_pieces ? partial_slots(k) : 0; }

int64_t piece_scratch_bytes(int64_t items, int64_t m_per_block, int64_t dv) {
    return items * m_per_block * (dv + 1) * (int64_t)sizeof(float);
}

// Tail split: the last round of a launch holds n_work mod slots items (all
// of them when n_work < slots).  Each is cut into as many key pieces as keep
// every slot busy, with at least kMinPieceTiles key tiles of 64 per piece
// (by the longest sequence's split) and at most sk::kMaxPieces.
struct TailPlan {
    uint32_t n_main;
    int pieces;
};
TailPlan plan_tail(const sk_problem& p, const sk::PartialKernel& k, int64_t n_work, const void* scratch,
                   int64_t scratch_bytes) {
    constexpr int64_t kMinPieceTiles = 8;
    TailPlan none{(uint32_t)n_work, 1};
    const int64_t slots = piece_slots(k);
    if (slots <= 0 || !scratch) return none;
    const int64_t tail = n_work % slots;
    if (tail == 0) return none;
    const int64_t split_keys = ((int64_t)p.max_seqlen_k + p.split_kv - 1) / p.split_kv;
    const int64_t tiles = (split_keys + 63) / 64;
    const int64_t pieces = std::min({slots / tail, tiles / kMinPieceTiles, (int64_t)sk::kMaxPieces});
    if (pieces < 2) return none;
    if (piece_scratch_bytes(tail * pieces, k.m_per_block, p.head_dim_v) > scratch_bytes) return none;
    return TailPlan{(uint32_t)(n_work - tail), (int)pieces};
}

// Automatic split count for split_kv = 0 (documented with sk_split_kv).
int32_t auto_split_kv(const sk_problem& p) {
    constexpr int64_t kMinKeys = 8192;
    constexpr int64_t kMaxAutoSplits = 8;
    if (p.max_seqlen_k < kMinKeys) return 1;
    sk_problem q = p;
    q.split_kv = 1;
    const sk::PartialKernel k = pick_partial(q);
    if (!k.launch || p.dtype == SK_F32) return 1;
    // 16-bit MFMA kernels: the fewest splits that give the 256-row kernel
    // one item per CU (the last round's remainder runs as key pieces), at
    // most 8.
    if (k.m_per_block > 1) {
        const int64_t cus = cu_count();
        if (cus <= 0) return 1;
        const int64_t per_split = query_blocks(p, 256) * p.num_heads;
        for (int64_t s = 1; s < kMaxAutoSplits; ++s)
            if (per_split * s >= cus) return (int32_t)s;
        return (int32_t)kMaxAutoSplits;
    }
    // The decode kernel: about one item per resident workgroup.
    const int64_t slots = partial_slots(k);
    const int64_t items = query_blocks(p, k.m_per_block) * p.num_heads;
    if (slots <= 0 || items <= 0 || items > slots) return 1;
    return (int32_t)std::clamp((slots + items / 2) / items, (int64_t)2, kMaxAutoSplits);
}

// The problem with split_kv resolved (split_kv = 0 -> the automatic count).
sk_problem resolved(const sk_problem& p) {
    sk_problem r = p;
    if (r.split_kv == 0) r.split_kv = auto_split_kv(p);
    return r;
}

// Split count of the backward's dQ pass.  dQ is a plain sum over key
// splits, so the count is free: one workgroup per CU runs a 128-row block's
// split, and S is chosen in 1..8 (at most one split per 512 keys) to
// minimise the rounds of workgroups per unit of work, ceil(items S / CUs) / S
// with items = query blocks x heads (smallest S on ties).  Without a device
// (CU count unknown) it is the problem's split count.
constexpr int kBwdQBlock = 128;
int32_t backward_dq_splits(const sk_problem& p) {
    const int64_t slots = cu_count();
    if (slots <= 0) return p.split_kv;
    int64_t blocks = (int64_t)p.batch * ((p.max_seqlen_q + kBwdQBlock - 1) / kBwdQBlock);
    if (p.cu_seqlens_q)
        blocks = std::min(blocks, ((int64_t)p.total_q + kBwdQBlock - 1) / kBwdQBlock + p.batch - 1);
    const int64_t items = std::max<int64_t>(blocks, 1) * p.num_heads;
    const int64_t max_s = std::clamp<int64_t>(p.max_seqlen_k / 512, 1, 8);
    int32_t best = 1;
    int64_t best_num = (items + slots - 1) / slots, best_den = 1;  // cost = num / den
    for (int64_t s = 2; s <= max_s; ++s) {
        const int64_t num = (items * s + slots - 1) / slots;
        if (num * best_den < best_num * s) {
            best = (int32_t)s;
            best_num = num;
            best_den = s;
        }
    }
    return best;
}

// Workspace of the backward: D [H][rows] f32, then the per-split dQ sums
// [H][S_dq][rows][D_qk] f32, each 256-byte aligned.
struct BackwardLayout {
    int64_t dvec_offset, dq_part_offset, total;
    int32_t dq_splits;
};
BackwardLayout backward_layout(const sk_problem& p) {
    auto round_up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t rows = rows_of(p);
    BackwardLayout w;
    w.dq_splits = backward_dq_splits(p);
    w.dvec_offset = 0;
    w.dq_part_offset = round_up((int64_t)p.num_heads * rows * (int64_t)sizeof(float));
    w.total = w.dq_part_offset +
              round_up((int64_t)p.num_heads * w.dq_splits * rows * p.head_dim_qk * (int64_t)sizeof(float));
    return w;
}

sk_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int32_t sk_abi_version(void) { return SK_ABI_VERSION; }

const char* sk_last_error(void) { return g_last_error.c_str(); }

const char* sk_status_string(sk_status status) {
    switch (status) {
        case SK_OK: return "SK_OK";
        case SK_ERR_INVALID_ARG: return "SK_ERR_INVALID_ARG";
        case SK_ERR_UNSUPPORTED: return "SK_ERR_UNSUPPORTED";
        case SK_ERR_HIP: return "SK_ERR_HIP";
    }
    return "SK_UNKNOWN_STATUS";
}

int64_t sk_rows(const sk_problem* p) {
    if (check_problem(p) != SK_OK) return -1;
    return rows_of(*p);
}

sk_status sk_workspace_bytes(const sk_problem* p, size_t* o_part_bytes, size_t* lse_part_bytes) {
    sk_status st = check_problem(p);
    if (st != SK_OK) return st;
    const sk_problem rp = resolved(*p);
    p = &rp;
    const size_t slots = (size_t)p->num_heads * p->split_kv * (size_t)rows_of(*p);
    if (o_part_bytes) *o_part_bytes = slots * p->head_dim_v * sizeof(float);
    if (lse_part_bytes) *lse_part_bytes = slots * sizeof(float);
    return ok();
}

int32_t sk_split_kv(const sk_problem* p) {
    if (check_problem(p) != SK_OK) return -1;
    ok();
    return resolved(*p).split_kv;
}

int64_t sk_partial_scratch_bytes(const sk_problem* p) {
    if (check_problem(p) != SK_OK) return -1;
    const sk::PartialKernel k = pick_partial(*p);
    const int64_t slots = k.launch ? piece_slots(k) : 0;
    ok();
    return slots > 0 ? piece_scratch_bytes(slots, k.m_per_block, p->head_dim_v) : 0;
}

int32_t sk_partial_m_per_block(const sk_problem* p) {
    if (check_problem(p) != SK_OK) return -1;
    const sk::PartialKernel k = pick_partial(*p);
    if (!k.launch) {
        fail(SK_ERR_UNSUPPORTED, "no partial kernel for dtype %d, head dims (%d, %d)", p->dtype, p->head_dim_qk,
             p->head_dim_v);
        return -1;
    }
    ok();
    return k.m_per_block;
}

sk_status sk_valid_split_counts(const sk_problem* p, int32_t* counts, void* stream) {
    sk_status st = check_problem(p);
    if (st != SK_OK) return st;
    const sk_problem rp = resolved(*p);
    p = &rp;
    if (p->batch == 0 || p->max_seqlen_q == 0 || rows_of(*p) == 0) return ok();
    if (!counts) return fail(SK_ERR_INVALID_ARG, "counts is NULL");
    sk::CountsArgs a;
    a.counts = counts;
    a.seqs = seq_table(*p);
    a.rows = rows_of(*p);
    const hipError_t ce = sk::check_record(&a.check);
    if (ce != hipSuccess) return hip_status(ce, "bounds-check record lookup");
    return hip_status(sk::launch_counts(a, p->batch, (hipStream_t)stream), "counts kernel launch");
}

// sk_attn_partial with the load-balance scratch given explicitly (NULL: every
// item runs whole).  `noalloc`: the scratch is the library's own, and a
// problem whose worst-case piece scratch exceeds it is rejected.
static sk_status partial_impl(const sk_problem* p, const void* q, const void* k, const void* v, float* o_part,
                              float* lse_part, void* stream, bool noalloc) {
    sk_status st = check_problem(p);
    if (st != SK_OK) return st;
    const sk_problem rp = resolved(*p);
    p = &rp;
    const sk::PartialKernel kern = pick_partial(*p);
    if (!kern.launch)
        return fail(SK_ERR_UNSUPPORTED, "no partial kernel for dtype %s with head dims (%d, %d)",
                    dtype_name(p->dtype), p->head_dim_qk, p->head_dim_v);
    const int64_t rows = rows_of(*p);
    if (p->batch == 0 || p->max_seqlen_q == 0 || rows == 0) return ok();
    if (!q || !k || !v || !o_part || !lse_part) return fail(SK_ERR_INVALID_ARG, "a tensor pointer is NULL");
    // Vector loads: 16-byte rows of Q/K/V, 16-byte rows of o_part.
    const int vec = 16 / elem_bytes(p->dtype);
    const int64_t qkv_strides[] = {p->q_stride_row, p->q_stride_head, p->q_stride_batch,
                                   p->k_stride_row, p->k_stride_head, p->k_stride_batch,
                                   p->v_stride_row, p->v_stride_head, p->v_stride_batch};
    for (int64_t s : qkv_strides)
        if (s % vec) return fail(SK_ERR_UNSUPPORTED, "Q/K/V strides must be multiples of %d elements", vec);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_part, 16) || !aligned(lse_part, 4))
        return fail(SK_ERR_UNSUPPORTED, "Q/K/V/o_part must be 16-byte aligned");
    // Key tiles are addressed with 32-bit byte offsets from the tile's first key.
    if (p->k_stride_row > ((int64_t)1 << 24) || p->v_stride_row > ((int64_t)1 << 24))
        return fail(SK_ERR_UNSUPPORTED, "K/V row strides above 2^24 elements are not supported");

    const int64_t n_tiles = (p->max_seqlen_q + kern.m_per_block - 1) / kern.m_per_block;
    const int64_t n_work = partial_work_items(*p, kern.m_per_block);
    if (n_work >= ((int64_t)1 << 31)) return fail(SK_ERR_UNSUPPORTED, "too many work items");

    sk::PartialArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.seqs = seq_table(*p);
    a.q_row = p->q_stride_row;
    a.q_head = p->q_stride_head;
    a.q_batch = p->q_stride_batch;
    a.k_row = p->k_stride_row;
    a.k_head = p->k_stride_head;
    a.k_batch = p->k_stride_batch;
    a.v_row = p->v_stride_row;
    a.v_head = p->v_stride_head;
    a.v_batch = p->v_stride_batch;
    a.rows = rows;
    a.heads = p->num_heads;
    a.n_tiles = (int32_t)n_tiles;
    a.n_work = (uint32_t)n_work;
    a.scale = p->softmax_scale;
    a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
    void* scratch = p->partial_scratch;
    int64_t scratch_bytes = p->partial_scratch_bytes;
    if (noalloc) {
        const int64_t slots = piece_slots(kern);
        const int64_t need = slots > 0 ? piece_scratch_bytes(slots, kern.m_per_block, p->head_dim_v) : 0;
        if (need > sk::kStaticScratchBytes)
            return fail(SK_ERR_UNSUPPORTED,
                        "sk_attn_partial_noalloc: this problem's load balance needs %lld bytes of scratch, above "
                        "the library's %lld",
                        (long long)need, (long long)sk::kStaticScratchBytes);
        scratch = nullptr;
        scratch_bytes = 0;
        if (need > 0) {
            const hipError_t e = sk::static_scratch(&scratch);
            if (e != hipSuccess) return hip_status(e, "static scratch lookup");
            scratch_bytes = sk::kStaticScratchBytes;
        }
    } else if (scratch && !aligned(scratch, 16)) {
        return fail(SK_ERR_INVALID_ARG, "partial_scratch must be 16-byte aligned");
    }
    const TailPlan plan = plan_tail(*p, kern, n_work, scratch, scratch_bytes);
    a.n_main = plan.n_main;
    a.pieces = plan.pieces;
    a.piece_o = nullptr;
    a.piece_l = nullptr;
    if (plan.pieces > 1) {
        const int64_t piece_rows = (n_work - plan.n_main) * (int64_t)plan.pieces * kern.m_per_block;
        a.piece_o = static_cast<float*>(scratch);
        a.piece_l = a.piece_o + piece_rows * p->head_dim_v;
    }
    a.batch = p->batch;
    a.pad_ = 0;
    const hipError_t ce = sk::check_record(&a.check);
    if (ce != hipSuccess) return hip_status(ce, "bounds-check record lookup");
    return hip_status(kern.launch(a, (hipStream_t)stream), "partial kernel launch");
}

sk_status sk_attn_partial(const sk_problem* p, const void* q, const void* k, const void* v, float* o_part,
                          float* lse_part, void* stream) {
    return partial_impl(p, q, k, v, o_part, lse_part, stream, false);
}

sk_status sk_attn_partial_noalloc(const sk_problem* p, const void* q, const void* k, const void* v, float* o_part,
                                  float* lse_part, void* stream) {
    return partial_impl(p, q, k, v, o_part, lse_part, stream, true);
}

sk_status sk_attn_combine(const sk_problem* p, const float* o_part, const float* lse_part, const int32_t* counts,
                          void* out, float* lse_out, void* stream) {
    sk_status st = check_problem(p);
    if (st != SK_OK) return st;
    const sk_problem rp = resolved(*p);
    p = &rp;
    const int64_t rows = rows_of(*p);
    if (p->batch == 0 || p->max_seqlen_q == 0 || rows == 0) return ok();
    if (!o_part || !lse_part || !out) return fail(SK_ERR_INVALID_ARG, "o_part, lse_part and out must not be NULL");
    if (p->head_dim_v % 4) return fail(SK_ERR_UNSUPPORTED, "head_dim_v must be a multiple of 4");
    const int64_t ostr[] = {p->o_stride_row, p->o_stride_head, p->o_stride_batch};
    for (int64_t s : ostr)
        if (s % 4) return fail(SK_ERR_UNSUPPORTED, "out strides must be multiples of 4 elements");
    if (!aligned(out, 4 * elem_bytes(p->out_dtype)) || !aligned(o_part, 16))
        return fail(SK_ERR_UNSUPPORTED, "out / o_part are not aligned for 4-element vectors");
    if (sk::combine_row_blocks(p->batch, p->max_seqlen_q, p->head_dim_v, p->cu_seqlens_q != nullptr) *
            p->num_heads >= ((int64_t)1 << 31))
        return fail(SK_ERR_UNSUPPORTED, "problem too large for the combine grid");
    sk::CombineArgs a;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.counts = counts;
    a.out = out;
    a.lse_out = lse_out;
    a.seqs = seq_table(*p);
    a.o_row = p->o_stride_row;
    a.o_head = p->o_stride_head;
    a.o_batch = p->o_stride_batch;
    a.rows = rows;
    a.heads = p->num_heads;
    a.dv = p->head_dim_v;
    a.batch = p->batch;
    a.row_blocks = 0;
    a.m_per_block = pick_partial(*p).m_per_block;  // 0 when no partial kernel exists for p
    a.pad_ = 0;
    const hipError_t ce = sk::check_record(&a.check);
    if (ce != hipSuccess) return hip_status(ce, "bounds-check record lookup");
    return hip_status(sk::launch_combine(a, p->out_dtype, (hipStream_t)stream), "combine kernel launch");
}

int64_t sk_check_violations(int64_t* first_site, int64_t* first_index, int64_t* first_limit) {
    sk::CheckRecord* rec = nullptr;
    const hipError_t e = sk::check_record(&rec);
    if (e != hipSuccess) {
        fail(SK_ERR_HIP, "locating the bounds-check record failed: %s", hipGetErrorString(e));
        return -1;
    }
    if (!rec) {
        fail(SK_ERR_UNSUPPORTED, "not a bounds-checked build (compiled without SK_CHECKED)");
        return -1;
    }
    sk::CheckRecord h{};
    if (hipMemcpy(&h, rec, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) {
        fail(SK_ERR_HIP, "reading the bounds-check record failed");
        return -1;
    }
    const sk::CheckRecord zero{};
    if (hipMemcpy(rec, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
        fail(SK_ERR_HIP, "resetting the bounds-check record failed");
        return -1;
    }
    if (first_site) *first_site = h.count ? (int64_t)h.site : 0;
    if (first_index) *first_index = h.count ? (int64_t)h.index : 0;
    if (first_limit) *first_limit = h.count ? (int64_t)h.limit : 0;
    ok();
    return (int64_t)h.count;
}

int64_t sk_backward_workspace_bytes(const sk_problem* p) {
    if (check_problem(p) != SK_OK) return -1;
    const sk_problem rp = resolved(*p);
    ok();
    const BackwardLayout w = backward_layout(rp);
    return w.total;
}

sk_status sk_attn_backward(const sk_problem* p, const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                           int64_t workspace_bytes, void* stream) {
    sk_status st = check_problem(p);
    if (st != SK_OK) return st;
    const sk_problem rp = resolved(*p);
    p = &rp;
    if (p->dtype == SK_F32) return fail(SK_ERR_UNSUPPORTED, "the backward needs bf16 or f16 storage (got f32)");
    if (p->out_dtype != p->dtype)
        return fail(SK_ERR_UNSUPPORTED, "the backward needs out_dtype == dtype (got %s, %s)", dtype_name(p->dtype),
                    dtype_name(p->out_dtype));
    const sk::BackwardKernel kern = sk::find_backward(p->dtype, p->head_dim_qk, p->head_dim_v);
    if (!kern.launch)
        return fail(SK_ERR_UNSUPPORTED, "no backward kernel for dtype %s with head dims (%d, %d)", dtype_name(p->dtype),
                    p->head_dim_qk, p->head_dim_v);
    const int64_t rows = rows_of(*p);
    if (p->batch == 0) return ok();
    if (workspace_bytes < 0) return fail(SK_ERR_INVALID_ARG, "workspace_bytes must be >= 0");
    const BackwardLayout w = backward_layout(*p);
    if (w.total > 0 && (!workspace || workspace_bytes < w.total))
        return fail(SK_ERR_INVALID_ARG, "workspace needs %lld bytes (got %lld)", (long long)w.total,
                    (long long)workspace_bytes);
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
        return fail(SK_ERR_INVALID_ARG, "a tensor pointer is NULL");
    // 16-byte vector loads of 16-bit rows; 8-byte stores of the gradients.
    const int64_t strides[] = {p->q_stride_row, p->q_stride_head, p->q_stride_batch, p->k_stride_row,
                               p->k_stride_head, p->k_stride_batch, p->v_stride_row, p->v_stride_head,
                               p->v_stride_batch, p->o_stride_row, p->o_stride_head, p->o_stride_batch};
    for (int64_t s : strides)
        if (s % 8) return fail(SK_ERR_UNSUPPORTED, "strides must be multiples of 8 elements");
    const void* ptrs[] = {q, k, v, out, dout, dq, dk, dv, workspace};
    for (const void* x : ptrs)
        if (x && !aligned(x, 16)) return fail(SK_ERR_UNSUPPORTED, "tensors and workspace must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(SK_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    // Tiles are addressed with 32-bit byte offsets from their first row.
    const int64_t row_strides[] = {p->q_stride_row, p->k_stride_row, p->v_stride_row, p->o_stride_row};
    for (int64_t s : row_strides)
        if (s > ((int64_t)1 << 24)) return fail(SK_ERR_UNSUPPORTED, "row strides above 2^24 elements are not supported");
    if (p->num_heads > 65535) return fail(SK_ERR_UNSUPPORTED, "num_heads above 65535 is not supported by the backward");
    if (kern.q_block != kBwdQBlock) return fail(SK_ERR_HIP, "internal: backward query block mismatch");
    const int64_t n_qtiles = ((int64_t)p->max_seqlen_q + kern.q_block - 1) / kern.q_block;
    const int64_t n_ktiles = ((int64_t)p->max_seqlen_k + kern.k_block - 1) / kern.k_block;
    if (n_qtiles * p->num_heads * w.dq_splits * p->batch >= ((int64_t)1 << 31) ||
        n_ktiles * p->num_heads * p->batch >= ((int64_t)1 << 31) ||
        ((int64_t)p->max_seqlen_q * (p->head_dim_qk / 4) + 255) / 256 > 0x7fffffff)
        return fail(SK_ERR_UNSUPPORTED, "problem too large for the backward grids");
    if ((p->max_seqlen_q == 0 || rows == 0) && p->max_seqlen_k == 0) return ok();

    sk::BackwardArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dvec = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.dvec_offset);
    a.dq_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.dq_part_offset);
    a.seqs = seq_table(*p);
    a.seqs.splits = nullptr;  // the dQ pass's own uniform split count
    a.seqs.s_max = w.dq_splits;
    a.q_row = p->q_stride_row;
    a.q_head = p->q_stride_head;
    a.q_batch = p->q_stride_batch;
    a.k_row = p->k_stride_row;
    a.k_head = p->k_stride_head;
    a.k_batch = p->k_stride_batch;
    a.v_row = p->v_stride_row;
    a.v_head = p->v_stride_head;
    a.v_batch = p->v_stride_batch;
    a.o_row = p->o_stride_row;
    a.o_head = p->o_stride_head;
    a.o_batch = p->o_stride_batch;
    a.rows = rows;
    a.heads = p->num_heads;
    a.n_qtiles = (int32_t)n_qtiles;
    a.n_ktiles = (int32_t)n_ktiles;
    a.batch = p->batch;
    a.scale = p->softmax_scale;
    a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
    const hipError_t ce = sk::check_record(&a.check);
    if (ce != hipSuccess) return hip_status(ce, "bounds-check record lookup");
    return hip_status(kern.launch(a, (hipStream_t)stream), "backward kernel launch");
}

}  // extern "C"
