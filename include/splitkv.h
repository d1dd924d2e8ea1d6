/*
 * libsplitkv: split-KV attention forward (and its backward) for AMD Instinct
 * MI355X (gfx950).
 *
 * The key axis of every (sequence, head) is divided into split_kv chunks.
 * sk_attn_partial computes one partial output O_s and one log-sum-exp L_s per
 * chunk; sk_attn_combine merges them into the attention output with the
 * NaN-safe f32 rule; sk_valid_split_counts gives the per-row number of splits
 * the merge reads.  The method is the one described on the page "Recombine
 * fully masked split-KV attention partials on the host" (rocmlirTriton pull
 * request #535); the packed variable-length batch and the num_splits knob
 * follow "[ASM][HIP][JIT][gfx942] Optimize long-context FMHA with split-KV"
 * (aiter pull request #5592).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates, frees and synchronises nothing; it only enqueues
 *     kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream).  Calls are asynchronous and thread-safe, except
 *     sk_attn_partial_noalloc, whose calls on one GPU share the library's
 *     own scratch (see there).
 *   - Arguments are checked on the host before anything is enqueued.  An
 *     invalid argument returns SK_ERR_INVALID_ARG, a valid request this
 *     build does not implement returns SK_ERR_UNSUPPORTED, and a failed
 *     launch returns SK_ERR_HIP; sk_last_error() then holds a message for the
 *     calling thread.  Nothing is written to device memory on error.
 *   - Device arrays named in sk_problem (cu_seqlens, per-sequence values) are
 *     read by the kernels; the host never dereferences them, so their values
 *     cannot be checked before launch.  They must be consistent with the
 *     scalar fields (see each field).
 *
 * Row numbering.  "Rows" are the packed query rows of the whole batch: with
 * cu_seqlens_q the row of (sequence b, query r) is cu_seqlens_q[b] + r; without
 * it (dense batch) it is b * max_seqlen_q + r.  sk_rows() returns their number.
 *
 * Partial buffers (written by sk_attn_partial, read by sk_attn_combine), f32:
 *   o_part   [num_heads][S_max][rows][head_dim_v]
 *   lse_part [num_heads][S_max][rows]
 * with S_max = sk_split_kv(p) (split_kv unless split_kv = 0).
 * i.e. the split axis sits right after the batch-head axis, as in the per-row
 * mask layout of the rocmlirTriton page ("Per-row mask layout").
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SK_ABI_VERSION 6

typedef enum sk_status {
    SK_OK = 0,
    SK_ERR_INVALID_ARG = 1,
    SK_ERR_UNSUPPORTED = 2,
    SK_ERR_HIP = 3
} sk_status;

/* Key visibility of query row q of a sequence with lastValid as below:
 *   NONE           keys 0 .. lastValid
 *   CAUSAL         keys 0 .. min(q, lastValid)                (top-left aligned)
 *   PREFIX_CAUSAL  keys 0 .. min(q + prefix_offset, lastValid)
 * (rocmlirTriton page, "Per-row valid-split counts": prefix_offset is 0 for
 * plain causal).  A row that sees no key is fully masked: output 0, LSE -inf. */
typedef enum sk_mask_mode {
    SK_MASK_NONE = 0,
    SK_MASK_CAUSAL = 1,
    SK_MASK_PREFIX_CAUSAL = 2
} sk_mask_mode;

typedef enum sk_dtype {
    SK_F32 = 0,
    SK_BF16 = 1,
    SK_F16 = 2  /* IEEE half: storage only; scores, softmax and the merge stay f32
                   (rocmlirTriton page, "f32 merge for f16/bf16") */
} sk_dtype;

typedef struct sk_problem {
    int32_t batch;          /* 0 <= B <= 65535: number of sequences */
    int32_t num_heads;      /* H >= 1 (query, key and value heads are equal) */
    int32_t max_seqlen_q;   /* dense: every Sq_b; varlen: >= every Sq_b */
    int32_t max_seqlen_k;   /* dense: every Sk_b; varlen: >= every Sk_b */
    int32_t total_q;        /* varlen (cu_seqlens_q != NULL): rows of Q / out,
                               = cu_seqlens_q[B]; ignored for a dense batch */
    int32_t head_dim_qk;    /* D_qk */
    int32_t head_dim_v;     /* D_v */
    int32_t split_kv;       /* S_max >= 1: splits per (sequence, head); 1 = unsplit
                               (aiter page: num_splits 2..8 force a split);
                               0 = automatic, see sk_split_kv() */
    int32_t n_per_block;    /* split granularity in keys (>= 1): the key tile
                               nPerBlock of the count formula */
    int32_t mask;           /* sk_mask_mode */
    int32_t dtype;          /* sk_dtype of Q, K, V */
    int32_t out_dtype;      /* sk_dtype of out */
    int64_t prefix_offset;  /* PREFIX_CAUSAL only (may be negative) */
    int64_t last_valid_kv_index; /* < 0: Sk_b - 1; otherwise min(value, Sk_b - 1) */
    float softmax_scale;    /* > 0, finite: scores are scale * q.k */
    int32_t reserved0;      /* must be 0 */
    const int32_t* cu_seqlens_q;          /* device [B+1] prefix sums, or NULL = dense */
    const int32_t* cu_seqlens_k;          /* device [B+1] prefix sums, or NULL = dense */
    const int32_t* split_kv_per_seq;      /* device [B], each in 1..split_kv, or NULL
                                             (must be NULL when split_kv = 0) */
    const int32_t* prefix_offset_per_seq; /* device [B] (PREFIX_CAUSAL), or NULL */
    const int32_t* last_valid_per_seq;    /* device [B] (< 0: Sk_b - 1), or NULL */
    /* Element strides.  The head dimension is contiguous (stride 1).  The batch
     * stride of a tensor is used only when its cu_seqlens pointer is NULL. */
    int64_t q_stride_row, q_stride_head, q_stride_batch;
    int64_t k_stride_row, k_stride_head, k_stride_batch;
    int64_t v_stride_row, v_stride_head, v_stride_batch;
    int64_t o_stride_row, o_stride_head, o_stride_batch;
    /* Optional device scratch for sk_attn_partial's load balance (or NULL).
     * When the last round of workgroups would leave CUs idle, the items of
     * that round are run as several workgroups over consecutive parts of
     * their keys, whose results sk_attn_partial merges before it returns
     * (the same log-sum-exp merge as sk_attn_combine).  The outputs then
     * differ from whole items only by where the weights are rounded to bf16
     * (each piece against its own running max).  It needs
     * partial_scratch_bytes >= sk_partial_scratch_bytes(p), 16-byte
     * alignment, and may not be shared by calls that can run at the same
     * time.  NULL (or too small) runs every item whole. */
    void* partial_scratch;
    int64_t partial_scratch_bytes;
    /* Sliding window (>= 0) or -1 for none.  The aiter page's split path
     * takes the caller's window without defining it; here a row q sees only
     * keys k >= q + off - window_left, with off = prefix_offset(_per_seq)
     * under PREFIX_CAUSAL and 0 otherwise (the position the causal rule
     * uses), on top of every other rule.  Counts do not change: the count
     * formula depends only on the last visible key. */
    int64_t window_left;
} sk_problem;

/* ABI version of the library (SK_ABI_VERSION of the header it was built from). */
int32_t sk_abi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* sk_last_error(void);

/* Human-readable name of a status code. */
const char* sk_status_string(sk_status status);

/* Number of packed query rows (see "Row numbering"), or -1 if `p` is invalid. */
int64_t sk_rows(const sk_problem* p);

/* The number of splits S_max every entry point uses for `p` (>= 1), or -1 if
 * `p` is invalid.  It is split_kv, or with split_kv = 0 the automatic choice
 * (aiter page, Technical Details: split only when the keys are long and the
 * query tiles alone do not fill the GPU), re-derived for this device.  With
 *   blocks(m) = query blocks of m rows: batch x blocks of the longest
 *               sequence, or for a packed batch at most ceil(total_q / m) +
 *               B - 1
 * S = 1 if max_seqlen_k < 8192.  Otherwise, for 16-bit storage with an MFMA
 * kernel (max_seqlen_q > 1 or head dims without a decode kernel), S is the
 * smallest count in 1..7 with blocks(256) x heads x S >= the device's CU
 * count (one item of the 256-row kernel per CU), else 8.  For the decode
 * kernel (one-row sequences), with
 *   items = blocks(1) x heads: one item per (sequence, head)
 *   slots = the decode kernel's resident workgroups on the device
 *   S     = clamp(round(slots / items), 2, 8)  if items <= slots, else 1.
 * The key threshold is the explicit 8192 of that page's contract (its review
 * notes a tile-rounded form that also split 8161..8191 keys).  f32 problems
 * and head dims without a 16-bit kernel stay unsplit.  The result depends on
 * the current device's CU count, so buffers must be sized with the same
 * device current. */
int32_t sk_split_kv(const sk_problem* p);

/* Bytes of the partial buffers sk_attn_partial writes and sk_attn_combine
 * reads (layout in the file header).  Either output pointer may be NULL. */
sk_status sk_workspace_bytes(const sk_problem* p, size_t* o_part_bytes, size_t* lse_part_bytes);

/* Bytes of partial_scratch that let sk_attn_partial balance its last round
 * on the current device (0: the kernel selected for `p` never uses it), or
 * -1 if `p` is invalid.  Depends on the device's CU count. */
int64_t sk_partial_scratch_bytes(const sk_problem* p);

/* Query rows per M block of the partial kernel selected for `p` (>= 1), or -1
 * if `p` is invalid or unsupported.  The kernel partitions each block's keys
 * with the count formula evaluated at the block's last row (rocmlirTriton
 * page, the paragraph on conservative counts), so the partials depend on it.
 * 1 for a 16-bit problem with max_seqlen_q = 1 and head dims 64/64 or
 * 128/128 (the decode kernel), 64 for f32.  Other 16-bit problems: 256 when
 * blocks(256) x num_heads x split_kv (resolved; blocks() as in sk_split_kv)
 * reaches the CU count of the current device, one item per CU, else 128 (and
 * 128 when no device is present).  Like the
 * automatic split count, the value depends on the current device, so every
 * call for one problem must see the same device current. */
int32_t sk_partial_m_per_block(const sk_problem* p);

/* Per-row valid-split counts (rocmlirTriton page, "Per-row valid-split
 * counts"):
 *   rowLast      = max(0, vis(q))  with vis(q) the row's last visible key
 *   keysPerSplit = nPerBlock * ceil(ceil((rowLast + 1) / nPerBlock) / S_b)
 *   count        = ceil((rowLast + 1) / keysPerSplit)
 * counts: device int32 [rows], written for every row of every sequence
 * (1 <= count <= S_b).  The count is head-independent. */
sk_status sk_valid_split_counts(const sk_problem* p, int32_t* counts, void* stream);

/* Per-split partial attention (rocmlirTriton page, Summary).  For every
 * sequence b, head h, split s < S_b and row: O_s and L_s (natural-log LSE of
 * the scaled scores) of softmax attention over the keys of split s of the
 * row's M block that the row may see.  Split s of a block covers keys
 * [s*kps, min((s+1)*kps, rowLast_blk + 1)) with kps the keys-per-split of the
 * block's last row.  A split that holds keys for the block but none the row
 * may see writes O_s = 0, L_s = -inf.  A split with no key for the whole
 * block is skipped without writing anything (real early exit, rocmlirTriton
 * page, review note on early exit): its slots keep their old contents, and
 * sk_attn_combine leaves them out of the merge.  So the buffers need no
 * clearing.
 * q, k, v: device, dtype; o_part, lse_part: device f32, layout in the header,
 * at least sk_workspace_bytes() bytes. */
sk_status sk_attn_partial(const sk_problem* p, const void* q, const void* k, const void* v,
                          float* o_part, float* lse_part, void* stream);

/* sk_attn_partial for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels and results as sk_attn_partial, except that the
 * load-balance scratch is the library's own instead of
 * p->partial_scratch (which is ignored): a static device array of 36 MiB
 * (37748736 bytes) that every GPU the library is loaded on holds until the
 * process ends.  It calls no allocator.  A problem whose worst-case piece
 * scratch, sk_partial_scratch_bytes(p), exceeds that size returns
 * SK_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU
 * shares that GPU's array and leaves the last call's contents in it (calls
 * need nothing cleared: each piece is written before it is read), so calls
 * that can overlap on one GPU (other streams, other threads) race and must
 * not be made. */
sk_status sk_attn_partial_noalloc(const sk_problem* p, const void* q, const void* k, const void* v,
                                  float* o_part, float* lse_part, void* stream);

/* NaN-safe f32 merge of the partials (rocmlirTriton page, "NaN-safe merge" and
 * "f32 merge for f16/bf16"), per (row, head) with c = count of the row:
 *   m   = max(max_{s<c} L_s, lowest finite f32)
 *   w_s = exp(L_s - m)
 *   O   = sum_{s<c} w_s O_s / max(sum_{s<c} w_s, 1)      (cast to out_dtype last)
 *   LSE = m + ln(sum_{s<c} w_s), or -inf when the sum is 0
 * Splits s >= c take no part in the merge, and neither do the splits
 * sk_attn_partial skipped: c is first capped at the number of splits that
 * hold a key for the row's M block (the block partition of
 * sk_partial_m_per_block; the skipped ones would have weight 0).  To keep
 * its loads in flight together, the kernel loads the slots of a row's first
 * splits (up to 4, 8, 16 or 32 by S_max) before it knows c, so slots past c
 * may be read; whatever they hold never reaches the result.  counts: device int32 [rows] from
 * sk_valid_split_counts, or NULL to evaluate the same formula inline.
 * out: device out_dtype with the o_stride_* layout, fully overwritten (a fully
 * masked row becomes 0).  lse_out: device f32 [num_heads][rows], or NULL to
 * skip it (the aiter page's return_lse=False). */
sk_status sk_attn_combine(const sk_problem* p, const float* o_part, const float* lse_part,
                          const int32_t* counts, void* out, float* lse_out, void* stream);

/* Backward of the merged attention (aiter page, review overview: the open
 * item on backward coverage for split-KV long-K attention).  The forward's
 * output is plain softmax attention over the keys each row may see, so with
 * P = exp(scale q.k - LSE) on those keys and 0 elsewhere:
 *   D  = rowsum(dO * O)
 *   dS = P * (dO V^T - D)
 *   dQ = softmax_scale dS K,  dK = softmax_scale dS^T Q,  dV = P^T dO
 * The dQ pass cuts each block of 128 query rows' keys into S_dq splits with
 * the count formula at the block's last row and sums the split results in
 * f32; S_dq (1..8) is chosen for the current device to fill whole rounds of
 * workgroups, and only the f32 summation order depends on it.  dK and dV are
 * computed per block of 128 keys over every row that sees one of them.
 * Storage: dtype SK_BF16 or SK_F16 (SK_F32: SK_ERR_UNSUPPORTED), out_dtype
 * must equal dtype; head dims (64, 64), (128, 128) or (192, 128).  P and dS
 * are rounded to the storage type before their products, which accumulate in
 * f32; the gradients are rounded to the storage type last.
 *   q, k, v    the forward's inputs (q_/k_/v_stride_*)
 *   out, dout  the forward's output and its gradient (o_stride_*)
 *   lse        f32 [num_heads][rows], the LSE sk_attn_combine wrote (natural
 *              log, -inf for a row that sees no key)
 *   dq         same layout as q; every row of every sequence is written
 *   dk, dv     same layouts as k and v; every key row of every sequence is
 *              written (keys no row sees get 0); rows of a packed K/V that
 *              belong to no sequence are left untouched
 *   workspace  device memory of at least sk_backward_workspace_bytes(p)
 *              bytes, 16-byte aligned; contents on entry do not matter; it
 *              may not be shared by calls that can run at the same time
 * Every tensor must be 16-byte aligned with strides that are multiples of 8
 * elements, and the row strides of q, k, v and the outputs must not exceed
 * 2^24 elements.  The result does not depend on split_kv beyond f32
 * summation order. */
sk_status sk_attn_backward(const sk_problem* p, const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* Bytes of workspace sk_attn_backward needs for `p` on the current device
 * (f32 D per (head, row) and one f32 dQ sum per (head, S_dq split, row, dim);
 * S_dq depends on the device's CU count), or -1 if `p` is invalid. */
int64_t sk_backward_workspace_bytes(const sk_problem* p);

/* Bounds-check report of a checked build of the library (compiled with
 * SK_CHECKED=1: split_kv_attention_amd.build.build_checked).  Its kernels
 * (counts, partial, piece merge, combine and the four backward kernels) test
 * every global index they derive from the problem and the device-side tables
 * against the logical extent it addresses, and skip the access when it falls
 * outside (a Q row reads as zeros; the other sites end the thread's work or
 * its item).  Sites: 1 work item (batch, head, split), 2 Q row (against
 * total_q), 3 last key row of a partial's key range (against
 * cu_seqlens_k[batch], or max_seqlen_k for dense K/V), 4 o_part / lse_part
 * slot, 5 key-piece scratch slot, 6 counts entry, 7 combine row (head,
 * sequence), 8 combine split slot (against split_kv), 9 backward work item,
 * 10 backward query row, 11 backward key row, 12 backward dQ split-sum
 * slot.  Returns the number of failed tests on the current device since the
 * previous call (each thread counts its own) and resets it; the first one's
 * site, index and limit go to the three pointers (each may be NULL).  It
 * synchronises with the device (blocking copies), so call it after the work
 * it reports on has finished.  A normal build returns -1 with
 * SK_ERR_UNSUPPORTED in sk_last_error; -1 with SK_ERR_HIP if the record
 * cannot be read. */
int64_t sk_check_violations(int64_t* first_site, int64_t* first_index, int64_t* first_limit);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_H */
