// Backward of split-KV attention: dQ, dK, dV of the merged output, for bf16
// or f16 storage with 16-bit MFMA and f32 accumulation.
//
// The aiter page "[ASM][HIP][JIT][gfx942] Optimize long-context FMHA with
// split-KV" leaves backward coverage of split-KV long-K attention open
// (review).  The merged output is plain attention over the visible keys, so
// its gradient is attention's: with P = exp(scale q.k - LSE) over the visible
// keys (LSE: the merged log-sum-exp of the forward),
//     D   = rowsum(dO * O)
//     dS  = P * (dO V^T - D)
//     dQ  = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
// Four kernels:
//  * bwd_rowdot: D per (row, head).
//  * bwd_dq: per (sequence, head, split, block of 128 query rows), the
//    forward's layout (4 waves, 32 query rows each, one query per lane):
//    S^T = K Q^T and dP^T = V dO^T (K, V rows from LDS, Q^T and dO^T in
//    registers), dS^T in registers as the B operand of dQ^T += K^T dS^T (K
//    read transposed from LDS).  The block's keys are cut into S_dq splits by
//    the count formula at its last row (S_dq chosen by the host to fill the
//    GPU), so a long key axis runs as many workgroups; each writes its dQ
//    sum to a workspace.
//  * bwd_dkdv: per (sequence, head, block of 128 keys), the same layout with
//    keys and queries swapped (one key per lane): S = Q K^T and dP = dO V^T
//    (Q, dO rows from LDS, K, V in registers), then dV^T += dO^T P and
//    dK^T += Q^T dS (Q, dO read transposed).  It loops over the 32-row query
//    tiles that can see a key of the block.
//  * bwd_dq_reduce: dQ = sum of the split sums (dQ is linear in the keys, so
//    the split merge of the forward reduces to a plain sum).
#include <float.h>

#include <type_traits>

#include "mfma_common.hpp"
#include "sk_common.hpp"

namespace sk {

namespace {

using namespace mfma;

constexpr int kThreads = 256;  // 4 waves
constexpr int kQB = 128;       // dQ kernel: query rows per workgroup (the split partition's M block)
constexpr int kKT = 64;        // dQ kernel: keys per tile
constexpr int kKB = 128;       // dK/dV kernel: keys per workgroup
constexpr int kQT = 32;        // dK/dV kernel: query rows per tile
constexpr float kLog2e = 1.4426950408889634f;

// log2-domain LSE of a row for P = exp2(s * scale log2 e - lse2); a row with
// no visible key (LSE = -inf) gets +inf, so all its weights are 0.
__device__ __forceinline__ float lse_log2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 r;
    r[0] = (T)a;  // round to nearest even
    r[1] = (T)b;
    r[2] = (T)c;
    r[3] = (T)d;
    *reinterpret_cast<t4*>(p) = r;
}

// Swizzle of the 16-byte chunks of a tile row for tiles read both ways: with
// 64 banks of 4 bytes, a 16-byte row read serves 16 lanes (16 rows, one
// chunk each) per cycle and a transposed 8-byte read 32 lanes (4 rows x 4
// consecutive chunks) per cycle.  Rows of 16 chunks all start in bank 0, so
// the XOR must make 16 consecutive rows distinct and give 4 consecutive rows
// different bits 2..3; rows of 8 or 24 chunks alternate between banks 0 and
// 32, so it must make the 8 even (and the 8 odd) rows of 16 distinct and give
// the two even (two odd) rows of 4 a different bit 2.  Both stay inside the
// row (XOR below 16 for 16 chunks, below 8 for 8 or 24) and repeat every 16
// rows.
template <int CH>
__device__ __forceinline__ int bt_swz(int r, int c) {
    if constexpr (CH % 16 == 0) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Reads of a row-major [rows][D] 16-bit tile in LDS whose 16-byte chunks are
// swizzled with bt_swz<D/8>: (a) the A operand of a 32x32x16 MFMA with the
// tile's rows as M (lane = row col, 8 consecutive D entries from k-step t),
// (b) the A operand with D as M and the rows as K, read transposed with
// ds_read_b64_tr_b16 in the row order the accumulator-to-B-operand mapping
// uses: step u of a 32-row block takes rows 16u + 4 half + 0..3 and
// 16u + 8 + 4 half + 0..3.
template <int D>
struct TileReads {
    static constexpr int CH = D / 8;
    static constexpr int kSpan = (CH % 16 == 0) ? 8 : 4;  // k-steps per repeating swizzle block
    // (a): per-lane bases for the k-steps of one 32-row block at row offset 0
    uint32_t row_addr[kSpan];
    // (b): per-lane bases of the two transposed reads for each 32-column block
    uint32_t tr_addr[D / 32][2];

    __device__ __forceinline__ void init(const uint16_t* tile, int lane) {
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int m = 0; m < kSpan; ++m) row_addr[m] = lds_addr(tile + col * D + bt_swz<CH>(col, 2 * m + half) * 8);
        const int s16 = lane & 15, g2 = (lane >> 4) & 1;
        const int r_a = half * 4 + (s16 >> 2);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            const int q = 4 * c + 2 * g2 + ((s16 & 3) >> 1);
            const int in = (s16 & 1) * 4;
            tr_addr[c][0] = lds_addr(tile + r_a * D + bt_swz<CH>(r_a, q) * 8 + in);
            tr_addr[c][1] = lds_addr(tile + (r_a + 8) * D + bt_swz<CH>(r_a + 8, q) * 8 + in);
        }
    }
};

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, N>{});
}

// acc[rb] += A(rows 32 rb .. 32 rb + 31 of the tile, reads (a)) * b[t] over
// the D / 16 k-steps.  PF k-steps of reads are in flight ahead of the MFMAs
// (one LDS read takes longer than the one or two MFMAs of a step); the reads
// go to a ring of PF + 1 buffers, so a buffer is refilled one step after the
// MFMA that read it.  side(t) runs after step t's MFMAs are issued.
template <typename E, int D, int NRB, int SLOT_OFS, int PF, typename Side>
__device__ __forceinline__ void gemm_rows(const TileReads<D>& tr, f32x16 (&acc)[NRB], const typename E::v8 (&b)[D / 16],
                                          Side&& side) {
    using v8 = typename E::v8;
    constexpr int kSpan = TileReads<D>::kSpan;
    constexpr int kSteps = D / 16;
    constexpr int P = PF < kSteps ? PF : kSteps;
    constexpr int R = P + 1;
    i32x4_t f[R][NRB];
    auto rd = [&](auto t_c) {
        constexpr int t = decltype(t_c)::value;
        static_for<NRB>([&](auto rb_c) {
            constexpr int rb = decltype(rb_c)::value;
            f[t % R][rb] = k_read<SLOT_OFS + (t / kSpan) * kSpan * 32 + rb * 32 * D * 2>(tr.row_addr[t % kSpan]);
        });
    };
    static_for<P>(rd);
    static_for<kSteps>([&](auto t_c) {
        constexpr int t = decltype(t_c)::value;
        // reads issued after step t's so far: steps t + 1 .. min(t + P - 1, kSteps - 1)
        constexpr int later = ((t + P - 1 < kSteps - 1) ? (t + P - 1) : (kSteps - 1)) - t;
        static_assert(later * NRB <= 15, "lgkmcnt range");
        i32x4_t(&x)[NRB] = f[t % R];
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(later * NRB) : "memory");
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) asm volatile("" : "+v"(x[rb]));  // no use above the wait
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[rb] = E::mfma(__builtin_bit_cast(v8, x[rb]), b[t], acc[rb]);
        if constexpr (t + P < kSteps) rd(std::integral_constant<int, t + P>{});
        side(t_c);
    });
}

struct NoSide {
    template <typename T>
    __device__ __forceinline__ void operator()(T) const {}
};

// Transposed reads of one step (16 tile rows at byte offset OFS) for every
// 32-column block c of D into x[2 c], x[2 c + 1].
template <int D, int OFS, int N>
__device__ __forceinline__ void tr_issue(const TileReads<D>& tr, s16x4 (&x)[N]) {
    static_assert(2 * (D / 32) <= N, "read buffer");
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        x[2 * c] = tr_read<OFS>(tr.tr_addr[c][0]);
        x[2 * c + 1] = tr_read<OFS>(tr.tr_addr[c][1]);
    }
}

// out[c] += A^T(x) * b for every 32-column block c of D, once at most LATER
// LDS reads (the ones issued after x's) are outstanding; side(c) runs after
// the MFMA of block c is issued, so that VALU work fills the MFMA pipe's
// time.
template <typename E, int D, int LATER, int N, typename Side>
__device__ __forceinline__ void tr_mfma(s16x4 (&x)[N], f32x16 (&out)[D / 32], const typename E::v8& b, Side&& side) {
    using v8 = typename E::v8;
    constexpr int NB = D / 32;
    static_assert(LATER <= 15, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(LATER) : "memory");
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) asm volatile("" : "+v"(x[i]));  // no use above the wait
    static_for<NB>([&](auto c_c) {
        constexpr int c = decltype(c_c)::value;
        const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(x[2 * c], x[2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        out[c] = E::mfma(a, b, out[c]);
        side(c_c);
    });
}

// Workgroups are dealt round-robin over the 8 XCDs (block b runs on XCD
// b % 8); this renumbering gives each XCD one contiguous range of logical
// blocks, so the blocks that share K/V (dQ: the query tiles of one split) or
// Q/dO (dK/dV: the key blocks of one head) share one L2.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t nb) {
    constexpr uint32_t kXcds = 8;
    const uint32_t x = b % kXcds;
    return x * (nb / kXcds) + min(x, nb % kXcds) + b / kXcds;
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O), one thread per (row, head)
// ---------------------------------------------------------------------------

template <typename T, int DV>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BackwardArgs a) {
    const int b = blockIdx.z, h = blockIdx.y;
    const int r = blockIdx.x * 256 + threadIdx.x;
    const Seq sq = load_seq(a.seqs, b);
    if (r >= sq.sq) return;
    const int64_t prow = sq.row0 + r;
    if (prow >= a.rows) return;
    if (!in_bounds(a.check, kSiteBwdRow, a.seqs.cu_q ? prow : (int64_t)b * a.seqs.max_sq + r, a.rows)) return;
    const int64_t o = (a.seqs.cu_q ? prow * a.o_row : (int64_t)b * a.o_batch + (int64_t)r * a.o_row) +
                      (int64_t)h * a.o_head;
    typedef T t8 __attribute__((ext_vector_type(8)));
    const t8* po = reinterpret_cast<const t8*>(reinterpret_cast<const T*>(a.out) + o);
    const t8* pd = reinterpret_cast<const t8*>(reinterpret_cast<const T*>(a.dout) + o);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < DV / 8; ++i) {
        const t8 x = po[i], y = pd[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf((float)x[j], (float)y[j], acc);
    }
    a.dvec[(int64_t)h * a.rows + prow] = acc;
}

// ---------------------------------------------------------------------------
// dQ per split
// ---------------------------------------------------------------------------

template <int DQK, int DV>
struct QCfg {
    static constexpr int K_ELEMS = kKT * DQK, V_ELEMS = kKT * DV;
    static constexpr int K_LOADS = kKT * (DQK / 8) / kThreads, V_LOADS = kKT * (DV / 8) / kThreads;
    static_assert(DQK % 64 == 0 && DV % 64 == 0, "head dims");
    static_assert((kKT * DQK / 8) % kThreads == 0 && (kKT * DV / 8) % kThreads == 0, "whole loads");
};

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BackwardArgs a) {
    using C = QCfg<DQK, DV>;
    using E = Elem<T>;
    using v8 = typename E::v8;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (C::K_ELEMS + C::V_ELEMS)];

    uint32_t w = xcd_contiguous(blockIdx.x, gridDim.x);
    const int tile = (int)(w % a.n_qtiles);
    w /= a.n_qtiles;
    const int head = (int)(w % a.heads);
    w /= a.heads;
    const int split = (int)(w % a.seqs.s_max);
    const int b = (int)(w / a.seqs.s_max);
    if (!in_bounds(a.check, kSiteBwdItem, b, a.batch) || !in_bounds(a.check, kSiteBwdItem, head, a.heads)) return;
    const Seq sq = load_seq(a.seqs, b);
    if (split >= sq.splits) return;
    const int r0 = tile * kQB;
    if (r0 >= sq.sq) return;
    const int mask = a.seqs.mask;
    int ks, ke;
    block_split_range(sq, mask, a.seqs.n_per_block, min(r0 + kQB, sq.sq) - 1, split, ks, ke);
    if (ks >= ke) return;  // no key for the whole block: not written, not summed
    if (!in_bounds(a.check, kSiteBwdKey, (sq.krow0 >= 0 ? sq.krow0 : 0) + ke - 1,
                   sq.krow0 >= 0 ? total_keys(a.seqs, a.batch) : (int64_t)a.seqs.max_sk))
        return;
    const int64_t win = a.seqs.window_left;
    {
        const int64_t lo_first = vis_first(sq, win, r0);
        if (lo_first > ks) ks = (int)min((int64_t)ke, ks + (lo_first - ks) / kKT * kKT);
    }

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int qrow = r0 + wave * 32 + col;
    const bool row_ok = qrow < sq.sq && sq.row0 + qrow < a.rows &&
                        in_bounds(a.check, kSiteBwdRow, a.seqs.cu_q ? sq.row0 + qrow : (int64_t)b * a.seqs.max_sq + qrow,
                                  a.rows);  // (rows: cu_seqlens past total_q)
    const int64_t prow = sq.row0 + qrow;
    const int vis_q = (int)max(min(vis_last(sq, mask, qrow), (int64_t)0x7fffffff), (int64_t)-1);
    const int lo_q = (int)min(vis_first(sq, win, qrow), (int64_t)0x7fffffff);

    const float lse2 = row_ok ? lse_log2(a.lse[(int64_t)head * a.rows + prow]) : INFINITY;
    const float dval = row_ok ? a.dvec[(int64_t)head * a.rows + prow] : 0.f;

    // Q^T and dO^T fragments (B operands): lane holds X[qrow][16t + 8 half .. +8]
    v8 qf[DQK / 16], df[DV / 16];
    {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             (a.seqs.cu_q ? prow * a.q_row : (int64_t)b * a.q_batch + (int64_t)qrow * a.q_row) +
                             (int64_t)head * a.q_head + half * 8;
        const uint16_t* dp = reinterpret_cast<const uint16_t*>(a.dout) +
                             (a.seqs.cu_q ? prow * a.o_row : (int64_t)b * a.o_batch + (int64_t)qrow * a.o_row) +
                             (int64_t)head * a.o_head + half * 8;
#pragma unroll
        for (int t = 0; t < DQK / 16; ++t)
            qf[t] = __builtin_bit_cast(v8, row_ok ? *reinterpret_cast<const uint4*>(qp + t * 16) : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int t = 0; t < DV / 16; ++t)
            df[t] = __builtin_bit_cast(v8, row_ok ? *reinterpret_cast<const uint4*>(dp + t * 16) : make_uint4(0, 0, 0, 0));
    }
    f32x16 dq[DQK / 32];
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c)
        for (int j = 0; j < 16; ++j) dq[c][j] = 0.f;

    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) +
                            (sq.krow0 >= 0 ? sq.krow0 * a.k_row : (int64_t)b * a.k_batch) + (int64_t)head * a.k_head;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) +
                            (sq.krow0 >= 0 ? sq.krow0 * a.v_row : (int64_t)b * a.v_batch) + (int64_t)head * a.v_head;
    // Tile DMA: load i of this thread fills chunk P = 256 i + tid (row P / CH,
    // swizzled chunk P % CH); rows past the split's end read as zeros.
    uint32_t k_off[C::K_LOADS], v_off[C::V_LOADS];
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
        const int P = i * kThreads + tid, r = P / (DQK / 8);
        k_off[i] = (uint32_t)(r * a.k_row + bt_swz<DQK / 8>(r, P % (DQK / 8)) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
        const int P = i * kThreads + tid, r = P / (DV / 8);
        v_off[i] = (uint32_t)(r * a.v_row + bt_swz<DV / 8>(r, P % (DV / 8)) * 8) * 2u;
    }
    uint16_t* const Ks = smem;
    uint16_t* const Vs = smem + 2 * C::K_ELEMS;
    // Buffer resources of the K and V tile at key kt (a tile at or past the
    // end has an empty range and loads zeros), and load i of the pair, K
    // loads first.  The loop issues a tile's loads one per k-step of the
    // previous tile's first GEMM: issued as one burst, they would hold the
    // wave before its first MFMA.
    struct TileRsrc {
        __amdgpu_buffer_rsrc_t k, v;
    };
    auto rsrc = [&](int kt) {
        const int rows = min(ke - kt, kKT);
        const uint32_t kb = rows > 0 ? (uint32_t)(((rows - 1) * a.k_row + DQK) * 2) : 0u;
        const uint32_t vb = rows > 0 ? (uint32_t)(((rows - 1) * a.v_row + DV) * 2) : 0u;
        return TileRsrc{tile_rsrc(kbase + (int64_t)kt * a.k_row, kb), tile_rsrc(vbase + (int64_t)kt * a.v_row, vb)};
    };
    auto load_one = [&](const TileRsrc& r, int slot, auto i_c) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i < C::K_LOADS)
            load_lds16(r.k, k_off[i], Ks + slot * C::K_ELEMS + (i * kThreads + wave * 64) * 8);
        else if constexpr (i < C::K_LOADS + C::V_LOADS)
            load_lds16(r.v, v_off[i - C::K_LOADS], Vs + slot * C::V_ELEMS + ((i - C::K_LOADS) * kThreads + wave * 64) * 8);
    };
    auto issue = [&](int kt, int slot) {
        const TileRsrc r = rsrc(kt);
        static_for<C::K_LOADS + C::V_LOADS>([&](auto i_c) { load_one(r, slot, i_c); });
    };
    static_assert(C::K_LOADS + C::V_LOADS <= DQK / 16, "one tile load per k-step of S^T = K Q^T");
    auto sync_tiles = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    };
    // LDS read bases of slot 0; slot 1 is a constant byte offset away
    TileReads<DQK> kr;
    TileReads<DV> vr;
    kr.init(Ks, lane);
    vr.init(Vs, lane);

    const int64_t vis_top = vis_last(sq, mask, r0);
    const int64_t full_last = min((int64_t)ke - kKT, vis_top - (kKT - 1));
    const int full_end = full_last < ks ? ks : (int)(ks + ((full_last - ks) / kKT + 1) * kKT);
    const int64_t lo_last = vis_first(sq, win, min(r0 + kQB, sq.sq) - 1);
    const int full_start = lo_last <= ks ? ks : (int)min((int64_t)ke, ks + ceil_div64(lo_last - ks, kKT) * kKT);
    const float cl2 = a.scale_log2;

    // One tile; loads(t) issues load t of the next tile into the other slot
    auto step = [&](int kt, auto slot_c, auto&& loads) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int KO = slot * C::K_ELEMS * 2, VO = slot * C::V_ELEMS * 2;  // slot byte offsets
        constexpr int NB = DQK / 32;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            for (int j = 0; j < 16; ++j) s[kb][j] = dp[kb][j] = 0.f;
        gemm_rows<E, DQK, 2, KO, 3>(kr, s, qf, loads);  // S^T = K Q^T
        if (kt >= full_end || kt < full_start) {
            const int lim = min(ke - 1, vis_q) - kt - half * 4, first = lo_q - kt - half * 4;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int rel = kb * 32 + (j >> 2) * 8 + (j & 3);
                    if (rel > lim || rel < first) s[kb][j] = -INFINITY;
                }
        }
        // dP^T = V dO^T; meanwhile P^T = exp2(S^T scale log2e - LSE log2e)
        // replaces S^T, 32 / (D_v / 16) elements per k-step
        gemm_rows<E, DV, 2, VO, 3>(vr, dp, df, [&](auto t_c) {
            constexpr int t = decltype(t_c)::value, per = 32 / (DV / 16);
#pragma unroll
            for (int e = t * per; e < (t + 1) * per; ++e)
                s[e >> 4][e & 15] = __builtin_amdgcn_exp2f(fmaf(s[e >> 4][e & 15], cl2, -lse2));
        });
        // dS^T = P^T * (dP^T - D) in GEMM1's B layout; dQ^T += K^T dS^T over
        // the tile's 64 keys in four steps of 16, each step's K^T reads
        // issued before the previous step's MFMAs and the next dS slice
        // computed under them
        v8 ds[2][2];
        auto ds_slice = [&](int kb, int h) {
#pragma unroll
            for (int j = 0; j < 8; ++j) ds[kb][h][j] = (T)(s[kb][8 * h + j] * (dp[kb][8 * h + j] - dval));
        };
        s16x4 xa[2 * NB], xb[2 * NB];
        tr_issue<DQK, KO + 0 * 16 * DQK * 2>(kr, xa);
        ds_slice(0, 0);
        tr_issue<DQK, KO + 1 * 16 * DQK * 2>(kr, xb);
        tr_mfma<E, DQK, 2 * NB>(xa, dq, ds[0][0], [&](auto c_c) {
            if constexpr (decltype(c_c)::value == 0) ds_slice(0, 1);
        });
        tr_issue<DQK, KO + 2 * 16 * DQK * 2>(kr, xa);
        tr_mfma<E, DQK, 2 * NB>(xb, dq, ds[0][1], [&](auto c_c) {
            if constexpr (decltype(c_c)::value == 0) ds_slice(1, 0);
        });
        tr_issue<DQK, KO + 3 * 16 * DQK * 2>(kr, xb);
        tr_mfma<E, DQK, 2 * NB>(xa, dq, ds[1][0], [&](auto c_c) {
            if constexpr (decltype(c_c)::value == 0) ds_slice(1, 1);
        });
        tr_mfma<E, DQK, 0>(xb, dq, ds[1][1], NoSide{});
    };

    // Tiles alternate between the two LDS slots; the loop takes them in
    // pairs so that each step's slot is a constant and the accumulators flow
    // through straight-line code.  A wave past the sequence's last row runs
    // on zero rows (its P is 0) instead of branching around the step.
    const int ntiles = ks < ke ? (ke - ks + kKT - 1) / kKT : 0;
    if (ntiles > 0) {
        issue(ks, 0);
        sync_tiles();
        int i = 0;
        for (; i + 2 <= ntiles; i += 2) {
            const int kt = ks + i * kKT;
            const TileRsrc r1 = rsrc(kt + kKT);
            step(kt, std::integral_constant<int, 0>{}, [&](auto t_c) { load_one(r1, 1, t_c); });
            sync_tiles();
            // past the last tile the range is empty (into a slot no step reads)
            const TileRsrc r0 = rsrc(kt + 2 * kKT);
            step(kt + kKT, std::integral_constant<int, 1>{}, [&](auto t_c) { load_one(r0, 0, t_c); });
            sync_tiles();
        }
        if (i < ntiles) step(ks + i * kKT, std::integral_constant<int, 0>{}, NoSide{});
    }

    if (!row_ok || prow >= a.rows) return;
    if (!in_bounds(a.check, kSiteBwdPart, ((int64_t)head * a.seqs.s_max + split) * a.rows + prow,
                   (int64_t)a.heads * a.seqs.s_max * a.rows))
        return;
    float* op = a.dq_part + (((int64_t)head * a.seqs.s_max + split) * a.rows + prow) * DQK + half * 4;
    const float sc = a.scale;
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            *reinterpret_cast<float4*>(op + c * 32 + jb * 8) =
                make_float4(dq[c][jb * 4] * sc, dq[c][jb * 4 + 1] * sc, dq[c][jb * 4 + 2] * sc, dq[c][jb * 4 + 3] * sc);
}

// dQ = sum of the split sums the block populated; one thread per (row, 4 dims)
template <typename T, int DQK>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(BackwardArgs a) {
    const int b = blockIdx.z, h = blockIdx.y;
    constexpr int kParts = DQK / 4;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int r = idx / kParts, part = idx % kParts;
    const Seq sq = load_seq(a.seqs, b);
    if (r >= sq.sq) return;
    const int64_t prow = sq.row0 + r;
    if (prow >= a.rows) return;
    const int n = block_populated_splits(sq, a.seqs.mask, a.seqs.n_per_block, kQB, r);
    if (!in_bounds(a.check, kSiteBwdRow, a.seqs.cu_q ? prow : (int64_t)b * a.seqs.max_sq + r, a.rows) ||
        (n > 0 && !in_bounds(a.check, kSiteBwdPart, ((int64_t)h * a.seqs.s_max + n - 1) * a.rows + prow,
                             (int64_t)a.heads * a.seqs.s_max * a.rows)))
        return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < n; ++s) {
        const float4 x = *reinterpret_cast<const float4*>(
            a.dq_part + (((int64_t)h * a.seqs.s_max + s) * a.rows + prow) * DQK + part * 4);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
    }
    const int64_t o = (a.seqs.cu_q ? prow * a.q_row : (int64_t)b * a.q_batch + (int64_t)r * a.q_row) +
                      (int64_t)h * a.q_head + part * 4;
    store4(reinterpret_cast<T*>(a.dq) + o, acc.x, acc.y, acc.z, acc.w);
}

// ---------------------------------------------------------------------------
// dK, dV per block of 128 keys
// ---------------------------------------------------------------------------

template <int DQK, int DV>
struct KCfg {
    static constexpr int Q_ELEMS = kQT * DQK, O_ELEMS = kQT * DV;
    static constexpr int Q_LOADS = kQT * (DQK / 8) / kThreads, O_LOADS = kQT * (DV / 8) / kThreads;
    static_assert((kQT * DQK / 8) % kThreads == 0 && (kQT * DV / 8) % kThreads == 0, "whole loads");
};

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BackwardArgs a) {
    using C = KCfg<DQK, DV>;
    using E = Elem<T>;
    using v8 = typename E::v8;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (C::Q_ELEMS + C::O_ELEMS)];
    __shared__ __attribute__((aligned(16))) float row_lse2[2][kQT];
    __shared__ __attribute__((aligned(16))) float row_d[2][kQT];

    uint32_t w = xcd_contiguous(blockIdx.x, gridDim.x);
    const int ktile = (int)(w % a.n_ktiles);
    w /= a.n_ktiles;
    const int head = (int)(w % a.heads);
    const int b = (int)(w / a.heads);
    if (!in_bounds(a.check, kSiteBwdItem, b, a.batch) || !in_bounds(a.check, kSiteBwdItem, head, a.heads)) return;
    const Seq sq = load_seq(a.seqs, b);
    const int k0 = ktile * kKB;
    if (k0 >= sq.sk) return;
    const int mask = a.seqs.mask;
    const int64_t win = a.seqs.window_left;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int key = k0 + wave * 32 + col;
    const int64_t krow = sq.krow0 >= 0 ? sq.krow0 + key : key;  // packed key row (dense: index in its batch)
    const bool key_ok = key < sq.sk && in_bounds(a.check, kSiteBwdKey, krow,
                                                 sq.krow0 >= 0 ? total_keys(a.seqs, a.batch) : (int64_t)a.seqs.max_sk);

    // K^T and V^T fragments (B operands): lane holds X[key][16t + 8 half .. +8]
    v8 kf[DQK / 16], vf[DV / 16];
    {
        const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k) +
                             (sq.krow0 >= 0 ? krow * a.k_row : (int64_t)b * a.k_batch + (int64_t)key * a.k_row) +
                             (int64_t)head * a.k_head + half * 8;
        const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v) +
                             (sq.krow0 >= 0 ? krow * a.v_row : (int64_t)b * a.v_batch + (int64_t)key * a.v_row) +
                             (int64_t)head * a.v_head + half * 8;
#pragma unroll
        for (int t = 0; t < DQK / 16; ++t)
            kf[t] = __builtin_bit_cast(v8, key_ok ? *reinterpret_cast<const uint4*>(kp + t * 16) : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int t = 0; t < DV / 16; ++t)
            vf[t] = __builtin_bit_cast(v8, key_ok ? *reinterpret_cast<const uint4*>(vp + t * 16) : make_uint4(0, 0, 0, 0));
    }
    f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c)
        for (int j = 0; j < 16; ++j) dk[c][j] = 0.f;
#pragma unroll
    for (int c = 0; c < DV / 32; ++c)
        for (int j = 0; j < 16; ++j) dv[c][j] = 0.f;

    // Rows q that see a key of [k0, k1): q + off >= k0 under a causal rule,
    // q + off - window <= k1 - 1 under a window; keys past lastValid are
    // seen by no row.
    const int k1 = (int)min((int64_t)k0 + kKB, sq.lv + 1);
    int q_lo = 0, q_hi = 0;
    if (k1 > k0) {
        // (clamped to the rows before the cast: the offset is 64-bit)
        q_lo = mask == SK_MASK_NONE ? 0 : (int)min(max((int64_t)0, (int64_t)k0 - sq.off), (int64_t)sq.sq);
        int64_t hi = sq.sq;
        if (win >= 0) hi = min(hi, (int64_t)k1 - sq.off + win);
        q_hi = (int)max(hi, (int64_t)q_lo);
    }
    // Every query tile the loop loads lies inside the sequence's rows.
    if (q_hi > q_lo && !in_bounds(a.check, kSiteBwdRow, (a.seqs.cu_q ? sq.row0 : (int64_t)b * a.seqs.max_sq) + q_hi - 1,
                                  a.rows))
        q_hi = q_lo;
    // This lane's key is visible to rows q in [q_first, q_first + q_span]
    // (q_span as unsigned: q is visible iff (unsigned)(q - q_first) <= q_span);
    // a key no row sees gets q_first = 2^31, q_span = 0, which no q < 2^31 meets.
    uint32_t q_first = 0x80000000u, q_span = 0;
    {
        const int64_t lo = mask == SK_MASK_NONE ? 0 : max((int64_t)0, (int64_t)key - sq.off);
        const int64_t hi = min((int64_t)sq.sq - 1, win >= 0 ? (int64_t)key - sq.off + win : (int64_t)sq.sq);
        if (key_ok && key <= sq.lv && lo <= hi) {
            q_first = (uint32_t)lo;
            q_span = (uint32_t)(hi - lo);
        }
    }
    // Rows [full_lo, full_hi] see every key of the block: a tile inside them
    // needs no mask (uniform over the workgroup).
    int full_lo = 1, full_hi = 0;
    {
        const int64_t kl = (int64_t)k0 + kKB - 1;  // the block's last key
        if (kl < sq.sk && kl <= sq.lv) {
            const int64_t lo = mask == SK_MASK_NONE ? 0 : max((int64_t)0, kl - sq.off);
            const int64_t hi = min((int64_t)sq.sq - 1, win >= 0 ? (int64_t)k0 - sq.off + win : (int64_t)sq.sq);
            if (lo <= hi) {
                full_lo = (int)lo;
                full_hi = (int)hi;
            }
        }
    }

    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q) +
                            (a.seqs.cu_q ? sq.row0 * a.q_row : (int64_t)b * a.q_batch) + (int64_t)head * a.q_head;
    const uint16_t* obase = reinterpret_cast<const uint16_t*>(a.dout) +
                            (a.seqs.cu_q ? sq.row0 * a.o_row : (int64_t)b * a.o_batch) + (int64_t)head * a.o_head;
    uint32_t q_off[C::Q_LOADS], o_off[C::O_LOADS];
#pragma unroll
    for (int i = 0; i < C::Q_LOADS; ++i) {
        const int P = i * kThreads + tid, r = P / (DQK / 8);
        q_off[i] = (uint32_t)(r * a.q_row + bt_swz<DQK / 8>(r, P % (DQK / 8)) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::O_LOADS; ++i) {
        const int P = i * kThreads + tid, r = P / (DV / 8);
        o_off[i] = (uint32_t)(r * a.o_row + bt_swz<DV / 8>(r, P % (DV / 8)) * 8) * 2u;
    }
    uint16_t* const Qs = smem;
    uint16_t* const Os = smem + 2 * C::Q_ELEMS;
    const float* lse_h = a.lse + (int64_t)head * a.rows + sq.row0;
    const float* d_h = a.dvec + (int64_t)head * a.rows + sq.row0;
    float pre_l = -INFINITY, pre_d = 0.f;  // this thread's row values of the next tile (threads 0..31)
    // Buffer resources of the Q and dO tile at row qt (a tile at or past the
    // end has an empty range and loads zeros), and load i of the pair, Q
    // loads first.  The loop issues a tile's loads one per k-step of the
    // previous tile's first GEMM: issued as one burst, they would hold the
    // wave before its first MFMA.
    struct TileRsrc {
        __amdgpu_buffer_rsrc_t q, o;
    };
    auto rsrc = [&](int qt) {
        const int rows = min(sq.sq - qt, kQT);
        const uint32_t qb = rows > 0 ? (uint32_t)(((rows - 1) * a.q_row + DQK) * 2) : 0u;
        const uint32_t ob = rows > 0 ? (uint32_t)(((rows - 1) * a.o_row + DV) * 2) : 0u;
        return TileRsrc{tile_rsrc(qbase + (int64_t)qt * a.q_row, qb), tile_rsrc(obase + (int64_t)qt * a.o_row, ob)};
    };
    auto load_one = [&](const TileRsrc& r, int slot, auto i_c) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i < C::Q_LOADS)
            load_lds16(r.q, q_off[i], Qs + slot * C::Q_ELEMS + (i * kThreads + wave * 64) * 8);
        else if constexpr (i < C::Q_LOADS + C::O_LOADS)
            load_lds16(r.o, o_off[i - C::Q_LOADS], Os + slot * C::O_ELEMS + ((i - C::Q_LOADS) * kThreads + wave * 64) * 8);
    };
    static_assert(C::Q_LOADS + C::O_LOADS <= DQK / 16, "one tile load per k-step of S = Q K^T");
    // the rows' LSE and D of the tile at qt (threads 0 .. kQT - 1)
    auto issue_rows = [&](int qt) {
        if (tid < kQT) {  // raw values: converted at sync time, so no wait here
            const bool ok = qt + tid < sq.sq;
            pre_l = ok ? lse_h[qt + tid] : -INFINITY;
            pre_d = ok ? d_h[qt + tid] : 0.f;
        }
    };
    auto sync_tiles = [&](int slot) {
        if (tid < kQT) {
            row_lse2[slot][tid] = lse_log2(pre_l);
            row_d[slot][tid] = pre_d;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    };
    // LDS read bases of slot 0; slot 1 is a constant byte offset away
    TileReads<DQK> qr;
    TileReads<DV> orr;
    qr.init(Qs, lane);
    orr.init(Os, lane);
    const float cl2 = a.scale_log2;

    // This lane holds rows qt + 8 g + 4 half + i of a tile (element
    // j = 4 g + i); their log2 LSE and D, four rows per load.  Plain loads
    // (the compiler tracks their completion), issued right after the barrier
    // and before the next tile's DMA, so they wait for no tile load.
    auto row_values = [&](int slot, float4 (&l4)[4], float4 (&d4)[4]) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            l4[g] = *reinterpret_cast<const float4*>(&row_lse2[slot][8 * g + 4 * half]);
            d4[g] = *reinterpret_cast<const float4*>(&row_d[slot][8 * g + 4 * half]);
        }
    };
    // One tile; loads(t) issues load t of the next tile into the other slot
    auto step = [&](int qt, auto slot_c, float4 (&l4)[4], float4 (&d4)[4], auto&& loads) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int QO = slot * C::Q_ELEMS * 2, OO = slot * C::O_ELEMS * 2;  // slot byte offsets
        constexpr int NBV = DV / 32, NBK = DQK / 32;
        // complete the row-value loads before the GEMM reads are issued
#pragma unroll
        for (int g = 0; g < 4; ++g)
            asm volatile("" ::"v"(l4[g].x), "v"(l4[g].y), "v"(l4[g].z), "v"(l4[g].w), "v"(d4[g].x), "v"(d4[g].y),
                         "v"(d4[g].z), "v"(d4[g].w));
        f32x16 sa[1], dpa[1];
        for (int j = 0; j < 16; ++j) sa[0][j] = dpa[0][j] = 0.f;
        gemm_rows<E, DQK, 1, QO, 3>(qr, sa, kf, loads);  // S = Q K^T (this lane: one key, 16 rows)
        f32x16& s = sa[0];
        if (!(qt >= full_lo && qt + kQT - 1 <= full_hi)) {
            const uint32_t base = (uint32_t)(qt + half * 4) - q_first;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (base + (uint32_t)((j >> 2) * 8 + (j & 3)) > q_span) s[j] = -INFINITY;
        }
        // dP = dO V^T; meanwhile P = exp2(S scale log2e - LSE log2e)
        // replaces S, 16 / (D_v / 16) elements per k-step
        v8 pf[2], dsf[2];
        gemm_rows<E, DV, 1, OO, 3>(orr, dpa, vf, [&](auto t_c) {
            constexpr int t = decltype(t_c)::value, per = 16 / (DV / 16);
#pragma unroll
            for (int j = t * per; j < (t + 1) * per; ++j) {
                const float l2 = (j & 3) == 0 ? l4[j >> 2].x : (j & 3) == 1 ? l4[j >> 2].y : (j & 3) == 2 ? l4[j >> 2].z : l4[j >> 2].w;
                s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], cl2, -l2));
                pf[j >> 3][j & 7] = (T)s[j];
            }
        });
        const f32x16& dp = dpa[0];
        auto ds_slice = [&](int h) {
#pragma unroll
            for (int j = 8 * h; j < 8 * h + 8; ++j) {
                const float dd = (j & 3) == 0 ? d4[j >> 2].x : (j & 3) == 1 ? d4[j >> 2].y : (j & 3) == 2 ? d4[j >> 2].z : d4[j >> 2].w;
                dsf[h][j & 7] = (T)(s[j] * (dp[j] - dd));
            }
        };
        // dV^T += dO^T P, then dK^T += Q^T dS over the tile's 32 rows, in
        // steps of 16 rows; each step's transposed reads are issued before
        // the previous step's MFMAs and dS is computed under the dV MFMAs
        s16x4 xa[2 * NBK], xb[2 * NBK];
        tr_issue<DV, OO>(orr, xa);
        tr_issue<DV, OO + 16 * DV * 2>(orr, xb);
        tr_mfma<E, DV, 2 * NBV>(xa, dv, pf[0], [&](auto c_c) {
            if constexpr (decltype(c_c)::value == 0) ds_slice(0);
        });
        tr_issue<DQK, QO>(qr, xa);
        tr_mfma<E, DV, 2 * NBK>(xb, dv, pf[1], [&](auto c_c) {
            if constexpr (decltype(c_c)::value == 0) ds_slice(1);
        });
        tr_issue<DQK, QO + 16 * DQK * 2>(qr, xb);
        tr_mfma<E, DQK, 2 * NBK>(xa, dk, dsf[0], NoSide{});
        tr_mfma<E, DQK, 0>(xb, dk, dsf[1], NoSide{});
    };

    // Tiles in pairs over the two LDS slots (constant slot per step, no
    // branch around the accumulators).
    const int ntiles = q_hi > q_lo ? (q_hi - q_lo + kQT - 1) / kQT : 0;
    if (ntiles > 0) {
        {
            const TileRsrc r = rsrc(q_lo);
            static_for<C::Q_LOADS + C::O_LOADS>([&](auto i_c) { load_one(r, 0, i_c); });
            issue_rows(q_lo);
        }
        sync_tiles(0);
        int i = 0;
        float4 l4[4], d4[4];
        for (; i + 2 <= ntiles; i += 2) {
            const int qt = q_lo + i * kQT;
            row_values(0, l4, d4);
            issue_rows(qt + kQT);
            const TileRsrc r1 = rsrc(qt + kQT);
            step(qt, std::integral_constant<int, 0>{}, l4, d4, [&](auto t_c) { load_one(r1, 1, t_c); });
            sync_tiles(1);
            row_values(1, l4, d4);
            // past the last tile the ranges are empty (into a slot no step
            // reads) and the row values are not used
            issue_rows(qt + 2 * kQT);
            const TileRsrc r0 = rsrc(qt + 2 * kQT);
            step(qt + kQT, std::integral_constant<int, 1>{}, l4, d4, [&](auto t_c) { load_one(r0, 0, t_c); });
            sync_tiles(0);
        }
        if (i < ntiles) {
            row_values(0, l4, d4);
            step(q_lo + i * kQT, std::integral_constant<int, 0>{}, l4, d4, NoSide{});
        }
    }

    if (!key_ok) return;
    T* kout = reinterpret_cast<T*>(a.dk) +
              (sq.krow0 >= 0 ? krow * a.k_row : (int64_t)b * a.k_batch + (int64_t)key * a.k_row) +
              (int64_t)head * a.k_head + half * 4;
    T* vout = reinterpret_cast<T*>(a.dv) +
              (sq.krow0 >= 0 ? krow * a.v_row : (int64_t)b * a.v_batch + (int64_t)key * a.v_row) +
              (int64_t)head * a.v_head + half * 4;
    const float sc = a.scale;
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            store4(kout + c * 32 + jb * 8, dk[c][jb * 4] * sc, dk[c][jb * 4 + 1] * sc, dk[c][jb * 4 + 2] * sc,
                   dk[c][jb * 4 + 3] * sc);
#pragma unroll
    for (int c = 0; c < DV / 32; ++c)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            store4(vout + c * 32 + jb * 8, dv[c][jb * 4], dv[c][jb * 4 + 1], dv[c][jb * 4 + 2], dv[c][jb * 4 + 3]);
}

// D, then dQ per split, dK/dV, and the dQ sum.  With no query row only dK/dV
// run (all zero); with no key the dQ pass writes nothing and the sum gives 0.
template <typename T, int DQK, int DV>
hipError_t launch(const BackwardArgs& a, hipStream_t stream) {
    const unsigned B = (unsigned)a.batch, H = (unsigned)a.heads;
    const bool has_rows = a.rows > 0 && a.seqs.max_sq > 0;
    if (has_rows) {
        hipLaunchKernelGGL((bwd_rowdot_kernel<T, DV>), dim3((a.seqs.max_sq + 255) / 256, H, B), dim3(256), 0, stream,
                           a);
        hipLaunchKernelGGL((bwd_dq_kernel<T, DQK, DV>), dim3((unsigned)a.n_qtiles * H * a.seqs.s_max * B),
                           dim3(kThreads), 0, stream, a);
    }
    if (a.n_ktiles > 0)
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, DQK, DV>), dim3((unsigned)a.n_ktiles * H * B), dim3(kThreads), 0,
                           stream, a);
    if (has_rows) {
        const unsigned reduce_blocks = (unsigned)(((int64_t)a.seqs.max_sq * (DQK / 4) + 255) / 256);
        hipLaunchKernelGGL((bwd_dq_reduce_kernel<T, DQK>), dim3(reduce_blocks, H, B), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename T>
BackwardKernel find_16(int d_qk, int d_v) {
    if (d_qk == 64 && d_v == 64) return {launch<T, 64, 64>, kQB, kKB};
    if (d_qk == 128 && d_v == 128) return {launch<T, 128, 128>, kQB, kKB};
    if (d_qk == 192 && d_v == 128) return {launch<T, 192, 128>, kQB, kKB};
    return {nullptr, 0, 0};
}

}  // namespace

BackwardKernel find_backward(int dtype, int d_qk, int d_v) {
    if (dtype == SK_BF16) return find_16<__bf16>(d_qk, d_v);
    if (dtype == SK_F16) return find_16<_Float16>(d_qk, d_v);
    return {nullptr, 0, 0};
}

}  // namespace sk
