// Split-KV partial attention, bf16 or f16 storage, 16-bit MFMA with f32
// accumulation.
//
// Per (sequence, head, split, block of 128 or 256 query rows) the kernel
// computes the partial output O_s and log-sum-exp L_s over the split's keys
// (rocmlirTriton page "Recombine fully masked split-KV attention partials on
// the host": Summary for the partials and the empty-split convention,
// "Per-row valid-split counts" for the block's key partition).  The workload
// it is tuned for is the long-context packed-varlen prefill of the aiter page
// "[ASM][HIP][JIT][gfx942] Optimize long-context FMHA with split-KV"
// (D_qk = 192, D_v = 128), re-designed for gfx950:
//
//  * 32 query rows per wave, in groups of 4 waves (one per SIMD).  GEMM0 is
//    computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K
//    (from LDS) is the A operand and Q^T (kept in registers for the whole key
//    loop) the B operand.  The accumulator then gives every lane ONE query
//    column and 16 keys, so the row max / row sum are in-lane reductions plus
//    one exchange between the two half-waves.
//  * The same accumulator layout is exactly the B operand layout (key-major,
//    query column per lane) GEMM1 needs for O^T = V^T P^T, so P never leaves
//    registers: it is rounded to bf16 in place.  V stays row-major in LDS and
//    its A operand is read with ds_read_b64_tr_b16, which hands each lane four
//    keys of one value column.
//  * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds,
//    no register staging), in two K and two or three V slots: the next tile
//    streams in while the current one is multiplied, with one barrier per
//    tile.  16-byte chunks are XOR-swizzled by row so both operand reads are
//    bank-conflict free.
//  * Large problems take two groups (8 waves, 256 rows, one workgroup per
//    CU): every tile is loaded once for twice the rows.  The second group
//    passes the tile's barrier between its GEMM0 and GEMM1, the first after
//    its GEMM1, so the two waves that share a SIMD (waves w and w + 4) run
//    opposite halves of the tile step: one's softmax beside the other's
//    MFMAs.  V then takes three LDS slots (one group still reads tile t - 1).
//  * Online softmax in base 2 with the scale folded into one FMA per score;
//    the reference max moves only when it grows by more than 2^8, and a row
//    with no visible key so far keeps m = -inf and zero weights.
//  * Work items are remapped so each XCD streams one (head, split) key range
//    through its own L2.
#include <float.h>

#include <atomic>
#include <type_traits>

#include "mfma_common.hpp"
#include "pieces.hpp"
#include "sk_common.hpp"

namespace sk {

namespace {

using namespace mfma;

constexpr int kGroupRows = 128;    // query rows per group of 4 waves
constexpr int kGroupThreads = 256;
constexpr int kBN = 64;            // keys per tile

template <int DQK, int DV, int G>
struct Cfg {
    static constexpr int kBM = G * kGroupRows;           // query rows per workgroup
    static constexpr int kThreads = G * kGroupThreads;
    static constexpr int V_SLOTS = G == 1 ? 2 : 3;       // LDS slots of V tiles
    static constexpr int KCH = DQK / 8;                 // 16-byte chunks per K row
    static constexpr int VCH = DV / 8;                  // 16-byte chunks per V row
    static constexpr int K_ELEMS = kBN * DQK;           // one K tile (bf16 elements)
    static constexpr int V_ELEMS = kBN * DV;            // one V tile
    static constexpr int LDS_ELEMS = 2 * K_ELEMS + V_SLOTS * V_ELEMS;
    static constexpr int K_LOADS = kBN * KCH / kThreads;  // 16-byte loads per thread per tile
    static constexpr int V_LOADS = kBN * VCH / kThreads;
    static constexpr int VG = (VCH / 4) < 4 ? (VCH / 4) : 4;  // V swizzle period (rows)
    static_assert(G == 1 || G == 2, "one or two groups of 4 waves");
    static_assert(DQK % 64 == 0 && DV % 32 == 0, "head dims must be multiples of 64 (QK) and 32 (V)");
    static_assert((kBN * KCH) % kThreads == 0 && (kBN * VCH) % kThreads == 0, "whole loads per thread");
    static_assert(K_LOADS + V_LOADS <= DQK / 16, "one tile load per GEMM0 step");
};

// Growth of the running max (in log2 units) tolerated before the output
// accumulator is rescaled.  Using a stale max m' <= m only changes the common
// factor 2^(m - m') of every weight and of their sum, so O = sum p V / sum p
// and LSE = m' + log(sum p) are unchanged; weights stay below 2^8.
constexpr float kRescaleThreshold = 8.0f;

template <typename T, int DQK, int DV, int G>
__global__ __launch_bounds__(G * kGroupThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void partial_bf16_kernel(PartialArgs a) {
    using C = Cfg<DQK, DV, G>;
    constexpr int kBM = C::kBM;
    constexpr int kThreads = C::kThreads;
    using E = Elem<T>;
    using bf16x8 = typename E::v8;  // operand vector of the storage type
    using bf16x2 = typename E::v2;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];

    // Workgroups past n_main run piece `piece` of tail item n_main + tail_i.
    uint32_t item = blockIdx.x;
    int piece = -1;
    uint32_t tail_i = 0;
    if (item >= a.n_main) {
        const uint32_t j = item - a.n_main, n_tail = a.n_work - a.n_main;
        tail_i = j % n_tail;
        piece = (int)(j / n_tail);
        item = a.n_main + tail_i;
    }
    const WorkItem it = decode_work(a, item);
    if (!in_bounds(a.check, kSiteWorkItem, it.batch, a.batch) || !in_bounds(a.check, kSiteWorkItem, it.head, a.heads) ||
        !in_bounds(a.check, kSiteWorkItem, it.split, a.seqs.s_max))
        return;
    const Seq sq = load_seq(a.seqs, it.batch);
    if (it.split >= sq.splits) return;
    const int r0 = it.tile * kBM;
    if (r0 >= sq.sq) return;
    const int mask = a.seqs.mask;

    // The block's key range for this split, from its last row.  A split
    // with no key for the whole block exits without writing anything: its
    // slots take no part in the merge (the combine merges only the block's
    // populated splits).
    int ks, ke;
    block_split_range(sq, mask, a.seqs.n_per_block, min(r0 + kBM, sq.sq) - 1, it.split, ks, ke);
    if (ks >= ke) return;
    if (!in_bounds(a.check, kSiteKeys, (sq.krow0 >= 0 ? sq.krow0 : 0) + ke - 1,
                   sq.krow0 >= 0 ? total_keys(a.seqs, a.batch) : (int64_t)a.seqs.max_sk))
        return;
    if (piece >= 0) {
        // piece p of P takes key tiles [nt p / P, nt (p + 1) / P) of the split
        const int nt = ks < ke ? (ke - ks + kBN - 1) / kBN : 0;
        const int lo = (int)((int64_t)nt * piece / a.pieces), hi = (int)((int64_t)nt * (piece + 1) / a.pieces);
        ke = min(ks + hi * kBN, ke);
        ks = min(ks + lo * kBN, ke);
    }
    // Sliding window: whole tiles below the first row's first visible key
    // (the smallest in the block) hold no key any row sees; start past them.
    const int64_t win = a.seqs.window_left;
    {
        const int64_t lo_first = vis_first(sq, win, r0);
        if (lo_first > ks) ks = (int)min((int64_t)ke, ks + (lo_first - ks) / kBN * kBN);
    }
    // Smallest visibility limit in the block (its first row): tiles entirely
    // below it and inside the split need no per-element mask.
    const int64_t vis_top = vis_last(sq, mask, r0);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA bases in SGPRs
    const bool late = G > 1 && wave >= 4;  // second group: barrier between GEMM0 and GEMM1
    const int lane = tid & 63;
    const int col = lane & 31;   // query column of this lane (and A-row for loads)
    const int half = lane >> 5;  // which 8-wide k slice / which 4 accumulator rows
    const int qrow = r0 + wave * 32 + col;
    const bool row_ok = qrow < sq.sq && sq.row0 + qrow < a.rows;  // (rows: cu_seqlens past total_q)
    const bool q_ok = row_ok && in_bounds(a.check, kSiteQRow,
                                          a.seqs.cu_q ? sq.row0 + qrow : (int64_t)it.batch * a.seqs.max_sq + qrow,
                                          a.rows);
    const bool wave_active = (r0 + wave * 32) < sq.sq;
    // Visibility limits of this lane's row, clamped into int range (keys are int).
    const int vis_q = (int)max(min(vis_last(sq, mask, qrow), (int64_t)0x7fffffff), (int64_t)-1);
    const int lo_q = (int)min(vis_first(sq, win, qrow), (int64_t)0x7fffffff);

    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) +
                            (sq.krow0 >= 0 ? sq.krow0 * a.k_row : (int64_t)it.batch * a.k_batch) +
                            (int64_t)it.head * a.k_head;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) +
                            (sq.krow0 >= 0 ? sq.krow0 * a.v_row : (int64_t)it.batch * a.v_batch) +
                            (int64_t)it.head * a.v_head;

    // Q^T fragments (B operand of GEMM0): lane holds Q[qrow][16t + 8*half .. +8].
    bf16x8 qf[DQK / 16];
    {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             (a.seqs.cu_q ? (sq.row0 + qrow) * a.q_row
                                          : (int64_t)it.batch * a.q_batch + (int64_t)qrow * a.q_row) +
                             (int64_t)it.head * a.q_head + half * 8;
#pragma unroll
        for (int t = 0; t < DQK / 16; ++t) {
            uint4 x = q_ok ? *reinterpret_cast<const uint4*>(qp + t * 16) : make_uint4(0, 0, 0, 0);
            qf[t] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 o[DV / 32];
#pragma unroll
    for (int c = 0; c < DV / 32; ++c)
        for (int j = 0; j < 16; ++j) o[c][j] = 0.f;
    float m_i = -INFINITY;  // reference max of raw scores (this lane's query)
    float l_i = 0.f;        // sum of weights over this half-wave's keys
    const float cl2 = a.scale_log2;

    // Direct HBM -> LDS tile loads (buffer_load ... lds).  Load i of this
    // thread fills LDS chunk P = kThreads i + tid of the tile (a wave covers
    // 64 consecutive chunks); the chunk holds row P / CH and, after the
    // swizzle, column chunk c of that row.  The byte offset from the tile's first key
    // is the same for every tile.
    uint32_t k_off[C::K_LOADS], v_off[C::V_LOADS];
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
        const int P = i * kThreads + tid;
        const int r = P / C::KCH;
        k_off[i] = (uint32_t)(r * a.k_row + k_swz<C::KCH>(r, P % C::KCH) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
        const int P = i * kThreads + tid;
        const int r = P / C::VCH;
        v_off[i] = (uint32_t)(r * a.v_row + v_swz<C::VG>(r, P % C::VCH) * 8) * 2u;
    }
    // LDS: K tiles in two slots, V tiles in two (one group) or three slots.
    // K runs one tile ahead of V: between tile t's softmax and its GEMM1,
    // GEMM0 of tile t + 1 reads the other K slot.  With two groups, the
    // second group's GEMM1 of tile t runs after the barrier that ends the
    // tile, beside the first group's GEMM1 of tile t + 1 and the DMA of
    // V(t + 2): three V slots.
    uint16_t* const Ks0 = smem;
    uint16_t* const Vs0 = smem + 2 * C::K_ELEMS;
    // The buffer range of a tile ends with the split's last key, so rows past
    // it read as zeros (finite): their scores are masked to -inf, weights 0.
    // A tile starting at or past the end has an empty range and loads zeros.
    auto tile_bytes = [&](int kt, int64_t row, int d) -> uint32_t {
        const int rows = min(ke - kt, kBN);
        return rows > 0 ? (uint32_t)(((rows - 1) * row + d) * 2) : 0u;
    };
    // K and V tiles are issued in key order: running source pointers.
    const uint16_t* k_src = kbase + (int64_t)ks * a.k_row;
    const uint16_t* v_src = vbase + (int64_t)ks * a.v_row;
    const int64_t k_step = (int64_t)kBN * a.k_row, v_step = (int64_t)kBN * a.v_row;
    const uint32_t k_full = (uint32_t)(((kBN - 1) * a.k_row + DQK) * 2);
    const uint32_t v_full = (uint32_t)(((kBN - 1) * a.v_row + DV) * 2);
    auto issue_k = [&](int kt, int slot) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(k_src, kt + kBN <= ke ? k_full : tile_bytes(kt, a.k_row, DQK));
        k_src += k_step;
        uint16_t* dst = Ks0 + slot * C::K_ELEMS;
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) load_lds16(r, k_off[i], dst + (i * kThreads + wave * 64) * 8);
    };
    auto issue_v = [&](int kt, int slot) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(v_src, kt + kBN <= ke ? v_full : tile_bytes(kt, a.v_row, DV));
        v_src += v_step;
        uint16_t* dst = Vs0 + slot * C::V_ELEMS;
#pragma unroll
        for (int i = 0; i < C::V_LOADS; ++i) load_lds16(r, v_off[i], dst + (i * kThreads + wave * 64) * 8);
    };
    // The same loads, one at a time: the buffer resources of a K and a V
    // tile, then load i of the pair (K loads first), so that the loads of a
    // tile can be spread over the steps of a GEMM.
    auto rsrc_k = [&](int kt) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(k_src, kt + kBN <= ke ? k_full : tile_bytes(kt, a.k_row, DQK));
        k_src += k_step;
        return r;
    };
    auto rsrc_v = [&](int kt) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(v_src, kt + kBN <= ke ? v_full : tile_bytes(kt, a.v_row, DV));
        v_src += v_step;
        return r;
    };
    auto issue_one = [&](__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int kslot, int vslot, auto i_c) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i < C::K_LOADS)
            load_lds16(rk, k_off[i], Ks0 + kslot * C::K_ELEMS + (i * kThreads + wave * 64) * 8);
        else if constexpr (i < C::K_LOADS + C::V_LOADS)
            load_lds16(rv, v_off[i - C::K_LOADS], Vs0 + vslot * C::V_ELEMS + ((i - C::K_LOADS) * kThreads + wave * 64) * 8);
    };
    auto sync_tiles = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's tile loads landed
        __syncthreads();                     // everyone's landed; every wave is done with the old slots
    };

    // Per-lane LDS read offsets (elements).  GEMM0: K row kb*32 + col, chunk
    // 2t + half.  GEMM1 (transpose read): source lane s = lane % 16 of each
    // 16-lane group addresses key (4h + s/4 [+8]) and value columns
    // 32c + 16 g2 + 4 (s%4) .. +3, g2 = (lane / 16) % 2.
    const int k_rd = col * DQK;
    const int s16 = lane & 15;
    const int g2 = (lane >> 4) & 1;
    const int v_key = half * 4 + (s16 >> 2);
    const int v_sw = 4 * ((s16 >> 2) % C::VG);
    const int v_q = 2 * g2 + ((s16 & 3) >> 1);
    const int v_in = (s16 & 1) * 4;

    // Tiles [full_start, full_end) lie inside the split, below every row's
    // last visible key and (with a window) at or above every row's first.
    const int64_t full_last = min((int64_t)ke - kBN, vis_top - (kBN - 1));  // last unmasked tile start
    const int full_end = full_last < ks ? ks : (int)(ks + ((full_last - ks) / kBN + 1) * kBN);
    const int64_t lo_last = vis_first(sq, win, min(r0 + kBM, sq.sq) - 1);  // the block's largest first key
    const int full_start = lo_last <= ks ? ks : (int)min((int64_t)ke, ks + ceil_div64(lo_last - ks, kBN) * kBN);

    // GEMM0: S^T[key][query] for the two 32-key blocks of tile Kb; K
    // fragments for step t + 1 are read while step t multiplies.
    auto gemm0 = [&](const uint16_t* Kb, f32x16(&sacc)[2], auto&& side) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
        // per-lane bases: chunk (2t + half) ^ f(row) with f < 16 (or < 8)
        // changes only the low 4 (3) bits, so t / 8 (t / 4) steps add whole
        // 256-byte (128-byte) blocks
        constexpr int kSpan = (C::KCH % 16 == 0) ? 8 : 4;  // steps per repeating block
        uint32_t kaddr[kSpan];
#pragma unroll
        for (int m = 0; m < kSpan; ++m) kaddr[m] = lds_addr(Kb + k_rd + (k_swz<C::KCH>(col, 2 * m + half) * 8));
        i32x4_t f[2][2];
        auto rd = [&](i32x4_t(&x)[2], auto t_c) {
            constexpr int t = decltype(t_c)::value;
            x[0] = k_read<(t / kSpan) * kSpan * 32>(kaddr[t % kSpan]);
            x[1] = k_read<(t / kSpan) * kSpan * 32 + 32 * DQK * 2>(kaddr[t % kSpan]);
        };
        auto mm = [&](i32x4_t(&x)[2], auto t_c) {
            constexpr int t = decltype(t_c)::value;
            sacc[0] = E::mfma(__builtin_bit_cast(bf16x8, x[0]), qf[t], sacc[0]);
            sacc[1] = E::mfma(__builtin_bit_cast(bf16x8, x[1]), qf[t], sacc[1]);
        };
        rd(f[0], std::integral_constant<int, 0>{});
        [&]<int... Step>(std::integer_sequence<int, Step...>) {
            (([&] {
                constexpr int t = Step;
                if constexpr (t + 1 < DQK / 16) {
                    rd(f[(t + 1) & 1], std::integral_constant<int, t + 1>{});
                    k_wait<2>(f[t & 1][0], f[t & 1][1]);
                } else {
                    k_wait<0>(f[t & 1][0], f[t & 1][1]);
                }
                mm(f[t & 1], std::integral_constant<int, t>{});
                side(std::integral_constant<int, t>{});
            }()),
             ...);
        }(std::make_integer_sequence<int, DQK / 16>{});
    };
    auto no_side = [](auto) {};

    // Masking of a tile from full_end on.  Accumulator element j of a lane
    // holds key kt + 32*kb + 8*(j/4) + 4*half + (j%4) for query column `col`.
    auto mask_tile = [&](int kt, f32x16(&sacc)[2]) {
        const int lim = min(ke - 1, vis_q) - kt - half * 4;  // last visible key, relative
        const int first = lo_q - kt - half * 4;               // first visible key, relative
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rel = kb * 32 + (j >> 2) * 8 + (j & 3);
                if (rel > lim || rel < first) sacc[kb][j] = -INFINITY;
            }
    };
    // Reference-max update from a tile's complete scores.  The reference max
    // moves only when it grew by more than the threshold for some row of the
    // wave; the output accumulated so far is rescaled before this tile's
    // weights are added.
    auto max_update = [&](const f32x16(&sacc)[2]) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
        mx = fmaxf(mx, other_half(mx));
        const float m_cand = fmaxf(m_i, mx);
        const bool grow = (m_cand - m_i) * cl2 > kRescaleThreshold;  // false while nothing is visible
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_cand : m_i;
            const float alpha = grow ? __builtin_amdgcn_exp2f((m_i - m_new) * cl2) : 1.0f;
            l_i *= alpha;
#pragma unroll
            for (int c = 0; c < DV / 32; ++c)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[c][j] *= alpha;
            m_i = m_new;
        }
    };
    // First tile and masked tiles take the reference-max update before their
    // weights.  Later unmasked tiles skip it: every row already has a finite
    // reference (the first tile was unmasked), their weights are computed
    // against it, and only if some row's weight sum leaves [0, 2^64] (a score
    // more than 64 / (scale log2 e) above the reference, or inf) the update
    // is taken and the weights recomputed.  Below that bound weights, sums
    // and the output accumulator stay far inside f32 / bf16 range, and the
    // result O = sum p V / sum p does not depend on the reference.
    auto prepare = [&](int kt, f32x16(&sacc)[2]) -> bool {
        const bool masked = kt >= full_end || kt < full_start;
        if (masked) {
            asm volatile("");  // a real branch: most tiles need no mask
            mask_tile(kt, sacc);
        }
        // the first unmasked tile too: rows may have seen nothing before it
        if (masked || kt == ks || kt == full_start) {
            max_update(sacc);
            return true;
        }
        return false;
    };

    // Weights of a tile (rounded to bf16, in GEMM1's B-operand layout) and
    // their row sum rs, which adds the rounded values so O is their exact
    // weighted mean.
    auto weights = [&](const f32x16(&sacc)[2], bf16x8(&pf)[2][2], float& rs) {
        const float mc = (m_i == -INFINITY) ? 0.f : m_i * cl2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                pf[kb][j >> 3][j & 7] = (T)__builtin_amdgcn_exp2f(fmaf(sacc[kb][j], cl2, -mc));
        const bf16x2 ones = {(T)1.0f, (T)1.0f};
        rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 8; j += 2)
                    rs = E::dot2(bf16x2{pf[kb][u][j], pf[kb][u][j + 1]}, ones, rs);
    };
    // Range check of weights computed without the max update (see prepare).
    auto check_weights = [&](bool max_taken, const f32x16(&sacc)[2], bf16x8(&pf)[2][2], float& rs) {
        if (!max_taken && __builtin_amdgcn_ballot_w64(!(rs <= 0x1p64f))) {
            max_update(sacc);
            weights(sacc, pf, rs);
        }
        l_i += rs;
    };
    // GEMM1: O^T[value][query] += V^T[value][key] P^T[key][query].
    // B element j' of step (kb, u) is key 32kb + 16u + 8(j'/4) + 4half + j'%4;
    // the two transpose reads give this lane's value column at keys
    // 32kb + 16u + 4half + 0..3 and + 8..11.  Step n + 1's reads are issued
    // before step n's MFMAs.
    auto gemm1 = [&](const uint16_t* Vb, const bf16x8(&pf)[2][2]) {
        static_assert(DV == 128 || DV == 64, "GEMM1 read schedule covers D_v of 64 and 128");
        uint32_t vaddr[DV / 32];
#pragma unroll
        for (int c = 0; c < DV / 32; ++c) vaddr[c] = lds_addr(Vb + v_key * DV + (((4 * c + v_q) ^ v_sw) * 8) + v_in);
        s16x4 xa[8], xb[8];
        auto issue_step = [&](s16x4(&x)[8], auto kb_c, auto u_c) {
            constexpr int kb = decltype(kb_c)::value, u = decltype(u_c)::value;
            constexpr int o0 = (kb * 32 + u * 16) * DV * 2, o1 = o0 + 8 * DV * 2;
#pragma unroll
            for (int c = 0; c < DV / 32; ++c) {
                x[2 * c] = tr_read<o0>(vaddr[c]);
                x[2 * c + 1] = tr_read<o1>(vaddr[c]);
            }
#pragma unroll
            for (int c = DV / 32; c < 4; ++c) x[2 * c] = x[2 * c + 1] = s16x4{0, 0, 0, 0};
        };
        auto mma_step = [&](s16x4(&x)[8], const bf16x8& p) {
#pragma unroll
            for (int c = 0; c < DV / 32; ++c) {
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x[2 * c], x[2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7));
                o[c] = E::mfma(va, p, o[c]);
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        constexpr int kReads = DV / 16;  // reads per step
        issue_step(xa, I0{}, I0{});
        issue_step(xb, I0{}, I1{});
        tr_wait<kReads>(xa);
        mma_step(xa, pf[0][0]);
        issue_step(xa, I1{}, I0{});
        tr_wait<kReads>(xb);
        mma_step(xb, pf[0][1]);
        issue_step(xb, I1{}, I1{});
        tr_wait<kReads>(xa);
        mma_step(xa, pf[1][0]);
        tr_wait<0>(xb);
        mma_step(xb, pf[1][1]);
    };

    // Pipeline.  Iteration i: the weights of tile i from its scores;
    // GEMM0(i+1) from K slot (i+1)%2 into the same score registers, with the
    // DMA of K(i+2) into K slot i%2 and of V(i+1) into the V slot after tile
    // i's spread over its steps; GEMM1(i); then tile i+1's mask / max update.
    // Every wave passes one barrier per iteration: the first group after
    // GEMM1(i), the second before it.  The loads a barrier covers were issued
    // before it by every wave (in GEMM0), and a slot is refilled only after
    // the barrier that follows its last reader: K(i) is last read by GEMM0(i)
    // in iteration i - 1; V(i - 2) by the second group's GEMM1(i - 2), which
    // runs between the barriers of iterations i - 2 and i - 1.
    const int ntiles = ks < ke ? (ke - ks + kBN - 1) / kBN : 0;
    if (ntiles > 0) {
        issue_k(ks, 0);
        issue_v(ks, 0);
        sync_tiles();
        issue_k(ks + kBN, 1);
        f32x16 sc[2];
        bool sc_max = true;  // whether tile sc took the reference-max update
        if (wave_active) {
            gemm0(Ks0, sc, no_side);
            sc_max = prepare(ks, sc);
        }
        sync_tiles();
        int vs_cur = 0, vs_next = 1;  // V slots of tiles i and i + 1
        for (int i = 0; i + 1 < ntiles; ++i) {
            const int kt = ks + i * kBN;
            // K(i + 2) and V(i + 1), one load per GEMM0 step: issued as one
            // burst, the loads of a CU's 8 waves queue in its memory pipeline
            // and hold each wave before its first MFMA.
            const __amdgpu_buffer_rsrc_t rk = rsrc_k(kt + 2 * kBN);
            const __amdgpu_buffer_rsrc_t rv = rsrc_v(kt + kBN);
            if (wave_active) {
                bf16x8 pf[2][2];
                float rs = 0.f;
                weights(sc, pf, rs);
                check_weights(sc_max, sc, pf, rs);
                gemm0(Ks0 + ((i + 1) & 1) * C::K_ELEMS, sc, [&](auto step_c) {
                    issue_one(rk, rv, i & 1, vs_next, step_c);
                });
                if (late) sync_tiles();
                gemm1(Vs0 + vs_cur * C::V_ELEMS, pf);
                sc_max = prepare(kt + kBN, sc);
                if (!late) sync_tiles();
            } else {
                [&]<int... L>(std::integer_sequence<int, L...>) {
                    (issue_one(rk, rv, i & 1, vs_next, std::integral_constant<int, L>{}), ...);
                }(std::make_integer_sequence<int, C::K_LOADS + C::V_LOADS>{});
                sync_tiles();
            }
            vs_cur = vs_next;
            vs_next = vs_next + 1 == C::V_SLOTS ? 0 : vs_next + 1;
        }
        if (wave_active) {
            bf16x8 pf[2][2];
            float rs;
            weights(sc, pf, rs);
            check_weights(sc_max, sc, pf, rs);
            gemm1(Vs0 + vs_cur * C::V_ELEMS, pf);
        }
    }

    if (!row_ok) return;
    const int64_t prow = sq.row0 + qrow;
    if (prow >= a.rows) return;
    const float l_tot = l_i + other_half(l_i);
    const bool empty = (m_i == -INFINITY);  // no visible key in this split
    const float inv = empty ? 0.f : 1.0f / l_tot;
    float* op;
    float* lp;
    if (piece < 0) {
        const int64_t slot = ((int64_t)it.head * a.seqs.s_max + it.split) * a.rows + prow;
        if (!in_bounds(a.check, kSitePartialSlot, slot, (int64_t)a.heads * a.seqs.s_max * a.rows)) return;
        op = a.o_part + slot * DV;
        lp = a.lse_part + slot;
    } else {
        const int64_t slot = ((int64_t)tail_i * a.pieces + piece) * kBM + wave * 32 + col;
        if (!in_bounds(a.check, kSitePieceSlot, slot, (int64_t)(a.n_work - a.n_main) * a.pieces * kBM)) return;
        op = a.piece_o + slot * DV;
        lp = a.piece_l + slot;
    }
    op += half * 4;
#pragma unroll
    for (int c = 0; c < DV / 32; ++c)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            *reinterpret_cast<float4*>(op + c * 32 + jb * 8) =
                make_float4(o[c][jb * 4] * inv, o[c][jb * 4 + 1] * inv, o[c][jb * 4 + 2] * inv, o[c][jb * 4 + 3] * inv);
    if (half == 0) *lp = empty ? -INFINITY : m_i * a.scale + logf(l_tot);
}

template <typename T, int DQK, int DV, int G>
hipError_t launch(const PartialArgs& a, hipStream_t stream) {
    const uint32_t n_tail = a.n_work - a.n_main;
    const uint32_t grid = a.n_main + n_tail * (uint32_t)a.pieces;
    hipLaunchKernelGGL((partial_bf16_kernel<T, DQK, DV, G>), dim3(grid), dim3(G * kGroupThreads), 0, stream, a);
    if (n_tail > 0) {
        launch_merge_pieces<G * kGroupRows, DV>(a, n_tail, stream);
    }
    return hipGetLastError();
}

// Resident workgroups per CU (the same on every gfx950 device; cached).
template <typename T, int DQK, int DV, int G>
int blocks_per_cu() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, partial_bf16_kernel<T, DQK, DV, G>, G * kGroupThreads, 0) !=
        hipSuccess)
        return 0;
    cached.store(n, std::memory_order_relaxed);
    return n;
}

template <typename T, int G>
PartialKernel find_partial_16(int d_qk, int d_v) {
    constexpr int bm = G * kGroupRows;
    if (d_qk == 64 && d_v == 64) return {launch<T, 64, 64, G>, bm, blocks_per_cu<T, 64, 64, G>, true};
    if (d_qk == 128 && d_v == 128) return {launch<T, 128, 128, G>, bm, blocks_per_cu<T, 128, 128, G>, true};
    if (d_qk == 192 && d_v == 128) return {launch<T, 192, 128, G>, bm, blocks_per_cu<T, 192, 128, G>, true};
    return {nullptr, 0, nullptr, false};
}

}  // namespace

PartialKernel find_partial_bf16(int d_qk, int d_v, bool two_groups) {
    return two_groups ? find_partial_16<__bf16, 2>(d_qk, d_v) : find_partial_16<__bf16, 1>(d_qk, d_v);
}
PartialKernel find_partial_f16(int d_qk, int d_v, bool two_groups) {
    return two_groups ? find_partial_16<_Float16, 2>(d_qk, d_v) : find_partial_16<_Float16, 1>(d_qk, d_v);
}

}  // namespace sk
