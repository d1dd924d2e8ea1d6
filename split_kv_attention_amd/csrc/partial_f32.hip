// Split-KV partial attention, f32 storage and f32 arithmetic (VALU).
//
// Computes, per (sequence, head, split, query block), the partial output O_s
// and log-sum-exp L_s of softmax attention over the split's keys, the method
// of the rocmlirTriton page "Recombine fully masked split-KV attention
// partials on the host" (Summary; the block partition in "Per-row valid-split
// counts").  gfx950 has no reduced-precision f32 matrix path that would keep
// an f32 problem at f32 accuracy, so this variant uses FMA on the vector ALUs:
// SUB lanes per query row (four, at least four values each), each holding
// a slice of the row's Q and of its output, with key/value tiles staged
// through LDS.  A score is SUB partial dot products summed across the row's
// lanes.  It serves small f32 problems; bf16 goes to MFMA.
#include "sk_common.hpp"

namespace sk {

namespace {

constexpr int kF32Rows = 64;  // query rows per workgroup

// Lanes per query row for head dims DQK, DV: four, or fewer where a lane
// would not get a whole float4 slice.  (On the tiny 64-dim workload four
// lanes per row took the kernel from 43 to 23 us, sixteen to 27 us; DPP row
// sums instead of LDS shuffles then to 21 us.)
template <int DQK, int DV>
constexpr int f32_sub() {
    constexpr int d = DQK < DV ? DQK : DV;
    return d / 4 < 4 ? d / 4 : 4;
}

// Sum over the SUB consecutive lanes of a row (SUB = 2 or 4: a half quad
// or a quad), every lane receiving it: DPP quad permutes, which exchange
// within the row's own lanes without a trip through LDS.
template <int SUB>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(SUB == 1 || SUB == 2 || SUB == 4, "a row's lanes sit in one quad");
    if constexpr (SUB >= 2)  // quad_perm [1, 0, 3, 2]: lane ^ 1
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
    if constexpr (SUB == 4)  // quad_perm [2, 3, 0, 1]: lane ^ 2
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
    return x;
}

template <int DQK, int DV, int BN>
__global__ __launch_bounds__((kF32Rows * f32_sub<DQK, DV>())) void partial_f32_kernel(PartialArgs a) {
    constexpr int SUB = f32_sub<DQK, DV>(), NT = kF32Rows * SUB;
    constexpr int QS = DQK / SUB, VS = DV / SUB;  // this lane's slice of a Q / output row
    static_assert(QS % 4 == 0 && VS % 4 == 0, "whole float4 slices");
    __shared__ float4 Ks[BN * DQK / 4];
    __shared__ float4 Vs[BN * DV / 4];

    const WorkItem it = decode_work(a, blockIdx.x);
    if (!in_bounds(a.check, kSiteWorkItem, it.batch, a.batch) || !in_bounds(a.check, kSiteWorkItem, it.head, a.heads) ||
        !in_bounds(a.check, kSiteWorkItem, it.split, a.seqs.s_max))
        return;
    const Seq sq = load_seq(a.seqs, it.batch);
    if (it.split >= sq.splits) return;
    const int r0 = it.tile * kF32Rows;
    if (r0 >= sq.sq) return;
    const int mask = a.seqs.mask;

    // Key range of this split for this block (the count formula at the
    // block's last row).  A split with no key for the whole block exits
    // without writing: the combine merges only the block's populated splits.
    int ks, ke;
    block_split_range(sq, mask, a.seqs.n_per_block, min(r0 + kF32Rows, sq.sq) - 1, it.split, ks, ke);
    if (ks >= ke) return;
    if (!in_bounds(a.check, kSiteKeys, (sq.krow0 >= 0 ? sq.krow0 : 0) + ke - 1,
                   sq.krow0 >= 0 ? total_keys(a.seqs, a.batch) : (int64_t)a.seqs.max_sk))
        return;
    // Sliding window: tiles below the first row's first visible key hold
    // nothing any row sees.
    const int64_t win = a.seqs.window_left;
    {
        const int64_t lo_first = vis_first(sq, win, r0);
        if (lo_first > ks) ks = (int)min((int64_t)ke, ks + (lo_first - ks) / BN * BN);
    }

    const int tid = threadIdx.x;
    const int sub = tid % SUB;
    const int qrow = r0 + tid / SUB;
    const bool row_ok = qrow < sq.sq && sq.row0 + qrow < a.rows;  // (rows: cu_seqlens past total_q)
    const bool q_ok = row_ok && in_bounds(a.check, kSiteQRow,
                                          a.seqs.cu_q ? sq.row0 + qrow : (int64_t)it.batch * a.seqs.max_sq + qrow,
                                          a.rows);
    const int64_t vis = vis_last(sq, mask, qrow);
    const int64_t lo = vis_first(sq, win, qrow);

    const float* qp = reinterpret_cast<const float*>(a.q) +
                      (a.seqs.cu_q ? (sq.row0 + qrow) * a.q_row : (int64_t)it.batch * a.q_batch + (int64_t)qrow * a.q_row) +
                      (int64_t)it.head * a.q_head + sub * QS;
    const float* kp = reinterpret_cast<const float*>(a.k) +
                      (sq.krow0 >= 0 ? sq.krow0 * a.k_row : (int64_t)it.batch * a.k_batch) + (int64_t)it.head * a.k_head;
    const float* vp = reinterpret_cast<const float*>(a.v) +
                      (sq.krow0 >= 0 ? sq.krow0 * a.v_row : (int64_t)it.batch * a.v_batch) + (int64_t)it.head * a.v_head;

    float qv[QS];
#pragma unroll
    for (int d = 0; d < QS; d += 4) {
        float4 x = q_ok ? *reinterpret_cast<const float4*>(qp + d) : make_float4(0.f, 0.f, 0.f, 0.f);
        qv[d] = x.x;
        qv[d + 1] = x.y;
        qv[d + 2] = x.z;
        qv[d + 3] = x.w;
    }
    float o[VS];
#pragma unroll
    for (int d = 0; d < VS; ++d) o[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c = a.scale_log2;

    for (int kt = ks; kt < ke; kt += BN) {
        __syncthreads();
        for (int i = tid; i < BN * DQK / 4; i += NT) {
            const int kr = i / (DQK / 4), col = i % (DQK / 4);
            const int key = kt + kr;
            Ks[i] = key < ke ? *reinterpret_cast<const float4*>(kp + (int64_t)key * a.k_row + col * 4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int i = tid; i < BN * DV / 4; i += NT) {
            const int kr = i / (DV / 4), col = i % (DV / 4);
            const int key = kt + kr;
            Vs[i] = key < ke ? *reinterpret_cast<const float4*>(vp + (int64_t)key * a.v_row + col * 4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();

        float sc[BN];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < QS / 4; ++d) {
                const float4 kk = Ks[j * (DQK / 4) + sub * (QS / 4) + d];
                dot = fmaf(qv[4 * d], kk.x, dot);
                dot = fmaf(qv[4 * d + 1], kk.y, dot);
                dot = fmaf(qv[4 * d + 2], kk.z, dot);
                dot = fmaf(qv[4 * d + 3], kk.w, dot);
            }
            dot = row_sum<SUB>(dot);
            const int key = kt + j;
            sc[j] = (key < ke && key <= vis && key >= lo) ? dot : -INFINITY;
            mx = fmaxf(mx, sc[j]);
        }
        // Online softmax in base 2; a row with nothing visible yet keeps
        // m = -inf and zero weights (no -inf - -inf).  The row's lanes hold
        // the same scores and take the same steps.
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f((m - m_use) * c);
        const float mc = m_use * c;
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            sc[j] = exp2f(fmaf(sc[j], c, -mc));
            rs += sc[j];
        }
        l = fmaf(l, alpha, rs);
        m = m_new;
#pragma unroll
        for (int d = 0; d < VS / 4; ++d) {
            float4 acc = make_float4(o[4 * d] * alpha, o[4 * d + 1] * alpha, o[4 * d + 2] * alpha, o[4 * d + 3] * alpha);
#pragma unroll
            for (int j = 0; j < BN; ++j) {
                const float4 vv = Vs[j * (DV / 4) + sub * (VS / 4) + d];
                acc.x = fmaf(sc[j], vv.x, acc.x);
                acc.y = fmaf(sc[j], vv.y, acc.y);
                acc.z = fmaf(sc[j], vv.z, acc.z);
                acc.w = fmaf(sc[j], vv.w, acc.w);
            }
            o[4 * d] = acc.x;
            o[4 * d + 1] = acc.y;
            o[4 * d + 2] = acc.z;
            o[4 * d + 3] = acc.w;
        }
    }

    if (!row_ok) return;
    const int64_t prow = sq.row0 + qrow;
    if (prow >= a.rows) return;
    // Empty split or fully masked row: O_s = 0, L_s = -inf.
    const bool empty = (m == -INFINITY);
    const float inv = empty ? 0.f : 1.0f / l;
    const int64_t slot = ((int64_t)it.head * a.seqs.s_max + it.split) * a.rows + prow;
    if (!in_bounds(a.check, kSitePartialSlot, slot, (int64_t)a.heads * a.seqs.s_max * a.rows)) return;
    float* op = a.o_part + slot * DV + sub * VS;
#pragma unroll
    for (int d = 0; d < VS; d += 4)
        *reinterpret_cast<float4*>(op + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
    if (sub == 0) a.lse_part[slot] = empty ? -INFINITY : m * a.scale + logf(l);
}

template <int DQK, int DV, int BN>
hipError_t launch(const PartialArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((partial_f32_kernel<DQK, DV, BN>), dim3(a.n_work), dim3(kF32Rows * f32_sub<DQK, DV>()), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

PartialKernel find_partial_f32(int d_qk, int d_v) {
    if (d_qk == 16 && d_v == 16) return {launch<16, 16, 32>, kF32Rows, nullptr, false};
    if (d_qk == 32 && d_v == 32) return {launch<32, 32, 32>, kF32Rows, nullptr, false};
    if (d_qk == 64 && d_v == 64) return {launch<64, 64, 32>, kF32Rows, nullptr, false};
    if (d_qk == 128 && d_v == 128) return {launch<128, 128, 16>, kF32Rows, nullptr, false};
    return {nullptr, 0, nullptr, false};
}

}  // namespace sk
