// Split-KV partial attention, bf16 storage, bf16 MFMA with f32 accumulation.
//
// Per (sequence, head, split, block of 128 query rows) the kernel computes the
// partial output O_s and log-sum-exp L_s over the split's keys (rocmlirTriton
// page "Recombine fully masked split-KV attention partials on the host":
// Summary for the partials and the empty-split convention, "Per-row
// valid-split counts" for the block's key partition).  The workload it is
// tuned for is the long-context packed-varlen prefill of the aiter page
// "[ASM][HIP][JIT][gfx942] Optimize long-context FMHA with split-KV"
// (D_qk = 192, D_v = 128), re-designed for gfx950:
//
//  * 4 waves, 32 query rows each.  GEMM0 is computed transposed, S^T = K Q^T,
//    with v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and Q^T
//    (kept in registers for the whole key loop) the B operand.  The
//    accumulator then gives every lane ONE query column and 16 keys, so the
//    row max / row sum are in-lane reductions plus one exchange between the
//    two half-waves.
//  * The same accumulator layout is exactly the B operand layout (key-major,
//    query column per lane) GEMM1 needs for O^T = V^T P^T, so P never leaves
//    registers: it is rounded to bf16 in place.  V is the A operand and is
//    staged transposed (V^T, key-contiguous) in LDS.
//  * Online softmax in base 2 with the scale folded into one FMA per score;
//    a row with no visible key so far keeps m = -inf and zero weights.
//  * K rows are padded by 16 bytes and V^T rows by 8 bytes in LDS so that the
//    128-bit and 64-bit operand reads are bank-conflict free.
//  * Next key tile is prefetched into registers while the current one is
//    multiplied; work items are remapped so each XCD streams one (head, split)
//    key range through its own L2.
#include "sk_common.hpp"

namespace sk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;    // query rows per workgroup
constexpr int kBN = 64;     // keys per tile
constexpr int kThreads = 256;

template <int DQK, int DV>
struct Cfg {
    static constexpr int KS = DQK + 8;                  // K row stride in LDS (bf16)
    static constexpr int VS = kBN + 4;                  // V^T row stride in LDS (bf16)
    static constexpr int K_CHUNKS = kBN * DQK / 8;      // 16-byte chunks of a K tile
    static constexpr int V_CHUNKS = (kBN / 4) * (DV / 8);  // (4 keys x 8 values) chunks of a V tile
    static constexpr int K_PER_T = (K_CHUNKS + kThreads - 1) / kThreads;
    static_assert(V_CHUNKS <= kThreads, "one V chunk per thread at most");
    static constexpr int LDS_ELEMS = kBN * KS + DV * VS;
    static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims must be multiples of 16 (QK) and 32 (V)");
};

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Growth of the running max (in log2 units) tolerated before the output
// accumulator is rescaled.  Using a stale max m' <= m only changes the common
// factor 2^(m - m') of every weight and of their sum, so O = sum p V / sum p
// and LSE = m' + log(sum p) are unchanged; weights stay below 2^8.
constexpr float kRescaleThreshold = 8.0f;

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void partial_bf16_kernel(PartialArgs a) {
    using C = Cfg<DQK, DV>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
    uint16_t* Ks = smem;                 // [kBN][KS]
    uint16_t* Vt = smem + kBN * C::KS;   // [DV][VS]

    const WorkItem it = decode_work(a);
    const Seq sq = load_seq(a.seqs, it.batch);
    if (it.split >= sq.splits) return;
    const int r0 = it.tile * kBM;
    if (r0 >= sq.sq) return;
    const int mask = a.seqs.mask;

    // The block's key range for this split, from its last row.
    const int last_row = min(r0 + kBM, sq.sq) - 1;
    const int64_t rl = row_last(sq, mask, last_row);
    const int64_t kps = keys_per_split(rl, a.seqs.n_per_block, sq.splits);
    // Split s covers [s*kps, (s+1)*kps) of the keys 0..rowLast.  Keys past
    // lastValid are never visible, so an empty key range (lastValid = -1)
    // gives an empty loop and no key is loaded.
    const int64_t kend = min(rl + 1, sq.lv + 1);
    const int ks = (int)min((int64_t)it.split * kps, kend);
    const int ke = (int)min((int64_t)(it.split + 1) * kps, kend);
    // Smallest visibility limit in the block (its first row): tiles entirely
    // below it and inside the split need no per-element mask.
    const int64_t vis_first = vis_last(sq, mask, r0);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 31;   // query column of this lane (and A-row for loads)
    const int half = lane >> 5;  // which 8-wide k slice / which 4 accumulator rows
    const int qrow = r0 + wave * 32 + col;
    const bool row_ok = qrow < sq.sq;
    const bool wave_active = (r0 + wave * 32) < sq.sq;
    // Visibility limit of this lane's row, clamped into int range (keys are int).
    const int vis_q = (int)max(min(vis_last(sq, mask, qrow), (int64_t)0x7fffffff), (int64_t)-1);

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
            uint4 x = row_ok ? *reinterpret_cast<const uint4*>(qp + t * 16) : make_uint4(0, 0, 0, 0);
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

    // Per-thread load assignment, fixed for every tile: K chunk i is row
    // kr[i], 8-element column kc[i]; V chunk is 4 keys (vq) x 8 values (vd).
    const int k_row32 = (int)a.k_row, v_row32 = (int)a.v_row;
    int kr[C::K_PER_T], kc[C::K_PER_T];
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
        const int c = min(tid + i * kThreads, C::K_CHUNKS - 1);
        kr[i] = c / (DQK / 8);
        kc[i] = (c % (DQK / 8)) * 8;
    }
    const int vc = min(tid, C::V_CHUNKS - 1);
    const int vq = vc % (kBN / 4), vd = vc / (kBN / 4);
    const bool v_loader = tid < C::V_CHUNKS;

    // Register staging of the next tile.  Rows past the split's end load the
    // split's last key instead (valid memory, finite values): their scores are
    // masked to -inf and their weights are 0.
    uint4 kreg[C::K_PER_T];
    uint4 vreg[4];
    auto gload = [&](int kt) {
        const uint16_t* kt_ptr = kbase + (int64_t)kt * a.k_row;
        const uint16_t* vt_ptr = vbase + (int64_t)kt * a.v_row;
        const int last = ke - 1 - kt;  // last loadable row of this tile
        if (last >= kBN - 1) {
#pragma unroll
            for (int i = 0; i < C::K_PER_T; ++i)
                kreg[i] = *reinterpret_cast<const uint4*>(kt_ptr + kr[i] * k_row32 + kc[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vreg[j] = *reinterpret_cast<const uint4*>(vt_ptr + (4 * vq + j) * v_row32 + vd * 8);
        } else {
#pragma unroll
            for (int i = 0; i < C::K_PER_T; ++i)
                kreg[i] = *reinterpret_cast<const uint4*>(kt_ptr + min(kr[i], last) * k_row32 + kc[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vreg[j] = *reinterpret_cast<const uint4*>(vt_ptr + min(4 * vq + j, last) * v_row32 + vd * 8);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i)
            if (C::K_CHUNKS % kThreads == 0 || tid + i * kThreads < C::K_CHUNKS)
                *reinterpret_cast<uint4*>(Ks + kr[i] * C::KS + kc[i]) = kreg[i];
        // V^T: four keys of one value column become one 8-byte row segment.
        if (v_loader) {
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
            const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
            const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
            const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint2 lo, hi;
                lo.x = pack_lo(w0[e], w1[e]);
                lo.y = pack_lo(w2[e], w3[e]);
                hi.x = pack_hi(w0[e], w1[e]);
                hi.y = pack_hi(w2[e], w3[e]);
                *reinterpret_cast<uint2*>(Vt + (vd * 8 + 2 * e) * C::VS + 4 * vq) = lo;
                *reinterpret_cast<uint2*>(Vt + (vd * 8 + 2 * e + 1) * C::VS + 4 * vq) = hi;
            }
        }
    };

    if (ks < ke) gload(ks);
    for (int kt = ks; kt < ke; kt += kBN) {
        __syncthreads();  // every wave is done with the previous tile
        lstore();
        __syncthreads();
        if (kt + kBN < ke) gload(kt + kBN);

        if (wave_active) {
            // GEMM0: S^T[key][query] for two 32-key blocks.
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
#pragma unroll
            for (int t = 0; t < DQK / 16; ++t) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + col) * C::KS + t * 16 + half * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sacc[kb], 0, 0, 0);
                }
            }
            // Accumulator element j of this lane holds key
            //   kt + 32*kb + 8*(j/4) + 4*half + (j%4)   for query column `col`.
            const bool full = (kt + kBN <= ke) && ((int64_t)kt + kBN - 1 <= vis_first);
            if (!full) {
                const int lim = min(ke - 1, vis_q) - kt - half * 4;  // last visible key, relative
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (kb * 32 + (j >> 2) * 8 + (j & 3) > lim) sacc[kb][j] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // Move the reference max only when it grew by more than the
            // threshold for some row of the wave (rare after the first tiles).
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
            const float mc = (m_i == -INFINITY) ? 0.f : m_i * cl2;

            // P (rounded to bf16) in the B-operand layout of GEMM1; the row
            // sum adds the rounded weights, so O is their exact weighted mean.
            bf16x8 pf[2][2];
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    bf16x2 p2;
                    p2[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][j], cl2, -mc));
                    p2[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][j + 1], cl2, -mc));
                    pf[kb][j >> 3][j & 7] = p2[0];
                    pf[kb][j >> 3][(j & 7) + 1] = p2[1];
                    l_i = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_i, false);
                }

            // GEMM1: O^T[value][query] += V^T[value][key] P^T[key][query].
            // B element j' of step (kb, u) is key 32kb + 16u + 8(j'/4) + 4half + j'%4,
            // so the A operand takes two 4-key runs of one V^T row.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int kofs = kb * 32 + u * 16 + half * 4;
#pragma unroll
                    for (int c = 0; c < DV / 32; ++c) {
                        const uint16_t* vr = Vt + (c * 32 + col) * C::VS + kofs;
                        uint4 va;
                        const uint2 x0 = *reinterpret_cast<const uint2*>(vr);
                        const uint2 x1 = *reinterpret_cast<const uint2*>(vr + 8);
                        va.x = x0.x;
                        va.y = x0.y;
                        va.z = x1.x;
                        va.w = x1.y;
                        o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pf[kb][u], o[c], 0, 0, 0);
                    }
                }
        }
    }

    if (!row_ok) return;
    const int64_t prow = sq.row0 + qrow;
    if (prow >= a.rows) return;
    const float l_tot = l_i + __shfl_xor(l_i, 32);
    const bool empty = (m_i == -INFINITY);  // no visible key in this split
    const float inv = empty ? 0.f : 1.0f / l_tot;
    const int64_t slot = ((int64_t)it.head * a.seqs.s_max + it.split) * a.rows + prow;
    float* op = a.o_part + slot * DV + half * 4;
#pragma unroll
    for (int c = 0; c < DV / 32; ++c)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            *reinterpret_cast<float4*>(op + c * 32 + jb * 8) =
                make_float4(o[c][jb * 4] * inv, o[c][jb * 4 + 1] * inv, o[c][jb * 4 + 2] * inv, o[c][jb * 4 + 3] * inv);
    if (half == 0) a.lse_part[slot] = empty ? -INFINITY : m_i * a.scale + logf(l_tot);
}

template <int DQK, int DV>
hipError_t launch(const PartialArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((partial_bf16_kernel<DQK, DV>), dim3(a.n_work), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

PartialKernel find_partial_bf16(int d_qk, int d_v) {
    if (d_qk == 64 && d_v == 64) return {launch<64, 64>, kBM};
    if (d_qk == 128 && d_v == 128) return {launch<128, 128>, kBM};
    if (d_qk == 192 && d_v == 128) return {launch<192, 128>, kBM};
    return {nullptr, 0};
}

}  // namespace sk
