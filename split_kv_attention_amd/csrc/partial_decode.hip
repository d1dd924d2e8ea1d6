// Split-KV partial attention for decode: one query row per sequence, bf16 or
// f16 storage, f32 arithmetic on the vector ALUs.
//
// The partial step of the rocmlirTriton page "Recombine fully masked split-KV
// attention partials on the host" (Summary; the block partition of "Per-row
// valid-split counts", whose block here is the sequence's single row), for
// problems whose sequences hold at most one query row, as in batched decode.
// There the work is a stream of K and V with about one FLOP per byte: an MFMA
// tile of 128 query rows would carry one useful row and stage every key
// through LDS.  Instead a workgroup of four waves takes one (sequence, head,
// split) and reads its keys straight into registers:
//   * a key's D values are spread over D / 8 consecutive lanes (16 bytes
//     each), so one load instruction covers 64 / (D / 8) whole key rows;
//   * each lane multiplies its 8 values by its slice of q and a DPP
//     butterfly over the key's lanes sums the score;
//   * every group of lanes keeps its own running max, weight sum and output
//     slice over the keys it loaded (an online softmax in base 2), and the
//     4 * 64 / (D / 8) group states are merged through LDS at the end.
// Every key of the split's visible range is loaded once; out-of-range lanes
// load the last visible key and take weight 0.
#include <atomic>

#include "sk_common.hpp"

namespace sk {

namespace {

constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecUnroll = 8;     // keys per lane group per step
constexpr float kLn2 = 0.69314718055994531f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two 16-bit values packed in a dword -> two floats (exact).
template <typename T>
__device__ __forceinline__ void unpack2(uint32_t x, float& lo, float& hi);
template <>
__device__ __forceinline__ void unpack2<__bf16>(uint32_t x, float& lo, float& hi) {
    lo = __uint_as_float(x << 16);
    hi = __uint_as_float(x & 0xffff0000u);
}
template <>
__device__ __forceinline__ void unpack2<_Float16>(uint32_t x, float& lo, float& hi) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 v = __builtin_bit_cast(h2, x);
    lo = (float)v[0];
    hi = (float)v[1];
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each group of L consecutive lanes (L = 8 or 16), every lane of
// the group receiving it: exchanges with lane ^ 1 and lane ^ 2 (quad
// permutes), then with the mirrored lane of the other quad in each 8-lane
// half-row, then (L = 16) of the other half in the 16-lane row.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L == 8 || L == 16, "lanes per key");
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (L == 16) x += dpp<0x140>(x);  // row_mirror
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void partial_decode_kernel(PartialArgs a) {
    constexpr int LPK = D / 8;             // lanes per key
    constexpr int G = 64 / LPK;            // keys per load instruction of a wave
    constexpr int CHUNK = G * kDecUnroll;  // keys per wave step
    constexpr int NS = kDecWaves * G;      // lane-group states merged at the end
    __shared__ float st_m[NS];
    __shared__ float st_l[NS];
    __shared__ float st_o[NS][D];

    const WorkItem it = decode_work(a, blockIdx.x);
    if (!in_bounds(a.check, kSiteWorkItem, it.batch, a.batch) || !in_bounds(a.check, kSiteWorkItem, it.head, a.heads) ||
        !in_bounds(a.check, kSiteWorkItem, it.split, a.seqs.s_max))
        return;
    const Seq sq = load_seq(a.seqs, it.batch);
    if (it.split >= sq.splits || sq.sq < 1) return;
    const int mask = a.seqs.mask;

    // The split's key range for the row (the count formula at the block's
    // last row, here row 0).  A split with no key exits without writing: the
    // combine merges only the populated splits.
    int ks, ke;
    block_split_range(sq, mask, a.seqs.n_per_block, 0, it.split, ks, ke);
    if (ks >= ke) return;
    if (!in_bounds(a.check, kSiteKeys, (sq.krow0 >= 0 ? sq.krow0 : 0) + ke - 1,
                   sq.krow0 >= 0 ? total_keys(a.seqs, a.batch) : (int64_t)a.seqs.max_sk))
        return;
    // Keys of the split the row sees: from the window's first key to the
    // mask's last, clamped so that ks <= kb <= kend <= ke whatever the
    // offset (an empty range leaves O_s = 0, L_s = -inf).
    const int64_t lo = max((int64_t)ks, vis_first(sq, a.seqs.window_left, 0));
    const int64_t hi = min((int64_t)ke, vis_last(sq, mask, 0) + 1);
    const int kb = (int)min(lo, (int64_t)ke);
    const int kend = (int)max(hi, (int64_t)kb);

    const int64_t row = sq.row0;
    const bool row_ok = row < a.rows &&
                        in_bounds(a.check, kSiteQRow, a.seqs.cu_q ? row : (int64_t)it.batch * a.seqs.max_sq, a.rows);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int grp = lane / LPK, part = lane % LPK;

    float q[8];
    {
        const T* qp = reinterpret_cast<const T*>(a.q) + (a.seqs.cu_q ? row * a.q_row : (int64_t)it.batch * a.q_batch) +
                      (int64_t)it.head * a.q_head + part * 8;
        const u32x4 x = row_ok ? *reinterpret_cast<const u32x4*>(qp) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) unpack2<T>(x[e], q[2 * e], q[2 * e + 1]);
    }
    const T* kbase = reinterpret_cast<const T*>(a.k) +
                     (sq.krow0 >= 0 ? sq.krow0 * a.k_row : (int64_t)it.batch * a.k_batch) +
                     (int64_t)it.head * a.k_head + part * 8;
    const T* vbase = reinterpret_cast<const T*>(a.v) +
                     (sq.krow0 >= 0 ? sq.krow0 * a.v_row : (int64_t)it.batch * a.v_batch) +
                     (int64_t)it.head * a.v_head + part * 8;
    const float c = a.scale_log2;

    float m = -INFINITY, l = 0.f;  // this group's running max (log2 units) and weight sum
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    for (int c0 = kb + wave * CHUNK; c0 < kend; c0 += kDecWaves * CHUNK) {
        u32x4 kx[kDecUnroll], vx[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const int key = min(c0 + u * G + grp, kend - 1);  // in range; weight 0 past kend
            kx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (int64_t)key * a.k_row));
            vx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + (int64_t)key * a.v_row));
        }
        float s[kDecUnroll];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float k0, k1;
                unpack2<T>(kx[u][e], k0, k1);
                dot = fmaf(q[2 * e], k0, dot);
                dot = fmaf(q[2 * e + 1], k1, dot);
            }
            dot = group_sum<LPK>(dot);
            s[u] = (c0 + u * G + grp < kend) ? dot * c : -INFINITY;
            mx = fmaxf(mx, s[u]);
        }
        // m = -inf until the group has seen a visible key: weights and the
        // rescale then use 0 as the reference (no -inf - -inf)
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const float p = __builtin_amdgcn_exp2f(s[u] - m_use);
            l += p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v0, v1;
                unpack2<T>(vx[u][e], v0, v1);
                o[2 * e] = fmaf(p, v0, o[2 * e]);
                o[2 * e + 1] = fmaf(p, v1, o[2 * e + 1]);
            }
        }
        m = m_new;
    }

    // Merge the lane groups: m = max of their maxima, weights 2^(m_g - m).
    const int g = wave * G + grp;
    if (part == 0) {
        st_m[g] = m;
        st_l[g] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) st_o[g][part * 8 + e] = o[e];
    __syncthreads();
    if (!row_ok || tid >= D) return;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i) M = fmaxf(M, st_m[i]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const float w = __builtin_amdgcn_exp2f(st_m[i] - M_use);
        L = fmaf(st_l[i], w, L);
        O = fmaf(st_o[i][tid], w, O);
    }
    // Nothing visible: O_s = 0, L_s = -inf.
    const bool empty = (M == -INFINITY);
    const int64_t slot = ((int64_t)it.head * a.seqs.s_max + it.split) * a.rows + row;
    if (!in_bounds(a.check, kSitePartialSlot, slot, (int64_t)a.heads * a.seqs.s_max * a.rows)) return;
    a.o_part[slot * D + tid] = empty ? 0.f : O / L;
    if (tid == 0) a.lse_part[slot] = empty ? -INFINITY : M * kLn2 + logf(L);
}

template <typename T, int D>
hipError_t launch(const PartialArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((partial_decode_kernel<T, D>), dim3(a.n_work), dim3(kDecThreads), 0, stream, a);
    return hipGetLastError();
}

// Resident workgroups per CU (cached; the same on every gfx950 device).
template <typename T, int D>
int blocks_per_cu() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, partial_decode_kernel<T, D>, kDecThreads, 0) != hipSuccess)
        return 0;
    cached.store(n, std::memory_order_relaxed);
    return n;
}

template <typename T>
PartialKernel find_decode(int d_qk, int d_v) {
    if (d_qk != d_v) return {nullptr, 0, nullptr, false};
    if (d_qk == 64) return {launch<T, 64>, 1, blocks_per_cu<T, 64>, false};
    if (d_qk == 128) return {launch<T, 128>, 1, blocks_per_cu<T, 128>, false};
    return {nullptr, 0, nullptr, false};
}

}  // namespace

PartialKernel find_partial_decode(int dtype, int d_qk, int d_v) {
    if (dtype == SK_BF16) return find_decode<__bf16>(d_qk, d_v);
    if (dtype == SK_F16) return find_decode<_Float16>(d_qk, d_v);
    return {nullptr, 0, nullptr, false};
}

}  // namespace sk
