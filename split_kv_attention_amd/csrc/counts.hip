// Per-row valid-split counts (rocmlirTriton page "Recombine fully masked
// split-KV attention partials on the host", section "Per-row valid-split
// counts").  One thread per query row; the count is head-independent.
#include "sk_common.hpp"

namespace sk {

__global__ __launch_bounds__(256) void counts_kernel(CountsArgs a) {
    const Seq s = load_seq(a.seqs, blockIdx.y);
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= s.sq || s.row0 + r >= a.rows) return;
    if (!in_bounds(a.check, kSiteCountsRow, s.row0 + r, a.rows)) return;
    a.counts[s.row0 + r] = valid_split_count(s, a.seqs.mask, a.seqs.n_per_block, r);
}

hipError_t launch_counts(const CountsArgs& a, int batch, hipStream_t stream) {
    const dim3 grid((a.seqs.max_sq + 255) / 256, batch);
    hipLaunchKernelGGL(counts_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sk
