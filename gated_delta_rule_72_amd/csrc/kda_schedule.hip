// kda_schedule.hip -- longest-first ordering of packed sequences for prefill.
#include "kda_internal.h"
#include "kda_schedule.h"

namespace kda {

// rank(n) = #{m : len_m > len_n} + #{m < n : len_m == len_n}; order[rank(n)] = n.
// A permutation by construction, so every rank is written exactly once.
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                       int32_t* __restrict__ order) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= n_seq) return;
    const int32_t len = cu[n + 1] - cu[n];
    int rank = 0;
    for (int m = 0; m < n_seq; ++m) {
        const int32_t lm = cu[m + 1] - cu[m];
        rank += (lm > len) || (lm == len && m < n);
    }
    order[rank] = n;
}

hipError_t launch_schedule(const int32_t* cu_seqlens, int n_seq, int32_t* order, hipStream_t stream) {
    hipLaunchKernelGGL(schedule_kernel, dim3((n_seq + 255) / 256), dim3(256), 0, stream, cu_seqlens,
                       n_seq, order);
    return hipGetLastError();
}

size_t prefill_workspace_bytes(int32_t n_seq, bool varlen) {
    if (!varlen) return 0;
    return ((static_cast<size_t>(n_seq) * sizeof(int32_t) + 255) / 256) * 256;
}

}  // namespace kda
