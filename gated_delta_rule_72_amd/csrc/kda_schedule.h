// kda_schedule.h -- how prefill workgroups map to (sequence, head, value-row
// block), shared by the prefill kernels.
//
// A "unit" is one (sequence, head) pair; its value rows are split into
// n_vblk independent blocks (the forget gate scales rows, so rows never
// interact).  Units are ordered longest sequence first (order[] from the
// schedule kernel; identity for equal lengths), so long scans start early.
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b goes to
// XCD b % 8); the mapping below puts all row blocks of a unit on one XCD, so
// the q/k tiles they all read are shared through that XCD's L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kNumXcd = 8;

struct Unit {
    int seq;    // sequence index (into cu_seqlens / S0 / S_T)
    int head;
    int vblk;   // block of value rows
    int64_t t0, t1;  // token range [t0, t1)
    bool valid;
};

// Grid size for n_units units of n_vblk blocks each (padded to whole XCD groups).
__host__ __device__ inline int64_t prefill_grid(int64_t n_units, int n_vblk) {
    return ((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * n_vblk;
}

__device__ inline Unit map_unit(int64_t b, int n_seq, int n_heads, int n_vblk, int n_tok,
                                const int32_t* cu_seqlens, const int32_t* order) {
    const int64_t group = static_cast<int64_t>(kNumXcd) * n_vblk;
    const int64_t g = b / group;
    const int64_t r = b % group;
    const int64_t unit = g * kNumXcd + (r % kNumXcd);
    Unit u;
    u.vblk = static_cast<int>(r / kNumXcd);
    u.valid = unit < static_cast<int64_t>(n_seq) * n_heads;
    if (!u.valid) return u;
    const int rank = static_cast<int>(unit / n_heads);
    u.head = static_cast<int>(unit % n_heads);
    u.seq = order ? order[rank] : rank;
    if (cu_seqlens) {
        u.t0 = cu_seqlens[u.seq];
        u.t1 = cu_seqlens[u.seq + 1];
    } else {
        const int64_t len = n_tok / n_seq;
        u.t0 = static_cast<int64_t>(u.seq) * len;
        u.t1 = u.t0 + len;
    }
    return u;
}

// Writes order[0..n_seq) = sequence indices sorted by length, longest first
// (ties by index).  Enqueued on `stream` before the prefill kernel.
hipError_t launch_schedule(const int32_t* cu_seqlens, int n_seq, int32_t* order, hipStream_t stream);

}  // namespace kda
