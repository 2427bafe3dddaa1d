// kda_segments.hip -- composition of segment states for sequence-parallel
// prefill of long sequences.
//
// Within a chunk the state update is affine in the entering state S (page
// "Kimi (AI)", section "Kimi Delta Attention (KDA)": the forget gate scales
// rows, and the predict / update steps act on S from the right):
//     S' = diag(gamma) S (I - K^T A^T K) + (terms that do not involve S),
// so over a segment of whole chunks
//     S_end = diag(Gamma) S_start M + dS,
// with Gamma the product of the segment's gates (per value row), M the product
// of the chunks' key-side factors (d_k x d_k, the same for every row), and dS
// the segment's end state from a zero start.  The prefill computes dS and M for
// every segment in parallel (two scans), this kernel walks the segments of
// each (sequence, head) in order to get every segment's true starting state,
// and a last scan reruns each segment from it.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One workgroup of 512 threads per (sequence, head, block of rows).  A row's
// d_k outputs are d_k / 4 column groups of four key channels, and each product
// S M is split over KS = 4 quarters of the reduction index k, so a thread
// accumulates 4 columns over d_k / 4 values of k and the quarters are summed
// through LDS (4 rows per workgroup at d_k = 128, 8 at 64).
// For segment g = 0 .. G-1 of sequence n:
//     S_start[n G + g] = S                      (S = S0[n], or zeros, for g = 0)
//     S = diag(gamma_g) S M_g + dS_g
// and S_T[n] = S after the last segment.  gamma_g is the segment's total decay
// per value row (the product of its gates), written by the scan that produced dS.
// M_{g+1}, dS_{g+1} and gamma_{g+1} are loaded into registers while segment g is
// composed, so a step waits only for its own LDS products.
// Layouts: dS, S_start [n_seq G, H, d_v, d_k]; M [n_seq G, H, d_k, d_k];
// gdecay [n_seq G, H, d_v]; S0, S_T [n_seq, H, d_v, d_k].
// range_flags [n_seq G, H, d_v / 64] (or null): segments whose scan met a chunk
// beyond the decay range of the factored form; their dS is not valid, so a
// workgroup whose rows belong to such a segment leaves S_T unwritten (S0 stays
// intact when S_T aliases it) for the token-recurrent pass that follows.
template <int DK, int DV>
__global__ __launch_bounds__(512) void combine_segments_kernel(
    const float* __restrict__ gdecay, const float* __restrict__ S0, const float* __restrict__ dS,
    const float* __restrict__ M, const int32_t* __restrict__ range_flags, int n_seq, int G, int n_heads,
    float* __restrict__ S_start, float* __restrict__ S_T) {
    constexpr int NT = 512;
    constexpr int KS = 4;                 // quarters of the reduction index
    constexpr int CG = DK / 4;            // column groups per row
    constexpr int ROWS = NT / (CG * KS);  // rows per workgroup
    constexpr int NRB = DV / ROWS;        // row blocks per head
    constexpr int KQ = DK / KS;           // values of k per quarter
    constexpr int MP = DK * DK / 4 / NT;  // 16-byte pieces of M per thread
    static_assert(DV % ROWS == 0, "rows per workgroup");
    __shared__ __align__(16) float Ms[DK * DK];
    __shared__ __align__(16) float Ss[ROWS * DK];
    __shared__ __align__(16) float Ps[KS * ROWS * DK];  // partial sums per quarter

    const int b = blockIdx.x;
    const int rblk = b % NRB, unit = b / NRB;
    const int h = unit % n_heads, n = unit / n_heads;
    if (n >= n_seq) return;
    const int tid = threadIdx.x;
    const int c4 = 4 * (tid % CG), r = (tid / CG) % ROWS, q = tid / (CG * ROWS);
    const bool owner = q == 0;  // the threads of quarter 0 hold the state
    const int i = rblk * ROWS + r;  // value row
    const int64_t H = n_heads;
    const int64_t row_off = static_cast<int64_t>(i) * DK + c4;
    auto seg_of = [&](int g) { return static_cast<int64_t>(n) * G + g; };

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if (owner && S0) s = *reinterpret_cast<const f32x4*>(S0 + (static_cast<int64_t>(n) * H + h) * DV * DK + row_off);
    f32x4 mreg[MP], dnext = {0.f, 0.f, 0.f, 0.f};
    float gnext = 1.f;
    auto load_next = [&](int g) {
        const int64_t sg = seg_of(g);
        const float* Mg = M + (sg * H + h) * DK * DK;
#pragma unroll
        for (int p = 0; p < MP; ++p) mreg[p] = *reinterpret_cast<const f32x4*>(Mg + 4 * (tid + NT * p));
        if (owner) {
            dnext = *reinterpret_cast<const f32x4*>(dS + (sg * H + h) * DV * DK + row_off);
            gnext = gdecay[(sg * H + h) * DV + i];
        }
    };
    load_next(0);
    for (int g = 0; g < G; ++g) {
        if (owner) {
            *reinterpret_cast<f32x4*>(S_start + (seg_of(g) * H + h) * DV * DK + row_off) = s;
            *reinterpret_cast<f32x4*>(Ss + r * DK + c4) = s;
        }
#pragma unroll
        for (int p = 0; p < MP; ++p) *reinterpret_cast<f32x4*>(Ms + 4 * (tid + NT * p)) = mreg[p];
        const f32x4 d = dnext;
        const float gam = gnext;
        if (g + 1 < G) load_next(g + 1);
        __syncthreads();
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int kk = 0; kk < KQ; ++kk) {
            const int k = q * KQ + kk;
            const float sk = Ss[r * DK + k];
            const f32x4 mk = *reinterpret_cast<const f32x4*>(Ms + k * DK + c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += sk * mk[e];
        }
        *reinterpret_cast<f32x4*>(Ps + (q * ROWS + r) * DK + c4) = acc;
        __syncthreads();  // partials complete; Ms and Ss are free for the next segment
        if (owner) {
            f32x4 t = *reinterpret_cast<const f32x4*>(Ps + r * DK + c4);
#pragma unroll
            for (int qq = 1; qq < KS; ++qq) {
                const f32x4 pq = *reinterpret_cast<const f32x4*>(Ps + (qq * ROWS + r) * DK + c4);
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] += pq[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] = gam * t[e] + d[e];
        }
        // Ps is rewritten only after the next segment's first barrier, which every
        // owner reaches after reading it here
    }
    bool beyond = false;
    if (range_flags) {
        const int vb = (rblk * ROWS) / 64;  // the scan's block of 64 rows that holds these rows
        for (int g = 0; g < G; ++g) beyond |= range_flags[(seg_of(g) * H + h) * (DV / 64) + vb] != 0;
    }
    if (owner && S_T && !beyond)
        *reinterpret_cast<f32x4*>(S_T + (static_cast<int64_t>(n) * H + h) * DV * DK + row_off) = s;
}

template <int DK, int DV>
hipError_t launch_combine_segments(const float* gdecay, const float* S0, const float* dS, const float* M,
                                   const int32_t* range_flags, int n_seq, int G, int n_heads, float* S_start,
                                   float* S_T, hipStream_t stream) {
    constexpr int NRB = DV / (512 / (DK / 4 * 4));
    const int64_t grid = static_cast<int64_t>(n_seq) * n_heads * NRB;
    hipLaunchKernelGGL((combine_segments_kernel<DK, DV>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream,
                       gdecay, S0, dS, M, range_flags, n_seq, G, n_heads, S_start, S_T);
    return hipGetLastError();
}

template hipError_t launch_combine_segments<128, 128>(const float*, const float*, const float*, const float*,
                                                      const int32_t*, int, int, int, float*, float*, hipStream_t);
template hipError_t launch_combine_segments<64, 64>(const float*, const float*, const float*, const float*,
                                                    const int32_t*, int, int, int, float*, float*, hipStream_t);

}  // namespace kda
