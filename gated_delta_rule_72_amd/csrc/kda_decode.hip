// kda_decode.hip -- one recurrent KDA step per (sequence, head), streaming the
// state from HBM exactly once.
//
// Page "Kimi (AI)", section "Kimi Delta Attention (KDA)": the state is d_v x d_k
// (rows are value channels, the forget gate diag(alpha_t) scales rows), so each
// row s_i evolves on its own:
//     a_i = s_i . k          (old row; the prediction is alpha_i a_i)
//     c_i = s_i . q
//     u_i = beta (v_i - alpha_i a_i)
//     s_i <- alpha_i s_i + u_i k
//     o_i = s_i(new) . q = alpha_i c_i + u_i (k . q)
// so one read and one write of S suffice; the read-out uses the updated state.
// With a scalar gate (Gated DeltaNet) alpha_i is the (sequence, head)'s one
// value for every row; without a gate (the delta rule) it is 1.  With the gate
// on key channels (S~ = S diag(alpha), alpha in R^{d_k}) the row is scaled
// elementwise first: s~_i = s_i (.) alpha, a_i = s~_i . k, c_i = s~_i . q,
// u_i = beta (v_i - a_i), s_i <- s~_i + u_i k, o_i = c_i + u_i (k . q).
//
// Layout of the work: one workgroup of 512 threads per 64 state rows of a
// (sequence, head); a head of 128 rows takes two.  Eight consecutive lanes own
// one row; lane j of the eight holds the float4 chunks j, j+8, j+16, ... of the
// row, so each load instruction of the group covers a contiguous 128-byte line.
// All state loads of a thread are issued before any arithmetic, and the state
// is read and written with non-temporal hints (regular loads and stores are
// 16% slower).  One row per thread leaves each thread few registers, so many
// workgroups stay resident and much of the state is in flight; 64 rows per
// workgroup measured 3% faster than 128, 32 the same as 64, 16 or 8 slower.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// state rows per workgroup (one per eight threads); a head of d_v rows takes
// d_v / decode_rows workgroups
constexpr int kDecodeRows = 64;
constexpr int decode_rows(int d_v) { return d_v < kDecodeRows ? d_v : kDecodeRows; }
constexpr int decode_threads(int d_v) { return 8 * decode_rows(d_v); }

template <typename T, int D_K, int D_V, int GATE>
__global__ __launch_bounds__(1024) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ S, T* __restrict__ o) {
    constexpr int ROWS_PER_PASS = decode_rows(D_V);  // row slots
    constexpr int P = 1;                            // rows per thread
    constexpr int NB = D_V / ROWS_PER_PASS;         // workgroups per head
    constexpr int M = D_K / 32;                     // float4 chunks per lane per row
    static_assert(D_V % ROWS_PER_PASS == 0 && D_K % 32 == 0, "unsupported head size");

    const int64_t head = blockIdx.x / NB;           // (b * H + h)
    const int lane8 = threadIdx.x & 7;
    const int slot = (blockIdx.x % NB) * ROWS_PER_PASS + (threadIdx.x >> 3);

    float* Sh = S + head * (int64_t)(D_V * D_K);
    const T* qh = q + head * D_K;
    const T* kh = k + head * D_K;

    // state rows first: the bulk of the traffic
    f32x4 s[P][M];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const float* row = Sh + (int64_t)(slot + p * ROWS_PER_PASS) * D_K;
#pragma unroll
        for (int m = 0; m < M; ++m)
            s[p][m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row) + lane8 + 8 * m);
    }
    f32x4 kk[M], qq[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        kk[m] = Elem<T>::load4(kh + 4 * (lane8 + 8 * m));
        qq[m] = Elem<T>::load4(qh + 4 * (lane8 + 8 * m));
    }
    if constexpr (GATE == GATE_KEY) {
        // s~ = s (.) alpha over key channels, in place
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const f32x4 ak = *reinterpret_cast<const f32x4*>(alpha + head * D_K + 4 * (lane8 + 8 * m));
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[p][m][e] *= ak[e];
        }
    }
    float vi[P], ai[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int i = slot + p * ROWS_PER_PASS;
        vi[p] = Elem<T>::load(v + head * D_V + i);
        // the row's gate; 1 for the key-channel gate, already applied to the state
        ai[p] = GATE == GATE_CHANNEL ? alpha[head * D_V + i] : GATE == GATE_SCALAR ? alpha[head] : 1.f;
    }
    const float bt = beta[head];

    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m)
        kq += kk[m][0] * qq[m][0] + kk[m][1] * qq[m][1] + kk[m][2] * qq[m][2] + kk[m][3] * qq[m][3];
    kq = sum8(kq);

#pragma unroll
    for (int p = 0; p < P; ++p) {
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a += s[p][m][e] * kk[m][e];
                c += s[p][m][e] * qq[m][e];
            }
        }
        a = sum8(a);
        c = sum8(c);
        const float u = bt * (vi[p] - ai[p] * a);
        float* row = Sh + (int64_t)(slot + p * ROWS_PER_PASS) * D_K;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            f32x4 n;
#pragma unroll
            for (int e = 0; e < 4; ++e) n[e] = ai[p] * s[p][m][e] + u * kk[m][e];
            __builtin_nontemporal_store(n, reinterpret_cast<f32x4*>(row) + lane8 + 8 * m);
        }
        if (lane8 == 0) Elem<T>::store(o + head * D_V + slot + p * ROWS_PER_PASS, ai[p] * c + u * kq);
    }
}

template <typename T, int D_K, int D_V, int GATE>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const int64_t heads = (int64_t)a.batch * a.n_heads;
    if (heads == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_step_kernel<T, D_K, D_V, GATE>), dim3((unsigned)(heads * (D_V / decode_rows(D_V)))),
                       dim3(decode_threads(D_V)), 0, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.alpha, a.beta, a.S, static_cast<T*>(a.o));
    return hipGetLastError();
}

template <typename T, int GATE>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_decode_t<T, 128, 128, GATE>(a, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_decode_t<T, 64, 64, GATE>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_decode_t<T, 128, 64, GATE>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_decode_t<T, 64, 128, GATE>(a, stream);
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs& a, hipStream_t stream) {
    switch (a.gate) {
        case GATE_CHANNEL: return launch_decode_g<T, GATE_CHANNEL>(a, stream);
        case GATE_SCALAR: return launch_decode_g<T, GATE_SCALAR>(a, stream);
        case GATE_NONE: return launch_decode_g<T, GATE_NONE>(a, stream);
        case GATE_KEY: return launch_decode_g<T, GATE_KEY>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_decode_dt<uint16_t>(a, stream) : launch_decode_dt<float>(a, stream);
}

}  // namespace kda
