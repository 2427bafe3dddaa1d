// kda_prefill_valu.hip -- KDA prefill token by token on the vector ALUs, with
// the state held in registers.
//
// The path of float32 inputs (fp32 arithmetic throughout), and of the gate on
// key channels for either input type.  Page "Kimi (AI)", section
// "Kimi Delta Attention (KDA)": the state is d_v x d_k with rows = value
// channels, and the forget gate diag(alpha_t) scales rows, so every row s_i of
// S evolves on its own.  For each token t of a sequence, in order:
//     a_i = s_i . k_t          (prediction before the gate: v~_i = alpha_i a_i)
//     c_i = s_i . q_t
//     u_i = beta_t (v_i - alpha_i a_i)
//     s_i <- alpha_i s_i + u_i k_t
//     o_i = s_i . q_t = alpha_i c_i + u_i (k_t . q_t)
// which is the three-step update followed by the read-out with the updated
// state -- the decode step, repeated over the sequence without leaving
// registers.
//
// Layout of the work: one wave per (sequence, head, block of 8 value rows).
// Eight consecutive lanes own one row; lane j of the eight holds the float4
// chunks j, j + 8, ... of the row (d_k / 32 chunks), so the dot products are
// 8-lane DPP reductions.  Each token's q, k (every lane its chunks), v and
// alpha (every lane its row) and beta are loaded three tokens ahead of their use.
// Rows are independent, so the d_v / 8 waves of a head run side by side on
// different CUs.  A token costs each wave about a hundred VALU instructions.
// A chunked fp32 form on the vector ALUs (32-token chunks, every small matrix
// product through LDS) measured 5.6x slower on the tiny fp32 workload (384 vs
// 69 us per call) and 8.5x slower at H = 8, T = 1024, d = 128 (3.1 vs 0.37 ms).
// No log of alpha is taken, so alpha = 0 is exact here.
// With the gate on key channels (S~ = S diag(alpha), alpha in R^{d_k}) each
// lane first scales its part of the row by its key channels' gates, s~ = s (.)
// alpha, and then a = s~ . k, c = s~ . q, u = beta (v - a), s <- s~ + u k,
// o = c + u (k . q): the per-token form needs no chunk algebra for it.  bf16
// inputs are widened to fp32 on load and o is rounded to nearest even.
// bf16 calls of at most 16 tokens per sequence (multi-token decode: a few new
// tokens for each of many sequences, the state continued in place) also run
// here: each state is read once and written once, as in the decode step, where
// the chunked path would spend a whole 64-token chunk on every sequence.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_schedule.h"

#include <type_traits>

namespace kda {

constexpr int ROWS_PER_WAVE = 8;

template <int DK, int GATE>
struct Token {
    f32x4 k[DK / 32], q[DK / 32];
    f32x4 ak[GATE == GATE_KEY ? DK / 32 : 1];  // key-channel gates (GATE_KEY only)
    float v, a, b;
};

template <typename T, int DK, int DV, int GATE>
__device__ __forceinline__ void load_token(Token<DK, GATE>& x, const T* __restrict__ q, const T* __restrict__ k,
                                           const T* __restrict__ v, const float* __restrict__ alpha,
                                           const float* __restrict__ beta, int64_t th, int i, int lane8) {
#pragma unroll
    for (int m = 0; m < DK / 32; ++m) {
        x.k[m] = Elem<T>::load4(k + th * DK + 4 * (lane8 + 8 * m));
        x.q[m] = Elem<T>::load4(q + th * DK + 4 * (lane8 + 8 * m));
        if constexpr (GATE == GATE_KEY)
            x.ak[m] = *reinterpret_cast<const f32x4*>(alpha + th * DK + 4 * (lane8 + 8 * m));
    }
    x.v = Elem<T>::load(v + th * DV + i);
    x.a = GATE == GATE_CHANNEL ? alpha[th * DV + i] : GATE == GATE_SCALAR ? alpha[th] : 1.f;
    x.b = beta[th];
}

template <typename T, int DK, int DV, int GATE, int D>
__global__ __launch_bounds__(64) void prefill_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int n_seq, int n_tok, int n_heads,
    T* __restrict__ o, float* __restrict__ S_T) {
    constexpr int NVB = DV / ROWS_PER_WAVE;
    constexpr int M = DK / 32;
    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int lane = threadIdx.x;
    const int lane8 = lane & 7;
    const int i = u.vblk * ROWS_PER_WAVE + (lane >> 3);  // value row of this lane
    const int64_t H = n_heads;
    const int h = u.head;

    const int64_t s_off = ((static_cast<int64_t>(u.seq) * H + h) * DV + i) * DK;
    f32x4 s[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        s[m] = S0 ? *reinterpret_cast<const f32x4*>(S0 + s_off + 4 * (lane8 + 8 * m)) : f32x4{0.f, 0.f, 0.f, 0.f};

    // one token of the recurrence for this lane's row
    auto step = [&](const Token<DK, GATE>& x, int64_t t) {
        if constexpr (GATE == GATE_KEY) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[m][e] *= x.ak[m][e];
        }
        float a0 = 0.f, a1 = 0.f, c0 = 0.f, c1 = 0.f, kq0 = 0.f, kq1 = 0.f;  // two partial sums each
#pragma unroll
        for (int m = 0; m < M; ++m) {
            a0 += s[m][0] * x.k[m][0] + s[m][2] * x.k[m][2];
            a1 += s[m][1] * x.k[m][1] + s[m][3] * x.k[m][3];
            c0 += s[m][0] * x.q[m][0] + s[m][2] * x.q[m][2];
            c1 += s[m][1] * x.q[m][1] + s[m][3] * x.q[m][3];
            kq0 += x.k[m][0] * x.q[m][0] + x.k[m][2] * x.q[m][2];
            kq1 += x.k[m][1] * x.q[m][1] + x.k[m][3] * x.q[m][3];
        }
        const float a = sum8(a0 + a1), c = sum8(c0 + c1), kq = sum8(kq0 + kq1);
        const float uu = x.b * (x.v - x.a * a);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[m][e] = x.a * s[m][e] + uu * x.k[m][e];
        if (lane8 == 0) Elem<T>::store(o + (t * H + h) * DV + i, x.a * c + uu * kq);
    };
    // a ring of D token buffers: each token is loaded D - 1 tokens ahead of its use
    // (the ring index is a compile-time constant in the unrolled body, so no
    // registers are copied); D = 1 loads each token just before its step
    Token<DK, GATE> tok[D];
#pragma unroll
    for (int j = 0; j < D - 1; ++j)
        if (u.t0 + j < u.t1) load_token<T, DK, DV, GATE>(tok[j], q, k, v, alpha, beta, (u.t0 + j) * H + h, i, lane8);
    for (int64_t t = u.t0; t < u.t1; t += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int64_t tt = t + j;
            if (tt + D - 1 < u.t1)
                load_token<T, DK, DV, GATE>(tok[(j + D - 1) % D], q, k, v, alpha, beta, (tt + D - 1) * H + h, i, lane8);
            if (tt < u.t1) step(tok[j], tt);
        }
    }
    if (S_T) {
#pragma unroll
        for (int m = 0; m < M; ++m) *reinterpret_cast<f32x4*>(S_T + s_off + 4 * (lane8 + 8 * m)) = s[m];
    }
}

// Ring depth for long calls (loads well ahead of their use), and for short bf16
// calls, where many waves in flight matter more than a deep ring: at d = 128
// depth 4 takes 214 VGPRs (two waves per SIMD), depth 2 128.  Multi-token decode
// of the decode workload's state, ms per call for 1 / 4 / 16 tokens: depth 4
// 0.248 / 0.408 / 1.05, depth 2 0.191 / 0.273 / 0.731, depth 1 0.199 / 0.275 / 0.710.
constexpr int kRingLong = 4;
constexpr int kRingShort = 2;

template <typename T, int DK, int DV, int GATE, int D>
static hipError_t launch_valu_d(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    constexpr int NVB = DV / ROWS_PER_WAVE;
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((prefill_valu_kernel<T, DK, DV, GATE, D>), dim3(static_cast<unsigned>(grid)), dim3(64), 0,
                       stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.alpha, a.beta, a.S0, a.cu_seqlens, order, a.n_seq, a.n_tok, a.n_heads,
                       static_cast<T*>(a.o), a.S_T);
    return hipGetLastError();
}

template <typename T, int DK, int DV, int GATE>
static hipError_t launch_valu_t(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    const bool short_call = std::is_same<T, uint16_t>::value && !a.cu_seqlens &&
                            a.n_tok <= static_cast<int64_t>(RECURRENT_MAX_TOKENS) * a.n_seq;
    return short_call ? launch_valu_d<T, DK, DV, GATE, kRingShort>(a, order, stream)
                      : launch_valu_d<T, DK, DV, GATE, kRingLong>(a, order, stream);
}

template <typename T, int GATE>
static hipError_t launch_valu_g(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_valu_t<T, 128, 128, GATE>(a, order, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_valu_t<T, 64, 64, GATE>(a, order, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_valu_t<T, 128, 64, GATE>(a, order, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_valu_t<T, 64, 128, GATE>(a, order, stream);
    return hipErrorInvalidValue;
}

// The token-recurrent prefill: float32 inputs, the key-channel gate, and bf16
// calls of a few tokens per sequence (multi-token decode).  The workspace holds
// only the longest-first schedule (packed input), at its start.
hipError_t launch_prefill_recurrent(const PrefillArgs& a, hipStream_t stream) {
    const int32_t* order = nullptr;
    if (a.cu_seqlens) {
        int32_t* ord = static_cast<int32_t*>(a.workspace);
        const hipError_t e = launch_schedule(a.cu_seqlens, a.n_seq, ord, stream);
        if (e != hipSuccess) return e;
        order = ord;
    }
    if (a.bf16) {
        switch (a.gate) {
            case GATE_CHANNEL: return launch_valu_g<uint16_t, GATE_CHANNEL>(a, order, stream);
            case GATE_SCALAR: return launch_valu_g<uint16_t, GATE_SCALAR>(a, order, stream);
            case GATE_NONE: return launch_valu_g<uint16_t, GATE_NONE>(a, order, stream);
            case GATE_KEY: return launch_valu_g<uint16_t, GATE_KEY>(a, order, stream);
        }
        return hipErrorInvalidValue;
    }
    switch (a.gate) {
        case GATE_CHANNEL: return launch_valu_g<float, GATE_CHANNEL>(a, order, stream);
        case GATE_SCALAR: return launch_valu_g<float, GATE_SCALAR>(a, order, stream);
        case GATE_NONE: return launch_valu_g<float, GATE_NONE>(a, order, stream);
        case GATE_KEY: return launch_valu_g<float, GATE_KEY>(a, order, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) { return launch_prefill_recurrent(a, stream); }

}  // namespace kda
