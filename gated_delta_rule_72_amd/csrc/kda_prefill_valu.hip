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
// Calls whose sequences average more than 16 tokens (dense bf16 calls: more
// than 8) take the staged form further down, which feeds the same per-row
// recurrence from tokens staged in LDS by blocks; the form below serves the
// shorter ones.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_schedule.h"
#include "kda_staged.h"

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

// Waves per workgroup of the ring form (8 rows each); a head of d_v rows takes
// d_v / (8 W) workgroups.  Eight waves (64 rows) per workgroup measured 7% slower
// on multi-token decode of 1 and 4 tokens (1% faster at 16).
constexpr int kRingWaves = 1;

template <typename T, int DK, int DV, int GATE, int D>
__global__ __launch_bounds__(64 * kRingWaves) void prefill_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int n_seq, int n_tok, int n_heads,
    T* __restrict__ o, float* __restrict__ S_T) {
    constexpr int RW = ROWS_PER_WAVE * kRingWaves;  // rows per workgroup
    constexpr int NVB = DV / RW;
    constexpr int M = DK / 32;
    static_assert(DV % RW == 0, "rows per workgroup");
    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int lane = threadIdx.x & 63;
    const int lane8 = lane & 7;
    const int i = u.vblk * RW + (threadIdx.x >> 6) * ROWS_PER_WAVE + (lane >> 3);  // value row of this lane
    const int64_t H = n_heads;
    const int h = u.head;

    const int64_t s_off = ((static_cast<int64_t>(u.seq) * H + h) * DV + i) * DK;
    f32x4 s[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        s[m] = S0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S0 + s_off + 4 * (lane8 + 8 * m)))
                  : f32x4{0.f, 0.f, 0.f, 0.f};

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
        for (int m = 0; m < M; ++m)
            __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(S_T + s_off + 4 * (lane8 + 8 * m)));
    }
}

// Ring depth for long calls (loads well ahead of their use), and for short bf16
// calls, where many waves in flight matter more than a deep ring: at d = 128
// depth 4 takes 214 VGPRs (two waves per SIMD), depth 2 128.  Multi-token decode
// of the decode workload's state, ms per call for 1 / 4 / 16 tokens: depth 4
// 0.248 / 0.408 / 1.05, depth 2 0.191 / 0.273 / 0.731, depth 1 0.199 / 0.275 / 0.710;
// with the state read and written non-temporally (each element is touched once),
// depth 2 0.169 / 0.251 / 0.666.
constexpr int kRingLong = 4;
constexpr int kRingShort = 2;

template <typename T, int DK, int DV, int GATE, int D>
static hipError_t launch_valu_d(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    constexpr int NVB = DV / (ROWS_PER_WAVE * kRingWaves);
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((prefill_valu_kernel<T, DK, DV, GATE, D>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * kRingWaves), 0,
                       stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.alpha, a.beta, a.S0, a.cu_seqlens, order, a.n_seq, a.n_tok, a.n_heads,
                       static_cast<T*>(a.o), a.S_T);
    return hipGetLastError();
}

// ------------------------------------------------------------ staged form --
// (kda_staged.h: the staged blocks and the body)
template <typename T, int DK, int DV, int GATE, int R, int L, bool CKPT>
__global__ __launch_bounds__(L * R) void prefill_staged_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int n_seq, int n_tok, int n_heads,
    T* __restrict__ o, float* __restrict__ S_T, float* __restrict__ ckpt,
    const int32_t* __restrict__ range_flags, int flag_segs) {
    __shared__ StageBuf<DK, GATE, R> buf[2];
    prefill_staged_body<T, DK, DV, GATE, R, L, CKPT>(buf, blockIdx.x, q, k, v, alpha, beta, S0, cu_seqlens, order,
                                                     n_seq, n_tok, n_heads, o, S_T, ckpt, range_flags, flag_segs);
}

template <typename T, int DK, int DV, int GATE, int R, int L = 8>
static hipError_t launch_staged_r(const PrefillArgs& a, const int32_t* order, hipStream_t stream, float* ckpt,
                                  const int32_t* range_flags = nullptr, int flag_segs = 1) {
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, DV / R);
    if (ckpt) {
        hipLaunchKernelGGL((prefill_staged_kernel<T, DK, DV, GATE, R, L, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(L * R), 0, stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), a.alpha, a.beta, a.S0, a.cu_seqlens, order, a.n_seq, a.n_tok,
                           a.n_heads, nullptr, nullptr, ckpt, range_flags, 1);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((prefill_staged_kernel<T, DK, DV, GATE, R, L, false>), dim3(static_cast<unsigned>(grid)), dim3(L * R),
                       0, stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.alpha, a.beta, a.S0, a.cu_seqlens, order, a.n_seq, a.n_tok, a.n_heads,
                       static_cast<T*>(a.o), a.S_T, ckpt, range_flags, flag_segs);
    return hipGetLastError();
}

// Rows per workgroup: 64 when that makes at least one workgroup per CU, else
// 32, else 16.  Below 64 a row gets 16 lanes, so a wave's share of a token is
// half as many instructions (against 8 lanes, ms per call: the key-channel gate
// at 1 x 4096 tokens, H = 8, d = 128, 1.41 -> 1.11, at 16 x 64 tokens, H = 4,
// 0.028 -> 0.025; fp32 1 x 1024, H = 8: 0.297 -> 0.246; the tiny fp32 workload
// 0.055 -> 0.050).  At 64 rows, 16 lanes (1024 threads) was 1% slower on the
// batched workload with the key-channel gate.
constexpr int kStagedSmallLanes = 16;
template <typename T, int DK, int DV, int GATE>
static hipError_t launch_staged(const PrefillArgs& a, const int32_t* order, hipStream_t stream,
                                float* ckpt = nullptr, const int32_t* range_flags = nullptr) {
    constexpr int64_t kCus = 256;
    const int64_t units = static_cast<int64_t>(a.n_seq) * a.n_heads;
    if (units * (DV / 64) >= kCus) return launch_staged_r<T, DK, DV, GATE, 64>(a, order, stream, ckpt, range_flags);
    if (units * (DV / 32) >= kCus)
        return launch_staged_r<T, DK, DV, GATE, 32, kStagedSmallLanes>(a, order, stream, ckpt, range_flags);
    return launch_staged_r<T, DK, DV, GATE, 16, kStagedSmallLanes>(a, order, stream, ckpt, range_flags);
}

template <typename T, int GATE>
static hipError_t launch_ckpt_g(const PrefillArgs& a, const int32_t* order, float* ckpt, hipStream_t stream,
                                const int32_t* rf) {
    if (a.d_k == 128 && a.d_v == 128) return launch_staged<T, 128, 128, GATE>(a, order, stream, ckpt, rf);
    if (a.d_k == 64 && a.d_v == 64) return launch_staged<T, 64, 64, GATE>(a, order, stream, ckpt, rf);
    if (a.d_k == 128 && a.d_v == 64) return launch_staged<T, 128, 64, GATE>(a, order, stream, ckpt, rf);
    if (a.d_k == 64 && a.d_v == 128) return launch_staged<T, 64, 128, GATE>(a, order, stream, ckpt, rf);
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_ckpt_t(const PrefillArgs& a, const int32_t* order, float* ckpt, hipStream_t stream,
                                const int32_t* rf) {
    switch (a.gate) {
        case GATE_CHANNEL: return launch_ckpt_g<T, GATE_CHANNEL>(a, order, ckpt, stream, rf);
        case GATE_SCALAR: return launch_ckpt_g<T, GATE_SCALAR>(a, order, ckpt, stream, rf);
        case GATE_NONE: return launch_ckpt_g<T, GATE_NONE>(a, order, ckpt, stream, rf);
        case GATE_KEY: return launch_ckpt_g<T, GATE_KEY>(a, order, ckpt, stream, rf);
    }
    return hipErrorInvalidValue;
}

// The backward's forward pass: the staged form run for its states only (a.o and
// a.S_T null), storing the state entering every block of 16 tokens into ckpt.
hipError_t launch_prefill_checkpoints(const PrefillArgs& a, const int32_t* order, float* ckpt, hipStream_t stream,
                                      const int32_t* range_flags) {
    static_assert(STAGE_TOKENS == STATE_CHECKPOINT_TOKENS, "checkpoint spacing");
    return a.bf16 ? launch_ckpt_t<uint16_t>(a, order, ckpt, stream, range_flags)
                  : launch_ckpt_t<float>(a, order, ckpt, stream, range_flags);
}

#ifndef KDA_STAGED_MIN_TOKENS
#define KDA_STAGED_MIN_TOKENS (STAGE_TOKENS + 1)
#endif
// Calls whose sequences average more than one staged block take the staged form.
constexpr int64_t kStagedMinTokens = KDA_STAGED_MIN_TOKENS;
constexpr int64_t kRingShortMaxTokens = 8;

template <typename T, int DK, int DV, int GATE>
static hipError_t launch_valu_t(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    // dense bf16 calls of at most 16 tokens per sequence (multi-token decode): the ring of
    // two up to 8 tokens, the staged form above that (ms per call on the decode workload's
    // state, ring / staged: 8 tokens 0.400 / 0.408, 12 tokens 0.534 / 0.515, 16 tokens
    // 0.666 / 0.623)
    const bool dense_bf16 = std::is_same<T, uint16_t>::value && !a.cu_seqlens;
    if (dense_bf16 && a.n_tok <= kRingShortMaxTokens * a.n_seq)
        return launch_valu_d<T, DK, DV, GATE, kRingShort>(a, order, stream);
    if (dense_bf16 || a.n_tok >= kStagedMinTokens * a.n_seq)
        return launch_staged<T, DK, DV, GATE>(a, order, stream);
    return launch_valu_d<T, DK, DV, GATE, kRingLong>(a, order, stream);
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

// The units of a chunked bf16 call that its scan marked as beyond the decay range,
// recomputed from S0 by the staged form (64 rows per workgroup, the scan's row
// blocks; sequences in index order).  No log of alpha is taken here, so alpha = 0
// and any strength of decay are exact.
template <int DK, int DV>
static hipError_t launch_fixup_t(const PrefillArgs& a, const int32_t* range_flags, int G, hipStream_t stream) {
    switch (a.gate) {
        case GATE_CHANNEL:
            return launch_staged_r<uint16_t, DK, DV, GATE_CHANNEL, 64>(a, nullptr, stream, nullptr, range_flags, G);
        case GATE_SCALAR:
            return launch_staged_r<uint16_t, DK, DV, GATE_SCALAR, 64>(a, nullptr, stream, nullptr, range_flags, G);
        case GATE_KEY:
            return launch_staged_r<uint16_t, DK, DV, GATE_KEY, 64>(a, nullptr, stream, nullptr, range_flags, G);
        default: return hipErrorInvalidValue;  // no gate: nothing decays, nothing is marked
    }
}

hipError_t launch_prefill_range_fixup(const PrefillArgs& a, const int32_t* range_flags, int G, hipStream_t stream) {
    if (!a.bf16 || a.n_tok <= 0) return hipSuccess;
    if (a.d_k == 128 && a.d_v == 128) return launch_fixup_t<128, 128>(a, range_flags, G, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_fixup_t<64, 64>(a, range_flags, G, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_fixup_t<128, 64>(a, range_flags, G, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_fixup_t<64, 128>(a, range_flags, G, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
