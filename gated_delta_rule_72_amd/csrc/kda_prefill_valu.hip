// kda_prefill_valu.hip -- chunkwise KDA prefill in fp32 on the vector ALUs.
//
// The float32-input path (fp32 arithmetic throughout, so its results sit at
// fp32 rounding of the recurrence).  Same chunk algebra as the bf16 MFMA path;
// written for clarity rather than speed.
//
// Chunk algebra (derived from the three-step update of page "Kimi (AI)",
// section "Kimi Delta Attention (KDA)"; rows of S are value channels, so the
// gate is a per-row scalar and commutes with everything on the key side).
// For a chunk of tokens 1..n entering with state S:
//   G[t,i]  = sum_{s<=t} log alpha[s,i]            cumulative log-decay per row
//   L       = strictly_lower(diag(beta) K K^T)      decay-free
//   A       = (I + L)^{-1} diag(beta)               unit-lower solve
//   X       = V (.) exp(-G)
//   U       = A X - (A K) S^T                       decay-normalised errors
//   O       = exp(G) (.) (Q S^T + tril(Q K^T) U)    tril keeps the diagonal
//   S'      = diag(exp(G[n,:])) (S + U^T K)
// A partial last chunk is padded with k = q = v = 0, alpha = 1, beta = 0
// tokens, which leave every quantity above unchanged.  GATE selects the
// layout of alpha: per value channel, one scalar per (token, head) for every
// row, or none (alpha = 1).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_schedule.h"

namespace kda {

template <typename T, int DK, int DV, int BV, int GATE>
__global__ __launch_bounds__(256) void prefill_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int n_seq, int n_tok, int n_heads,
    T* __restrict__ o, float* __restrict__ S_T) {
    constexpr int C = PREFILL_CHUNK_F32;
    constexpr int NT = 256;
    constexpr int NVB = DV / BV;
    constexpr int KP = DK + 1;  // padded row pitch
    __shared__ float Ks[C][KP];
    __shared__ float Qs[C][KP];
    __shared__ float Ws[C][KP];
    __shared__ float Ss[BV][KP];
    __shared__ float Xs[C][BV];
    __shared__ float Us[C][BV];
    __shared__ float Gs[C][BV];
    __shared__ float Ls[C][C + 1];
    __shared__ float As[C][C + 1];
    __shared__ float Ps[C][C + 1];
    __shared__ float bs[C];
    __shared__ float gam[BV];

    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int h = u.head;
    const int i0 = u.vblk * BV;  // first value row of this block
    const int64_t H = n_heads;

    // state rows i0 .. i0+BV-1 of this (sequence, head)
    const int64_t s_off = ((static_cast<int64_t>(u.seq) * H + h) * DV + i0) * DK;
    for (int x = tid; x < BV * DK; x += NT) {
        const int i = x / DK, j = x % DK;
        Ss[i][j] = S0 ? S0[s_off + x] : 0.f;
    }

    for (int64_t tc = u.t0; tc < u.t1; tc += C) {
        const int n = static_cast<int>(min<int64_t>(C, u.t1 - tc));
        __syncthreads();  // previous chunk done with every buffer
        for (int x = tid; x < C * DK; x += NT) {
            const int t = x / DK, j = x % DK;
            const int64_t g = ((tc + t) * H + h) * DK + j;
            Ks[t][j] = t < n ? Elem<T>::load(k + g) : 0.f;
            Qs[t][j] = t < n ? Elem<T>::load(q + g) : 0.f;
        }
        for (int x = tid; x < C * BV; x += NT) {
            const int t = x / BV, i = x % BV;
            const int64_t g = ((tc + t) * H + h) * DV + i0 + i;
            Xs[t][i] = t < n ? Elem<T>::load(v + g) : 0.f;
            if constexpr (GATE == GATE_CHANNEL) Gs[t][i] = t < n ? logf(alpha[g]) : 0.f;
            else if constexpr (GATE == GATE_SCALAR) Gs[t][i] = t < n ? logf(alpha[(tc + t) * H + h]) : 0.f;
            else Gs[t][i] = 0.f;
        }
        if (tid < C) bs[tid] = tid < n ? beta[(tc + tid) * H + h] : 0.f;
        __syncthreads();

        // cumulative log-decay per row; K K^T and Q K^T in parallel
        if (tid < BV) {
            float acc = 0.f;
            for (int t = 0; t < C; ++t) {
                acc += Gs[t][tid];
                Gs[t][tid] = acc;
            }
            gam[tid] = expf(acc);
        }
        for (int x = tid; x < C * C; x += NT) {
            const int t = x / C, s = x % C;
            float kk = 0.f, qk = 0.f;
            if (s <= t) {
                for (int j = 0; j < DK; ++j) {
                    kk += Ks[t][j] * Ks[s][j];
                    qk += Qs[t][j] * Ks[s][j];
                }
            }
            Ls[t][s] = s < t ? bs[t] * kk : 0.f;
            Ps[t][s] = qk;
        }
        __syncthreads();

        // (I + L)^{-1} by forward substitution, one column per thread;
        // X = V exp(-G) meanwhile
        if (tid < C) {
            const int c = tid;
            for (int r = 0; r < C; ++r) {
                float x = (r == c) ? 1.f : 0.f;
                for (int s = c; s < r; ++s) x -= Ls[r][s] * As[s][c];
                As[r][c] = r < c ? 0.f : x;
            }
        }
        for (int x = tid; x < C * BV; x += NT) {
            const int t = x / BV, i = x % BV;
            Xs[t][i] *= expf(-Gs[t][i]);
        }
        __syncthreads();
        for (int x = tid; x < C * C; x += NT) {
            const int t = x / C, s = x % C;
            As[t][s] *= bs[s];
        }
        __syncthreads();

        // W = A K, U0 = A X
        for (int x = tid; x < C * DK; x += NT) {
            const int t = x / DK, j = x % DK;
            float acc = 0.f;
            for (int s = 0; s <= t; ++s) acc += As[t][s] * Ks[s][j];
            Ws[t][j] = acc;
        }
        for (int x = tid; x < C * BV; x += NT) {
            const int t = x / BV, i = x % BV;
            float acc = 0.f;
            for (int s = 0; s <= t; ++s) acc += As[t][s] * Xs[s][i];
            Us[t][i] = acc;
        }
        __syncthreads();

        // U = U0 - W S^T
        for (int x = tid; x < C * BV; x += NT) {
            const int t = x / BV, i = x % BV;
            float acc = 0.f;
            for (int j = 0; j < DK; ++j) acc += Ws[t][j] * Ss[i][j];
            Us[t][i] -= acc;
        }
        __syncthreads();

        // O = exp(G) (Q S^T + tril(Q K^T) U)
        for (int x = tid; x < C * BV; x += NT) {
            const int t = x / BV, i = x % BV;
            if (t >= n) continue;
            float acc = 0.f;
            for (int j = 0; j < DK; ++j) acc += Qs[t][j] * Ss[i][j];
            for (int s = 0; s <= t; ++s) acc += Ps[t][s] * Us[s][i];
            Elem<T>::store(o + ((tc + t) * H + h) * DV + i0 + i, expf(Gs[t][i]) * acc);
        }
        __syncthreads();

        // S <- diag(gamma) (S + U^T K)
        for (int x = tid; x < BV * DK; x += NT) {
            const int i = x / DK, j = x % DK;
            float acc = Ss[i][j];
            for (int t = 0; t < C; ++t) acc += Us[t][i] * Ks[t][j];
            Ss[i][j] = gam[i] * acc;
        }
    }
    __syncthreads();
    if (S_T) {
        for (int x = tid; x < BV * DK; x += NT) S_T[s_off + x] = Ss[x / DK][x % DK];
    }
}

template <typename T, int DK, int DV, int GATE>
static hipError_t launch_valu_t(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    constexpr int BV = 32;
    constexpr int NVB = DV / BV;
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((prefill_valu_kernel<T, DK, DV, BV, GATE>), dim3(static_cast<unsigned>(grid)),
                       dim3(256), 0, stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.alpha, a.beta,
                       a.S0, a.cu_seqlens, order, a.n_seq, a.n_tok, a.n_heads,
                       static_cast<T*>(a.o), a.S_T);
    return hipGetLastError();
}

template <typename T, int GATE>
static hipError_t launch_valu_g(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_valu_t<T, 128, 128, GATE>(a, order, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_valu_t<T, 64, 64, GATE>(a, order, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_valu_t<T, 128, 64, GATE>(a, order, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_valu_t<T, 64, 128, GATE>(a, order, stream);
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_valu_dt(const PrefillArgs& a, hipStream_t stream) {
    const int32_t* order = nullptr;
    if (a.cu_seqlens) {
        int32_t* ord = static_cast<int32_t*>(a.workspace);
        const hipError_t e = launch_schedule(a.cu_seqlens, a.n_seq, ord, stream);
        if (e != hipSuccess) return e;
        order = ord;
    }
    switch (a.gate) {
        case GATE_CHANNEL: return launch_valu_g<T, GATE_CHANNEL>(a, order, stream);
        case GATE_SCALAR: return launch_valu_g<T, GATE_SCALAR>(a, order, stream);
        case GATE_NONE: return launch_valu_g<T, GATE_NONE>(a, order, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    return launch_valu_dt<float>(a, stream);
}

}  // namespace kda
