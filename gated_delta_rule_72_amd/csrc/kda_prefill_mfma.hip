// kda_prefill_mfma.hip -- fused chunkwise KDA prefill for bf16 inputs on
// CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Method: page "Kimi (AI)", section "Kimi Delta Attention (KDA)" -- the state S
// is d_v x d_k (rows = value channels) and the forget gate diag(alpha_t) scales
// its rows.  A per-row scalar decay commutes with everything on the key side,
// so within a chunk of C tokens (S entering the chunk):
//   G[t,i] = sum_{s<=t} log alpha[s,i]          (per-row cumulative log-decay)
//   L      = strictly_lower(diag(beta) K K^T)    (decay-free beta-weighted Gram)
//   A      = (I + L)^{-1} diag(beta)             (unit-lower WY/UT solve)
//   U      = A (V (.) e^{-G}) - (A K) S^T        (decay-normalised errors)
//   O      = e^{G} (.) (Q S^T + tril(Q K^T) U)   (tril keeps the diagonal: o_t = S_t q_t)
//   S'     = diag(e^{G[C-1,:]}) (S + U^T K)
// The decayed Gram of value row i is D_i L D_i^{-1} with D_i = diag(e^{G[:,i]}),
// so one decay-free solve serves every row; the decay moves onto V, O and S as
// elementwise scalings.  Chunks that cross the end of a sequence are padded
// with k = q = v = 0, alpha = 1, beta = 0 tokens, which change nothing.
//
// Work decomposition: one workgroup of 8 waves per (sequence, head, block of
// 64 value rows); the workgroup walks its sequence chunk by chunk, holding S^T
// in fp32 MFMA accumulators (one 32x32 tile per wave) across the whole scan,
// with a bf16 copy in LDS as the operand of Q S^T and W S^T.  The next chunk's
// q/k/v/alpha/beta are loaded into registers while the current chunk computes.
//
// Precision: q, k, v are exact bf16 inputs.  Computed operands are carried as
// hi + lo bf16 pairs (x = hi + lo to ~2^-16 relative) where the error budget
// needs it -- A, V e^{-G}, U and P = tril(Q K^T) -- and as single bf16 for
// W = A K and S (the state itself stays fp32).  Products of split operands
// take three MFMAs (hi*hi + lo*hi + hi*lo).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_schedule.h"

namespace kda {
namespace {

constexpr int C = PREFILL_CHUNK_BF16;  // 64 tokens per chunk
constexpr int BV = 64;                 // value rows per workgroup
constexpr int NW = 8;                  // waves per workgroup
constexpr int NT = NW * 64;            // threads per workgroup
constexpr int PAD = 8;                 // bf16 row padding (16 bytes) against bank conflicts

// ------------------------------------------------------------- MFMA helpers
// v_mfma_f32_32x32x16_bf16 operand layout: lane l supplies row (l & 31) of A
// (column (l & 31) of B) and the 8 consecutive reduction indices starting at
// 8 * (l >> 5).  Both operands are read from LDS buffers stored
// "reduction-index contiguous": A as [m][k], B as [n][k].
__device__ __forceinline__ bf16x8 frag(const uint16_t* base, int pitch, int row0, int k0, int lane) {
    const uint16_t* p = base + (row0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulator layout of a 32x32 tile: register r of lane l holds
// D[row = 8*(r/4) + 4*(l>>5) + (r&3)][col = l & 31].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Shared-memory layout (bytes).  Regions are reused across the phases of a
// chunk; the comments give each region's tenants in order.
template <int DK>
struct Smem {
    static constexpr int KP = DK + PAD;     // pitch of [t][j] bf16 rows
    static constexpr int CP = C + PAD;      // pitch of [x][t] bf16 rows (length C)
    static constexpr int LP = C + 4;        // pitch of C x C fp32 rows
    static constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
    // R0: K as [t][j] (Gram products) -> solve scratch X fp32 [t][s] -> -W bf16 [t][j]
    static constexpr int R0 = 0;
    static constexpr int R0_SZ = max3(C * KP * 2, C * LP * 4, 0);
    // R1: Q as [t][j]
    static constexpr int R1 = R0 + R0_SZ;
    static constexpr int R1_SZ = C * KP * 2;
    // R2: K^T as [j][t]
    static constexpr int R2 = R1 + R1_SZ;
    static constexpr int R2_SZ = DK * CP * 2;
    // R3: L fp32 [t][s] -> U^T hi, lo bf16 [i][t]
    static constexpr int R3 = R2 + R2_SZ;
    static constexpr int R3_SZ = max3(C * LP * 4, 2 * BV * CP * 2, 0);
    // R4: solve temporaries fp32 -> A hi, lo bf16 [t][s]
    static constexpr int R4 = R3 + R3_SZ;
    static constexpr int R4_SZ = 2 * C * CP * 2;
    // R5: P = tril(Q K^T) hi, lo bf16 [t][s]
    static constexpr int R5 = R4 + R4_SZ;
    static constexpr int R5_SZ = 2 * C * CP * 2;
    // R6: V^T raw bf16 [i][t] -> X^T = (V e^{-G})^T hi, lo bf16 [i][t]
    static constexpr int R6 = R5 + R5_SZ;
    static constexpr int R6_SZ = 2 * BV * CP * 2;
    // R7: S bf16 [i][j] (operand copy of the fp32 state)
    static constexpr int R7 = R6 + R6_SZ;
    static constexpr int R7_SZ = BV * KP * 2;
    // R8: G fp32 [t][i]
    static constexpr int R8 = R7 + R7_SZ;
    static constexpr int R8_SZ = C * BV * 4;
    // R9: beta [C], gamma [BV], partial scan sums [8][BV]
    static constexpr int R9 = R8 + R8_SZ;
    static constexpr int R9_SZ = (C + BV + 8 * BV) * 4;
    static constexpr int TOTAL = R9 + R9_SZ;
};

}  // namespace

template <int DK, int DV>
__global__ __launch_bounds__(NT) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int n_seq, int n_tok, int n_heads,
    uint16_t* __restrict__ o, float* __restrict__ S_T) {
    using SM = Smem<DK>;
    static_assert(SM::TOTAL <= 160 * 1024, "LDS budget");
    static_assert(DK == 64 || DK == 128, "d_k");
    constexpr int NVB = DV / BV;
    constexpr int KP = SM::KP, CP = SM::CP, LP = SM::LP;
    constexpr int JT = DK / 32;          // 32-wide tiles along d_k
    constexpr int KQ_CHUNKS = C * DK / 8;  // 16-byte pieces of a K (or Q) chunk
    constexpr int KQ_PER_T = (KQ_CHUNKS + NT - 1) / NT;
    constexpr int A_CHUNKS = C * BV / 4;   // float4 pieces of an alpha block
    constexpr int A_PER_T = A_CHUNKS / NT;
    static_assert(A_CHUNKS % NT == 0 && C * BV / 8 == NT, "thread mapping");

    __shared__ __align__(16) unsigned char smem[SM::TOTAL];
    uint16_t* Kc = reinterpret_cast<uint16_t*>(smem + SM::R0);
    float* Xs = reinterpret_cast<float*>(smem + SM::R0);
    uint16_t* Wn = reinterpret_cast<uint16_t*>(smem + SM::R0);
    uint16_t* Qc = reinterpret_cast<uint16_t*>(smem + SM::R1);
    uint16_t* Kt = reinterpret_cast<uint16_t*>(smem + SM::R2);
    float* Lf = reinterpret_cast<float*>(smem + SM::R3);
    uint16_t* Ut_hi = reinterpret_cast<uint16_t*>(smem + SM::R3);
    uint16_t* Ut_lo = Ut_hi + BV * CP;
    float* Rtmp = reinterpret_cast<float*>(smem + SM::R4);
    uint16_t* A_hi = reinterpret_cast<uint16_t*>(smem + SM::R4);
    uint16_t* A_lo = A_hi + C * CP;
    uint16_t* P_hi = reinterpret_cast<uint16_t*>(smem + SM::R5);
    uint16_t* P_lo = P_hi + C * CP;
    uint16_t* Xt_hi = reinterpret_cast<uint16_t*>(smem + SM::R6);
    uint16_t* Xt_lo = Xt_hi + BV * CP;
    uint16_t* Sb = reinterpret_cast<uint16_t*>(smem + SM::R7);
    float* Gs = reinterpret_cast<float*>(smem + SM::R8);
    float* bs = reinterpret_cast<float*>(smem + SM::R9);
    float* gam = bs + C;
    float* psum = gam + BV;

    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t H = n_heads;
    const int h = u.head;
    const int i0 = u.vblk * BV;

    // ---- state: wave w owns S^T tile (j-tile jt, i-tile it) in fp32 accumulators
    const bool owns_s = wave < 2 * JT;
    const int s_jt = wave % JT, s_it = wave / JT;
    const int64_t s_base = ((static_cast<int64_t>(u.seq) * H + h) * DV + i0) * DK;
    f32x16 accS = {};
    if (owns_s) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = 32 * s_jt + acc_row(r, lane), i = 32 * s_it + (lane & 31);
            accS[r] = S0 ? S0[s_base + static_cast<int64_t>(i) * DK + j] : 0.f;
        }
    }

    // ---- register prefetch of one chunk's inputs
    u16x8 pk[KQ_PER_T], pq[KQ_PER_T], pv;
    f32x4 pa[A_PER_T];
    float pb = 0.f;
    auto prefetch = [&](int64_t tc, int n) {
#pragma unroll
        for (int p = 0; p < KQ_PER_T; ++p) {
            const int idx = tid + NT * p;
            const int t = idx / (DK / 8), c = idx % (DK / 8);
            pk[p] = u16x8{};
            pq[p] = u16x8{};
            if (idx < KQ_CHUNKS && t < n) {
                const int64_t g = ((tc + t) * H + h) * DK + 8 * c;
                pk[p] = *reinterpret_cast<const u16x8*>(k + g);
                pq[p] = *reinterpret_cast<const u16x8*>(q + g);
            }
        }
        {
            const int t = tid / (BV / 8), c = tid % (BV / 8);
            pv = u16x8{};
            if (t < n) pv = *reinterpret_cast<const u16x8*>(v + ((tc + t) * H + h) * DV + i0 + 8 * c);
        }
#pragma unroll
        for (int p = 0; p < A_PER_T; ++p) {
            const int idx = tid + NT * p;
            const int t = idx / (BV / 4), c = idx % (BV / 4);
            pa[p] = f32x4{1.f, 1.f, 1.f, 1.f};
            if (t < n) pa[p] = *reinterpret_cast<const f32x4*>(alpha + ((tc + t) * H + h) * DV + i0 + 4 * c);
        }
        if (tid < C) pb = tid < n ? beta[(tc + tid) * H + h] : 0.f;
    };

    auto chunk_len = [&](int64_t tc) { return static_cast<int>(min<int64_t>(C, u.t1 - tc)); };

    if (u.t0 < u.t1) prefetch(u.t0, chunk_len(u.t0));

    // bf16 copy of the entering state for the S-side products
    auto write_state_copy = [&]() {
        if (owns_s) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                // registers 4rb..4rb+3 hold 4 consecutive j of one i
                const int j = 32 * s_jt + 8 * rb + 4 * (lane >> 5), i = 32 * s_it + (lane & 31);
                u16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = f32_to_bf16_bits(accS[4 * rb + e]);
                *reinterpret_cast<u16x4*>(Sb + i * KP + j) = w;
            }
        }
    };
    write_state_copy();

    for (int64_t tc = u.t0; tc < u.t1; tc += C) {
        const int n = chunk_len(tc);
        __syncthreads();  // B0: the previous chunk is done with every buffer

        // ================= P0: stage the prefetched chunk into LDS
#pragma unroll
        for (int p = 0; p < KQ_PER_T; ++p) {
            const int idx = tid + NT * p;
            if (idx < KQ_CHUNKS) {
                const int t = idx / (DK / 8), c = idx % (DK / 8);
                *reinterpret_cast<u16x8*>(Kc + t * KP + 8 * c) = pk[p];
                *reinterpret_cast<u16x8*>(Qc + t * KP + 8 * c) = pq[p];
#pragma unroll
                for (int e = 0; e < 8; ++e) Kt[(8 * c + e) * CP + t] = pk[p][e];
            }
        }
        {
            const int t = tid / (BV / 8), c = tid % (BV / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) Xt_hi[(8 * c + e) * CP + t] = pv[e];  // raw V^T
        }
#pragma unroll
        for (int p = 0; p < A_PER_T; ++p) {
            const int idx = tid + NT * p;
            const int t = idx / (BV / 4), c = idx % (BV / 4);
            f32x4 la;
#pragma unroll
            for (int e = 0; e < 4; ++e) la[e] = __logf(pa[p][e]);
            *reinterpret_cast<f32x4*>(Gs + t * BV + 4 * c) = la;
        }
        if (tid < C) bs[tid] = pb;
        // next chunk's loads fly while this one computes
        if (tc + C < u.t1) prefetch(tc + C, chunk_len(tc + C));
        __syncthreads();  // B1

        // ================= P1: local scans of G; Gram products on waves 0..5
        const int gi = tid % BV, gpart = tid / BV;  // column i, rows 8*gpart .. 8*gpart+7
        float gl[8];
        {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc += Gs[(8 * gpart + e) * BV + gi];
                gl[e] = acc;
            }
            psum[gpart * BV + gi] = acc;
        }
        if (wave < 6) {
            // tiles (0,0), (1,0), (1,1) of L (waves 0-2) and of P (waves 3-5)
            const int tileid = wave % 3;
            const int tb = tileid == 0 ? 0 : 1, sb = tileid == 2 ? 1 : 0;
            const uint16_t* Aop = wave < 3 ? Kc : Qc;
            f32x16 acc = {};
#pragma unroll
            for (int kk = 0; kk < DK; kk += 16)
                acc = mfma(frag(Aop, KP, 32 * tb, kk, lane), frag(Kc, KP, 32 * sb, kk, lane), acc);
            const int col = 32 * sb + (lane & 31);
            if (wave < 3) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * tb + acc_row(r, lane);
                    Lf[row * LP + col] = col < row ? bs[row] * acc[r] : 0.f;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * tb + acc_row(r, lane);
                    uint16_t hi, lo;
                    split_bf16(col <= row ? acc[r] : 0.f, hi, lo);
                    P_hi[row * CP + col] = hi;
                    P_lo[row * CP + col] = lo;
                }
            }
        } else if (wave == 6) {
            // upper-right 32x32 block of P is zero
            for (int x = lane; x < 32 * 32; x += 64) {
                const int row = x / 32, col = 32 + x % 32;
                P_hi[row * CP + col] = 0;
                P_lo[row * CP + col] = 0;
            }
        }
        __syncthreads();  // B2

        // ================= P2: finish G, gamma, X = V e^{-G}; diagonal 16x16 inverses
        {
            float off = 0.f;
            for (int p = 0; p < gpart; ++p) off += psum[p * BV + gi];
            uint16_t xh[8], xl[8];
            const u16x8 vraw = *reinterpret_cast<const u16x8*>(Xt_hi + gi * CP + 8 * gpart);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = gl[e] + off;
                Gs[(8 * gpart + e) * BV + gi] = g;
                split_bf16(bf16_bits_to_f32(vraw[e]) * __expf(-g), xh[e], xl[e]);
            }
            if (gpart == 7) gam[gi] = __expf(gl[7] + off);
            u16x8 wh, wl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wh[e] = xh[e];
                wl[e] = xl[e];
            }
            *reinterpret_cast<u16x8*>(Xt_hi + gi * CP + 8 * gpart) = wh;
            *reinterpret_cast<u16x8*>(Xt_lo + gi * CP + 8 * gpart) = wl;
        }
        if (wave == 0) {
            // T_b = (I + L_bb)^{-1} for the four 16x16 diagonal blocks; lane = (block, column)
            const int b = lane >> 4, c = lane & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= Lf[(16 * b + r) * LP + 16 * b + s] * x[s];
                x[r] = r < c ? 0.f : acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Xs[(16 * b + r) * LP + 16 * b + c] = x[r];
        }
        __syncthreads();  // B3

        // ================= P3: off-diagonal blocks of (I + L)^{-1}, block row by block row
        // X[bi, :bi] = T_bi * ( - sum_{m < bi} L[bi, m] X[m, :bi] )
#pragma unroll 1
        for (int bi = 1; bi < 4; ++bi) {
            const int ncol = 16 * bi;
            for (int x = tid; x < 16 * ncol; x += NT) {
                const int r = x / ncol, col = x % ncol;
                const int mstart = col / 16;
                float acc = 0.f;
                for (int s = 16 * mstart; s < 16 * bi; ++s)
                    acc -= Lf[(16 * bi + r) * LP + s] * Xs[s * LP + col];
                Rtmp[r * 48 + col] = acc;
            }
            __syncthreads();
            for (int x = tid; x < 16 * ncol; x += NT) {
                const int r = x / ncol, col = x % ncol;
                float acc = 0.f;
                for (int s = 0; s <= r; ++s) acc += Xs[(16 * bi + r) * LP + 16 * bi + s] * Rtmp[s * 48 + col];
                Xs[(16 * bi + r) * LP + col] = acc;
            }
            __syncthreads();
        }
        // A = X diag(beta) as hi/lo bf16, zero above the diagonal
        for (int x = tid; x < C * C; x += NT) {
            const int t = x / C, s = x % C;
            uint16_t hi, lo;
            split_bf16(s <= t ? Xs[t * LP + s] * bs[s] : 0.f, hi, lo);
            A_hi[t * CP + s] = hi;
            A_lo[t * CP + s] = lo;
        }
        __syncthreads();  // B4

        // ================= P4: W = A K (all waves), U0 = A X (waves 0..3)
        {
            // W tiles: (tb, jb); 2*JT tiles over the waves
            f32x16 accW = {};
            const bool has_w = wave < 2 * JT;
            const int w_tb = wave / JT, w_jb = wave % JT;
            if (has_w) {
#pragma unroll
                for (int kk = 0; kk < 64; kk += 16) {
                    if (kk < 32 * (w_tb + 1)) {
                        const bf16x8 bk = frag(Kt, CP, 32 * w_jb, kk, lane);
                        accW = mfma(frag(A_hi, CP, 32 * w_tb, kk, lane), bk, accW);
                        accW = mfma(frag(A_lo, CP, 32 * w_tb, kk, lane), bk, accW);
                    }
                }
            }
            f32x16 accU = {};
            const int u_tb = wave >> 1, u_ib = wave & 1;  // waves 0..3
            if (wave < 4) {
#pragma unroll
                for (int kk = 0; kk < 64; kk += 16) {
                    if (kk < 32 * (u_tb + 1)) {
                        const bf16x8 ah = frag(A_hi, CP, 32 * u_tb, kk, lane);
                        const bf16x8 al = frag(A_lo, CP, 32 * u_tb, kk, lane);
                        const bf16x8 xh = frag(Xt_hi, CP, 32 * u_ib, kk, lane);
                        const bf16x8 xl = frag(Xt_lo, CP, 32 * u_ib, kk, lane);
                        accU = mfma(ah, xh, accU);
                        accU = mfma(al, xh, accU);
                        accU = mfma(ah, xl, accU);
                    }
                }
            }
            // -W as bf16 [t][j] into R0 (the solve scratch is dead after B4)
            if (has_w) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = 32 * w_tb + acc_row(r, lane), j = 32 * w_jb + (lane & 31);
                    Wn[t * KP + j] = f32_to_bf16_bits(-accW[r]);
                }
            }
            __syncthreads();  // B5

            // ============= P5: U = U0 - W S^T (waves 0..3); Q S^T (waves 4..7)
            f32x16 accO = {};
            const int o_tb = (wave - 4) >> 1, o_ib = (wave - 4) & 1;
            if (wave < 4) {
#pragma unroll
                for (int kk = 0; kk < DK; kk += 16)
                    accU = mfma(frag(Wn, KP, 32 * u_tb, kk, lane), frag(Sb, KP, 32 * u_ib, kk, lane), accU);
                // U^T hi/lo [i][t]: registers 4rb..4rb+3 are 4 consecutive t of one i
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int t = 32 * u_tb + 8 * rb + 4 * (lane >> 5), i = 32 * u_ib + (lane & 31);
                    u16x4 wh, wl;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint16_t hi, lo;
                        split_bf16(accU[4 * rb + e], hi, lo);
                        wh[e] = hi;
                        wl[e] = lo;
                    }
                    *reinterpret_cast<u16x4*>(Ut_hi + i * CP + t) = wh;
                    *reinterpret_cast<u16x4*>(Ut_lo + i * CP + t) = wl;
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < DK; kk += 16)
                    accO = mfma(frag(Qc, KP, 32 * o_tb, kk, lane), frag(Sb, KP, 32 * o_ib, kk, lane), accO);
            }
            __syncthreads();  // B6

            // ============= P6: O = e^G (Q S^T + P U) (waves 4..7); S^T += K^T U, decay (all)
            if (wave >= 4) {
#pragma unroll
                for (int kk = 0; kk < 64; kk += 16) {
                    if (kk < 32 * (o_tb + 1)) {
                        const bf16x8 ph = frag(P_hi, CP, 32 * o_tb, kk, lane);
                        const bf16x8 pl = frag(P_lo, CP, 32 * o_tb, kk, lane);
                        const bf16x8 uh = frag(Ut_hi, CP, 32 * o_ib, kk, lane);
                        const bf16x8 ul = frag(Ut_lo, CP, 32 * o_ib, kk, lane);
                        accO = mfma(ph, uh, accO);
                        accO = mfma(pl, uh, accO);
                        accO = mfma(ph, ul, accO);
                    }
                }
                const int i = 32 * o_ib + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = 32 * o_tb + acc_row(r, lane);
                    if (t < n) {
                        const float val = __expf(Gs[t * BV + i]) * accO[r];
                        o[((tc + t) * H + h) * DV + i0 + i] = f32_to_bf16_bits(val);
                    }
                }
            }
            if (owns_s) {
#pragma unroll
                for (int kk = 0; kk < 64; kk += 16) {
                    const bf16x8 kt = frag(Kt, CP, 32 * s_jt, kk, lane);
                    accS = mfma(kt, frag(Ut_hi, CP, 32 * s_it, kk, lane), accS);
                    accS = mfma(kt, frag(Ut_lo, CP, 32 * s_it, kk, lane), accS);
                }
                const float gm = gam[32 * s_it + (lane & 31)];
#pragma unroll
                for (int r = 0; r < 16; ++r) accS[r] *= gm;
            }
            write_state_copy();  // Sb is not read again in this chunk (last reader: P5)
        }
    }

    if (S_T && owns_s) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = 32 * s_jt + acc_row(r, lane), i = 32 * s_it + (lane & 31);
            S_T[s_base + static_cast<int64_t>(i) * DK + j] = accS[r];
        }
    }
}

template <int DK, int DV>
static hipError_t launch_mfma_t(const PrefillArgs& a, const int32_t* order, hipStream_t stream) {
    constexpr int NVB = DV / BV;
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((prefill_mfma_kernel<DK, DV>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0,
                       stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.alpha, a.beta, a.S0, a.cu_seqlens, order,
                       a.n_seq, a.n_tok, a.n_heads, static_cast<uint16_t*>(a.o), a.S_T);
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const int32_t* order = nullptr;
    if (a.cu_seqlens) {
        int32_t* ord = static_cast<int32_t*>(a.workspace);
        const hipError_t e = launch_schedule(a.cu_seqlens, a.n_seq, ord, stream);
        if (e != hipSuccess) return e;
        order = ord;
    }
    if (a.d_k == 128 && a.d_v == 128) return launch_mfma_t<128, 128>(a, order, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_mfma_t<64, 64>(a, order, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_mfma_t<128, 64>(a, order, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_mfma_t<64, 128>(a, order, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
