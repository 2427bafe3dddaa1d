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
//   U      = A (V (.) e^{-G} - K S^T)            (decay-normalised errors)
//   O      = e^{G} (.) (Q S^T + tril(Q K^T) U)   (tril keeps the diagonal: o_t = S_t q_t)
//   S'     = diag(e^{G[C-1,:]}) (S + U^T K)
// The decayed Gram of value row i is D_i L D_i^{-1} with D_i = diag(e^{G[:,i]}),
// so one decay-free solve serves every row; the decay moves onto V, O and S as
// elementwise scalings.  Token rows past the end of a sequence read as k = q =
// v = 0, beta = 0 and log alpha = 0, which change nothing.
//
// Work decomposition: one workgroup of 8 waves per (sequence, head, block of
// 64 value rows) walks its sequence chunk by chunk, holding S^T in fp32 MFMA
// accumulators (one 32x32 tile per wave) for the whole scan, with a bf16 copy
// in LDS as the operand of Q S^T and K S^T.  The S-independent solve runs on
// waves 0-3 while waves 4-7 form Q S^T and K S^T.  The next chunk's inputs are
// loaded into registers while the current chunk computes; barriers order LDS
// only, so those loads (and the output stores) stay in flight across them.
//
// Precision: q, k, v are exact bf16 inputs.  Computed operands are carried as
// hi + lo bf16 pairs (x = hi + lo to ~2^-16 relative) where the error budget
// needs it -- A, V e^{-G} - K S^T, U and P = tril(Q K^T) -- and S is a single
// bf16 copy of the fp32 state.  A product of two split operands takes three
// MFMAs (hi*hi + lo*hi + hi*lo).  The solve itself runs in fp32 (VALU forward
// substitution on 16x16 diagonal blocks, fp32 MFMA for the off-diagonal blocks).
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
// word 3 of a gfx9 buffer resource: raw (untyped) 32-bit data
constexpr int kBufferWord3 = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- MFMA helpers
// v_mfma_f32_32x32x16_bf16 operand layout: lane l supplies row (l & 31) of A
// (column (l & 31) of B) and the 8 consecutive reduction indices starting at
// 8 * (l >> 5).  Both operands are read from LDS buffers stored
// "reduction-index contiguous": A as [m][k], B as [n][k].
__device__ __forceinline__ bf16x8 frag(const uint16_t* base, int pitch, int row0, int k0, int lane) {
    const uint16_t* p = base + (row0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// The same for v_mfma_f32_16x16x32_bf16: row (l & 15), reduction indices 8 * (l >> 4) ...
__device__ __forceinline__ bf16x8 frag16(const uint16_t* base, int pitch, int row0, int k0, int lane) {
    const uint16_t* p = base + (row0 + (lane & 15)) * pitch + k0 + 8 * (lane >> 4);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16f(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Accumulator layout of a 32x32 tile: register r of lane l holds
// D[row = 8*(r/4) + 4*(l>>5) + (r&3)][col = l & 31]; of a 16x16 tile: register
// r holds D[4*(l>>4) + r][l & 15].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Compiler-only fence: the LDS operand loads above it are issued before the
// matrix instructions below it, so their latencies overlap instead of each
// MFMA waiting for its own freshly issued load.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Order this wave's own LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Buffer resource over [p, p + bytes): loads past the end return 0 and stores
// past the end are dropped, so a chunk's rows beyond its sequence need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kBufferWord3);
}

// Shared-memory layout (bytes).  Regions are reused across the phases of a
// chunk; the comments give each region's tenants in order.  Each region is its
// own __shared__ array, so the compiler knows that accesses to different
// regions never alias and can move loads ahead of unrelated stores.
template <int DK>
struct Smem {
    static constexpr int KP = DK + PAD;     // pitch of [t][j] bf16 rows
    static constexpr int CP = C + PAD;      // pitch of [x][t] bf16 rows (length C)
    // pitch of C x C fp32 rows: 80 = 16 mod 64 makes the column-wise operand
    // loads of the fp32 matrix-core solve (rows 4k + g, columns m) hit distinct banks
    static constexpr int LP = C + 16;
    static constexpr int RP = 48;           // pitch of the 32 x 32 solve temporary
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    static constexpr int HILO = 2 * C * CP * 2;  // a C x C (or BV x C) hi/lo bf16 pair
    // R0: K [t][j] -> solve temporary (fp32 32 x RP) -> A hi/lo [t][s]
    static constexpr int R0 = 0;
    static constexpr int R0_SZ = mx(mx(C * KP * 2, 32 * RP * 4), HILO);
    // R1: Q [t][j] -> Y^T hi/lo [i][t]
    static constexpr int R1 = R0 + R0_SZ;
    static constexpr int R1_SZ = mx(C * KP * 2, HILO);
    // R2: K^T [j][t]
    static constexpr int R2 = R1 + R1_SZ;
    static constexpr int R2_SZ = DK * CP * 2;
    // R3: L fp32 [t][s] -> U^T hi/lo [i][t]
    static constexpr int R3 = R2 + R2_SZ;
    static constexpr int R3_SZ = mx(C * LP * 4, HILO);
    // R4: (I + L)^{-1} fp32 [t][s] -> O bf16 [t][i] (stored at the next chunk)
    static constexpr int R4 = R3 + R3_SZ;
    static constexpr int R4_SZ = mx(C * LP * 4, C * (BV + PAD) * 2);
    // R5: P = tril(Q K^T) hi/lo [t][s]
    static constexpr int R5 = R4 + R4_SZ;
    static constexpr int R5_SZ = HILO;
    // R6: V bf16 [t][i] as loaded
    static constexpr int R6 = R5 + R5_SZ;
    static constexpr int R6_SZ = C * (BV + PAD) * 2;
    // R7: S bf16 [i][j] (operand copy of the fp32 state)
    static constexpr int R7 = R6 + R6_SZ;
    static constexpr int R7_SZ = BV * KP * 2;
    // R8: log alpha -> per-part local prefix sums -> G, fp32 [t][i]
    static constexpr int GP = BV + 4;       // pitch of G rows
    static constexpr int R8 = R7 + R7_SZ;
    static constexpr int R8_SZ = C * GP * 4;
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
    constexpr int KP = SM::KP, CP = SM::CP, LP = SM::LP, GP = SM::GP, RP = SM::RP;
    constexpr int OP = BV + PAD;           // pitch of the staged O and V rows
    constexpr int JT = DK / 32;            // 32-wide tiles along d_k

    __shared__ __align__(16) unsigned char r0[SM::R0_SZ];
    __shared__ __align__(16) unsigned char r1[SM::R1_SZ];
    __shared__ __align__(16) unsigned char r2[SM::R2_SZ];
    __shared__ __align__(16) unsigned char r3[SM::R3_SZ];
    __shared__ __align__(16) unsigned char r4[SM::R4_SZ];
    __shared__ __align__(16) unsigned char r5[SM::R5_SZ];
    __shared__ __align__(16) unsigned char r6[SM::R6_SZ];
    __shared__ __align__(16) unsigned char r7[SM::R7_SZ];
    __shared__ __align__(16) unsigned char r8[SM::R8_SZ];
    __shared__ __align__(16) unsigned char r9[SM::R9_SZ];
    uint16_t* Kc = reinterpret_cast<uint16_t*>(r0);
    float* Rtmp = reinterpret_cast<float*>(r0);
    uint16_t* A_hi = reinterpret_cast<uint16_t*>(r0);
    uint16_t* A_lo = A_hi + C * CP;
    uint16_t* Qc = reinterpret_cast<uint16_t*>(r1);
    uint16_t* Yt_hi = reinterpret_cast<uint16_t*>(r1);
    uint16_t* Yt_lo = Yt_hi + BV * CP;
    uint16_t* Kt = reinterpret_cast<uint16_t*>(r2);
    float* Lf = reinterpret_cast<float*>(r3);
    uint16_t* Ut_hi = reinterpret_cast<uint16_t*>(r3);
    uint16_t* Ut_lo = Ut_hi + BV * CP;
    float* Xs = reinterpret_cast<float*>(r4);
    uint16_t* Os = reinterpret_cast<uint16_t*>(r4);
    uint16_t* P_hi = reinterpret_cast<uint16_t*>(r5);
    uint16_t* P_lo = P_hi + C * CP;
    uint16_t* Vr = reinterpret_cast<uint16_t*>(r6);
    uint16_t* Sb = reinterpret_cast<uint16_t*>(r7);
    float* Gs = reinterpret_cast<float*>(r8);
    float* bs = reinterpret_cast<float*>(r9);
    float* gam = bs + C;
    float* psum = gam + BV;

    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform: keep it (and every tile offset derived from it) scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t H = n_heads;
    const int h = u.head;
    const int i0 = u.vblk * BV;
    const int64_t row_qk = H * DK, row_v = H * DV;  // element strides between tokens

    // ---- state: wave w owns S^T tile (j-tile s_jt, i-tile s_it) in fp32 accumulators
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

    // ---- register prefetch of one chunk's inputs; every load moves 16 bytes
    // per lane, so one wave instruction covers 1 KB of whole cache lines.
    // K, Q: thread (row pair tp, 16-byte chunk c) holds rows 2tp, 2tp+1 (with
    // d_k = 64 the upper four waves repeat the lower four).
    // V: thread (row td/8, 8 values at 8*(td%8)); alpha: rows td/16 and 32 + td/16,
    // 4 values at 4*(td%16); beta: wave 0, lane = token.
    const int kq_tp = lane & 31, kq_c = (2 * wave + (lane >> 5)) % (DK / 8);
    const int gpart = wave;
    u32x4 pk0 = {}, pk1 = {}, pq0 = {}, pq1 = {}, pv = {};
    f32x4 pa0 = {}, pa1 = {};
    float pb = 0.f;
    // Rows past the sequence end read as zeros through the buffer range, so
    // no load needs a per-row branch.
    auto prefetch = [&](int64_t tc, int n) {
        const int64_t tok0 = tc * H + h;  // (token tc, head h) row index
        {
            const int64_t bytes = ((n - 1) * row_qk + DK) * 2;
            const auto rk = make_rsrc(k + tok0 * DK, bytes);
            const auto rq = make_rsrc(q + tok0 * DK, bytes);
            const int off0 = static_cast<int>((2 * kq_tp) * row_qk + 8 * kq_c) * 2;
            const int off1 = off0 + static_cast<int>(row_qk) * 2;
            pk0 = __builtin_amdgcn_raw_buffer_load_b128(rk, off0, 0, 0);
            pk1 = __builtin_amdgcn_raw_buffer_load_b128(rk, off1, 0, 0);
            pq0 = __builtin_amdgcn_raw_buffer_load_b128(rq, off0, 0, 0);
            pq1 = __builtin_amdgcn_raw_buffer_load_b128(rq, off1, 0, 0);
        }
        {
            const auto rv = make_rsrc(v + tok0 * DV + i0, ((n - 1) * row_v + BV) * 2);
            pv = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>((tid >> 3) * row_v + 8 * (tid & 7)) * 2, 0, 0);
            const auto ra = make_rsrc(alpha + tok0 * DV + i0, ((n - 1) * row_v + BV) * 4);
            const int offa = static_cast<int>((tid >> 4) * row_v + 4 * (tid & 15)) * 4;
            pa0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, offa, 0, 0));
            pa1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, offa + static_cast<int>(32 * row_v) * 4, 0, 0));
        }
        if (wave == 0) {  // beta of token `lane`: one cache line per token, so one wave only
            const auto rb = make_rsrc(beta + tok0, ((n - 1) * H + 1) * 4);
            pb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(lane * H) * 4, 0, 0));
        }
    };

    auto chunk_len = [&](int64_t tc) { return static_cast<int>(min<int64_t>(C, u.t1 - tc)); };

    // staged O rows of a finished chunk -> global, one 16-byte store per thread
    auto store_o = [&](int64_t tc, int n, int td) {
        const int t = td >> 3, c = td & 7;
        const u32x4 val = *reinterpret_cast<const u32x4*>(Os + t * OP + 8 * c);
        const auto ro = make_rsrc(o + (tc * H + h) * DV + i0, ((n - 1) * row_v + BV) * 2);
        __builtin_amdgcn_raw_buffer_store_b128(val, ro, static_cast<int>(t * row_v + 8 * c) * 2, 0, 0);
    };

    if (u.t0 < u.t1) prefetch(u.t0, chunk_len(u.t0));

    // bf16 copy of the state for the S-side products (S^T registers 4rb..4rb+3
    // hold 4 consecutive key channels j of one value row i)
    auto write_state_copy = [&](int ln) {
        if (owns_s) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int j = 32 * s_jt + 8 * rb + 4 * (ln >> 5), i = 32 * s_it + (ln & 31);
                uint2 w;
                w.x = pack_bf16(accS[4 * rb], accS[4 * rb + 1]);
                w.y = pack_bf16(accS[4 * rb + 2], accS[4 * rb + 3]);
                *reinterpret_cast<uint2*>(Sb + i * KP + j) = w;
            }
        }
    };
    write_state_copy(lane);

    int64_t prev_tc = -1;
    int prev_n = 0;
    for (int64_t tc = u.t0; tc < u.t1; tc += C) {
        const int n = chunk_len(tc);
        // Lane-derived values are recomputed every chunk from an opaque copy of
        // the lane id, so the compiler does not hoist dozens of loop-invariant
        // LDS addresses into registers (which spills).
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int ln = lane_o;
        const int td = ln + 64 * wave;
        const int g16 = ln >> 4, m16 = ln & 15;
        block_sync();  // the previous chunk is done with every buffer

        // ======== stage this chunk; log-decay local scan (into G); previous
        // chunk's O out; next chunk's loads in (they fly while this chunk computes)
        {
            const int rr = 2 * (ln & 31), c = (2 * wave + (ln >> 5)) % (DK / 8);
            *reinterpret_cast<u32x4*>(Kc + rr * KP + 8 * c) = pk0;
            *reinterpret_cast<u32x4*>(Kc + (rr + 1) * KP + 8 * c) = pk1;
            *reinterpret_cast<u32x4*>(Qc + rr * KP + 8 * c) = pq0;
            *reinterpret_cast<u32x4*>(Qc + (rr + 1) * KP + 8 * c) = pq1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // bf16 e of row rr (low half) and of row rr + 1 (high half)
                const uint32_t lo = pk0[e >> 1] >> (16 * (e & 1)), hi = pk1[e >> 1] >> (16 * (e & 1));
                *reinterpret_cast<uint32_t*>(Kt + (8 * c + e) * CP + rr) = (lo & 0xffffu) | (hi << 16);
            }
        }
        if (td < C) bs[td] = pb;
        *reinterpret_cast<u32x4*>(Vr + (td >> 3) * OP + 8 * (td & 7)) = pv;
        {
            // log alpha, 0 for rows past the sequence end (they read as alpha = 0)
            const int t = td >> 4, c = 4 * (td & 15);
            f32x4 l0, l1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l0[e] = t < n ? __logf(pa0[e]) : 0.f;
                l1[e] = t + 32 < n ? __logf(pa1[e]) : 0.f;
            }
            *reinterpret_cast<f32x4*>(Gs + t * GP + c) = l0;
            *reinterpret_cast<f32x4*>(Gs + (t + 32) * GP + c) = l1;
        }
        if (prev_tc >= 0) store_o(prev_tc, prev_n, td);
        if (tc + C < u.t1) prefetch(tc + C, chunk_len(tc + C));
        block_sync();

        // ======== Gram products.  Wave 0: the four 16x16 diagonal blocks of L and
        // their inverses T_b = (I + L_bb)^{-1} (forward substitution, lane =
        // (block, column)).  Waves 1-3: the rest of L = strictly_lower(diag(beta)
        // K K^T) (tile (1,0) and the two sub-diagonal 16x16 blocks).  Waves 4-6:
        // P = tril(Q K^T) as hi/lo bf16, formed transposed (D[s][t]) so that each
        // lane holds 4 consecutive s of one row t.
        // local prefix sums of log alpha: thread (column ln, rows 8*gpart .. 8*gpart+7)
        {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc += Gs[(8 * gpart + e) * GP + ln];
                Gs[(8 * gpart + e) * GP + ln] = acc;
            }
            psum[gpart * BV + ln] = acc;
        }
        if (wave == 0) {
            f32x4 d[4] = {};
            bf16x8 kf[4][DK / 32];
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) kf[b][kk] = frag16(Kc, KP, 16 * b, 32 * kk, ln);
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
                for (int b = 0; b < 4; ++b) d[b] = mfma16(kf[b][kk], kf[b][kk], d[b]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + 16 * b + 4 * g16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * g16 + r;  // within the block
                    Lf[(16 * b + row) * LP + 16 * b + m16] = m16 < row ? b4[r] * d[b][r] : 0.f;
                }
            }
            wave_lds_sync();
            const int b = g16, c = m16;
            const float* Lb = Lf + (16 * b) * LP + 16 * b;
            // Row pieces of the strictly lower block are loaded in two batches
            // (rows 1-9, then rows 10-15 once rows 0-5 are done), so no LDS round
            // trip sits inside the dependent substitution chain.
            f32x4 lrow[36];
            auto load_rows = [&](int r_lo, int r_hi) {
#pragma unroll
                for (int r = 1, p = 0; r < 16; ++r)
#pragma unroll
                    for (int s4 = 0; s4 < r; s4 += 4, ++p)
                        if (r >= r_lo && r < r_hi) lrow[p] = *reinterpret_cast<const f32x4*>(Lb + r * LP + s4);
            };
            float x[16];
            auto solve_rows = [&](int r_lo, int r_hi) {
#pragma unroll
                for (int r = 0, p = 0; r < 16; ++r) {
                    float acc0 = (r == c) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                    for (int s4 = 0; s4 < r; s4 += 4, ++p) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (r >= r_lo && r < r_hi && s4 + e < r) {
                                if (e & 1) acc1 -= lrow[p][e] * x[s4 + e];
                                else acc0 -= lrow[p][e] * x[s4 + e];
                            }
                        }
                    }
                    if (r >= r_lo && r < r_hi) x[r] = acc0 + acc1;  // zero for r < c
                }
            };
            load_rows(1, 10);
            issue_fence();
            solve_rows(0, 6);
            load_rows(10, 16);
            issue_fence();
            solve_rows(6, 16);
#pragma unroll
            for (int r = 0; r < 16; ++r) Xs[(16 * b + r) * LP + 16 * b + c] = x[r];
        } else if (wave == 1) {
            // tile (1,0): rows 32-63 x cols 0-31
            f32x16 acc = {};
            bf16x8 fa[DK / 16], fb[DK / 16];
#pragma unroll
            for (int kk = 0; kk < DK / 16; ++kk) {
                fa[kk] = frag(Kc, KP, 32, 16 * kk, ln);
                fb[kk] = frag(Kc, KP, 0, 16 * kk, ln);
            }
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < DK / 16; ++kk) acc = mfma(fa[kk], fb[kk], acc);
            f32x4 b4[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) b4[rb] = *reinterpret_cast<const f32x4*>(bs + 32 + 8 * rb + 4 * (ln >> 5));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 + acc_row(r, ln);
                Lf[row * LP + (ln & 31)] = b4[r >> 2][r & 3] * acc[r];
            }
        } else if (wave < 4) {
            // the 16x16 blocks (16..31, 0..15) (wave 2) and (48..63, 32..47) (wave 3)
            const int R = wave == 2 ? 16 : 48, Cc = R - 16;
            f32x4 d = {};
            bf16x8 fa[DK / 32], fb[DK / 32];
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                fa[kk] = frag16(Kc, KP, R, 32 * kk, ln);
                fb[kk] = frag16(Kc, KP, Cc, 32 * kk, ln);
            }
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) d = mfma16(fa[kk], fb[kk], d);
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + R + 4 * g16);
#pragma unroll
            for (int r = 0; r < 4; ++r) Lf[(R + 4 * g16 + r) * LP + Cc + m16] = b4[r] * d[r];
        } else if (wave < 7) {
            // P^T tiles (s-tile, t-tile) = (0,0), (0,1), (1,1)
            const int sb = wave == 6 ? 1 : 0, tb = wave == 4 ? 0 : 1;
            f32x16 acc = {};
            bf16x8 fa[DK / 16], fb[DK / 16];
#pragma unroll
            for (int kk = 0; kk < DK / 16; ++kk) {
                fa[kk] = frag(Kc, KP, 32 * sb, 16 * kk, ln);
                fb[kk] = frag(Qc, KP, 32 * tb, 16 * kk, ln);
            }
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < DK / 16; ++kk) acc = mfma(fa[kk], fb[kk], acc);
            const int t = 32 * tb + (ln & 31);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int s0 = 32 * sb + 8 * rb + 4 * (ln >> 5);
                float pv4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pv4[e] = s0 + e <= t ? acc[4 * rb + e] : 0.f;
                uint2 wh, wl;
                split_bf16x2(pv4[0], pv4[1], wh.x, wl.x);
                split_bf16x2(pv4[2], pv4[3], wh.y, wl.y);
                *reinterpret_cast<uint2*>(P_hi + t * CP + s0) = wh;
                *reinterpret_cast<uint2*>(P_lo + t * CP + s0) = wl;
            }
        }
        block_sync();

        // ======== finish G and gamma (all waves, thread = (column ln, 8 rows));
        // solve level 2 (waves 0, 1): X[R, Cc] = -T_R L[R, Cc] T_Cc for the 16x16
        // blocks (16, 0) and (48, 32); waves 4-7: O^T = S Q^T and K S^T
        {
            float off = 0.f;
            for (int p = 0; p < gpart; ++p) off += psum[p * BV + ln];
#pragma unroll
            for (int e = 0; e < 8; ++e) Gs[(8 * gpart + e) * GP + ln] += off;
            if (gpart == 7) gam[ln] = __expf(Gs[63 * GP + ln]);
        }
        f32x16 accO = {}, accY = {};
        const int o_ib = (wave - 4) >> 1, o_tb = (wave - 4) & 1;  // O^T tile (i-tile, t-tile)
        const int y_tb = o_tb, y_ib = o_ib;  // (K S^T) tile (t-tile, i-tile): shares the S operand
        if (wave < 2) {
            const int R = 16 * (2 * wave + 1), Cc = 16 * (2 * wave);
            float la[4], xa[4], ta[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                la[kk] = Lf[(R + m16) * LP + Cc + 4 * kk + g16];
                xa[kk] = Xs[(Cc + 4 * kk + g16) * LP + Cc + m16];
                ta[kk] = Xs[(R + m16) * LP + R + 4 * g16 + kk];
            }
            issue_fence();
            f32x4 y = {};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) y = mfma16f(la[kk], xa[kk], y);
            // y (row 4*g16 + r, column m16) feeds the next product directly as its B
            // operand: step r uses reduction index 4*g16 + r, matched on the A side
            f32x4 z = {};
#pragma unroll
            for (int r = 0; r < 4; ++r) z = mfma16f(ta[r], y[r], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) Xs[(R + 4 * g16 + r) * LP + Cc + m16] = -z[r];
        } else if (wave >= 4) {
            // two batches of four reduction steps bound the operand registers
#pragma unroll
            for (int half = 0; half < DK / 64; ++half) {
                bf16x8 fs[4], fq[4], fk[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k0 = 64 * half + 16 * kk;
                    fs[kk] = frag(Sb, KP, 32 * o_ib, k0, ln);
                    fq[kk] = frag(Qc, KP, 32 * o_tb, k0, ln);
                    fk[kk] = frag(Kc, KP, 32 * y_tb, k0, ln);
                }
                issue_fence();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    accO = mfma(fs[kk], fq[kk], accO);
                    accY = mfma(fk[kk], fs[kk], accY);
                }
            }
        }
        block_sync();

        // ======== solve level 3a (waves 0-3): Y2 = L[32:64, 0:32] X[0:32, 0:32], one
        // 16x16 quadrant (qr, qc) per wave, into Rtmp [32][RP]; waves 4-7:
        // Y = V e^{-G} - K S^T -> Y^T hi/lo [i][t]
        const int qr = wave >> 1, qc = wave & 1;
        if (wave < 4) {
            float la[8], xa[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                la[kk] = Lf[(32 + 16 * qr + m16) * LP + 4 * kk + g16];
                xa[kk] = Xs[(4 * kk + g16) * LP + 16 * qc + m16];
            }
            issue_fence();
            f32x4 y = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (kk >= 4 * qc)  // X[0:32, 0:32] is lower triangular by 16x16 blocks
                    y = mfma16f(la[kk], xa[kk], y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Rtmp[(16 * qr + 4 * g16 + r) * RP + 16 * qc + m16] = y[r];
        } else {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                // registers 4rb..4rb+3: 4 consecutive t of one i
                const int t = 32 * y_tb + 8 * rb + 4 * (ln >> 5), i = 32 * y_ib + (ln & 31);
                float xv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xv[e] = bf16_bits_to_f32(Vr[(t + e) * OP + i]) * __expf(-Gs[(t + e) * GP + i]);
                uint2 wh, wl;
                split_bf16x2(xv[0] - accY[4 * rb], xv[1] - accY[4 * rb + 1], wh.x, wl.x);
                split_bf16x2(xv[2] - accY[4 * rb + 2], xv[3] - accY[4 * rb + 3], wh.y, wl.y);
                *reinterpret_cast<uint2*>(Yt_hi + i * CP + t) = wh;
                *reinterpret_cast<uint2*>(Yt_lo + i * CP + t) = wl;
            }
        }
        block_sync();

        // ======== solve level 3b (waves 0-3): X[32:64, 0:32] = -X[32:64, 32:64] Y2
        if (wave < 4) {
            float xa[8], ra[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                xa[kk] = Xs[(32 + 16 * qr + m16) * LP + 32 + 4 * kk + g16];
                ra[kk] = Rtmp[(4 * kk + g16) * RP + 16 * qc + m16];
            }
            issue_fence();
            f32x4 z = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (kk < 4 * (qr + 1))  // X[32:64, 32:64] is lower triangular by blocks
                    z = mfma16f(xa[kk], ra[kk], z);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Xs[(32 + 16 * qr + 4 * g16 + r) * LP + 16 * qc + m16] = -z[r];
        }
        block_sync();

        // ======== A = (I + L)^{-1} diag(beta) as hi/lo bf16, zero above the diagonal;
        // each thread converts 8 consecutive entries of one row
        {
            const int t = td >> 3, s0 = 8 * (td & 7);
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(Xs + t * LP + s0);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(Xs + t * LP + s0 + 4);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(bs + s0);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(bs + s0 + 4);
            float av[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = e < 4 ? x0[e] * b0[e] : x1[e - 4] * b1[e - 4];
                av[e] = s0 + e <= t ? xv : 0.f;
            }
            u32x4 wh, wl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t a, b;
                split_bf16x2(av[2 * e], av[2 * e + 1], a, b);
                wh[e] = a;
                wl[e] = b;
            }
            *reinterpret_cast<u32x4*>(A_hi + t * CP + s0) = wh;
            *reinterpret_cast<u32x4*>(A_lo + t * CP + s0) = wl;
        }
        block_sync();

        // ======== U = A Y (waves 0-3) -> U^T hi/lo [i][t]
        if (wave < 4) {
            const int u_tb = wave >> 1, u_ib = wave & 1;
            f32x16 accU = {};
            bf16x8 ah[4], al[4], yh[4], yl[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 * (u_tb + 1)) {  // A is lower triangular
                    ah[kk] = frag(A_hi, CP, 32 * u_tb, 16 * kk, ln);
                    al[kk] = frag(A_lo, CP, 32 * u_tb, 16 * kk, ln);
                    yh[kk] = frag(Yt_hi, CP, 32 * u_ib, 16 * kk, ln);
                    yl[kk] = frag(Yt_lo, CP, 32 * u_ib, 16 * kk, ln);
                }
            }
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 * (u_tb + 1)) {
                    accU = mfma(ah[kk], yh[kk], accU);
                    accU = mfma(al[kk], yh[kk], accU);
                    accU = mfma(ah[kk], yl[kk], accU);
                }
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int t = 32 * u_tb + 8 * rb + 4 * (ln >> 5), i = 32 * u_ib + (ln & 31);
                uint2 wh, wl;
                split_bf16x2(accU[4 * rb], accU[4 * rb + 1], wh.x, wl.x);
                split_bf16x2(accU[4 * rb + 2], accU[4 * rb + 3], wh.y, wl.y);
                *reinterpret_cast<uint2*>(Ut_hi + i * CP + t) = wh;
                *reinterpret_cast<uint2*>(Ut_lo + i * CP + t) = wl;
            }
        }
        block_sync();

        // ======== O^T = e^G (S Q^T + U^T P^T) staged as bf16 O [t][i] (waves 4-7);
        // S^T = diag(gamma)(S^T + K^T U) (all waves)
        if (wave >= 4) {
            bf16x8 uh[4], ul[4], ph[4], pl[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 * (o_tb + 1)) {  // P is lower triangular
                    uh[kk] = frag(Ut_hi, CP, 32 * o_ib, 16 * kk, ln);
                    ul[kk] = frag(Ut_lo, CP, 32 * o_ib, 16 * kk, ln);
                    ph[kk] = frag(P_hi, CP, 32 * o_tb, 16 * kk, ln);
                    pl[kk] = frag(P_lo, CP, 32 * o_tb, 16 * kk, ln);
                }
            }
            const int tq = 32 * o_tb + (ln & 31);
            f32x4 g4[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                g4[rb] = *reinterpret_cast<const f32x4*>(Gs + tq * GP + 32 * o_ib + 8 * rb + 4 * (ln >> 5));
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 * (o_tb + 1)) {
                    accO = mfma(uh[kk], ph[kk], accO);
                    accO = mfma(ul[kk], ph[kk], accO);
                    accO = mfma(uh[kk], pl[kk], accO);
                }
            }
            const int t = tq;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int i = 32 * o_ib + 8 * rb + 4 * (ln >> 5);
                uint2 w;
                w.x = pack_bf16(__expf(g4[rb][0]) * accO[4 * rb], __expf(g4[rb][1]) * accO[4 * rb + 1]);
                w.y = pack_bf16(__expf(g4[rb][2]) * accO[4 * rb + 2], __expf(g4[rb][3]) * accO[4 * rb + 3]);
                *reinterpret_cast<uint2*>(Os + t * OP + i) = w;
            }
        }
        if (owns_s) {
            bf16x8 kt[4], uh[4], ul[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                kt[kk] = frag(Kt, CP, 32 * s_jt, 16 * kk, ln);
                uh[kk] = frag(Ut_hi, CP, 32 * s_it, 16 * kk, ln);
                ul[kk] = frag(Ut_lo, CP, 32 * s_it, 16 * kk, ln);
            }
            const float gm = gam[32 * s_it + (ln & 31)];
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                accS = mfma(kt[kk], uh[kk], accS);
                accS = mfma(kt[kk], ul[kk], accS);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) accS[r] *= gm;
        }
        write_state_copy(ln);  // the last readers of the old copy were S Q^T and K S^T
        prev_tc = tc;
        prev_n = n;
    }
    if (prev_tc >= 0) {
        block_sync();
        store_o(prev_tc, prev_n, tid);
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
