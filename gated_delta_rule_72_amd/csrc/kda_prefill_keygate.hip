// kda_prefill_keygate.hip -- chunkwise prefill for bf16 inputs with the forget
// gate on key channels (S~ = S diag(alpha_t), alpha_t in R^{d_k}), on CDNA4
// matrix cores (bf16 MFMA with fp32 accumulation).
//
// Method: page "Kimi (AI)", section "Kimi Delta Attention (KDA)" -- the three
// steps (forget gating, prediction, delta update) per token, with the gate
// diagonal on the key side of the d_v x d_k state, the channel-wise forgetting
// the transcript page "Per dins de Kimi K3 ..." describes.  Within a chunk of
// C tokens (S entering the chunk, all per key channel j):
//   G[t,j]  = sum_{s<=t} log2 alpha[s,j]                 (base-2 log-decays)
//   M[t,r]  = sum_j k_t[j] k_r[j] 2^{G[t,j] - G[r,j]}    (r < t, decayed Gram)
//   Pd[t,r] = sum_j q_t[j] k_r[j] 2^{G[t,j] - G[r,j]}    (r <= t)
//   A       = (I + strictly_lower(diag(beta) M))^{-1} diag(beta)
//   U       = A (V - Kh S^T),          Kh = K (.) 2^{G}
//   O       = Qh S^T + Pd U,           Qh = Q (.) 2^{G}
//   S'      = S diag(2^{G[C-1,:]}) + U^T Kt,   Kt = K (.) 2^{G[C-1,:] - G}
// Unlike the value-row gate, the decay sits on the contraction index of K K^T,
// so it cannot be factored out of the solve: every chunk has its own decayed
// Gram.  Every factor the scan needs (2^{G}, 2^{G[C-1] - G}, the gamma of the
// state) is a power of two of a non-positive exponent, so the scan has no range
// limit; only the Grams pair a decay with its inverse.
//
// Two kernels.
// keygate_solve_kernel, one workgroup per (chunk, head), all in parallel: M and
// Pd on MFMA from exponent-scaled operands, the solve for A (kda_solve.h), and
// A and Pd written as solved records.  The chunk is cut into four 16-token
// sub-chunks, one per wave.  A block (a, b) of sub-chunks b < a pairs rows t of
// a with rows r of b through the reference point just before sub-chunk a:
//   2^{G_t - G_r} = 2^{G_t - G_ref} 2^{G_ref - G_r},  both factors <= 1,
// so off the diagonal nothing can overflow.  A diagonal block takes its
// reference at its own 8th token: one factor of each pair exceeds 1 by at most
// the decay of half a sub-chunk.  A chunk where some channel decays by more than
// 2^-KG_RANGE over such a half (alpha = 0 and NaN included) is marked, and its
// (sequence, head) is recomputed token by token (the range fixup).
// keygate_scan_kernel: one workgroup of 8 waves per (sequence, head, block of 64
// value rows) walks the chunks with S^T in fp32 MFMA accumulators, as the
// value-row scan does (kda_prefill_mfma.hip); the loader waves read alpha on the
// key channels and form Kh, Qh, Kt and gamma while staging the chunk.
//
// Precision: Kh and Qh are single bf16 (their rounding reaches the state only
// through the delta rule's own correction, or only the output); Kt, A, Pd, the
// errors Y and U are hi + lo bf16 pairs (x = hi + lo to ~2^-16); S is a single
// bf16 copy of the fp32 state.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_schedule.h"
#include "kda_solve.h"

namespace kda {

namespace {

// Largest log2-decay magnitude over half a sub-chunk that the diagonal Gram blocks
// accept; their operands then stay within 2^{+-64} of k and q.
constexpr float KG_RANGE = 64.f;
constexpr int KG_SUB = 16;  // tokens per sub-chunk (one wave of the solve kernel)
constexpr int KG_MID = 7;   // reference token of a diagonal block, within its sub-chunk

// The 32x32 block of a solved record that holds rows 16 tt .. 16 tt + 15 and
// columns 32 kh .. 32 kh + 31 (kh = 1 only for tt >= 2).
__device__ __forceinline__ int record_block(int tt, int kh) { return tt < 2 ? 0 : (kh ? 2 : 1); }

// hi + lo bf16 split of 8 floats, as two MFMA operands
__device__ __forceinline__ void split8f(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t a, b;
        split_bf16x2(x[2 * e], x[2 * e + 1], a, b);
        h[e] = a;
        l[e] = b;
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ f32x4 mfma_hilo(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma16(ah, bh, c);
    c = mfma16(al, bh, c);
    return mfma16(ah, bl, c);
}

// element x of 8 bf16 packed in four words (low half first)
__device__ __forceinline__ float bf16_elem(const u32x4& w, int x) {
    return x & 1 ? __uint_as_float(w[x >> 1] & 0xffff0000u) : __uint_as_float(w[x >> 1] << 16);
}

}  // namespace

// ============================================================================
// keygate_solve_kernel: A and Pd of one (chunk, head) per workgroup of 4 waves.
// Wave a owns sub-chunk a: lane (g = lane / 16, m = lane % 16) holds token
// 16 a + m at key channels 32 kk + 8 g .. +7 (kk = 0 .. d_k/32 - 1), the layout of
// a v_mfma_f32_16x16x32_bf16 operand row, loaded straight from global memory.
// Its local log2-decay prefix P[t] (over the sub-chunk, inclusive) is a scan
// across the 16 lanes of a DPP row.  Blocks are formed transposed (D[r][t], so a
// lane holds four consecutive r of one t) and written as whole 8- or 16-byte
// rows of L and of the Pd record.
// ============================================================================
template <int DK>
__global__ __launch_bounds__(256, 3) void keygate_solve_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_off,
    int n_seq, int n_tok, int n_heads, uint16_t* __restrict__ arec, uint16_t* __restrict__ prec,
    int32_t* __restrict__ cmark) {
    constexpr int NK = DK / 32;      // 32-channel reduction steps
    constexpr int RBP = DK + 4;      // pitch (fp32) of the right-operand bases
    constexpr int RB_BYTES = 3 * KG_SUB * RBP * 4;
    constexpr int XS_BYTES = C * LP * 4;
    constexpr int RFP = DK + PAD;    // pitch (bf16) of the one-reference right operands
    constexpr int RF_BYTES = 2 * 3 * KG_SUB * RFP * 2;
    constexpr int U1 = RB_BYTES > XS_BYTES ? RB_BYTES : XS_BYTES;
    constexpr int UX = U1 > RF_BYTES ? U1 : RF_BYTES;
    // the right operands (either form) are dead once L is formed, so X reuses their
    // space; the 32x32 temporary of the solve reuses rows 0-16 of L
    __shared__ __align__(16) unsigned char rx_[UX];
    __shared__ __align__(16) float Lf[C * LP];
    __shared__ __align__(16) float Tt[4 * DK];  // sub-chunk totals of log2 alpha
    __shared__ __align__(16) float bs[C];
    __shared__ int marks[4];
    static_assert(32 * SOLVE_RP <= 17 * LP, "temporary fits in rows 0-16 of L");
    float* RBs = reinterpret_cast<float*>(rx_);  // [3][16][RBP]: K (.) 2^{T_b - P_b} of sub-chunks 0-2
    uint16_t* RFh = reinterpret_cast<uint16_t*>(rx_);  // [48][RFP] hi, then lo: one-reference right operands
    uint16_t* RFl = RFh + 3 * KG_SUB * RFP;
    float* Xs = reinterpret_cast<float*>(rx_);

    const int64_t H = n_heads;
    const int item = blockIdx.x;
    if (item >= first_chunk(n_seq, n_seq, n_tok, chunk_off) * n_heads) return;
    const int gc = item / n_heads, h = item % n_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // = sub-chunk a
    const int g = lane >> 4, m16 = lane & 15;
    const ChunkRef ch = chunk_ref(gc, n_seq, n_tok, cu_seqlens, chunk_off);  // ch.n >= 1
    const int t = KG_SUB * wave + m16;  // this lane's token within the chunk
    const int64_t tok0 = ch.t0 * H + h;
    const int64_t row_bytes = ((ch.n - 1) * H * DK + DK) * 2;
    const auto rk = make_rsrc(k + tok0 * DK, row_bytes);
    const auto rq = make_rsrc(q + tok0 * DK, row_bytes);
    const auto ra = make_rsrc(alpha + tok0 * DK, 2 * row_bytes);
    const auto rbt = make_rsrc(beta + tok0, ((ch.n - 1) * H + 1) * 4);

    // ---- loads: k, q, alpha of this lane's token and channels (rows past the end read 0)
    u32x4 kf[NK], qf[NK];
    float P[NK][8];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int e = static_cast<int>(t * H * DK + 32 * kk + 8 * g);
        kf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, e * 2, 0, 0);
        qf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, e * 2, 0, 0);
        const u32x4 a0 = __builtin_amdgcn_raw_buffer_load_b128(ra, e * 4, 0, 0);
        const u32x4 a1 = __builtin_amdgcn_raw_buffer_load_b128(ra, e * 4 + 16, 0, 0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            P[kk][x] = __uint_as_float(a0[x]);
            P[kk][4 + x] = __uint_as_float(a1[x]);
        }
    }
    const float bt =
        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rbt, static_cast<int>(t * H) * 4, 0, 0));
    auto kv = [&](int kk, int x) { return bf16_elem(kf[kk], x); };
    auto qv = [&](int kk, int x) { return bf16_elem(qf[kk], x); };

    // ---- local inclusive prefix of log2 alpha over the sub-chunk (rows past the end
    // contribute 0): Hillis-Steele over the 16 lanes of each DPP row
    const bool live = t < ch.n;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            float v = live ? __builtin_amdgcn_logf(P[kk][x]) : 0.f;
            v += dpp_mov<0x111>(v);  // row_shr:1 (lanes shifted in from outside the row read 0)
            v += dpp_mov<0x112>(v);  // row_shr:2
            v += dpp_mov<0x114>(v);  // row_shr:4
            v += dpp_mov<0x118>(v);  // row_shr:8
            P[kk][x] = v;
        }

    // ---- the sub-chunk totals T (lane 15 of each row holds P[15]) and beta
    if (m16 == 15) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
            for (int x = 0; x < 8; ++x) Tt[wave * DK + 32 * kk + 8 * g + x] = P[kk][x];
    }
    if (g == 0) bs[t] = bt;
    block_sync();  // totals

    // ---- one reference for the whole chunk (the end of token 31) when both halves
    // of the chunk decay by at most 2^-KG_RANGE on every channel; the same test on
    // the same totals in every wave, so the choice is uniform.  (False for NaN.)
    bool half_ok = true;
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) {
        const int j = (DK / 64) * lane + c;
        half_ok = half_ok && Tt[j] + Tt[DK + j] >= -KG_RANGE && Tt[2 * DK + j] + Tt[3 * DK + j] >= -KG_RANGE;
    }
    const bool whole = __builtin_amdgcn_ballot_w64(!half_ok) == 0;

    uint16_t* prec_c = prec + static_cast<int64_t>(item) * (A_RECORD_BYTES / 2);
    // one transposed 16x16 block (rows r = 16 b + 4g + e, column t = 16 a + m16) into
    // L (scaled by beta_t, strictly lower) and into the Pd record (lower, diagonal
    // included)
    auto put_block = [&](int b, const f32x4& mT, const f32x4& pT) {
        const int s0 = KG_SUB * b + 4 * g;
        f32x4 lv, pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lv[e] = s0 + e < t ? bt * mT[e] : 0.f;
            pv[e] = s0 + e <= t ? pT[e] : 0.f;
        }
        *reinterpret_cast<f32x4*>(Lf + t * LP + s0) = lv;
        const int blk = record_block(wave, b >= 2);
        uint16_t* dst = prec_c + blk * 2 * A_BLOCK_ELEMS + (t & 31) * 32 + (s0 & 31);
        uint2 wh, wl;
        split_bf16x2(pv[0], pv[1], wh.x, wl.x);
        split_bf16x2(pv[2], pv[3], wh.y, wl.y);
        *reinterpret_cast<uint2*>(dst) = wh;
        *reinterpret_cast<uint2*>(dst + A_BLOCK_ELEMS) = wl;
    };
    // the zero quadrants of the Pd record: rows 0-15 x cols 16-31 and rows 32-47 x cols 48-63
    if (wave == 0 || wave == 2) {
        uint16_t* dst = prec_c + (wave == 0 ? 0 : 2) * 2 * A_BLOCK_ELEMS + m16 * 32 + 16 + 4 * g;
        *reinterpret_cast<uint2*>(dst) = uint2{0u, 0u};
        *reinterpret_cast<uint2*>(dst + A_BLOCK_ELEMS) = uint2{0u, 0u};
    }

    bool any_bad = false;
    if (whole) {
        // ======== one reference: d_t = G_t - G_31 (a sum over the tokens between, from
        // the local prefix and whole sub-chunk totals; |d_t| <= KG_RANGE), left operands
        // k_t, q_t times 2^{d_t}, right operand k_r times 2^{-d_r}.  The right
        // operands of sub-chunks 0-2 go to LDS (hi/lo) for the waves after them.
        bf16x8 lkh[NK], lkl[NK], lqh[NK], lql[NK];
        f32x4 mT = {}, pT = {};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int j0 = 32 * kk + 8 * g;
            float lk[8], lq[8], rr[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int j = j0 + x;
                const float d = wave == 0   ? (P[kk][x] - Tt[j]) - Tt[DK + j]
                                : wave == 1 ? P[kk][x] - Tt[DK + j]
                                : wave == 2 ? P[kk][x]
                                            : P[kk][x] + Tt[2 * DK + j];
                const float up = __builtin_amdgcn_exp2f(d), dn = __builtin_amdgcn_exp2f(-d);
                lk[x] = kv(kk, x) * up;
                lq[x] = qv(kk, x) * up;
                rr[x] = kv(kk, x) * dn;
            }
            bf16x8 rh, rl;
            split8f(lk, lkh[kk], lkl[kk]);
            split8f(lq, lqh[kk], lql[kk]);
            split8f(rr, rh, rl);
            if (wave < 3) {
                *reinterpret_cast<bf16x8*>(RFh + (KG_SUB * wave + m16) * RFP + j0) = rh;
                *reinterpret_cast<bf16x8*>(RFl + (KG_SUB * wave + m16) * RFP + j0) = rl;
            }
            mT = mfma_hilo(rh, rl, lkh[kk], lkl[kk], mT);
            pT = mfma_hilo(rh, rl, lqh[kk], lql[kk], pT);
        }
        put_block(wave, mT, pT);
        block_sync();  // right operands
        if (wave > 0) {
            f32x4 mB[3] = {}, pB[3] = {};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    if (b >= wave) continue;
                    const bf16x8 rh = frag16(RFh, RFP, KG_SUB * b, 32 * kk, lane);
                    const bf16x8 rl = frag16(RFl, RFP, KG_SUB * b, 32 * kk, lane);
                    mB[b] = mfma_hilo(rh, rl, lkh[kk], lkl[kk], mB[b]);
                    pB[b] = mfma_hilo(rh, rl, lqh[kk], lql[kk], pB[b]);
                }
            }
#pragma unroll
            for (int b = 0; b < 3; ++b)
                if (b < wave) put_block(b, mB[b], pB[b]);
        }
    } else {
        // ======== sub-chunk references: the right-operand bases k_r 2^{T - P[r]} of
        // sub-chunks 0-2, and the range check of the diagonal block's exponents
        // P[t] - P[mid]
        const int src_mid = ((lane & ~15) + KG_MID) * 4;
        auto bcast = [](int src, float v) {
            return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
        };
        bool bad = false;
        float* rbase = RBs + (wave * KG_SUB + m16) * RBP;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            float rb8[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float pm = bcast(src_mid, P[kk][x]), pe = Tt[wave * DK + 32 * kk + 8 * g + x];
                // (false for NaN too)
                bad = bad || !(P[kk][x] - pm <= KG_RANGE) || !(pm - P[kk][x] <= KG_RANGE);
                rb8[x] = kv(kk, x) * __builtin_amdgcn_exp2f(pe - P[kk][x]);
            }
            if (wave < 3) {
                *reinterpret_cast<f32x4*>(rbase + 32 * kk + 8 * g) = f32x4{rb8[0], rb8[1], rb8[2], rb8[3]};
                *reinterpret_cast<f32x4*>(rbase + 32 * kk + 8 * g + 4) = f32x4{rb8[4], rb8[5], rb8[6], rb8[7]};
            }
        }
        any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;

        // ---- diagonal block (a, a): left operands k_t, q_t times 2^{P[t] - P[mid]}, right
        // operand k_r times 2^{P[mid] - P[r]}, all from this lane's registers
        {
            f32x4 mT = {}, pT = {};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                float lk[8], lq[8], rr[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float d = P[kk][x] - bcast(src_mid, P[kk][x]);
                    const float up = __builtin_amdgcn_exp2f(d), dn = __builtin_amdgcn_exp2f(-d);
                    lk[x] = kv(kk, x) * up;
                    lq[x] = qv(kk, x) * up;
                    rr[x] = kv(kk, x) * dn;
                }
                bf16x8 lkh, lkl, lqh, lql, rh, rl;
                split8f(lk, lkh, lkl);
                split8f(lq, lqh, lql);
                split8f(rr, rh, rl);
                mT = mfma_hilo(rh, rl, lkh, lkl, mT);
                pT = mfma_hilo(rh, rl, lqh, lql, pT);
            }
            put_block(wave, mT, pT);
        }
        block_sync();  // right-operand bases

        // ---- blocks (a, b), b < a: left operands k_t, q_t times 2^{P[t]}, right operands
        // the bases of sub-chunk b times 2^{T_{b+1} + .. + T_{a-1}} (taken for b = a-1
        // down to 0, the sum growing by one total each step)
        if (wave > 0) {
            f32x4 mB[3] = {}, pB[3] = {};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                float lk[8], lq[8], carry[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float up = __builtin_amdgcn_exp2f(P[kk][x]);
                    lk[x] = kv(kk, x) * up;
                    lq[x] = qv(kk, x) * up;
                    carry[x] = 0.f;
                }
                bf16x8 lkh, lkl, lqh, lql;
                split8f(lk, lkh, lkl);
                split8f(lq, lqh, lql);
#pragma unroll
                for (int b = 2; b >= 0; --b) {
                    if (b >= wave) continue;
                    const float* src = RBs + (b * KG_SUB + m16) * RBP + 32 * kk + 8 * g;
                    const f32x4 r0 = *reinterpret_cast<const f32x4*>(src);
                    const f32x4 r1 = *reinterpret_cast<const f32x4*>(src + 4);
                    float rr[8];
#pragma unroll
                    for (int x = 0; x < 8; ++x)
                        rr[x] = (x < 4 ? r0[x] : r1[x - 4]) * __builtin_amdgcn_exp2f(carry[x]);
                    bf16x8 rh, rl;
                    split8f(rr, rh, rl);
                    mB[b] = mfma_hilo(rh, rl, lkh, lkl, mB[b]);
                    pB[b] = mfma_hilo(rh, rl, lqh, lql, pB[b]);
#pragma unroll
                    for (int x = 0; x < 8; ++x) carry[x] += Tt[b * DK + 32 * kk + 8 * g + x];
                }
            }
#pragma unroll
            for (int b = 0; b < 3; ++b)
                if (b < wave) put_block(b, mB[b], pB[b]);
        }
    }
    if (lane == 0) marks[wave] = any_bad ? 1 : 0;
    block_sync();  // L complete; the right-operand bases are dead (X takes their space)
    if (tid == 0) cmark[item] = marks[0] | marks[1] | marks[2] | marks[3];

    // ---- A = (I + L)^{-1} diag(beta) -> the A record
    float x[16];
    if (wave == 0) solve_diag_blocks(Lf, lane, x);
    assemble_inverse(Xs, Lf, Lf, x, wave, lane);
    write_solve_record<true>(arec + static_cast<int64_t>(item) * (A_RECORD_BYTES / 2), Xs, bs, tid);
}

// ============================================================================
// keygate_scan_kernel: the S-dependent chunk products, one workgroup of 8 waves
// per (sequence, head, block of 64 value rows); the roles and the three barriers
// per chunk are those of the value-row scan:
//   chain waves 0, 1 (32 value rows each, S^T in registers):
//       Y = V - Kh S^T,  U = A Y,  S^T <- diag(gamma) S^T + Kt^T U
//   out waves 2, 3:  O^T = S Qh^T + U^T Pd^T
//   loader waves 4-7: one chunk ahead, the loads; then log2 alpha and its prefix
//       over their 16 token rows (lane = d_k / 64 key channels), and at staging
//       Kh, Qh, Kt (hi/lo), gamma, V^T and the two solved records into LDS.
// The solved records are staged compactly (three 32x32 blocks of pitch CB).
// A unit with a marked chunk does not write S_T and is recomputed token by token.
// ============================================================================
template <int DK>
struct KgScanSmem {
    static constexpr int KP = DK + PAD;         // pitch of Kh and Kt rows [t][j]
    static constexpr int QP = DK + 2 * PAD;     // pitch of Qh and S rows
    static constexpr int OP = BV + PAD;         // pitch of O rows [t][i]
    static constexpr int VP = C + PAD;          // pitch of V^T rows [i][t]
    static constexpr int CB = 32 + PAD;         // pitch of the compact solved blocks
    static constexpr int RKH = C * KP * 2;
    static constexpr int RKT = 2 * C * KP * 2;  // Kt hi, lo
    static constexpr int RQ = C * QP * 2;
    static constexpr int RS = BV * QP * 2;
    static constexpr int RREC = 2 * 3 * 32 * CB * 2;
    static constexpr int RU = 2 * BV * CP * 2;  // U^T hi/lo [i][t]
    static constexpr int RV = BV * VP * 2;
    static constexpr int RO = C * OP * 2;
    static constexpr int RT = 2 * 4 * DK * 4;   // loader-wave totals of log2 alpha, two chunks
    static constexpr int RB = DK * 4;           // gamma
    static constexpr int TOTAL = RKH + RKT + RQ + RS + 2 * RREC + RU + RV + RO + RT + RB;
};

template <int DK, int DV>
__global__ __launch_bounds__(512) void keygate_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ arec,
    const uint16_t* __restrict__ prec, const int32_t* __restrict__ cmark, int n_seq, int n_tok, int n_heads,
    uint16_t* __restrict__ o, float* __restrict__ S_T, int32_t* __restrict__ range_flags) {
    using SM = KgScanSmem<DK>;
    static_assert(SM::TOTAL <= 160 * 1024, "LDS budget");
    static_assert(DK == 64 || DK == 128, "d_k");
    constexpr int NVB = DV / BV;
    constexpr int KP = SM::KP, QP = SM::QP, OP = SM::OP, VP = SM::VP, CB = SM::CB;
    constexpr int NJ = DK / 16;   // 16-row tiles of S^T along j
    constexpr int NM = DK / 32;   // 32-wide reduction steps over j
    constexpr int CPL = DK / 64;  // key channels per loader lane

    __shared__ __align__(16) unsigned char rkh_[SM::RKH];
    __shared__ __align__(16) unsigned char rkt_[SM::RKT];
    __shared__ __align__(16) unsigned char rq_[SM::RQ];
    __shared__ __align__(16) unsigned char rs_[SM::RS];
    __shared__ __align__(16) unsigned char ra_[SM::RREC];
    __shared__ __align__(16) unsigned char rp_[SM::RREC];
    __shared__ __align__(16) unsigned char ru_[SM::RU];
    __shared__ __align__(16) unsigned char rv_[SM::RV];
    __shared__ __align__(16) unsigned char ro_[SM::RO];
    __shared__ __align__(16) unsigned char rt_[SM::RT];
    __shared__ __align__(16) unsigned char rb_[SM::RB];
    uint16_t* Kh = reinterpret_cast<uint16_t*>(rkh_);
    uint16_t* Kt_hi = reinterpret_cast<uint16_t*>(rkt_);
    uint16_t* Kt_lo = Kt_hi + C * KP;
    uint16_t* Qh = reinterpret_cast<uint16_t*>(rq_);
    uint16_t* Sx = reinterpret_cast<uint16_t*>(rs_);
    uint16_t* A_hi = reinterpret_cast<uint16_t*>(ra_);
    uint16_t* A_lo = A_hi + 3 * 32 * CB;
    uint16_t* P_hi = reinterpret_cast<uint16_t*>(rp_);
    uint16_t* P_lo = P_hi + 3 * 32 * CB;
    uint16_t* Ux_hi = reinterpret_cast<uint16_t*>(ru_);
    uint16_t* Ux_lo = Ux_hi + BV * CP;
    uint16_t* VT = reinterpret_cast<uint16_t*>(rv_);
    uint16_t* Os = reinterpret_cast<uint16_t*>(ro_);
    float* Tot = reinterpret_cast<float*>(rt_);  // [2][4][DK]
    float* gam = reinterpret_cast<float*>(rb_);

    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wave < 2;
    const bool outw = wave == 2 || wave == 3;
    const bool loader = wave >= 4;
    const int w4 = wave - 4;         // loader wave index: token rows 16 w4 .. +15
    const int rb = 32 * (wave & 1);  // first of the 32 value rows of a chain or out wave
    const int64_t H = n_heads;
    const int h = u.head;
    const int i0 = u.vblk * BV;
    const int64_t row_qk = H * DK, row_v = H * DV;
    const int chunk0 = first_chunk(u.seq, n_seq, n_tok, chunk_off);
    const int64_t s_base = ((static_cast<int64_t>(u.seq) * H + h) * DV + i0) * DK;

    // One register array for every role's long-lived values: chain waves keep S^T at
    // [NJ ib + jt] and the U^T packs at CARRY0 + ..; out waves the O^T accumulators at
    // CARRY0 + ..; loader waves the loaded k, q (16 words: token r, CPL channels),
    // log2 alpha (16 CPL floats), v, the two solved records.
    constexpr int CARRY0 = 2 * NJ;
    constexpr int NA = A_RECORD_PIECES / 256;
    constexpr int PK0 = 0, PQ0 = 4, PL0 = 8, PV0 = PL0 + 4 * CPL, PA0 = PV0 + 4, PP0 = PA0 + NA;
    constexpr int RN = (CARRY0 + 8 > PP0 + NA) ? CARRY0 + 8 : PP0 + NA;
    f32x4 R[RN];
#pragma unroll
    for (int x = 0; x < RN; ++x) R[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (chain && S0) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const float* src =
                S0 + s_base + static_cast<int64_t>(rb + 16 * ib + (lane & 15)) * DK + 4 * (lane >> 4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) R[(ib) * NJ + (jt)] = *reinterpret_cast<const f32x4*>(src + 16 * jt);
        }
    }
    // negated bf16 copy of S as the B operand of Kh (-S)^T for the 32-wide j step m
    auto neg_state = [&](int ib, int m) {
        u32x4 w;
        w[0] = pack_bf16(-R[(ib) * NJ + (2 * m)][0], -R[(ib) * NJ + (2 * m)][1]);
        w[1] = pack_bf16(-R[(ib) * NJ + (2 * m)][2], -R[(ib) * NJ + (2 * m)][3]);
        w[2] = pack_bf16(-R[(ib) * NJ + (2 * m + 1)][0], -R[(ib) * NJ + (2 * m + 1)][1]);
        w[3] = pack_bf16(-R[(ib) * NJ + (2 * m + 1)][2], -R[(ib) * NJ + (2 * m + 1)][3]);
        return __builtin_bit_cast(bf16x8, w);
    };
    auto pack_state = [&](int ln) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            uint16_t* dst = Sx + (rb + 16 * ib + (ln & 15)) * QP + 4 * (ln >> 4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                uint2 w;
                w.x = pack_bf16(R[(ib) * NJ + (jt)][0], R[(ib) * NJ + (jt)][1]);
                w.y = pack_bf16(R[(ib) * NJ + (jt)][2], R[(ib) * NJ + (jt)][3]);
                *reinterpret_cast<uint2*>(dst + 16 * jt) = w;
            }
        }
    };
    // word r of the loaded k (q): token 16 w4 + r, channels CPL ln .. (bf16, low half first)
    auto kword = [&](int base, int r) { return __float_as_uint(R[base + r / 4][r % 4]); };
    auto lval = [&](int r, int c) { return R[PL0 + (CPL * r + c) / 4][(CPL * r + c) % 4]; };
    auto lset = [&](int r, int c, float x) { R[PL0 + (CPL * r + c) / 4][(CPL * r + c) % 4] = x; };

    // ---- the loads of one chunk (loader waves), one chunk ahead; every load is issued
    // unconditionally, a chunk past the end getting empty buffer ranges
    int32_t mark_next = 0;
    auto prefetch = [&](int64_t tc, int n, int gc) {
        const int ht = tid - 256;
        const int64_t tok0 = tc * H + h;
        const bool any = n > 0;
        const int64_t qk_bytes = any ? ((n - 1) * row_qk + DK) * 2 : 0;
        const auto rk = make_rsrc(k + tok0 * DK, qk_bytes);
        const auto rq = make_rsrc(q + tok0 * DK, qk_bytes);
        const auto ra = make_rsrc(alpha + tok0 * DK, 2 * qk_bytes);
        const auto rv = make_rsrc(v + tok0 * DV + i0, any ? ((n - 1) * row_v + BV) * 2 : 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = static_cast<int>((16 * w4 + r) * row_qk + CPL * lane);
            if constexpr (CPL == 2) {
                R[PK0 + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, e * 2, 0, 0));
                R[PQ0 + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rq, e * 2, 0, 0));
                const auto a2 = __builtin_amdgcn_raw_buffer_load_b64(ra, e * 4, 0, 0);
                lset(r, 0, __uint_as_float(a2[0]));
                lset(r, 1, __uint_as_float(a2[1]));
            } else {
                R[PK0 + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b16(rk, e * 2, 0, 0));
                R[PQ0 + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b16(rq, e * 2, 0, 0));
                lset(r, 0, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, e * 4, 0, 0)));
            }
            const int ev = static_cast<int>((16 * w4 + r) * row_v + lane);
            R[PV0 + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b16(rv, ev * 2, 0, 0));
        }
        const int64_t rec_off = (static_cast<int64_t>(gc) * n_heads + h) * (A_RECORD_BYTES / 2);
        const auto rra = make_rsrc(arec + rec_off, any ? A_RECORD_BYTES : 0);
        const auto rrp = make_rsrc(prec + rec_off, any ? A_RECORD_BYTES : 0);
#pragma unroll
        for (int p = 0; p < NA; ++p) {
            R[PA0 + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rra, (ht + 256 * p) * 16, 0, 0));
            R[PP0 + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rrp, (ht + 256 * p) * 16, 0, 0));
        }
        const auto rm = make_rsrc(cmark + static_cast<int64_t>(gc) * n_heads + h, any ? 4 : 0);
        mark_next = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(rm, 0, 0, 0));
    };

    auto chunk_len = [&](int64_t tc) { return static_cast<int>(max<int64_t>(0, min<int64_t>(C, u.t1 - tc))); };

    auto store_o = [&](int64_t tc, int n, int ln) {
        const auto ro = make_rsrc(o + (tc * H + h) * DV + i0, n > 0 ? ((n - 1) * row_v + BV) * 2 : 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int idx = ln + 64 * (wave - 2) + 128 * p, t = idx >> 3, c = idx & 7;
            const u32x4 val = *reinterpret_cast<const u32x4*>(Os + t * OP + 8 * c);
            __builtin_amdgcn_raw_buffer_store_b128(val, ro, static_cast<int>(t * row_v + 8 * c) * 2, 0, 0);
        }
    };

    // one 16-byte piece of a solved record -> its compact [3][32][CB] hi/lo blocks
    auto stage_rec = [&](uint16_t* hi, u32x4 val, int piece) {
        const int b = piece >> 8, half = (piece >> 7) & 1, row = (piece >> 2) & 31, c8 = 8 * (piece & 3);
        *reinterpret_cast<u32x4*>(hi + half * 3 * 32 * CB + (b * 32 + row) * CB + c8) = val;
    };
    // the stacked (frag_st) and plain (frag16) operands of rows 16 tt .. +15 at columns
    // 32 kh .. +31 of a compact solved matrix
    auto rec_st = [&](const uint16_t* base, int tt, int kh, int ln) {
        return frag_st(base + record_block(tt, kh) * 32 * CB, CB, 16 * (tt & 1), 0, ln);
    };
    auto rec_16 = [&](const uint16_t* base, int tt, int kh, int ln) {
        return frag16(base + record_block(tt, kh) * 32 * CB, CB, 16 * (tt & 1), 0, ln);
    };

    // ---- log-decays on the key channels: local_scan turns the loaded alpha of a
    // loader wave's 16 token rows into the inclusive prefix of log2 alpha over them
    // (rows past the sequence end contribute 0) and publishes the wave's totals;
    // finalize (after a barrier) adds the totals of the other loader waves:
    //   G[t]      = (totals of the waves before) + prefix[t]
    //   G[63] - G[t] = (own total - prefix[t]) + (totals of the waves after)
    // each a sum of nonpositive terms taken over whole runs, never the difference of
    // two long sums.
    bool beyond = false;  // loader waves: a chunk of the unit is marked
    auto local_scan = [&](int n, int par, int ln) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float run = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                run += 16 * w4 + r < n ? __builtin_amdgcn_logf(lval(r, c)) : 0.f;
                lset(r, c, run);
            }
            Tot[(par * 4 + w4) * DK + CPL * ln + c] = run;
        }
        beyond = beyond || mark_next != 0;
    };
    auto finalize = [&](int par, int ln) {
        float pre[CPL], suf[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            pre[c] = 0.f;
            suf[c] = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float tb = Tot[(par * 4 + b) * DK + CPL * ln + c];
                if (b < w4) pre[c] += tb;
                if (b > w4) suf[c] += tb;
            }
            if (w4 == 3) gam[CPL * ln + c] = __builtin_amdgcn_exp2f(pre[c] + lval(15, c));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 16 * w4 + r;
            float kh[CPL], qh[CPL], kt[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float g = lval(r, c);
                const float up = __builtin_amdgcn_exp2f(g + pre[c]);
                const float dn = __builtin_amdgcn_exp2f((lval(15, c) - g) + suf[c]);
                const uint32_t kw = kword(PK0, r), qw = kword(PQ0, r);
                const float kx = c ? __uint_as_float(kw & 0xffff0000u) : __uint_as_float(kw << 16);
                const float qx = c ? __uint_as_float(qw & 0xffff0000u) : __uint_as_float(qw << 16);
                kh[c] = kx * up;
                qh[c] = qx * up;
                kt[c] = kx * dn;
            }
            if constexpr (CPL == 2) {
                uint32_t th, tl;
                split_bf16x2(kt[0], kt[1], th, tl);
                *reinterpret_cast<uint32_t*>(Kh + t * KP + 2 * ln) = pack_bf16(kh[0], kh[1]);
                *reinterpret_cast<uint32_t*>(Qh + t * QP + 2 * ln) = pack_bf16(qh[0], qh[1]);
                *reinterpret_cast<uint32_t*>(Kt_hi + t * KP + 2 * ln) = th;
                *reinterpret_cast<uint32_t*>(Kt_lo + t * KP + 2 * ln) = tl;
            } else {
                uint32_t th, tl;
                split_bf16x2(kt[0], 0.f, th, tl);
                Kh[t * KP + ln] = static_cast<uint16_t>(pack_bf16(kh[0], 0.f));
                Qh[t * QP + ln] = static_cast<uint16_t>(pack_bf16(qh[0], 0.f));
                Kt_hi[t * KP + ln] = static_cast<uint16_t>(th);
                Kt_lo[t * KP + ln] = static_cast<uint16_t>(tl);
            }
        }
    };
    // the loaded records and v -> LDS (v transposed: lane = value row, 16 token columns)
    auto stage = [&](int ln) {
        const int ht = ln + 64 * w4;
#pragma unroll
        for (int p = 0; p < NA; ++p) {
            stage_rec(A_hi, __builtin_bit_cast(u32x4, R[PA0 + p]), ht + 256 * p);
            stage_rec(P_hi, __builtin_bit_cast(u32x4, R[PP0 + p]), ht + 256 * p);
        }
        u32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            auto vb = [&](int r) { return __float_as_uint(R[PV0 + r / 4][r % 4]) & 0xffffu; };
            w0[e] = vb(2 * e) | (vb(2 * e + 1) << 16);
            w1[e] = vb(8 + 2 * e) | (vb(9 + 2 * e) << 16);
        }
        *reinterpret_cast<u32x4*>(VT + ln * VP + 16 * w4) = w0;
        *reinterpret_cast<u32x4*>(VT + ln * VP + 16 * w4 + 8) = w1;
    };

    if (loader) {
        prefetch(u.t0, chunk_len(u.t0), chunk0);
        local_scan(chunk_len(u.t0), 0, lane);
    }
    if (chain) pack_state(lane);

    int64_t prev_tc = u.t0;
    int prev_n = 0;
    const int n_chunks = static_cast<int>((u.t1 - u.t0 + C - 1) / C);
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t tc = u.t0 + static_cast<int64_t>(c) * C;
        const int gc = chunk0 + c;
        const int n = chunk_len(tc);
        // lane-derived values are rebuilt every chunk from an opaque copy of the lane
        // id, so the compiler does not hoist loop-invariant LDS addresses (which spills)
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int ln = lane_o;
        const int g = ln >> 4, m16 = ln & 15;
        block_sync();  // the previous chunk is done with every buffer

        // ======== the loaders stage this chunk; the out waves store the previous O
        if (loader) {
            stage(ln);
            finalize(c & 1, ln);
        } else if (outw) {
            store_o(prev_tc, prev_n, ln);
        }
        block_sync();

        if (chain) {
            // ======== Y = V - Kh S^T, then U = A Y, for value rows i = rb + 16 ib + m16
            f32x4 Y[2][4];
            bf16x8 kf[2][4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) kf[0][tt] = frag_st(Kh, KP, 16 * tt, 0, ln);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const uint2 w = *reinterpret_cast<const uint2*>(VT + (rb + 16 * ib + m16) * VP + 16 * tt + 4 * g);
                    Y[ib][tt] = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                      __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
                }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + 1 < NM) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) kf[(m + 1) & 1][tt] = frag_st(Kh, KP, 16 * tt, 32 * (m + 1), ln);
                }
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const bf16x8 sb = neg_state(ib, m);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) Y[ib][tt] = mfma16(kf[m & 1][tt], sb, Y[ib][tt]);
                }
            }
            bf16x8 af[2][4];
            af[0][0] = rec_st(A_hi, 0, 0, ln);
            af[0][1] = rec_st(A_lo, 0, 0, ln);
            issue_fence();
            bf16x8 Yh[2][2], Yl[2][2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                split_stack(Y[ib][0], Y[ib][1], Yh[ib][0], Yl[ib][0]);
                split_stack(Y[ib][2], Y[ib][3], Yh[ib][1], Yl[ib][1]);
            }
            f32x4 U[2][4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x8* cur = af[tt & 1];
                bf16x8* nxt = af[(tt + 1) & 1];
                if (tt + 1 < 4) {
                    nxt[0] = rec_st(A_hi, tt + 1, 0, ln);
                    nxt[1] = rec_st(A_lo, tt + 1, 0, ln);
                    if (tt + 1 >= 2) {
                        nxt[2] = rec_st(A_hi, tt + 1, 1, ln);
                        nxt[3] = rec_st(A_lo, tt + 1, 1, ln);
                    }
                }
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    f32x4 acc = mfma16(cur[0], Yh[ib][0], f32x4{0.f, 0.f, 0.f, 0.f});
                    acc = mfma16(cur[1], Yh[ib][0], acc);
                    acc = mfma16(cur[0], Yl[ib][0], acc);
                    if (tt >= 2) {
                        acc = mfma16(cur[2], Yh[ib][1], acc);
                        acc = mfma16(cur[3], Yh[ib][1], acc);
                        acc = mfma16(cur[2], Yl[ib][1], acc);
                    }
                    U[ib][tt] = acc;
                }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i = rb + 16 * ib + m16;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    bf16x8 uh, ul;
                    split_stack(U[ib][2 * m], U[ib][2 * m + 1], uh, ul);
                    R[CARRY0 + 2 * ib + m] = __builtin_bit_cast(f32x4, uh);
                    R[CARRY0 + 4 + 2 * ib + m] = __builtin_bit_cast(f32x4, ul);
                    const u32x4 wh = __builtin_bit_cast(u32x4, uh), wl = __builtin_bit_cast(u32x4, ul);
                    *reinterpret_cast<uint2*>(Ux_hi + i * CP + 32 * m + 4 * g) = uint2{wh[0], wh[1]};
                    *reinterpret_cast<uint2*>(Ux_hi + i * CP + 32 * m + 16 + 4 * g) = uint2{wh[2], wh[3]};
                    *reinterpret_cast<uint2*>(Ux_lo + i * CP + 32 * m + 4 * g) = uint2{wl[0], wl[1]};
                    *reinterpret_cast<uint2*>(Ux_lo + i * CP + 32 * m + 16 + 4 * g) = uint2{wl[2], wl[3]};
                }
            }
        } else if (outw) {
            // ======== O^T = S Qh^T for value rows rb + 16 ib + 4g + r and tokens 16 tt + m16
            f32x4 Oacc[2][4];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) Oacc[ib][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                bf16x8 sf[2], qf[4];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) sf[ib] = frag16(Sx, QP, rb + 16 * ib, 32 * m, ln);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) qf[tt] = frag16(Qh, QP, 16 * tt, 32 * m, ln);
                issue_fence();
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) Oacc[ib][tt] = mfma16(sf[ib], qf[tt], Oacc[ib][tt]);
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) R[CARRY0 + 4 * ib + tt] = Oacc[ib][tt];
        } else {
            // ======== the loaders issue the next chunk's loads
            prefetch(tc + C, chunk_len(tc + C), gc + 1);
        }
        block_sync();

        if (chain) {
            // ======== S^T <- diag(gamma) S^T + Kt^T U: the key-channel decay scales the
            // rows j of S^T; Kt^T (rows j, reduction t) through the transposing read
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                const f32x4 g4 = *reinterpret_cast<const f32x4*>(gam + 16 * jt + 4 * g);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) R[(ib) * NJ + (jt)] *= g4;
            }
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                bf16x8 th[2], tl[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    th[m] = frag_tr_st(Kt_hi, KP, 16 * jt, 32 * m, ln);
                    tl[m] = frag_tr_st(Kt_lo, KP, 16 * jt, 32 * m, ln);
                }
                issue_fence();
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const bf16x8 uh = __builtin_bit_cast(bf16x8, R[CARRY0 + 2 * ib + m]);
                        const bf16x8 ul = __builtin_bit_cast(bf16x8, R[CARRY0 + 4 + 2 * ib + m]);
                        R[(ib) * NJ + (jt)] = mfma_hilo(th[m], tl[m], uh, ul, R[(ib) * NJ + (jt)]);
                    }
            }
            pack_state(ln);
        } else if (outw) {
            // ======== O^T += U^T Pd^T (Pd is lower triangular: t-tiles 0, 1 need s < 32),
            // staged as bf16 [t][i]
            f32x4 Oacc[2][4];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) Oacc[ib][tt] = R[CARRY0 + 4 * ib + tt];
            bf16x8 uh[2][2], ul[2][2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    uh[ib][m] = frag16(Ux_hi, CP, rb + 16 * ib, 32 * m, ln);
                    ul[ib][m] = frag16(Ux_lo, CP, rb + 16 * ib, 32 * m, ln);
                }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const bf16x8 ph0 = rec_16(P_hi, tt, 0, ln), pl0 = rec_16(P_lo, tt, 0, ln);
                bf16x8 ph1 = {}, pl1 = {};
                if (tt >= 2) {
                    ph1 = rec_16(P_hi, tt, 1, ln);
                    pl1 = rec_16(P_lo, tt, 1, ln);
                }
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    Oacc[ib][tt] = mfma_hilo(uh[ib][0], ul[ib][0], ph0, pl0, Oacc[ib][tt]);
                    if (tt >= 2) Oacc[ib][tt] = mfma_hilo(uh[ib][1], ul[ib][1], ph1, pl1, Oacc[ib][tt]);
                }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int t = 16 * tt + m16, i = rb + 16 * ib + 4 * g;
                    uint2 w;
                    w.x = pack_bf16(Oacc[ib][tt][0], Oacc[ib][tt][1]);
                    w.y = pack_bf16(Oacc[ib][tt][2], Oacc[ib][tt][3]);
                    *reinterpret_cast<uint2*>(Os + t * OP + i) = w;
                }
        }
        if (loader) local_scan(chunk_len(tc + C), (c + 1) & 1, ln);
        prev_tc = tc;
        prev_n = n;
    }
    __shared__ int beyond_s[4];
    if (loader && lane == 0) beyond_s[w4] = beyond ? 1 : 0;
    block_sync();
    const bool unit_beyond = (beyond_s[0] | beyond_s[1] | beyond_s[2] | beyond_s[3]) != 0;
    if (outw) store_o(prev_tc, prev_n, lane);  // (n = 0: nothing is stored)
    if (tid == 0) range_flags[(static_cast<int64_t>(u.seq) * H + h) * NVB + u.vblk] = unit_beyond ? 1 : 0;
    if (S_T && chain && !unit_beyond) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            float* dst = S_T + s_base + static_cast<int64_t>(rb + 16 * ib + (lane & 15)) * DK + 4 * (lane >> 4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) *reinterpret_cast<f32x4*>(dst + 16 * jt) = R[(ib) * NJ + (jt)];
        }
    }
}

// ---------------------------------------------------------------- launchers
static size_t kg_align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the key-gate bf16 prefill (each part 256-byte aligned):
//   order      n_seq int32       longest-first schedule (packed input)
//   chunk_off  n_seq + 1 int32   first chunk of every sequence (packed input)
//   flags      n_seq x H x (d_v / 64) int32: units recomputed token by token
//   marks      chunks x H int32: chunks beyond the range of the decayed Grams
//   A records, Pd records: chunks x H x A_RECORD_BYTES each
// with chunks bounded by n_tok / C + n_seq.
struct KgLayout {
    size_t order, chunk_off, flags, marks, arec, prec, total;
};

static KgLayout kg_layout(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_v) {
    const size_t mc = static_cast<size_t>(n_tok) / C + n_seq;
    KgLayout L;
    L.order = 0;
    L.chunk_off = L.order + kg_align256(static_cast<size_t>(n_seq) * 4);
    L.flags = L.chunk_off + kg_align256((static_cast<size_t>(n_seq) + 1) * 4);
    L.marks = L.flags + kg_align256(static_cast<size_t>(n_seq) * n_heads * (d_v / BV) * 4);
    L.arec = L.marks + kg_align256(mc * n_heads * 4);
    L.prec = L.arec + kg_align256(mc * n_heads * A_RECORD_BYTES);
    L.total = L.prec + kg_align256(mc * n_heads * A_RECORD_BYTES);
    return L;
}

size_t prefill_keygate_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    (void)d_k;
    return kg_layout(n_seq, n_tok, n_heads, d_v).total;
}

template <int DK, int DV>
static hipError_t launch_keygate_t(const PrefillArgs& a, hipStream_t stream) {
    constexpr int NVB = DV / BV;
    const KgLayout L = kg_layout(a.n_seq, a.n_tok, a.n_heads, DV);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* order = reinterpret_cast<int32_t*>(ws + L.order);
    int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
    int32_t* rflags = reinterpret_cast<int32_t*>(ws + L.flags);
    int32_t* marks = reinterpret_cast<int32_t*>(ws + L.marks);
    uint16_t* arec = reinterpret_cast<uint16_t*>(ws + L.arec);
    uint16_t* prec = reinterpret_cast<uint16_t*>(ws + L.prec);
    const int64_t mc = static_cast<int64_t>(a.n_tok) / C + a.n_seq;
    const int32_t* cu = a.cu_seqlens;
    hipError_t e;
    if (cu) {
        if ((e = launch_schedule(cu, a.n_seq, order, stream)) != hipSuccess) return e;
        if ((e = launch_chunk_offsets(cu, a.n_seq, a.n_tok, chunk_off, stream)) != hipSuccess) return e;
    } else {
        order = nullptr;
        chunk_off = nullptr;  // equal lengths: the kernels compute the offsets
    }
    if (a.n_tok > 0) {
        // one workgroup per (chunk, head) of the bound; those past the last chunk return
        hipLaunchKernelGGL((keygate_solve_kernel<DK>), dim3(static_cast<unsigned>(mc * a.n_heads)), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.alpha,
                           a.beta, cu, chunk_off, a.n_seq, a.n_tok, a.n_heads, arec, prec, marks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((keygate_scan_kernel<DK, DV>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.alpha, a.S0, cu, order, chunk_off, arec, prec, marks,
                       a.n_seq, a.n_tok, a.n_heads, static_cast<uint16_t*>(a.o), a.S_T, rflags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // units with a marked chunk (S_T left unwritten) are recomputed token by token;
    // the pass returns at once for the others
    return launch_prefill_range_fixup(a, rflags, 1, stream);
}

hipError_t launch_prefill_keygate(const PrefillArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_keygate_t<128, 128>(a, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_keygate_t<64, 64>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_keygate_t<128, 64>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_keygate_t<64, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
