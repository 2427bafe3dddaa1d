// kda_backward_chunk.hip -- the chunked backward of the bf16 prefill on CDNA4
// matrix cores (value-channel, scalar and no gate).
//
// The transcript page ("Per dins de Kimi K3 ..."), where it turns to training,
// says the model is trained with the chunk-wise parallel algorithm; this is that
// algorithm's backward for the recurrence of page "Kimi (AI)", section "Kimi
// Delta Attention (KDA)" (rows of the d_v x d_k state decayed by alpha).  Within
// a chunk of C tokens entered with state S (the forward's factored form, in
// natural-log units G = cumsum log alpha per value row, X = V e^{-G},
// T = (I + L)^{-1}, L = strictly_lower(diag(beta) K K^T)):
//     Y  = X - K S^T,   U = T (beta (.) Y),   O~ = Q S^T + P U   (P = tril(Q K^T)),
//     O  = e^{G} (.) O~,   S' = diag(gamma) (S + U^T K)          (gamma = e^{G_last}).
// Given dO and D = dL/dS' (the gradient of the state leaving the chunk):
//     dO~ = dO (.) e^{G},  dZ = D diag(gamma)          [written transposed, d_k x d_v]
//     dU  = P^T dO~ + K dZ^T,   dYb = T^T dU,   dY = beta (.) dYb
//     dL/dS = dZ + dO~^T Q - dY^T K                   (carried to the chunk before)
//     dV  = dY (.) e^{-G}
//     dQ  = dO~ S + dP K,            dP  = tril(dO~ U^T)
//     dK  = U dZ - dY S + dP^T Q + (dKK + dKK^T) K,   dKK = -strictly_lower(dY U^T)
//     dbeta_t = (1 / beta_t) sum_i dYb[t,i] U[t,i]    (U_t / beta_t is the error before beta)
//     dG  = dO~ (.) O~ - dY (.) X,  plus on the chunk's last token
//           sum_j dZ[i,j] S[i,j] + sum_t U[t,i] (K dZ^T)[t,i]   (the gradient through gamma)
//     dalpha = (reverse cumulative sum of dG over the chunk) / alpha
// (checked in fp64 against the token-by-token chain rule of the backward oracle).
//
// Passes, all on the caller's stream:
//   1. the forward: the chunk solve, storing both A and T = (I + L)^{-1} (no beta
//      factor) and marking units with |beta| below 2^-20, then the 32-token scan in
//      its checkpoint variant, which stores the state entering every 64-token chunk
//      (no outputs) and marks units beyond the factored form's range or with a gate
//      below 2^-5;
//   2. (the marks are only ever set; they are cleared before pass 1);
//   3. bwd_state_scan_kernel: per (sequence, head, 64 value rows), the chunks in
//      reverse, carrying dL/dS^T in fp32 MFMA accumulators -- the forward scan's
//      chain transposed (K dZ^T, T^T dU, K^T dY on the critical path) -- and
//      storing D for every chunk;
//   4. bwd_chunk_grad_kernel: every (chunk, head) at once, all value rows in one
//      workgroup, so the sums over rows (dq, dk, dbeta) need no atomics;
//   5. the units marked in passes 1-2 (the whole (sequence, head)) run the
//      token-recurrent backward instead, which is exact there.
// Precision: q, k, v are exact bf16; every other matrix operand is carried as a
// hi + lo bf16 pair (three MFMAs per product, two when one side is exact), so the
// gradients keep fp32-level agreement with the fp64 oracle.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_schedule.h"

namespace kda {
namespace {

// 8 floats (a: reduction indices 0-3, b: 4-7 of an operand) -> hi + lo bf16x8
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_bf16x2(a[0], a[1], h0, l0);
    split_bf16x2(a[2], a[3], h1, l1);
    split_bf16x2(b[0], b[1], h2, l2);
    split_bf16x2(b[2], b[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

// hi + lo split of an accumulator tile's four values, as two packed bf16x4 (uint2)
__device__ __forceinline__ void split4(const f32x4& a, uint2& hi, uint2& lo) {
    split_bf16x2(a[0], a[1], hi.x, lo.x);
    split_bf16x2(a[2], a[3], hi.y, lo.y);
}

// hi*hi + lo*hi + hi*lo of a split product
__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma16(ah, bh, c);
    c = mfma16(al, bh, c);
    return mfma16(ah, bl, c);
}

__device__ __forceinline__ bool unit_marked(const int32_t* __restrict__ flags, int seq, int h, int64_t H, int nvb) {
    bool m = false;
    for (int vb = 0; vb < nvb; ++vb) m |= flags[(static_cast<int64_t>(seq) * H + h) * nvb + vb] != 0;
    return m;
}

}  // namespace

// ============================================================================
// bwd_state_scan_kernel: one workgroup of 8 waves per (sequence, head, block of 64
// value rows), chunks last to first.
// - Chain waves (0-3): wave w owns value rows i0 + 16 w .. +15 and carries D^T (d_k x 16,
//   rows j = 16 jt + 4g + r of tile jt, column = the lane's row) in accumulators.  Per
//   chunk: store D, dZ = D gamma, dU = K dZ + P^T dO~, dYb = T^T dU, dY = beta dYb, then
//   D <- dZ + Q^T dO~ - K^T dY.
// - Helper waves (4-7) prepare the chunk before meanwhile: K and Q into the other of two
//   buffers; G and dO~^T [i][t], gamma (helper h: token rows 16 h .. +15, a lane per value
//   row); P = tril(Q K^T); T and beta.  Each of dO~^T and gamma, P, and T and beta has one
//   buffer, rewritten once the chain has read it.  Each input's loads for the chunk after
//   that are issued as soon as its registers are free.
// Four barriers per chunk:  D | chain: D store, K dZ  -- helpers: stage K, Q; log2 alpha
// prefix  | A | chain: P^T dO~  -- helpers: dO~^T, gamma  | B | chain: T^T dU  --
// helpers: P  | C | chain: D update  -- helpers: T, beta  | D.
// ============================================================================
template <int DK, int DV, int GATE>
__global__ __launch_bounds__(512) void bwd_state_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ dO, const float* __restrict__ dS_T,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ order, const int32_t* __restrict__ chunk_off,
    const uint16_t* __restrict__ trec, int32_t* __restrict__ range_flags, int n_seq, int n_tok, int n_heads,
    float* __restrict__ gck, float* __restrict__ dS0) {
    constexpr int NVB = DV / 64;
    constexpr int KP = DK + PAD;
    constexpr int NJ = DK / 16;
    constexpr int NM = DK / 32;
    constexpr int XP = C + 8;              // pitch of dO~^T rows (fp32)
    constexpr int PPR = DK / 8;            // 16-byte pieces per row of q or k
    constexpr int NKQ = C * PPR / 256;     // ... per helper thread
    constexpr int NREC = A_RECORD_PIECES / 256;
    __shared__ __align__(16) uint16_t Kc[2][C * KP];
    __shared__ __align__(16) uint16_t Qc[2][C * KP];
    __shared__ __align__(16) uint16_t T_hi[C * CP];
    __shared__ __align__(16) uint16_t T_lo[C * CP];
    __shared__ __align__(16) uint16_t P_hi[C * CP];
    __shared__ __align__(16) uint16_t P_lo[C * CP];
    __shared__ __align__(16) float dOT[64 * XP];
    __shared__ __align__(16) float bs[C];
    __shared__ __align__(16) float gam[64];
    __shared__ __align__(16) float Tot[4 * 64];

    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int64_t H = n_heads;
    const int h = u.head;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wave < 4;
    const int hw = wave & 3;      // chain: rows 16 hw ..; helper: token rows 16 hw ..
    const int htid = tid & 255;   // thread index among the chain or the helper waves
    if (unit_marked(range_flags, u.seq, h, H, NVB)) {
        // the whole (sequence, head) goes to the token-recurrent pass: mark every block of it
        if (tid < NVB) range_flags[(static_cast<int64_t>(u.seq) * H + h) * NVB + tid] = 1;
        return;
    }
    const int i0 = u.vblk * 64;
    const int iw = i0 + 16 * hw;  // first value row of a chain wave
    const int64_t row_qk = H * DK, row_v = H * DV;
    const int chunk0 = first_chunk(u.seq, n_seq, n_tok, chunk_off);
    const int n_chunks = static_cast<int>((u.t1 - u.t0 + C - 1) / C);

    // the upper-right 32x32 block of T is not part of a record, and the helpers write only the
    // 16x16 tiles of P on and below the diagonal: the rest is zeroed once and read as such
    for (int x = tid; x < 32 * 32; x += 512) {
        T_hi[(x >> 5) * CP + 32 + (x & 31)] = 0;
        T_lo[(x >> 5) * CP + 32 + (x & 31)] = 0;
    }
    for (int x = tid; x < C * C; x += 512) {
        const int t = x / C, s = x % C;
        if ((s >> 4) > (t >> 4)) P_hi[t * CP + s] = P_lo[t * CP + s] = 0;
    }

    // One register array holds each role's long-lived values -- the chain's D^T, or a
    // helper's loaded inputs -- so the allocator, which cannot know that a wave keeps one
    // role, does not keep both sets live at once (likewise X4: the chain's dU, a helper's
    // log2-decay prefix).
    constexpr int OK_ = 0, OQ = NKQ, OA = 2 * NKQ, OD = OA + 4, OR = OD + 4, OB = OR + NREC;
    constexpr int NRR = OB + 1 > NJ ? OB + 1 : NJ;
    f32x4 RR[NRR];
    f32x4* R = RR;  // chain: D^T tiles
    auto rk = [&](int p) -> f32x4& { return RR[OK_ + p]; };
    auto rq = [&](int p) -> f32x4& { return RR[OQ + p]; };
    auto rr = [&](int p) -> f32x4& { return RR[OR + p]; };
    // scalar members (an element of a vector cannot be bound to a reference)
    auto ra = [&](int r) { return RR[OA + (r >> 2)][r & 3]; };
    auto rd = [&](int r) { return RR[OD + (r >> 2)][r & 3]; };
    const int64_t s_base = ((static_cast<int64_t>(u.seq) * H + h) * DV + iw + (lane & 15)) * DK + 4 * (lane >> 4);
#pragma unroll
    for (int x = 0; x < NRR; ++x) RR[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (chain && dS_T) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) R[jt] = *reinterpret_cast<const f32x4*>(dS_T + s_base + 16 * jt);
    }

    // ---- a helper's inputs of one chunk, in registers (a chunk index outside 0 .. n_chunks - 1
    // loads nothing)
    auto chunk_len = [&](int c) {
        return c < 0 || c >= n_chunks ? 0 : static_cast<int>(min<int64_t>(C, u.t1 - (u.t0 + static_cast<int64_t>(c) * C)));
    };
    auto chunk_tok0 = [&](int c) { return (u.t0 + static_cast<int64_t>(c < 0 ? 0 : c) * C) * H + h; };
    auto fetch_kq = [&](int c) {
        const int n = chunk_len(c);
        const int64_t tok0 = chunk_tok0(c);
        const int64_t bqk = n > 0 ? ((n - 1) * row_qk + DK) * 2 : 0;
        const auto rk_ = make_rsrc(k + tok0 * DK, bqk);
        const auto rq_ = make_rsrc(q + tok0 * DK, bqk);
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int idx = htid + 256 * p;
            const int off = static_cast<int>((idx / PPR) * row_qk + 8 * (idx % PPR)) * 2;
            rk(p) = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk_, off, 0, 0));
            rq(p) = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq_, off, 0, 0));
        }
    };
    auto fetch_ad = [&](int c) {
        const int n = chunk_len(c);
        const int64_t tok0 = chunk_tok0(c);
        const int64_t bv = n > 0 ? ((n - 1) * row_v + 64) * 4 : 0;
        const auto ra_ = GATE == GATE_CHANNEL ? make_rsrc(alpha + tok0 * DV + i0, bv)
                         : GATE == GATE_SCALAR ? make_rsrc(alpha + tok0, n > 0 ? ((n - 1) * H + 1) * 4 : 0)
                                               : make_rsrc(alpha, 0);
        const auto rd_ = make_rsrc(dO + tok0 * DV + i0, bv);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 16 * hw + r;
            const int e = static_cast<int>(t * row_v + lane);
            if constexpr (GATE != GATE_NONE) {
                const int ea = GATE == GATE_CHANNEL ? e : static_cast<int>(t * H);
                RR[OA + (r >> 2)][r & 3] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra_, ea * 4, 0, 0));
            }
            RR[OD + (r >> 2)][r & 3] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd_, e * 4, 0, 0));
        }
    };
    auto fetch_tb = [&](int c) {
        const int n = chunk_len(c);
        const int64_t tok0 = chunk_tok0(c);
        const uint16_t* recp = trec + (static_cast<int64_t>(chunk0 + (c < 0 ? 0 : c)) * n_heads + h) * (A_RECORD_BYTES / 2);
        const auto rr_ = make_rsrc(recp, n > 0 ? A_RECORD_BYTES : 0);
#pragma unroll
        for (int p = 0; p < NREC; ++p) {
            // (an all-zero piece reads past the range: zero, no memory traffic)
            const int pc = htid + 256 * p;
            const int off = record_piece_zero(pc) ? A_RECORD_BYTES : pc * 16;
            rr(p) = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr_, off, 0, 0));
        }
        const auto rb_ = make_rsrc(beta + tok0, n > 0 ? ((n - 1) * H + 1) * 4 : 0);
        RR[OB][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb_, static_cast<int>(lane * H) * 4, 0, 0));
    };
    if (!chain) {
        fetch_kq(n_chunks - 1);
        fetch_ad(n_chunks - 1);
        fetch_tb(n_chunks - 1);
    }

    // Iteration c: the chain walks chunk c (none at c = n_chunks), the helpers prepare
    // chunk c - 1 (none at c = 0).
    for (int c = n_chunks; c >= 0; --c) {
        const bool work = c < n_chunks;  // the chain has a chunk
        const bool prep = c > 0;         // the helpers have one
        const int cb = c & 1;            // K, Q buffer of chunk c; chunk c - 1 uses the other
        const int nprep = chunk_len(c - 1);
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int ln = lane_o, g = ln >> 4, m16 = ln & 15;
        const uint16_t* Kw = Kc[cb];
        const uint16_t* Qw = Qc[cb];
        block_sync();  // D: chunk c is staged; the chain is done with chunk c + 1

        // ======== D -> A.  chain: D store, dZ = D gamma, dO~ operands, K dZ^T.  helpers: stage
        // K, Q of chunk c - 1 (then load those of c - 2); log2-alpha prefix
        f32x4 X4[4];
        f32x4* dU = X4;  // chain
        auto G16 = [&](int r) { return X4[r >> 2][r & 3]; };  // helpers: log2-decay prefix
        bf16x8 oh[2], ol[2];
        if (chain && work) {
            float* dst = gck + ((static_cast<int64_t>(chunk0 + c) * H + h) * DV + iw + m16) * DK + 4 * g;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) *reinterpret_cast<f32x4*>(dst + 16 * jt) = R[jt];
            const float gm = gam[16 * hw + m16];
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) R[jt] *= gm;  // dZ^T
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float* src = dOT + (16 * hw + m16) * XP + 32 * m + 4 * g;
                split8(*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 16), oh[m], ol[m]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) dU[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                bf16x8 zh, zl;
                split_stack(R[2 * m], R[2 * m + 1], zh, zl);
                bf16x8 kf[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) kf[tt] = frag_st(Kw, KP, 16 * tt, 32 * m, ln);
                issue_fence();
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    dU[tt] = mfma16(kf[tt], zh, dU[tt]);
                    dU[tt] = mfma16(kf[tt], zl, dU[tt]);
                }
            }
        }
        if (!chain && prep) {
#pragma unroll
            for (int p = 0; p < NKQ; ++p) {
                const int idx = htid + 256 * p;
                *reinterpret_cast<f32x4*>(Kc[cb ^ 1] + (idx / PPR) * KP + 8 * (idx % PPR)) = rk(p);
                *reinterpret_cast<f32x4*>(Qc[cb ^ 1] + (idx / PPR) * KP + 8 * (idx % PPR)) = rq(p);
            }
            fetch_kq(c - 2);
            float run = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (GATE != GATE_NONE) run += 16 * hw + r < nprep ? __builtin_amdgcn_logf(ra(r)) : 0.f;
                X4[r >> 2][r & 3] = run;
            }
            Tot[hw * 64 + ln] = run;
        }
        block_sync();  // A: the chain has read gamma and dO~^T; K, Q and the totals of c - 1 are in

        // ======== A -> B.  chain: dU += P^T dO~.  helpers: dO~^T = (dO e^{G})^T and gamma of c - 1
        if (chain && work) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (st >= 2 && m == 0) continue;  // P^T[s][t] = 0 for t < s
                    const bf16x8 ph = frag_tr_st(P_hi, CP, 16 * st, 32 * m, ln), pl = frag_tr_st(P_lo, CP, 16 * st, 32 * m, ln);
                    dU[st] = mfma3(ph, pl, oh[m], ol[m], dU[st]);
                }
        }
        if (!chain && prep) {
            float carry = 0.f;
#pragma unroll
            for (int w = 0; w < 3; ++w) carry += w < hw ? Tot[w * 64 + ln] : 0.f;
            float* dst = dOT + ln * XP + 16 * hw;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = rd(4 * p + e) * __builtin_amdgcn_exp2f(G16(4 * p + e) + carry);
                *reinterpret_cast<f32x4*>(dst + 4 * p) = x;
            }
            if (hw == 3) gam[ln] = __builtin_amdgcn_exp2f(G16(15) + carry);
            fetch_ad(c - 2);
        }
        block_sync();  // B: the chain is done with P

        // ======== B -> C.  chain: dYb = T^T dU, dY = beta dYb.  helpers: P of c - 1
        f32x4 dY[4];
        if (chain && work) {
            bf16x8 uh[2], ul[2];
            split_stack(dU[0], dU[1], uh[0], ul[0]);
            split_stack(dU[2], dU[3], uh[1], ul[1]);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                dY[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (st >= 2 && m == 0) continue;  // T^T[s][t] = 0 for t < s
                    const bf16x8 th = frag_tr_st(T_hi, CP, 16 * st, 32 * m, ln), tl = frag_tr_st(T_lo, CP, 16 * st, 32 * m, ln);
                    dY[st] = mfma3(th, tl, uh[m], ul[m], dY[st]);
                }
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + 16 * st + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) dY[st][e] *= -b4[e];  // negated for the K^T product
            }
        }
        if (!chain && prep) {
            // P = tril(Q K^T) as D[s][t] = K Q^T tiles: the 10 tiles with s-tile <= t-tile,
            // helper hw taking tiles hw, hw + 4, hw + 8; a lane holds four consecutive s of one
            // t, written as P[t][s .. s+3]
            const uint16_t* Kn = Kc[cb ^ 1];
            const uint16_t* Qn = Qc[cb ^ 1];
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int e = hw + 4 * x;
                if (e < 10) {
                    const int tt = e < 1 ? 0 : e < 3 ? 1 : e < 6 ? 2 : 3;
                    const int st = e - tt * (tt + 1) / 2;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < NM; ++m)
                        acc = mfma16(frag16(Kn, KP, 16 * st, 32 * m, ln), frag16(Qn, KP, 16 * tt, 32 * m, ln), acc);
                    const int t = 16 * tt + m16, s0 = 16 * st + 4 * g;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) acc[q4] = s0 + q4 <= t ? acc[q4] : 0.f;
                    uint2 wh, wl;
                    split4(acc, wh, wl);
                    *reinterpret_cast<uint2*>(P_hi + (16 * tt + m16) * CP + 16 * st + 4 * g) = wh;
                    *reinterpret_cast<uint2*>(P_lo + (16 * tt + m16) * CP + 16 * st + 4 * g) = wl;
                }
            }
        }
        block_sync();  // C: the chain is done with T and beta

        // ======== C -> D.  chain: D^T <- dZ^T + Q^T dO~ - K^T dY.  helpers: T, beta of c - 1
        if (chain && work) {
            bf16x8 yh[2], yl[2];
            split_stack(dY[0], dY[1], yh[0], yl[0]);
            split_stack(dY[2], dY[3], yh[1], yl[1]);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const bf16x8 aq = frag_tr_st(Qw, KP, 16 * jt, 32 * m, ln);
                    const bf16x8 ak = frag_tr_st(Kw, KP, 16 * jt, 32 * m, ln);
                    R[jt] = mfma16(aq, oh[m], R[jt]);
                    R[jt] = mfma16(aq, ol[m], R[jt]);
                    R[jt] = mfma16(ak, yh[m], R[jt]);
                    R[jt] = mfma16(ak, yl[m], R[jt]);
                }
            }
        }
        if (!chain && prep) {
#pragma unroll
            for (int p = 0; p < NREC; ++p) *reinterpret_cast<f32x4*>(record_piece_dst(T_hi, T_lo, htid + 256 * p)) = rr(p);
            if (hw == 0) bs[ln] = RR[OB][0];
            fetch_tb(c - 2);
        }
    }
    if (chain && dS0) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) *reinterpret_cast<f32x4*>(dS0 + s_base + 16 * jt) = R[jt];
    }
}

// ============================================================================
// bwd_chunk_grad_kernel: one workgroup of 8 waves per (chunk, head), all d_v value
// rows.  Phase A (wave w owns value rows 16 w .. +15, every token of the chunk):
// Y, U, O~, K dZ^T, dO~, dU, dYb, dY and the row-local gradients dV, dalpha, and
// each wave's share of dbeta.  Phase B (wave w owns key channels of dq and dk):
// in rounds of 64 value rows, the packs of U, dO~ and dY go through LDS for the
// sums over rows -- dP, dKK and the S- and dZ-side terms of dq and dk -- then the
// C x C terms (dP K, dP^T Q, (dKK + dKK^T) K).
// ============================================================================
template <int DK, int DV>
struct GradSmem {
    static constexpr int KP = DK + PAD;
    static constexpr int GP = C + 4;                 // pitch of G^T rows (fp32)
    static constexpr int RKQ = 2 * C * KP * 2;       // K, Q [t][j]
    static constexpr int BUF = C * CP * 2;           // one [64][CP] bf16 buffer
    static constexpr int UA = 4 * BUF + DV * GP * 4; // phase A: T, P hi/lo; G^T
    static constexpr int UB = 10 * BUF;              // phase B: U, dO~, dY (hi/lo, 64 rows); dP, dKK hi/lo
    static constexpr int UO = 2 * C * (DV + 4) * 4;  // dV, dalpha rows [t][i] after phase A
    static constexpr int RU0 = UA > UB ? UA : UB;
    static constexpr int RU = RU0 > UO ? RU0 : UO;
    static constexpr int RS = (C + DV + 8 * DV + 2 * 8 * C) * 4;  // beta, gamma, cumsum totals, row partials
    static constexpr int TOTAL = RKQ + RU + RS;
};

template <int DK, int DV, int GATE>
__global__ __launch_bounds__(512) void bwd_chunk_grad_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ dO,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ trec,
    const float* __restrict__ sck, const float* __restrict__ gck, const int32_t* __restrict__ range_flags, int n_seq,
    int n_tok, int n_heads, int max_chunks, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dalpha, float* __restrict__ dbeta) {
    using SM = GradSmem<DK, DV>;
    static_assert(SM::TOTAL <= 160 * 1024, "LDS budget");
    constexpr int NVB = DV / 64;
    constexpr int KP = SM::KP, GP = SM::GP;
    constexpr int NM = DK / 32;
    constexpr int NWA = DV / 16;            // waves of phase A
    constexpr int NR = DV / 64;             // rounds of phase B
    constexpr int NJT = DK / 16;            // key-channel tiles of dq, dk
    constexpr int TPW = NJT >= 8 ? 4 : 2;   // t-tiles per wave in phase B
    constexpr int PPR = DK / 8;
    constexpr int NKQ = C * PPR / 512;
    __shared__ __align__(16) unsigned char smem[SM::TOTAL];
    uint16_t* Kc = reinterpret_cast<uint16_t*>(smem);
    uint16_t* Qc = Kc + C * KP;
    unsigned char* ur = smem + SM::RKQ;
    // phase A
    uint16_t* T_hi = reinterpret_cast<uint16_t*>(ur);
    uint16_t* T_lo = T_hi + C * CP;
    uint16_t* P_hi = T_lo + C * CP;
    uint16_t* P_lo = P_hi + C * CP;
    float* GT = reinterpret_cast<float*>(ur + 4 * SM::BUF);
    // phase B
    uint16_t* UT_hi = reinterpret_cast<uint16_t*>(ur);
    uint16_t* UT_lo = UT_hi + C * CP;
    uint16_t* OT_hi = UT_lo + C * CP;
    uint16_t* OT_lo = OT_hi + C * CP;
    uint16_t* YT_hi = OT_lo + C * CP;
    uint16_t* YT_lo = YT_hi + C * CP;
    uint16_t* dP_hi = YT_lo + C * CP;
    uint16_t* dP_lo = dP_hi + C * CP;
    uint16_t* dK_hi = dP_lo + C * CP;  // dKK
    uint16_t* dK_lo = dK_hi + C * CP;
    float* bs = reinterpret_cast<float*>(ur + SM::RU);
    float* gam = bs + C;
    float* Tot = gam + DV;
    float* red = Tot + 8 * DV;   // [8][C] dbeta partials
    float* red2 = red + 8 * C;   // [8][C] scalar-gate dalpha partials

    const int64_t H = n_heads;
    const int total = min(first_chunk(n_seq, n_seq, n_tok, chunk_off), max_chunks);
    const int n_items = total * n_heads;  // (chunk, head) pairs, chunk-major
    const int64_t row_qk = H * DK, row_v = H * DV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, m16 = lane & 15;

    // The workgroup stays resident (one per CU) and walks the items it + k gridDim.x; the
    // next item's global inputs are loaded while the current one finishes.
    struct Item {
        int64_t tok0;
        int gc, h, n;
        int marked;  // computed by the token-recurrent pass instead
    };
    auto item_info = [&](int it) {
        Item x;
        x.gc = it / n_heads;
        x.h = it % n_heads;
        const ChunkRef ch = chunk_ref(x.gc, n_seq, n_tok, cu_seqlens, chunk_off);
        x.n = ch.n;
        x.tok0 = ch.t0 * H + x.h;
        x.marked = unit_marked(range_flags, ch.seq, x.h, H, NVB);
        return x;
    };
    constexpr int NRP = (A_RECORD_PIECES + 511) / 512;
    u32x4 pk[NKQ], pq[NKQ], prec[NRP];
    float pb, pa[NVB][8];
    f32x4 pS[NM][2], pD[NM][2];
    float pV[4][4], pdO[4][4];
    // The global inputs of the staging (K, Q, the T record, beta and alpha): loaded for the
    // next item while the current one finishes.  All loads are buffer loads: ranges end at the
    // chunk's last token, and an item that is not loaded (none left, or marked) gets empty
    // ranges, so every register is written and every load returns 0 without touching memory.
    // Each resource is uniform over the wave (a per-lane base would make the compiler loop over
    // the distinct bases, waiting for each load in turn); the lane's position is in the offset.
    auto fetch_stage = [&](const Item& x, bool valid) __attribute__((always_inline)) {
        // offsets from an opaque copy of the thread index, recomputed at every call (hoisted
        // out of the item loop they would hold registers throughout)
        int tid_f = tid;
        asm volatile("" : "+v"(tid_f));
        const int tid = tid_f, lane = tid & 63;
        const int g = lane >> 4, m16 = lane & 15;
        const int nn = valid ? x.n : 0;
        const int64_t bqk = nn > 0 ? ((nn - 1) * row_qk + DK) * 2 : 0;
        const auto rk_ = make_rsrc(k + x.tok0 * DK, bqk);
        const auto rq_ = make_rsrc(q + x.tok0 * DK, bqk);
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int idx = tid + 512 * p;
            const int off = static_cast<int>((idx / PPR) * row_qk + 8 * (idx % PPR)) * 2;
            pk[p] = __builtin_amdgcn_raw_buffer_load_b128(rk_, off, 0, 0);
            pq[p] = __builtin_amdgcn_raw_buffer_load_b128(rq_, off, 0, 0);
        }
        const auto rr_ = make_rsrc(trec + (static_cast<int64_t>(x.gc) * n_heads + x.h) * (A_RECORD_BYTES / 2),
                                   valid ? A_RECORD_BYTES : 0);
#pragma unroll
        for (int p = 0; p < NRP; ++p) {
            // (all-zero pieces and pieces past the record read past the range: zero)
            const int pc = tid + 512 * p;
            const int off = pc >= A_RECORD_PIECES || record_piece_zero(pc) ? A_RECORD_BYTES : pc * 16;
            prec[p] = __builtin_amdgcn_raw_buffer_load_b128(rr_, off, 0, 0);
        }
        const auto rb_ = make_rsrc(beta + x.tok0, nn > 0 ? ((nn - 1) * H + 1) * 4 : 0);
        pb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb_, static_cast<int>(tid * H) * 4, 0, 0));
        // alpha at token rows t = 8 w + r, value rows i = lane + 64 xv
        if constexpr (GATE != GATE_NONE) {
            const auto ra_ = GATE == GATE_CHANNEL ? make_rsrc(alpha + x.tok0 * DV, nn > 0 ? ((nn - 1) * row_v + DV) * 4 : 0)
                                                  : make_rsrc(alpha + x.tok0, nn > 0 ? ((nn - 1) * H + 1) * 4 : 0);
#pragma unroll
            for (int xv = 0; xv < NVB; ++xv)
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int t = 8 * wave + r;
                    const int off = GATE == GATE_CHANNEL ? static_cast<int>(t * row_v) + lane + 64 * xv : static_cast<int>(t * H);
                    pa[xv][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra_, off * 4, 0, 0));
                }
        }
    };
    // phase A's inputs: rows i = 16 w + m16 of S and D (key channels 8g + 32m .. +7), and V,
    // dO at the tile rows t = 16 tt + 4g + e
    auto fetch_a = [&](const Item& x) __attribute__((always_inline)) {
        int tid_f = tid;
        asm volatile("" : "+v"(tid_f));
        const int lane = tid_f & 63;
        const int g = lane >> 4, m16 = lane & 15;
        const bool rows = wave < NWA;
        const int nn = x.n;
        const int i = 16 * wave + m16;
        const int64_t unit = (static_cast<int64_t>(x.gc) * H + x.h) * DV * DK;
        const auto rs_ = make_rsrc(sck + unit, rows ? DV * DK * 4 : 0);
        const auto rz_ = make_rsrc(gck + unit, rows ? DV * DK * 4 : 0);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int off = (i * DK + 8 * g + 32 * m + 4 * hf) * 4;
                pS[m][hf] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_, off, 0, 0));
                pD[m][hf] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rz_, off, 0, 0));
            }
        const auto rv = make_rsrc(v + x.tok0 * DV, rows && nn > 0 ? ((nn - 1) * row_v + DV) * 2 : 0);
        const auto rdo = make_rsrc(dO + x.tok0 * DV, rows && nn > 0 ? ((nn - 1) * row_v + DV) * 4 : 0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int off = static_cast<int>((16 * tt + 4 * g + e) * row_v) + i;
                pV[tt][e] = bf16_bits_to_f32(
                    static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rv, off * 2, 0, 0)));
                pdO[tt][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdo, off * 4, 0, 0));
            }
    };

    int it = blockIdx.x;
    if (it >= n_items) return;
    Item cur = item_info(it);
    fetch_stage(cur, !cur.marked);
    while (true) {
    // the thread index passes through an empty asm every item, so the compiler cannot hoist
    // the body's lane-dependent addresses out of the loop (they would stay live throughout)
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    {
    const int tid = tid_o, lane = tid & 63;
    const int g = lane >> 4, m16 = lane & 15;
    const int it_next = it + static_cast<int>(gridDim.x);
    if (cur.marked) {
        // computed by the token-recurrent pass, which adds the row sums into zeros
        for (int x = tid; x < cur.n * DK; x += 512) {
            const int64_t e = (cur.tok0 + static_cast<int64_t>(x / DK) * H) * DK + x % DK;
            dq[e] = 0.f;
            dk[e] = 0.f;
        }
        if (tid < cur.n) {
            dbeta[cur.tok0 + tid * H] = 0.f;
            if (GATE == GATE_SCALAR) dalpha[cur.tok0 + tid * H] = 0.f;
        }
        if (it_next >= n_items) break;
        it = it_next;
        cur = item_info(it);
        fetch_stage(cur, !cur.marked);
        continue;
    }
    const int gc = cur.gc, h = cur.h, n = cur.n;
    const int64_t tok0 = cur.tok0;
    const bool more = it_next < n_items;
    Item nxt = cur;
    if (more) nxt = item_info(it_next);  // scalar loads, in flight under this item
    fetch_a(cur);                        // arrives under the staging

    // ======== staging: K, Q, T, beta; the upper-right 32x32 block of T is zero
#pragma unroll
    for (int p = 0; p < NRP; ++p)
        if (tid + 512 * p < A_RECORD_PIECES)
            *reinterpret_cast<u32x4*>(record_piece_dst(T_hi, T_lo, tid + 512 * p)) = prec[p];
    for (int x = tid; x < 32 * 32; x += 512) {
        T_hi[(x >> 5) * CP + 32 + (x & 31)] = 0;
        T_lo[(x >> 5) * CP + 32 + (x & 31)] = 0;
    }
    if (tid < C) bs[tid] = tid < n ? pb : 0.f;
#pragma unroll
    for (int p = 0; p < NKQ; ++p) {
        const int idx = tid + 512 * p;
        *reinterpret_cast<u32x4*>(Kc + (idx / PPR) * KP + 8 * (idx % PPR)) = pk[p];
        *reinterpret_cast<u32x4*>(Qc + (idx / PPR) * KP + 8 * (idx % PPR)) = pq[p];
    }
    // G: wave w sums log2 alpha over token rows 8 w .. +7, lane = value row (two rows per lane at d_v = 128)
    float Gl[NVB][8];
#pragma unroll
    for (int x = 0; x < NVB; ++x) {
        const int i = lane + 64 * x;
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (GATE != GATE_NONE) run += 8 * wave + r < n ? __builtin_amdgcn_logf(pa[x][r]) : 0.f;
            Gl[x][r] = run;
        }
        Tot[wave * DV + i] = run;
    }
    block_sync();
#pragma unroll
    for (int x = 0; x < NVB; ++x) {
        const int i = lane + 64 * x;
        float carry = 0.f;
        for (int w = 0; w < wave; ++w) carry += Tot[w * DV + i];
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = Gl[x][e] + carry;
            b[e] = Gl[x][4 + e] + carry;
        }
        *reinterpret_cast<f32x4*>(GT + i * GP + 8 * wave) = a;
        *reinterpret_cast<f32x4*>(GT + i * GP + 8 * wave + 4) = b;
        if (wave == 7) gam[i] = __builtin_amdgcn_exp2f(b[3]);
    }
    {
        // P = tril(Q K^T) as D[s][t] = K Q^T tiles: wave w the t-tile w / 2 and s-tiles 2 (w % 2) .. +1
        const int tt = wave >> 1;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int st = 2 * (wave & 1) + x;
            uint2 wh = {0u, 0u}, wl = {0u, 0u};
            if (st <= tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    acc = mfma16(frag16(Kc, KP, 16 * st, 32 * m, lane), frag16(Qc, KP, 16 * tt, 32 * m, lane), acc);
                const int t = 16 * tt + m16, s0 = 16 * st + 4 * g;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = s0 + e <= t ? acc[e] : 0.f;
                split4(acc, wh, wl);
            }
            *reinterpret_cast<uint2*>(P_hi + (16 * tt + m16) * CP + 16 * st + 4 * g) = wh;
            *reinterpret_cast<uint2*>(P_lo + (16 * tt + m16) * CP + 16 * st + 4 * g) = wl;
        }
    }
    block_sync();

    // ======== phase A
    // packs of U, dO~ and dY ([t] four per tile, hi and lo) for phase B; dV and a value-channel
    // dalpha at the tile rows, written out through LDS after the phase
    uint2 pU[4][2], pO[4][2], pY[4][2];
    f32x4 rdV[4], rdA[4];
    if (wave < NWA) {
        const int i = 16 * wave + m16;
        // S (state entering the chunk) and D (gradient of the state leaving it), row i,
        // key channels 8g + 32m .. +7: the B operands of K S^T, Q S^T and K dZ^T
        bf16x8 sh[NM], sl[NM], zh[NM], zl[NM];
        const float gm = gam[i];
        float part = 0.f;  // sum_j dZ[i,j] S[i,j], then + sum_t U[t,i] (K dZ^T)[t,i]
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const f32x4 s0 = pS[m][0], s1 = pS[m][1];
            f32x4 z0 = pD[m][0], z1 = pD[m][1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z0[e] *= gm;
                z1[e] *= gm;
                part += z0[e] * s0[e] + z1[e] * s1[e];
            }
            split8(s0, s1, sh[m], sl[m]);
            split8(z0, z1, zh[m], zl[m]);
        }
        f32x4 KS[4], QS[4], KZ[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) KS[tt] = QS[tt] = KZ[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const bf16x8 kf = frag16(Kc, KP, 16 * tt, 32 * m, lane), qf = frag16(Qc, KP, 16 * tt, 32 * m, lane);
                KS[tt] = mfma16(kf, sh[m], KS[tt]);
                KS[tt] = mfma16(kf, sl[m], KS[tt]);
                QS[tt] = mfma16(qf, sh[m], QS[tt]);
                QS[tt] = mfma16(qf, sl[m], QS[tt]);
                KZ[tt] = mfma16(kf, zh[m], KZ[tt]);
                KZ[tt] = mfma16(kf, zl[m], KZ[tt]);
            }
        }
        // X = V e^{-G}, Y = X - K S^T, Yb = beta Y (tile rows t = 16 tt + 4g + r)
        f32x4 X[4], Yb[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f32x4 G4 = *reinterpret_cast<const f32x4*>(GT + i * GP + 16 * tt + 4 * g);
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + 16 * tt + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                X[tt][e] = pV[tt][e] * __builtin_amdgcn_exp2f(-G4[e]);
                Yb[tt][e] = b4[e] * (X[tt][e] - KS[tt][e]);
            }
        }
        // U = T Yb, O~ = Q S^T + P U
        bf16x8 ah[2], al[2];
        split_stack(Yb[0], Yb[1], ah[0], al[0]);
        split_stack(Yb[2], Yb[3], ah[1], al[1]);
        f32x4 U[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            U[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (m == 1 && tt < 2) continue;  // T[t][s] = 0 for s > t
                U[tt] = mfma3(frag_st(T_hi, CP, 16 * tt, 32 * m, lane), frag_st(T_lo, CP, 16 * tt, 32 * m, lane), ah[m],
                              al[m], U[tt]);
            }
        }
        split_stack(U[0], U[1], ah[0], al[0]);
        split_stack(U[2], U[3], ah[1], al[1]);
        f32x4 Ot[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            Ot[tt] = QS[tt];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (m == 1 && tt < 2) continue;
                Ot[tt] = mfma3(frag_st(P_hi, CP, 16 * tt, 32 * m, lane), frag_st(P_lo, CP, 16 * tt, 32 * m, lane), ah[m],
                               al[m], Ot[tt]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) part += U[tt][e] * KZ[tt][e];
            split4(U[tt], pU[tt][0], pU[tt][1]);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);  // the column's sum over all four groups
        // dO~ = dO e^{G}; dU = K dZ^T + P^T dO~
        f32x4 dOt[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f32x4 G4 = *reinterpret_cast<const f32x4*>(GT + i * GP + 16 * tt + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) dOt[tt][e] = pdO[tt][e] * __builtin_amdgcn_exp2f(G4[e]);
            split4(dOt[tt], pO[tt][0], pO[tt][1]);
        }
        split_stack(dOt[0], dOt[1], ah[0], al[0]);
        split_stack(dOt[2], dOt[3], ah[1], al[1]);
        f32x4 dU[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            dU[st] = KZ[st];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (st >= 2 && m == 0) continue;  // P^T[s][t] = 0 for t < s
                dU[st] = mfma3(frag_tr_st(P_hi, CP, 16 * st, 32 * m, lane), frag_tr_st(P_lo, CP, 16 * st, 32 * m, lane),
                               ah[m], al[m], dU[st]);
            }
        }
        // dYb = T^T dU; dY = beta dYb; this wave's part of dbeta_t = sum_i dYb U / beta
        split_stack(dU[0], dU[1], ah[0], al[0]);
        split_stack(dU[2], dU[3], ah[1], al[1]);
        f32x4 dY[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            dY[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (st >= 2 && m == 0) continue;
                dY[st] = mfma3(frag_tr_st(T_hi, CP, 16 * st, 32 * m, lane), frag_tr_st(T_lo, CP, 16 * st, 32 * m, lane),
                               ah[m], al[m], dY[st]);
            }
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + 16 * st + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pb = sum16(dY[st][e] * U[st][e]);
                if (m16 == 0) red[wave * C + 16 * st + 4 * g + e] = pb;
                dY[st][e] *= b4[e];
            }
            split4(dY[st], pY[st][0], pY[st][1]);
        }
        // dV = dY e^{-G}; dG = dO~ O~ - dY X (+ the gradient through gamma on the last token);
        // dg = reverse cumulative sum of dG over the chunk; dalpha = dg / alpha
        float dG[4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f32x4 G4 = *reinterpret_cast<const f32x4*>(GT + i * GP + 16 * tt + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tt + 4 * g + e;
                rdV[tt][e] = dY[tt][e] * __builtin_amdgcn_exp2f(-G4[e]);
                dG[tt][e] = dOt[tt][e] * Ot[tt][e] - dY[tt][e] * X[tt][e] + (t == n - 1 ? part : 0.f);
            }
        }
        if constexpr (GATE != GATE_NONE) {
            float tile_tot[4], loc[4][4], excl[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                loc[tt][3] = dG[tt][3];
#pragma unroll
                for (int e = 2; e >= 0; --e) loc[tt][e] = dG[tt][e] + loc[tt][e + 1];
                const float tg = loc[tt][0];
                const float y1 = __shfl_down(tg, 16), y2 = __shfl_down(tg, 32), y3 = __shfl_down(tg, 48);
                excl[tt] = (g < 3 ? y1 : 0.f) + (g < 2 ? y2 : 0.f) + (g < 1 ? y3 : 0.f);
                float tot = tg + __shfl_xor(tg, 16);
                tile_tot[tt] = tot + __shfl_xor(tot, 32);
            }
            float carry = 0.f;
#pragma unroll
            for (int tt = 3; tt >= 0; --tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * g + e;
                    const float dg = loc[tt][e] + excl[tt] + carry;
                    if constexpr (GATE == GATE_CHANNEL) {
                        // alpha_t = 2^{G_t - G_{t-1}} from the staged log2-decays (rounding ~1e-7 |G|)
                        const float gp = t > 0 ? GT[i * GP + t - 1] : 0.f;
                        rdA[tt][e] = dg * __builtin_amdgcn_exp2f(gp - GT[i * GP + t]);
                    } else {
                        const float ps = sum16(dg);
                        if (m16 == 0) red2[wave * C + t] = ps;
                    }
                }
                carry += tile_tot[tt];
            }
        }
    }
    block_sync();  // phase A done: T, P and G^T are dead
    // phase B's B operands of its first round (value rows 0-63 of S and D at this lane's key
    // channel), issued now so that they arrive under the dV stores
    const int jt = wave % NJT, tt0 = (wave / NJT) * TPW;
    const int jc = 16 * jt + m16;  // this lane's key channel (B-operand column)
    const float* sbase = sck + (static_cast<int64_t>(gc) * H + h) * DV * DK + jc;
    const float* gbase = gck + (static_cast<int64_t>(gc) * H + h) * DV * DK + jc;
    f32x4 cs[2][2], cz[2][2];  // [m][half]: rows 64 r + 32 m + 16 half + 4 g .. +3
    auto load_sd = [&](int r) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t row = 64 * r + 32 * m + 16 * x + 4 * g + e;
                    cs[m][x][e] = sbase[row * DK];
                    cz[m][x][e] = gbase[row * DK];
                }
    };
    load_sd(0);
    {
        // dV (and a value-channel dalpha) through LDS as whole token rows [t][i], stored as
        // 16-byte pieces of each row: the tile layout has 4 tokens of one row per lane
        constexpr int VP = DV + 4;
        float* sv = reinterpret_cast<float*>(ur);
        float* sa = sv + C * VP;
        if (wave < NWA) {
            const int i = 16 * wave + m16;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * g + e;
                    sv[t * VP + i] = rdV[tt][e];
                    if constexpr (GATE == GATE_CHANNEL) sa[t * VP + i] = rdA[tt][e];
                }
        }
        block_sync();
        const auto rdv = make_rsrc(dv + tok0 * DV, ((n - 1) * row_v + DV) * 4);
        const auto rda = make_rsrc(dalpha + tok0 * DV, GATE == GATE_CHANNEL ? ((n - 1) * row_v + DV) * 4 : 0);
        for (int x = tid; x < C * DV / 4; x += 512) {
            const int t = x / (DV / 4), c4 = 4 * (x % (DV / 4));
            const int off = static_cast<int>(t * row_v + c4) * 4;
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(sv + t * VP + c4), rdv, off, 0, 0);
            if constexpr (GATE == GATE_CHANNEL)
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(sa + t * VP + c4), rda, off, 0, 0);
        }
        block_sync();  // the staging rows are read before phase B reuses the space
    }
    if (tid < n) {
        float sb = 0.f, sa = 0.f;
        for (int w = 0; w < NWA; ++w) {
            sb += red[w * C + tid];
            if (GATE == GATE_SCALAR) sa += red2[w * C + tid];
        }
        dbeta[tok0 + tid * H] = sb / bs[tid];
        if (GATE == GATE_SCALAR) dalpha[tok0 + tid * H] = sa / alpha[tok0 + tid * H];
    }

    // ======== phase B
    f32x4 DQ[TPW], DK_[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) DQ[x] = DK_[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    // dP and dKK tiles over rows: the 10 lower 16x16 tiles of each, 20 in all, wave w takes w, w + 8, w + 16
    f32x4 PT[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) PT[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto lower_tile = [](int e, int& tr, int& tc) {
        tr = e < 1 ? 0 : e < 3 ? 1 : e < 6 ? 2 : 3;
        tc = e - tr * (tr + 1) / 2;
    };
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (wave >= 4 * r && wave < 4 * r + 4) {
            const int il = 16 * (wave - 4 * r) + m16;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int o = il * CP + 16 * tt + 4 * g;
                *reinterpret_cast<uint2*>(UT_hi + o) = pU[tt][0];
                *reinterpret_cast<uint2*>(UT_lo + o) = pU[tt][1];
                *reinterpret_cast<uint2*>(OT_hi + o) = pO[tt][0];
                *reinterpret_cast<uint2*>(OT_lo + o) = pO[tt][1];
                *reinterpret_cast<uint2*>(YT_hi + o) = pY[tt][0];
                *reinterpret_cast<uint2*>(YT_lo + o) = pY[tt][1];
            }
        }
        block_sync();
        // dP += dO~ U^T, dKK += dY U^T over this round's 64 rows
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int e = wave + 8 * x;
            if (e < 20) {
                int tr, tc;
                lower_tile(e % 10, tr, tc);
                const uint16_t* Ah = e < 10 ? OT_hi : YT_hi;
                const uint16_t* Al = e < 10 ? OT_lo : YT_lo;
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    PT[x] = mfma3(frag_tr_st(Ah, CP, 16 * tr, 32 * m, lane), frag_tr_st(Al, CP, 16 * tr, 32 * m, lane),
                                  frag_tr_st(UT_hi, CP, 16 * tc, 32 * m, lane), frag_tr_st(UT_lo, CP, 16 * tc, 32 * m, lane),
                                  PT[x]);
            }
        }
        // dq += dO~ S, dk += U dZ - dY S over this round's rows: B operands (column j, stacked rows i)
        // from the state and gradient checkpoints
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const f32x4 s0 = cs[m][0], s1 = cs[m][1];
            f32x4 z0 = cz[m][0], z1 = cz[m][1];
            const int ib = 64 * r + 32 * m + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z0[e] *= gam[ib + e];
                z1[e] *= gam[ib + 16 + e];
            }
            bf16x8 sh, sl, nh, nl, zh, zl;
            split8(s0, s1, sh, sl);
            split8(-s0, -s1, nh, nl);
            split8(z0, z1, zh, zl);
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int tt = tt0 + x;
                DQ[x] = mfma3(frag_tr_st(OT_hi, CP, 16 * tt, 32 * m, lane), frag_tr_st(OT_lo, CP, 16 * tt, 32 * m, lane), sh,
                              sl, DQ[x]);
                DK_[x] = mfma3(frag_tr_st(UT_hi, CP, 16 * tt, 32 * m, lane), frag_tr_st(UT_lo, CP, 16 * tt, 32 * m, lane),
                               zh, zl, DK_[x]);
                DK_[x] = mfma3(frag_tr_st(YT_hi, CP, 16 * tt, 32 * m, lane), frag_tr_st(YT_lo, CP, 16 * tt, 32 * m, lane),
                               nh, nl, DK_[x]);
            }
        }
        if (r + 1 < NR) load_sd(r + 1);  // the next round's, under this round's barrier
        block_sync();  // the round's buffers are read
    }
    fetch_stage(nxt, more && !nxt.marked);  // the next item's, under this item's last phase
    // dP (lower, diagonal kept) and dKK (strictly lower, negated) -> LDS [t][s]; their upper tiles are zero
    for (int x = tid; x < 6 * 256; x += 512) {
        const int tile = x >> 8, y = x & 255;
        const int tr = tile < 3 ? 0 : tile < 5 ? 1 : 2, tc = tile < 3 ? 1 + tile : tile < 5 ? tile - 1 : 3;
        const int o = (16 * tr + (y >> 4)) * CP + 16 * tc + (y & 15);
        dP_hi[o] = dP_lo[o] = dK_hi[o] = dK_lo[o] = 0;
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        const int e = wave + 8 * x;
        if (e < 20) {
            int tr, tc;
            lower_tile(e % 10, tr, tc);
            const bool isP = e < 10;
            uint16_t* Dh = isP ? dP_hi : dK_hi;
            uint16_t* Dl = isP ? dP_lo : dK_lo;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = 16 * tr + 4 * g + rr, s = 16 * tc + m16;
                const float val = isP ? (s <= t ? PT[x][rr] : 0.f) : (s < t ? -PT[x][rr] : 0.f);
                const uint16_t hb = f32_to_bf16_bits(val);
                Dh[t * CP + s] = hb;
                Dl[t * CP + s] = f32_to_bf16_bits(val - bf16_bits_to_f32(hb));
            }
        }
    }
    block_sync();
    // dq += dP K; dk += dP^T Q + dKK K + dKK^T K (B operands: column j, stacked rows s)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const bf16x8 bk = frag_tr_st(Kc, KP, 16 * jt, 32 * m, lane);
        const bf16x8 bq = frag_tr_st(Qc, KP, 16 * jt, 32 * m, lane);
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int tt = tt0 + x;
            if (m == 0 || tt >= 2) {  // dP[t][s], dKK[t][s] = 0 for s > t
                DQ[x] = mfma16(frag_st(dP_hi, CP, 16 * tt, 32 * m, lane), bk, DQ[x]);
                DQ[x] = mfma16(frag_st(dP_lo, CP, 16 * tt, 32 * m, lane), bk, DQ[x]);
                DK_[x] = mfma16(frag_st(dK_hi, CP, 16 * tt, 32 * m, lane), bk, DK_[x]);
                DK_[x] = mfma16(frag_st(dK_lo, CP, 16 * tt, 32 * m, lane), bk, DK_[x]);
            }
            if (m == 1 || tt < 2) {  // dP^T[t][s], dKK^T[t][s] = 0 for s < t
                DK_[x] = mfma16(frag_tr_st(dP_hi, CP, 16 * tt, 32 * m, lane), bq, DK_[x]);
                DK_[x] = mfma16(frag_tr_st(dP_lo, CP, 16 * tt, 32 * m, lane), bq, DK_[x]);
                DK_[x] = mfma16(frag_tr_st(dK_hi, CP, 16 * tt, 32 * m, lane), bk, DK_[x]);
                DK_[x] = mfma16(frag_tr_st(dK_lo, CP, 16 * tt, 32 * m, lane), bk, DK_[x]);
            }
        }
    }
    const auto rdq = make_rsrc(dq + tok0 * DK, ((n - 1) * row_qk + DK) * 4);
    const auto rdk = make_rsrc(dk + tok0 * DK, ((n - 1) * row_qk + DK) * 4);
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * (tt0 + x) + 4 * g + e;
            const int off = static_cast<int>(t * row_qk + jc) * 4;
            // (__float_as_uint on the element value: a bit_cast of an ext-vector subscript
            // reads element 0 with this compiler)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(DQ[x][e]), rdq, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(DK_[x][e]), rdk, off, 0, 0);
        }
    }
    if (!more) break;
    it = it_next;
    cur = nxt;
    block_sync();  // every wave is done with this item's LDS before the next one's staging
    }
    }
}

// ---------------------------------------------------------------- launchers
template <int DK, int DV, int GATE>
static hipError_t launch_bwd_chunk_t(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream) {
    constexpr int NVB = DV / 64;
    const int64_t grid1 = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((bwd_state_scan_kernel<DK, DV, GATE>), dim3(static_cast<unsigned>(grid1)), dim3(512), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.alpha, a.beta, a.dO,
                       a.dS_T, a.cu_seqlens, b.order, b.chunk_off, b.rec, b.flags, a.n_seq, a.n_tok, a.n_heads, b.gck,
                       a.dS0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_tok == 0) return e;
    // one resident workgroup per CU (the LDS allows no more), each looping over (chunk, head) items
    int dev = 0, n_cu = 0;
    if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t grid2 = std::min<int64_t>(b.max_chunks * static_cast<int64_t>(a.n_heads), n_cu);
    hipLaunchKernelGGL((bwd_chunk_grad_kernel<DK, DV, GATE>), dim3(static_cast<unsigned>(grid2)), dim3(512), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.alpha, a.beta, a.dO, a.cu_seqlens, b.chunk_off, b.rec,
                       b.sck, b.gck, b.flags, a.n_seq, a.n_tok, a.n_heads, static_cast<int>(b.max_chunks), a.dq, a.dk,
                       a.dv, a.dalpha, a.dbeta);
    return hipGetLastError();
}

template <int GATE>
static hipError_t launch_bwd_chunk_g(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_bwd_chunk_t<128, 128, GATE>(a, b, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_bwd_chunk_t<64, 64, GATE>(a, b, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_bwd_chunk_t<128, 64, GATE>(a, b, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_bwd_chunk_t<64, 128, GATE>(a, b, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_backward_chunk_passes(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream) {
    switch (a.gate) {
        case GATE_CHANNEL: return launch_bwd_chunk_g<GATE_CHANNEL>(a, b, stream);
        case GATE_SCALAR: return launch_bwd_chunk_g<GATE_SCALAR>(a, b, stream);
        case GATE_NONE: return launch_bwd_chunk_g<GATE_NONE>(a, b, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
