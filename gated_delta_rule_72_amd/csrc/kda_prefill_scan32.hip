// kda_prefill_scan32.hip -- the S-dependent chunk products of the bf16 prefill
// (value-channel, scalar or no gate) in steps of 32 tokens, with every staged
// input double-buffered so that the staging of one step overlaps the matrix work
// of the step before.
//
// The recurrence is that of page "Kimi (AI)", section "Kimi Delta Attention
// (KDA)", in the chunk form written out in kda_prefill_mfma.hip, applied to half
// chunks: a 64-token chunk's system (I + L) is lower triangular, so the two 32x32
// diagonal blocks of its solved record A = (I + L)^{-1} diag(beta) are exactly the
// solved systems of its two halves.  The chunk solve therefore serves this scan with
// the records' diagonal blocks (0 and 2), and chunks are numbered as there.
//
// A 16x16 MFMA accumulator tile holds, in lane (column n = l % 16, group g = l / 16),
// rows 4g..4g+3.  Two tiles stacked along the row index give a lane the 8 rows
// {4g..4g+3, 16+4g..16+4g+3}; taken as the 8 reduction indices of a
// v_mfma_f32_16x16x32_bf16 B operand (the A operand reads the same indices, two
// 8-byte pieces per lane), Y, U and S feed the next product straight from the
// accumulators.
//
// One workgroup of 8 waves per (sequence, head, block of 64 value rows):
// - chain waves (0, 1) own 32 value rows each and keep S^T in fp32 accumulators;
//   per step: Y = X - K S^T, U = A Y (A, Y as hi + lo), then
//   S^T <- diag(gamma) (S^T + K^T U).  They form -Y = K S^T - X from the staged -X and
//   the bf16 copy of S that the S update already packed, and U = (-A)(-Y) from the
//   staged -A, so no sign flips sit on their path;
// - out waves (2, 3): O^T = 2^G (S Q^T + U^T P^T) for the same rows, with P = tril(Q K^T)
//   formed from the same K and Q fragments and kept in registers; O staged as bf16 rows
//   and stored at the next step;
// - loader waves (4-7) prepare the next step: K, Q and the A block into LDS, the
//   decay 2^G as prefix products of the gates (8 token rows per wave, a lane per value
//   row), X^T = V 2^{-G} and gamma; their loads are issued two steps ahead.
// Two barriers per step.  B0: step s is staged.  Chain: Y, U, the U^T copy  --  out:
// store O of s - 1, S Q^T and P  --  loaders: stage K, Q, A of s + 1, local prefix.  B1.
// Chain: S^T update, the S copy for step s + 1  --  out: U^T P^T, 2^G, stage O  --
// loaders: finish G, X^T, gamma of s + 1, load s + 3.
// K, Q, A, X^T, G and gamma alternate between two buffers by step parity; the S copy,
// the U^T copy and the O rows have one buffer each (written and read in alternate
// phases).
//
// CKPT (the chunked backward's forward pass): the chain waves store the state entering
// every 64-token chunk (every even step) into ckpt ([chunk, H, d_v, d_k] fp32, global
// chunk numbering) and form K S^T from a hi + lo copy of the state (the checkpoints feed
// dq and dk directly, where one bf16 copy's rounding is not damped by any decay); the
// output side is left out (no q, no P, no O: the out waves only keep the barriers).  A
// unit is marked when a 64-token chunk's decay is below 2^-100, the range of the
// backward's chunk form, or one of its gates is below 2^-5 (the backward's
// dalpha = dg / alpha would amplify its rounding there); marks are only set, since the
// backward clears them beforehand and its chunk solve may already have set some.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_schedule.h"

namespace kda {
namespace {

constexpr int H32 = 32;            // tokens per step
template <int V>
struct Parity {
    static constexpr int value = V;
};
// Range: X = V 2^{-G} and U grow like 2^{-G} inside a step, so the factored form holds
// only while every row's decay over a step stays above RANGE32_MIN (alpha in [0, 1]: the
// step's total is its smallest prefix).  Wave 7 checks each step's totals; a unit with
// any step beyond the range (alpha = 0 gives 0) is marked in range_flags[unit] and does
// not write S_T, so that S0 is intact when S_T aliases it, and a token-recurrent pass
// recomputes exactly the marked units afterwards.  Above the limit 2^{-G} stays below
// 2^{100}: fp32 and bf16 (same exponent range) keep it, and the products with A, P and
// K add at most a few powers of two.
constexpr float RANGE32_MIN = 0x1p-100f;

template <int DK>
struct Scan32Smem {
    static constexpr int KP = DK + PAD;       // K rows (bf16)
    static constexpr int QP = DK + 2 * PAD;   // Q rows (bf16)
    static constexpr int SXP = DK + PAD;      // S rows (bf16): 4 (mod 8) dwords, conflict-free for the
                                              // chain's 8-byte writes (0 (mod 8) suits Q's 16-byte reads)
    static constexpr int AP = H32 + PAD;      // A and U^T rows of 32 (bf16)
    static constexpr int XP = H32 + 4;        // X^T rows (fp32)
    static constexpr int GP = BV + 4;         // 2^G rows (fp32)
    static constexpr int OP = BV + PAD;       // O rows (bf16)
    static constexpr int RK = H32 * KP * 2;
    static constexpr int RQ = H32 * QP * 2;
    static constexpr int RA = 2 * H32 * AP * 2;  // hi, lo
    static constexpr int RX = BV * XP * 4;
    static constexpr int RG = H32 * GP * 4;
    static constexpr int RB = BV * 4;
    static constexpr int RS = BV * SXP * 2;
    static constexpr int RU = 2 * BV * AP * 2;
    static constexpr int RO = H32 * OP * 2;
    static constexpr int RT = 2 * 4 * BV * 4;
    static constexpr int TOTAL = 2 * (RK + RQ + RA + RX + RG + RB) + RS + RU + RO + RT;
};

// The scan of the unit that workgroup `block` maps to (the kernels below).  alpha null with a
// gate: every gate is 1 (the transitions' pass, launched together with a gated pass).
template <int DK, int DV, int GATE, bool NOOUT, bool SPLIT, bool CKPT>
__device__ __forceinline__ void scan32_body(
    int64_t block, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ arec,
    int n_seq, int n_tok, int n_heads, uint16_t* __restrict__ o, float* __restrict__ S_T, int flags,
    float* __restrict__ gdecay, int32_t* __restrict__ range_flags, float* __restrict__ ckpt,
    const int32_t* __restrict__ skip_flags, int skip_segs) {
    static_assert(!CKPT || (NOOUT && SPLIT), "the checkpoint variant has no output side and splits the state");
    using SM = Scan32Smem<DK>;
    static_assert(SM::TOTAL <= 160 * 1024, "LDS budget");
    static_assert(DK == 64 || DK == 128, "d_k");
    constexpr int NVB = DV / BV;
    constexpr int KP = SM::KP, QP = SM::QP, SXP = SM::SXP, AP = SM::AP, XP = SM::XP, GP = SM::GP, OP = SM::OP;
    constexpr int NJ = DK / 16;   // 16-row tiles of S^T along j
    constexpr int NM = DK / 32;   // 32-wide reduction steps over j
    constexpr int PPR = DK / 8;   // 16-byte pieces per row of q or k
    constexpr int NKQ = H32 * PPR / 256;  // pieces of K (and of Q) per loader thread

    __shared__ __align__(16) uint16_t Kb[2][H32 * KP];
    __shared__ __align__(16) uint16_t Qb[2][H32 * QP];
    __shared__ __align__(16) uint16_t Ab[2][2 * H32 * AP];  // hi rows, then lo rows
    __shared__ __align__(16) float Xb[2][BV * XP];          // X^T [i][t]
    __shared__ __align__(16) float Gb[2][H32 * GP];          // 2^G [t][i]
    __shared__ __align__(16) float gamb[2][BV];
    __shared__ __align__(16) uint16_t Sx[BV * SXP];           // S [i][j], bf16
    __shared__ __align__(16) uint16_t Ux[2 * BV * AP];       // U^T [i][t] hi rows, then lo rows
    __shared__ __align__(16) uint16_t Os[H32 * OP];          // O [t][i], bf16
    __shared__ __align__(16) float Tot[2][BV][4];           // loader totals, per value row
    __shared__ int beyond_s[4];

    const Unit u = map_unit(block, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // chain waves and their 16-row blocks: two waves of 32 rows, or without an output side
    // (no out waves) four of 16, which halves each chain wave's dependent work per step
    constexpr int NCH = NOOUT ? 4 : 2;
    constexpr int NIB = 4 / NCH;
    const bool chain = wave < NCH;
    const bool outw = !NOOUT && (wave == 2 || wave == 3);
    const bool loader = wave >= 4;
    const int rb = 16 * NIB * (wave & (NCH - 1));  // first of the value rows of a chain or out wave
    const int lw = wave - 4;         // loader index: token rows 8 lw .. +7
    const int64_t H = n_heads;
    const int h = u.head;
    const int i0 = u.vblk * BV;
    if (skip_flags) {
        // a unit of a sequence that another pass recomputes token by token: any of the
        // skip_segs segments of its sequence marked for this block of rows (one per lane)
        const int64_t n0 = u.seq / skip_segs * static_cast<int64_t>(skip_segs);
        bool m = false;
        for (int g = lane; g < skip_segs; g += 64) m |= skip_flags[((n0 + g) * H + h) * NVB + u.vblk] != 0;
        if (__ballot(m) != 0) return;
    }
    const int64_t row_qk = H * DK, row_v = H * DV;
    const int chunk0 = first_chunk(u.seq, n_seq, n_tok, chunk_off);
    const int n_steps = static_cast<int>((u.t1 - u.t0 + H32 - 1) / H32);
    // tokens of step s (0 outside the unit's steps)
    auto step_len = [&](int s) {
        return s < 0 ? 0
                     : static_cast<int>(max<int64_t>(0, min<int64_t>(H32, u.t1 - (u.t0 + static_cast<int64_t>(s) * H32))));
    };

    // ---- one register array holds each role's long-lived values: the chain's S^T
    // (at NJ ib + jt), U^T packs (CU0 ..) and bf16 copy of S (SP0 .., then its lo part at
    // SPL0 .. under SPLIT), the out waves' O^T accumulators and P operands (CU0 ..), the
    // loaders' pieces of two steps (set x at LS0 + LSN x)
    constexpr int CU0 = NIB * NJ;
    constexpr int SP0 = CU0 + 4;
    constexpr int SPL0 = SP0 + NIB * NJ / 2;
    constexpr int LK = 0, LQ = NKQ, LA = 2 * NKQ, LV = LA + 1, LL = LV + 2, LSN = LL + 2;
    constexpr int LS0 = 0;
    constexpr int SPE = SPLIT ? SPL0 + NIB * NJ / 2 : SP0 + NIB * NJ / 2;
    constexpr int RC = (CU0 + 8 > SPE) ? CU0 + 8 : SPE;
    constexpr int RN = (RC > LS0 + 2 * LSN) ? RC : LS0 + 2 * LSN;
    f32x4 R[RN];
#pragma unroll
    for (int x = 0; x < RN; ++x) R[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t s_base = ((static_cast<int64_t>(u.seq) * H + h) * DV + i0) * DK;
    // (S0 is loaded here, before the role dispatch, rather than in the chain's own prologue:
    // measured with the fetch counters, that order costs the scan about 7% fewer HBM reads)
    if (chain && (flags & SCAN_S0_IDENTITY)) {
        // S0 = I (d_v = d_k): row i holds 1 at key channel i
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            const int row = i0 + rb + 16 * ib + (lane & 15);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) R[ib * NJ + jt][e] = row == 16 * jt + 4 * (lane >> 4) + e ? 1.f : 0.f;
        }
    } else if (chain && S0) {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            const float* src = S0 + s_base + static_cast<int64_t>(rb + 16 * ib + (lane & 15)) * DK + 4 * (lane >> 4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) R[ib * NJ + jt] = *reinterpret_cast<const f32x4*>(src + 16 * jt);
        }
    }
    // S [i][j] as bf16 for the out waves (lane holds j = 16 jt + 4g .. +3 of row i), and the
    // same words kept as the B operands of K S^T: for the 32-wide j step m the stacked pair
    // of tiles 2m, 2m + 1 is R[SP0 + (NJ / 2) ib + m]; tile jt of both row blocks, first
    // scaled by gamma (the decay of the step)
    auto pack_tile = [&](int jt, int ln) {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
            uint2 w;
            if constexpr (SPLIT) {
                uint2 wl;
                split_bf16x2(R[ib * NJ + jt][0], R[ib * NJ + jt][1], w.x, wl.x);
                split_bf16x2(R[ib * NJ + jt][2], R[ib * NJ + jt][3], w.y, wl.y);
                R[SPL0 + (NJ / 2) * ib + jt / 2][2 * (jt & 1)] = __uint_as_float(wl.x);
                R[SPL0 + (NJ / 2) * ib + jt / 2][2 * (jt & 1) + 1] = __uint_as_float(wl.y);
            } else {
                w.x = pack_bf16(R[ib * NJ + jt][0], R[ib * NJ + jt][1]);
                w.y = pack_bf16(R[ib * NJ + jt][2], R[ib * NJ + jt][3]);
            }
            if constexpr (!NOOUT) {
                uint16_t* dst = Sx + (rb + 16 * ib + (ln & 15)) * SXP + 4 * (ln >> 4);
                *reinterpret_cast<uint2*>(dst + 16 * jt) = w;
            }
            R[SP0 + (NJ / 2) * ib + jt / 2][2 * (jt & 1)] = __uint_as_float(w.x);
            R[SP0 + (NJ / 2) * ib + jt / 2][2 * (jt & 1) + 1] = __uint_as_float(w.y);
        }
    };
    auto scale_pack = [&](int jt, const float (&gm)[NIB], int ln) {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) R[ib * NJ + jt] *= gm[ib];
        pack_tile(jt, ln);
    };
    auto pack_state = [&](int ln) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) pack_tile(jt, ln);
    };

    // ---- a loader's loads of step s into register set x (a step past the end loads
    // nothing: empty ranges), in two parts issued at different points: K, Q and the A block
    // (loader thread ht holds 16-byte pieces ht + 256 p of K and Q, row-major, and piece ht
    // of the step's A block: 32 rows of 4 pieces, hi then lo), then V and alpha (token rows
    // 8 lw .. +7, lane = value row).
    auto step_tok0 = [&](int s) {
        const int sc = step_len(s) > 0 ? s : 0;
        return (u.t0 + static_cast<int64_t>(sc) * H32) * H + h;
    };
    auto fetch_kqa = [&](int s, int x) {
        const int ht = tid - 256;
        const int n = step_len(s);
        const bool any = n > 0;
        const int sc = any ? s : 0;
        const int64_t tok0 = step_tok0(s);
        const int64_t bqk = any ? ((n - 1) * row_qk + DK) * 2 : 0;
        const auto rk_ = make_rsrc(k + tok0 * DK, bqk);
        const auto rq_ = make_rsrc(q + tok0 * DK, bqk);
        const int b0 = LS0 + LSN * x;
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int idx = ht + 256 * p;
            const int off = static_cast<int>((idx / PPR) * row_qk + 8 * (idx % PPR)) * 2;
            R[b0 + LK + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk_, off, 0, 0));
            if constexpr (!NOOUT)
                R[b0 + LQ + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq_, off, 0, 0));
        }
        // block 2 (s % 2) of the chunk's record: rows 0-31 x cols 0-31 for the first
        // half, rows 32-63 x cols 32-63 for the second; each block is hi then lo.  The
        // forward's records are packed (pieces above the diagonal left out), the backward's
        // whole; either way the threads of all-zero pieces read past the range, which
        // returns zero without touching memory.
        constexpr bool TRI = !CKPT;
        const int64_t rec = static_cast<int64_t>(chunk0 + sc / 2) * n_heads + h;
        const uint16_t* blk = TRI ? arec + rec * (A_TRI_RECORD_BYTES / 2) + (sc & 1) * A_TRI_BLOCK_ELEMS
                                  : arec + rec * (A_RECORD_BYTES / 2) + (sc & 1) * 2 * (2 * A_BLOCK_ELEMS);
        constexpr int blk_bytes = TRI ? A_TRI_BLOCK_ELEMS * 2 : 2 * A_BLOCK_ELEMS * 2;
        const auto ra_ = make_rsrc(blk, any ? blk_bytes : 0);
        const int pc = ht & 3, prow = (ht >> 2) & 31;
        const int aoff = pc > (prow >> 3) ? blk_bytes
                         : TRI             ? ((ht >> 7) * A_TRI_PIECES + tri_piece(prow, pc)) * 16
                                           : ht * 16;
        R[b0 + LA] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra_, aoff, 0, 0));
    };
    auto fetch_vl = [&](int s, int x) {
        const int n = step_len(s);
        const bool any = n > 0;
        const int64_t tok0 = step_tok0(s);
        const int b0 = LS0 + LSN * x;
        // (v reads as zero when the flag asks for it: an empty range)
        const auto rv = make_rsrc(v + tok0 * DV + i0, any && !(flags & SCAN_ZERO_V) ? ((n - 1) * row_v + BV) * 2 : 0);
        // (without alpha -- a gated instantiation run with every gate 1 -- an empty range:
        // the loads return 0 and touch no memory, and local_scan takes 1 for them)
        const bool gl = any && alpha != nullptr;
        const auto rl = GATE == GATE_CHANNEL && gl ? make_rsrc(alpha + tok0 * DV + i0, ((n - 1) * row_v + BV) * 4)
                        : GATE == GATE_SCALAR && gl ? make_rsrc(alpha + tok0, ((n - 1) * H + 1) * 4)
                                                    : make_rsrc(alpha, 0);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e = static_cast<int>((8 * lw + r) * row_v + lane);
            // the bf16 bits, zero-extended (shifted into place where they are used)
            R[b0 + LV + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b16(rv, e * 2, 0, 0));
            if constexpr (GATE != GATE_NONE) {
                const int ea = GATE == GATE_CHANNEL ? e : static_cast<int>((8 * lw + r) * H);
                R[b0 + LL + r / 4][r % 4] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, ea * 4, 0, 0));
            }
        }
    };
    auto fetch = [&](int s, int x) {
        fetch_kqa(s, x);
        fetch_vl(s, x);
    };
    // stage K, Q and the A block of step s (set x) into buffer par, A with its sign flipped
    auto stage = [&](int x, int par, int ln) {
        const int ht = ln + 64 * lw;
        const int b0 = LS0 + LSN * x;
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int idx = ht + 256 * p;
            *reinterpret_cast<f32x4*>(Kb[par] + (idx / PPR) * KP + 8 * (idx % PPR)) = R[b0 + LK + p];
            if constexpr (!NOOUT)
                *reinterpret_cast<f32x4*>(Qb[par] + (idx / PPR) * QP + 8 * (idx % PPR)) = R[b0 + LQ + p];
        }
        // piece ht: half ht / 128, row (ht / 4) % 32, columns 8 (ht % 4) ..
        const u32x4 na = __builtin_bit_cast(u32x4, R[b0 + LA]) ^ 0x80008000u;
        *reinterpret_cast<u32x4*>(Ab[par] + ((ht >> 7) * H32 + ((ht >> 2) & 31)) * AP + 8 * (ht & 3)) = na;
    };
    // The decay as products (no logarithms): each loader's inclusive prefix product of the
    // gates over its 8 token rows, in the alpha registers, and V over that product in the V
    // registers (one reciprocal, then suffix products); the loader's total to Tot[par][lw].
    // Rows past the sequence end contribute 1.  Within a step nothing underflows: a step
    // whose total decay is below 2^-100 marks the unit for the recurrent pass, and every
    // prefix is at least the total.
    // loaders: some step (CKPT: some 64-token chunk, or one gate) of some row of the unit is
    // beyond the range
    bool beyond = false;
    float prev_tot = 1.f;  // wave 7, CKPT: the decay of the chunk's first step
    float gprod = 1.f;     // wave 7: the row's total decay over the unit's steps
    auto local_scan = [&](int n, int x, int par, int ln) {
        const int b0 = LS0 + LSN * x;
        float a[8];
        float run = 1.f, amin = 1.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            a[r] = GATE != GATE_NONE && alpha && 8 * lw + r < n ? R[b0 + LL + r / 4][r % 4] : 1.f;
            run *= a[r];
            amin = fminf(amin, a[r]);
            R[b0 + LL + r / 4][r % 4] = run;
        }
        // (also true for a NaN gate)
        if constexpr (CKPT) beyond = beyond || __builtin_amdgcn_ballot_w64(!(amin >= 0x1p-5f)) != 0;
        float inv = __builtin_amdgcn_rcpf(run);  // 1 / prefix of row 7, then of rows 6, 5, ..
#pragma unroll
        for (int r = 7; r >= 0; --r) {
            R[b0 + LV + r / 4][r % 4] = __uint_as_float(__float_as_uint(R[b0 + LV + r / 4][r % 4]) << 16) * inv;
            inv *= a[r];
        }
        Tot[par][ln][lw] = run;
    };
    // after a barrier: multiply in the totals of the loaders before, write 2^G [t][i],
    // -X^T [i][t] and (wave 7) gamma
    auto finalize = [&](int x, int par, int ln) {
        const int b0 = LS0 + LSN * x;
        const f32x4 tl = *reinterpret_cast<const f32x4*>(&Tot[par][ln][0]);
        float carry = 1.f;
#pragma unroll
        for (int b = 0; b < 3; ++b) carry *= b < lw ? tl[b] : 1.f;
        const float nic = -__builtin_amdgcn_rcpf(carry);
        float* xt = Xb[par] + ln * XP + 8 * lw;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if constexpr (!NOOUT) Gb[par][(8 * lw + 4 * p + e) * GP + ln] = R[b0 + LL + p][e] * carry;
            *reinterpret_cast<f32x4*>(xt + 4 * p) = R[b0 + LV + p] * nic;
        }
        if (lw == 3) {
            const float tot = R[b0 + LL + 1][3] * carry;
            gamb[par][ln] = tot;
            gprod *= tot;  // (steps outside the unit contribute 1)
            // (also true for a NaN total)
            if constexpr (CKPT) {
                // a chunk is the step pair (even, odd): its decay is the product of theirs
                if (par == 0) prev_tot = tot;
                else beyond = beyond || __builtin_amdgcn_ballot_w64(!(prev_tot * tot >= RANGE32_MIN)) != 0;
            } else {
                beyond = beyond || __builtin_amdgcn_ballot_w64(!(tot >= RANGE32_MIN)) != 0;
            }
        }
    };
    // staged O rows of a finished step -> global by the out waves, two 16-byte pieces
    // per thread (n = 0: nothing is stored)
    auto store_o = [&](int s, int ln) {
        const int n = step_len(s);
        const int64_t tc = u.t0 + static_cast<int64_t>(n > 0 ? s : 0) * H32;
        const auto ro = make_rsrc(o + (tc * H + h) * DV + i0, n > 0 ? ((n - 1) * row_v + BV) * 2 : 0);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int idx = ln + 64 * (wave - 2) + 128 * p, t = idx >> 3, c = idx & 7;
            const u32x4 val = *reinterpret_cast<const u32x4*>(Os + t * OP + 8 * c);
            __builtin_amdgcn_raw_buffer_store_b128(val, ro, static_cast<int>(t * row_v + 8 * c) * 2, 0, 0);
        }
    };

    // one step; the parity (LDS buffers, register set) is a compile-time constant, so that
    // the register array is indexed statically (a run-time index would put it in memory)
    auto body = [&](int s, auto parity, auto role) __attribute__((always_inline)) {
        constexpr int par = decltype(parity)::value;
        constexpr int ROLE = decltype(role)::value;
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int ln = lane_o;
        const int g = ln >> 4, m16 = ln & 15;
        const uint16_t* Kc = Kb[par];
        block_sync();  // B0: step s is staged

        if constexpr (ROLE == 0) {
            if constexpr (CKPT && par == 0) {
                // the state entering chunk s / 2, [i][j] rows of 16-byte pieces
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    float* dst = ckpt + ((static_cast<int64_t>(chunk0 + s / 2) * H + h) * DV + i0 + rb + 16 * ib + m16) * DK +
                                 4 * g;
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) *reinterpret_cast<f32x4*>(dst + 16 * jt) = R[ib * NJ + jt];
                }
            }
            // ======== -Y = K S^T - X, U = (-A)(-Y) for value rows i = rb + 16 ib + m16 (lane
            // column); rows t = 16 tt + 4g + r of tile tt
            f32x4 Y[NIB][2];
            const float* XT = Xb[par];
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    Y[ib][tt] = *reinterpret_cast<const f32x4*>(XT + (rb + 16 * ib + m16) * XP + 16 * tt + 4 * g);
            bf16x8 kf[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) kf[0][tt] = frag_st(Kc, KP, 16 * tt, 0, ln);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + 1 < NM) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) kf[(m + 1) & 1][tt] = frag_st(Kc, KP, 16 * tt, 32 * (m + 1), ln);
                }
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    const bf16x8 sb = __builtin_bit_cast(bf16x8, R[SP0 + (NJ / 2) * ib + m]);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) Y[ib][tt] = mfma16(kf[m & 1][tt], sb, Y[ib][tt]);
                    if constexpr (SPLIT) {
                        const bf16x8 sl = __builtin_bit_cast(bf16x8, R[SPL0 + (NJ / 2) * ib + m]);
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt) Y[ib][tt] = mfma16(kf[m & 1][tt], sl, Y[ib][tt]);
                    }
                }
            }
            const uint16_t* Ah = Ab[par];
            const uint16_t* Al = Ab[par] + H32 * AP;
            bf16x8 af[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                af[tt][0] = frag_st(Ah, AP, 16 * tt, 0, ln);
                af[tt][1] = frag_st(Al, AP, 16 * tt, 0, ln);
            }
            issue_fence();
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) {
                bf16x8 yh, yl;
                split_stack(Y[ib][0], Y[ib][1], yh, yl);
                f32x4 U[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    f32x4 acc = mfma16(af[tt][0], yh, f32x4{0.f, 0.f, 0.f, 0.f});
                    acc = mfma16(af[tt][1], yh, acc);
                    U[tt] = mfma16(af[tt][0], yl, acc);
                }
                // U^T packs (t = 4g .. +3 in words 0, 1; 16 + 4g .. +3 in words 2, 3) for the
                // state update, and the U^T [i][t] copy for the out waves
                bf16x8 uh, ul;
                split_stack(U[0], U[1], uh, ul);
                R[CU0 + ib] = __builtin_bit_cast(f32x4, uh);
                R[CU0 + 2 + ib] = __builtin_bit_cast(f32x4, ul);
                if constexpr (!NOOUT) {
                    const int i = rb + 16 * ib + m16;
                    const u32x4 wh = __builtin_bit_cast(u32x4, uh), wl = __builtin_bit_cast(u32x4, ul);
                    *reinterpret_cast<uint2*>(Ux + i * AP + 4 * g) = uint2{wh[0], wh[1]};
                    *reinterpret_cast<uint2*>(Ux + i * AP + 16 + 4 * g) = uint2{wh[2], wh[3]};
                    *reinterpret_cast<uint2*>(Ux + (BV + i) * AP + 4 * g) = uint2{wl[0], wl[1]};
                    *reinterpret_cast<uint2*>(Ux + (BV + i) * AP + 16 + 4 * g) = uint2{wl[2], wl[3]};
                }
            }
        } else if constexpr (ROLE == 1 && !NOOUT) {
            // ======== the previous step's O out; O^T = S Q^T for value rows rb + 16 ib + 4g + r
            // (tile rows) and tokens t = 16 tt + m16 (tile column)
            store_o(s - 1, ln);  // (none before the first step)
            // P = tril(Q K^T) as 16x16 tiles D[s][t] = K Q^T (a lane holds four consecutive s of
            // one t): (t-tile, s-tile) = (0, 0), (1, 0), (1, 1) from the same K and Q fragments
            const uint16_t* Qc = Qb[par];
            f32x4 Oacc[2][2], Pt[3];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) Oacc[ib][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < 3; ++x) Pt[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                bf16x8 sf[2], qf[2], kf[2];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) sf[ib] = frag16(Sx, SXP, rb + 16 * ib, 32 * m, ln);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    qf[tt] = frag16(Qc, QP, 16 * tt, 32 * m, ln);
                    kf[tt] = frag16(Kc, KP, 16 * tt, 32 * m, ln);
                }
                issue_fence();
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) Oacc[ib][tt] = mfma16(sf[ib], qf[tt], Oacc[ib][tt]);
                Pt[0] = mfma16(kf[0], qf[0], Pt[0]);
                Pt[1] = mfma16(kf[0], qf[1], Pt[1]);
                Pt[2] = mfma16(kf[1], qf[1], Pt[2]);
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) R[CU0 + 2 * ib + tt] = Oacc[ib][tt];
            // keep s <= t; then the stacked B operands of U^T P^T per t-tile (s-tile 0 for
            // reduction indices 4g .., s-tile 1 for 16 + 4g ..; the tile (0, 1) is zero)
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int tt = x == 0 ? 0 : 1, st = x == 2 ? 1 : 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) Pt[x][e] = 16 * st + 4 * g + e <= 16 * tt + m16 ? Pt[x][e] : 0.f;
            }
            bf16x8 ph, pl;
            split_stack(Pt[0], f32x4{0.f, 0.f, 0.f, 0.f}, ph, pl);
            R[CU0 + 4] = __builtin_bit_cast(f32x4, ph);
            R[CU0 + 5] = __builtin_bit_cast(f32x4, pl);
            split_stack(Pt[1], Pt[2], ph, pl);
            R[CU0 + 6] = __builtin_bit_cast(f32x4, ph);
            R[CU0 + 7] = __builtin_bit_cast(f32x4, pl);
        } else if constexpr (ROLE == 2) {
            // ======== the next step's K, Q, A (then those loads of the step after the next) and
            // the local prefix products of its gates (past the last step: an empty step, which
            // nothing reads; no branch keeps the compiler's counts of outstanding loads exact)
            stage(par ^ 1, par ^ 1, ln);
            fetch_kqa(s + 3, par ^ 1);
            local_scan(step_len(s + 1), par ^ 1, par ^ 1, ln);
        }
        block_sync();  // B1

        if constexpr (ROLE == 0) {
            // ======== S^T += K^T U, then the decay: the K^T operand (rows j, reduction t) from
            // row-major K through the transposing read, tile jt + 1 read while jt computes;
            // tile jt - 1 is scaled and packed while tile jt's products run
            float gm[NIB];
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) gm[ib] = gamb[par][rb + 16 * ib + m16];
            bf16x8 kt[2];
            kt[0] = frag_tr_st(Kc, KP, 0, 0, ln);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                if (jt + 1 < NJ) kt[(jt + 1) & 1] = frag_tr_st(Kc, KP, 16 * (jt + 1), 0, ln);
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    R[ib * NJ + jt] = mfma16(kt[jt & 1], __builtin_bit_cast(bf16x8, R[CU0 + ib]), R[ib * NJ + jt]);
                    R[ib * NJ + jt] = mfma16(kt[jt & 1], __builtin_bit_cast(bf16x8, R[CU0 + 2 + ib]), R[ib * NJ + jt]);
                }
                if (jt > 0) scale_pack(jt - 1, gm, ln);
            }
            scale_pack(NJ - 1, gm, ln);
        } else if constexpr (ROLE == 1 && !NOOUT) {
            // ======== O^T += U^T P^T (U^T rows with the stacked reduction order of the P
            // operands), then O = 2^{G} O staged as bf16 [t][i]
            bf16x8 uh[2], ul[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                uh[ib] = frag_st(Ux, AP, rb + 16 * ib, 0, ln);
                ul[ib] = frag_st(Ux + BV * AP, AP, rb + 16 * ib, 0, ln);
            }
            issue_fence();
            const float* Gc = Gb[par];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 ph = __builtin_bit_cast(bf16x8, R[CU0 + 4 + 2 * tt]);
                const bf16x8 pl = __builtin_bit_cast(bf16x8, R[CU0 + 5 + 2 * tt]);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    f32x4 acc = R[CU0 + 2 * ib + tt];
                    acc = mfma16(uh[ib], ph, acc);
                    acc = mfma16(ul[ib], ph, acc);
                    acc = mfma16(uh[ib], pl, acc);
                    const int t = 16 * tt + m16, i = rb + 16 * ib + 4 * g;
                    const f32x4 g4 = *reinterpret_cast<const f32x4*>(Gc + t * GP + i);
                    uint2 w;
                    w.x = pack_bf16(g4[0] * acc[0], g4[1] * acc[1]);
                    w.y = pack_bf16(g4[2] * acc[2], g4[3] * acc[3]);
                    *reinterpret_cast<uint2*>(Os + t * OP + i) = w;
                }
            }
        } else if constexpr (ROLE == 2) {
            // ======== the next step's G, X^T and gamma; then the V and alpha loads of the step
            // after the next
            finalize(par ^ 1, par ^ 1, ln);
            fetch_vl(s + 3, par ^ 1);
        }
    };
    // Each role runs its own copy of the loop (the same barriers in the same order), so
    // the compiler counts each role's outstanding loads and stores on its own path: in one
    // shared loop the role branches rejoin and it falls back to waiting for all of them,
    // which would undo the loaders' loads two steps ahead.
    auto run = [&](auto role) __attribute__((always_inline)) {
        constexpr int ROLE = decltype(role)::value;
        // prologue: step 0 staged, steps 1 and 2 in flight
        if constexpr (ROLE == 2) {
            fetch(0, 0);
            fetch(1, 1);
            stage(0, 0, lane);
            local_scan(step_len(0), 0, 0, lane);
        }
        if constexpr (ROLE == 0) pack_state(lane);
        block_sync();
        if constexpr (ROLE == 2) {
            finalize(0, 0, lane);
            fetch(2, 0);
        }
        // an even number of steps, so that the loop body has no branch: a last step past the
        // end is empty (K, X and U zero, gamma one) and leaves the state as it is
        for (int s = 0; s < n_steps; s += 2) {
            body(s, Parity<0>{}, role);
            body(s + 1, Parity<1>{}, role);
        }
    };
    // Each role ends in its own branch (one barrier each), so that values of one role are
    // not kept live through the others' loops; the chain waves are the critical path and
    // issue first on the SIMDs they share with loaders.
    auto unit_beyond = [&]() {
        return (beyond_s[0] | beyond_s[1] | beyond_s[2] | beyond_s[3]) != 0;
    };
    if (chain) {
        __builtin_amdgcn_s_setprio(3);
        run(Parity<0>{});
        __builtin_amdgcn_s_setprio(0);
        block_sync();
        if (S_T && !unit_beyond()) {
            float* st = S_T + (static_cast<int64_t>(u.seq) * H + h) * DV * DK;
            if (NOOUT && SPLIT && !CKPT && (flags & SCAN_STATE_DFRAG)) {  // (fragment orders: the paired passes only)
                // the chain registers are already in accumulator order: 1 KB per store
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt)
                        reinterpret_cast<f32x4*>(st)[dfrag_index((i0 + rb + 16 * ib) / 16, jt, lane, NJ)] =
                            R[ib * NJ + jt];
            } else if (NOOUT && SPLIT && !CKPT && (flags & SCAN_STATE_AFRAG)) {
                // Element (row rw + (lane & 15), column 16 jt + 4 (lane >> 4) + e) of S belongs
                // to fragment lane 16 ((lane & 15) >> 2) + 4 (lane >> 4) + e at stacked position
                // (lane & 3) + 4 ((rw / 16) & 1).  Each element is split into hi + lo bf16 (one
                // 32-bit word), and a 4 x 4 transpose of the words within each quad of lanes
                // gives lane q the four positions of fragment lane ... + q: 8 bytes of hi and 8
                // of lo per tile.
                uint16_t* sb = reinterpret_cast<uint16_t*>(st);
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    const int rw = i0 + rb + 16 * ib;
                    const int fl = 16 * ((lane & 15) >> 2) + 4 * (lane >> 4) + (lane & 3);
                    const int hb = 4 * ((rw >> 4) & 1);
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) {
                        u32x4 a;  // hi | lo << 16
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            uint32_t hi, lo;
                            split_bf16x2(R[ib * NJ + jt][e], 0.f, hi, lo);
                            a[e] = (hi & 0xffffu) | (lo << 16);
                        }
                        quad_transpose4(a, lane);
                        const u32x2 hi2 = {(a[0] & 0xffffu) | (a[1] << 16), (a[2] & 0xffffu) | (a[3] << 16)};
                        const u32x2 lo2 = {(a[0] >> 16) | (a[1] & 0xffff0000u), (a[2] >> 16) | (a[3] & 0xffff0000u)};
                        *reinterpret_cast<u32x2*>(sb + afrag_index(jt, rw >> 5, 0, fl, NJ) * 8 + hb) = hi2;
                        *reinterpret_cast<u32x2*>(sb + afrag_index(jt, rw >> 5, 1, fl, NJ) * 8 + hb) = lo2;
                    }
                }
            } else {
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    float* dst = S_T + s_base + static_cast<int64_t>(rb + 16 * ib + (lane & 15)) * DK + 4 * (lane >> 4);
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) *reinterpret_cast<f32x4*>(dst + 16 * jt) = R[ib * NJ + jt];
                }
            }
        }
    } else if (outw) {
        run(Parity<1>{});
        block_sync();
        if constexpr (!NOOUT) store_o(((n_steps + 1) & ~1) - 1, lane);  // (an empty last step stores nothing)
    } else {
        // (the loaders one level above the out waves: ~1% on the batched workload)
        __builtin_amdgcn_s_setprio(1);
        run(Parity<2>{});
        __builtin_amdgcn_s_setprio(0);
        if (lane == 0) beyond_s[lw] = beyond ? 1 : 0;
        block_sync();
        if (range_flags && lw == 0 && lane == 0 && (!CKPT || unit_beyond()))
            range_flags[(static_cast<int64_t>(u.seq) * H + h) * NVB + u.vblk] = unit_beyond() ? 1 : 0;
        // the unit's total decay per value row, when asked for (the sequence-parallel path
        // composes segments with it)
        if (gdecay && lw == 3) gdecay[(static_cast<int64_t>(u.seq) * H + h) * DV + i0 + lane] = gprod;
    }
}

template <int DK, int DV, int GATE, bool NOOUT = false, bool SPLIT = false, bool CKPT = false>
__global__ __launch_bounds__(512) void scan32_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ arec,
    int n_seq, int n_tok, int n_heads, uint16_t* __restrict__ o, float* __restrict__ S_T, int flags,
    float* __restrict__ gdecay, int32_t* __restrict__ range_flags, float* __restrict__ ckpt,
    const int32_t* __restrict__ skip_flags, int skip_segs) {
    scan32_body<DK, DV, GATE, NOOUT, SPLIT, CKPT>(blockIdx.x, q, k, v, alpha, S0, cu_seqlens, order, chunk_off, arec,
                                                  n_seq, n_tok, n_heads, o, S_T, flags, gdecay, range_flags, ckpt,
                                                  skip_flags, skip_segs);
}

// The arguments of one output-free pass.
struct Scan32PassArgs {
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const int32_t* cu_seqlens;
    const int32_t* order;
    const int32_t* chunk_off;
    const uint16_t* arec;
    int n_seq, n_tok, n_heads;
    float* S_T;
    int flags;
    float* gdecay;
    int32_t* range_flags;
};

// Two output-free passes with the state split (NOOUT, SPLIT), over units of the same
// count, in one launch: blocks below nb1 run the first, the rest the second.  Both run the
// same code on the same LDS variables (48 KB a workgroup), so a CU holds a workgroup of
// each at once and the two passes' latency-bound steps overlap, where one after the other
// they would each leave the CUs half used.
template <int DK, int DV, int GATE>
__global__ __launch_bounds__(512) void scan32_pair_kernel(Scan32PassArgs p1, Scan32PassArgs p2, int nb1) {
    const bool first = static_cast<int>(blockIdx.x) < nb1;
    const Scan32PassArgs& p = first ? p1 : p2;
    scan32_body<DK, DV, GATE, true, true, false>(first ? blockIdx.x : blockIdx.x - nb1, nullptr, p.k, p.v, p.alpha,
                                                 nullptr, p.cu_seqlens, p.order, p.chunk_off, p.arec, p.n_seq,
                                                 p.n_tok, p.n_heads, nullptr, p.S_T, p.flags, p.gdecay,
                                                 p.range_flags, nullptr, nullptr, 1);
}

}  // namespace

template <int DK, int DV, int GATE, bool NOOUT, bool SPLIT>
hipError_t launch_scan32_pass(const PrefillArgs& a, int n_units_seq, const int32_t* cu, const int32_t* order,
                              const int32_t* chunk_off, const uint16_t* arec, const float* S0, float* S_T, int flags,
                              float* gdecay, int32_t* range_flags, hipStream_t stream, const int32_t* skip_flags,
                              int skip_segs) {
    constexpr int NVB = DV / BV;
    const int64_t grid = prefill_grid(static_cast<int64_t>(n_units_seq) * a.n_heads, NVB);
    hipLaunchKernelGGL((scan32_kernel<DK, DV, GATE, NOOUT, SPLIT>), dim3(static_cast<unsigned>(grid)), dim3(512), 0,
                       stream, NOOUT ? nullptr : static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.alpha, S0, cu,
                       cu ? order : nullptr, chunk_off, arec, n_units_seq, a.n_tok, a.n_heads,
                       NOOUT ? nullptr : static_cast<uint16_t*>(a.o), S_T, flags, gdecay, range_flags, nullptr,
                       skip_flags, skip_segs);
    return hipGetLastError();
}

template <int DK, int DV, int GATE>
hipError_t launch_scan32_pair(const PrefillArgs& a, int n_units_seq, const int32_t* cu, const int32_t* order,
                              const int32_t* chunk_off, const uint16_t* arec, float* dS, float* gdecay,
                              int32_t* range_flags, float* Mf, hipStream_t stream) {
    static_assert(DK == DV, "the transitions are d_k x d_k");
    constexpr int NVB = DV / BV;
    const int64_t nb1 = prefill_grid(static_cast<int64_t>(n_units_seq) * a.n_heads, NVB);
    Scan32PassArgs p1;
    p1.k = static_cast<const uint16_t*>(a.k);
    p1.v = static_cast<const uint16_t*>(a.v);
    p1.alpha = a.alpha;
    p1.cu_seqlens = cu;
    p1.order = cu ? order : nullptr;
    p1.chunk_off = chunk_off;
    p1.arec = arec;
    p1.n_seq = n_units_seq;
    p1.n_tok = a.n_tok;
    p1.n_heads = a.n_heads;
    p1.S_T = dS;
    p1.flags = SCAN_STATE_DFRAG;
    p1.gdecay = gdecay;
    p1.range_flags = range_flags;
    Scan32PassArgs p2 = p1;
    p2.alpha = nullptr;  // no gate
    p2.S_T = Mf;
    p2.flags = SCAN_ZERO_V | SCAN_S0_IDENTITY | SCAN_STATE_AFRAG;
    p2.gdecay = nullptr;
    p2.range_flags = nullptr;
    hipLaunchKernelGGL((scan32_pair_kernel<DK, DV, GATE>), dim3(static_cast<unsigned>(2 * nb1)), dim3(512), 0, stream,
                       p1, p2, static_cast<int>(nb1));
    return hipGetLastError();
}

template <int DK, int DV, int GATE>
hipError_t launch_scan32_ckpt(const BackwardArgs& a, const int32_t* order, const int32_t* chunk_off,
                              const uint16_t* arec, int32_t* range_flags, float* ckpt, hipStream_t stream) {
    constexpr int NVB = DV / BV;
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, NVB);
    const int32_t* cu = a.cu_seqlens;
    hipLaunchKernelGGL((scan32_kernel<DK, DV, GATE, true, true, true>), dim3(static_cast<unsigned>(grid)), dim3(512),
                       0, stream, nullptr, static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       a.alpha, a.S0, cu, cu ? order : nullptr, chunk_off, arec, a.n_seq, a.n_tok, a.n_heads, nullptr,
                       nullptr, 0, nullptr, range_flags, ckpt, nullptr, 1);
    return hipGetLastError();
}

#define KDA_SCAN32_PASS(DK, DV, GATE, NOOUT, SPLIT)                                                                \
    template hipError_t launch_scan32_pass<DK, DV, GATE, NOOUT, SPLIT>(                                           \
        const PrefillArgs&, int, const int32_t*, const int32_t*, const int32_t*, const uint16_t*, const float*,  \
        float*, int, float*, int32_t*, hipStream_t, const int32_t*, int);
// the output pass and the segments' end-state pass for each gate; the transitions' pass
// (no gate, state split) where d_v = d_k
#define KDA_SCAN32_G(DK, DV, GATE)             \
    KDA_SCAN32_PASS(DK, DV, GATE, false, false) \
    KDA_SCAN32_PASS(DK, DV, GATE, true, false)
#define KDA_SCAN32(DK, DV)                  \
    KDA_SCAN32_G(DK, DV, GATE_CHANNEL)      \
    KDA_SCAN32_G(DK, DV, GATE_SCALAR)       \
    KDA_SCAN32_G(DK, DV, GATE_NONE)
KDA_SCAN32(128, 128)
KDA_SCAN32(64, 64)
KDA_SCAN32(128, 64)
KDA_SCAN32(64, 128)
#undef KDA_SCAN32
#undef KDA_SCAN32_G
#undef KDA_SCAN32_PASS
#define KDA_SCAN32_PAIR(DK, GATE)                                                                                   \
    template hipError_t launch_scan32_pair<DK, DK, GATE>(const PrefillArgs&, int, const int32_t*, const int32_t*,  \
                                                         const int32_t*, const uint16_t*, float*, float*, int32_t*, \
                                                         float*, hipStream_t);
KDA_SCAN32_PAIR(128, GATE_CHANNEL)
KDA_SCAN32_PAIR(128, GATE_SCALAR)
KDA_SCAN32_PAIR(128, GATE_NONE)
KDA_SCAN32_PAIR(64, GATE_CHANNEL)
KDA_SCAN32_PAIR(64, GATE_SCALAR)
KDA_SCAN32_PAIR(64, GATE_NONE)
#undef KDA_SCAN32_PAIR
#define KDA_SCAN32_CKPT(DK, DV, GATE)                                                                               \
    template hipError_t launch_scan32_ckpt<DK, DV, GATE>(const BackwardArgs&, const int32_t*, const int32_t*,      \
                                                         const uint16_t*, int32_t*, float*, hipStream_t);
#define KDA_SCAN32_CKPT_G(DK, DV)         \
    KDA_SCAN32_CKPT(DK, DV, GATE_CHANNEL) \
    KDA_SCAN32_CKPT(DK, DV, GATE_SCALAR)  \
    KDA_SCAN32_CKPT(DK, DV, GATE_NONE)
KDA_SCAN32_CKPT_G(128, 128)
KDA_SCAN32_CKPT_G(64, 64)
KDA_SCAN32_CKPT_G(128, 64)
KDA_SCAN32_CKPT_G(64, 128)
#undef KDA_SCAN32_CKPT_G
#undef KDA_SCAN32_CKPT

}  // namespace kda
