// kda_prefill_mfma.hip -- chunkwise KDA prefill for bf16 inputs on CDNA4
// matrix cores (bf16 MFMA with fp32 accumulation).
//
// Method: page "Kimi (AI)", section "Kimi Delta Attention (KDA)" -- the state S
// is d_v x d_k (rows = value channels) and the forget gate diag(alpha_t) scales
// its rows.  A per-row scalar decay commutes with everything on the key side,
// so within a chunk of C tokens (S entering the chunk):
//   G[t,i] = sum_{s<=t} log alpha[s,i]          (per-row cumulative log-decay; kept in log2 units)
//   L      = strictly_lower(diag(beta) K K^T)    (decay-free beta-weighted Gram)
//   A      = (I + L)^{-1} diag(beta)             (unit-lower WY/UT solve)
//   U      = A (V (.) e^{-G} - K S^T)            (decay-normalised errors)
//   O      = e^{G} (.) (Q S^T + tril(Q K^T) U)   (tril keeps the diagonal: o_t = S_t q_t)
//   S'     = diag(e^{G[C-1,:]}) (S + U^T K)
// The decayed Gram of value row i is D_i L D_i^{-1} with D_i = diag(e^{G[:,i]}),
// so one decay-free solve serves every row; the decay moves onto V, O and S as
// elementwise scalings.  Token rows past the end of a sequence read as k = q =
// v = 0, beta = 0 and log alpha = 0, which change nothing.
// The gate comes in three layouts (template parameter GATE): one value per
// value channel (KDA), one per (token, head) shared by every row (the
// scalar-gated delta rule, Gated DeltaNet, which KDA refines), or none (the
// delta rule, G = 0).  Only the loads of alpha and the log of G differ.
//
// Two kernels.  A depends on k and beta only, never on S, so chunk_solve_kernel
// solves it for every (chunk, head) at once and hands it to the scan through
// the workspace as hi/lo bf16.  scan_kernel then walks each sequence chunk by
// chunk with only the S-dependent products on its critical path: one
// workgroup of 8 waves per (sequence, head, block of 64 value rows) holds S^T
// in fp32 MFMA accumulators for the whole scan, with three workgroup barriers
// per chunk.  Calls with few (sequence, head) units cut every sequence into
// segments that the same scan runs in parallel, composed in between
// (kda_segments.hip; the launcher at the end of this file).
//
// Precision: q, k, v are exact bf16 inputs.  Computed operands are carried as
// hi + lo bf16 pairs (x = hi + lo to ~2^-16 relative) where the error budget
// needs it -- A, V e^{-G} - K S^T, U and P = tril(Q K^T) -- and S is a single
// bf16 copy of the fp32 state.  A product of two split operands takes three
// MFMAs (hi*hi + lo*hi + hi*lo).  The solve runs in fp32: VALU forward
// substitution on 16x16 diagonal blocks, fp32 MFMA for the off-diagonal blocks.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_schedule.h"
#include "kda_solve.h"

namespace kda {

// ============================================================================
// chunk_offsets_kernel: chunk_off[m] = sum_{m' < m} ceil(len_m' / C) for
// m = 0 .. n_seq; one workgroup.
// ============================================================================
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                             int n_tok, int32_t* __restrict__ chunk_off) {
    __shared__ int32_t part[1024];
    const int tid = static_cast<int>(threadIdx.x);
    int32_t carry = 0;
    for (int base = 0; base < n_seq; base += 1024) {
        const int m = base + tid;
        int32_t cnt = 0;
        if (m < n_seq) {
            const int64_t len = seq_start(m + 1, n_seq, n_tok, cu) - seq_start(m, n_seq, n_tok, cu);
            cnt = static_cast<int32_t>((len + C - 1) / C);
        }
        part[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan
            const int32_t add = tid >= d ? part[tid - d] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        if (m < n_seq) chunk_off[m] = carry + part[tid] - cnt;
        carry += part[1023];
        __syncthreads();
    }
    if (tid == 0) chunk_off[n_seq] = carry;
}

hipError_t launch_chunk_offsets(const int32_t* cu_seqlens, int n_seq, int n_tok, int32_t* chunk_off,
                                hipStream_t stream) {
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, n_seq, n_tok, chunk_off);
    return hipGetLastError();
}

// ============================================================================
// segment_cu_kernel: the token offsets of the segments of the sequence-parallel
// prefill.  Sequence n (tokens s0 .. s1-1, c = ceil((s1 - s0) / C) chunks) becomes
// G segments of ceil(c / G) whole chunks each (the last ones shorter or empty):
// cu_seg[n G + g] = min(s0 + g ceil(c / G) C, s1) and cu_seg[n_seq G] = n_tok.
// One thread per sequence.
// ============================================================================
__global__ __launch_bounds__(256) void segment_cu_kernel(const int32_t* __restrict__ cu, int n_seq, int n_tok,
                                                         int G, int32_t* __restrict__ cu_seg) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= n_seq) return;
    const int64_t s0 = seq_start(n, n_seq, n_tok, cu), s1 = seq_start(n + 1, n_seq, n_tok, cu);
    const int64_t per = ((s1 - s0 + C - 1) / C + G - 1) / G;  // chunks per segment
    for (int g = 0; g < G; ++g)
        cu_seg[static_cast<int64_t>(n) * G + g] = static_cast<int32_t>(min<int64_t>(s0 + g * per * C, s1));
    if (n == n_seq - 1) cu_seg[static_cast<int64_t>(n_seq) * G] = static_cast<int32_t>(s1);
}

// ============================================================================
// chunk_solve_kernel: A = (I + L)^{-1} diag(beta) of every (chunk, head), each
// written as the A record described above.  Workgroups of 4 waves loop over the
// (chunk, head) items, four per CU, loading the next item's K and beta while
// they solve the current one.  The inverse X = (I + L)^{-1} is built by blocks:
// 16x16 diagonal blocks by forward substitution, then X21 = -X22 L21 X11 at 16
// and at 32 rows.
// ============================================================================
// STORE_T (the chunked backward): a second record, in trec, holds T = (I + L)^{-1}
// itself, without the diag(beta) factor, and a chunk with a token whose |beta| is
// below 2^-20 marks every row block of its (sequence, head) in range_flags (n_vblk
// blocks per head): the backward divides by beta there and leaves such units to
// its token-recurrent pass.
// HALVES (the 32-token scan): only the two diagonal 32x32 blocks of each record, the
// solved systems of the chunk's two halves; block 1 is neither formed nor written.
template <int DK, bool STORE_T = false, bool HALVES = false>
__global__ __launch_bounds__(256, 4) void chunk_solve_kernel(
    const uint16_t* __restrict__ k, const float* __restrict__ beta, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ chunk_off, int n_seq, int n_tok, int n_heads, int max_chunks,
    uint16_t* __restrict__ arec, uint16_t* __restrict__ trec = nullptr, int32_t* __restrict__ range_flags = nullptr,
    int n_vblk = 0) {
    constexpr int KP = DK + PAD;
    constexpr int KX = (C * KP * 2 > C * LP * 4) ? C * KP * 2 : C * LP * 4;
    // K is dead once L is formed, so X reuses its space; the 32x32 temporary of
    // the last level reuses rows 0-16 of L, which only the 16-row level reads.
    // 35 KB in all, so four workgroups share a CU.
    __shared__ __align__(16) unsigned char kx_[KX];  // K [t][j], then X = (I + L)^{-1} [t][s]
    __shared__ __align__(16) float Lf[C * LP];       // L [t][s]
    __shared__ __align__(16) float bs[C];
    static_assert(32 * SOLVE_RP <= 17 * LP, "temporary fits in rows 0-16 of L");
    uint16_t* Kc = reinterpret_cast<uint16_t*>(kx_);
    float* Xs = reinterpret_cast<float*>(kx_);
    float* Rtmp = Lf;

    const int64_t H = n_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int total = min(first_chunk(n_seq, n_seq, n_tok, chunk_off), max_chunks) * n_heads;  // items

    // ---- loads of one item's K and beta into registers (rows past the sequence
    // end read as zero; an item past the last gets empty ranges)
    constexpr int PIECES = C * DK / 8 / 256;  // 16-byte pieces of K per thread
    u32x4 pk[PIECES];
    float pb;
    auto fetch = [&](int w) {
        const bool any = w < total;
        const int wc = any ? w : 0;
        const ChunkRef ch = chunk_ref(wc / n_heads, n_seq, n_tok, cu_seqlens, chunk_off);
        const int64_t tok0 = ch.t0 * H + wc % n_heads;
        const auto rk = make_rsrc(k + tok0 * DK, any ? ((ch.n - 1) * H * DK + DK) * 2 : 0);
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int idx = tid + 256 * p, t = idx / (DK / 8), c = idx % (DK / 8);
            pk[p] = __builtin_amdgcn_raw_buffer_load_b128(rk, static_cast<int>(t * H * DK + 8 * c) * 2, 0, 0);
        }
        const auto rb = make_rsrc(beta + tok0, any ? ((ch.n - 1) * H + 1) * 4 : 0);
        pb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(lane * H) * 4, 0, 0));
    };

    fetch(blockIdx.x);
    for (int w = blockIdx.x; w < total; w += gridDim.x) {
    // lane-derived values are rebuilt every item from an opaque copy of the lane
    // id, so the compiler does not hoist dozens of loop-invariant LDS addresses
    // into registers (which spills)
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int tid = lane_o + 64 * wave, g16 = lane_o >> 4, m16 = lane_o & 15;
    const int lane = lane_o;
    const int gc = w / n_heads, h = w % n_heads;
#pragma unroll
    for (int p = 0; p < PIECES; ++p) {
        const int idx = tid + 256 * p, t = idx / (DK / 8), c = idx % (DK / 8);
        *reinterpret_cast<u32x4*>(Kc + t * KP + 8 * c) = pk[p];
    }
    if (tid < C) bs[tid] = pb;
    if constexpr (STORE_T) {
        if (wave == 0) {
            const ChunkRef ch = chunk_ref(gc, n_seq, n_tok, cu_seqlens, chunk_off);
            const bool tiny = lane < ch.n && !(fabsf(pb) >= 0x1p-20f);
            if (__builtin_amdgcn_ballot_w64(tiny) != 0 && lane < n_vblk)
                range_flags[(static_cast<int64_t>(ch.seq) * n_heads + h) * n_vblk + lane] = 1;
        }
    }
    block_sync();
    fetch(w + gridDim.x);

    // ---- L = strictly_lower(diag(beta) K K^T).  Wave 0: the four 16x16 diagonal
    // blocks, then their inverses T_b = (I + L_bb)^{-1} (lane = (block, column)),
    // kept in registers until K's space is free.
    // Wave 1: rows 32-63 x cols 0-31.  Waves 2, 3: the blocks (16..31, 0..15) and
    // (48..63, 32..47).
    float x[16];
    if (wave == 0) {
        f32x4 d[4] = {};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            bf16x8 kf[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) kf[b] = frag16(Kc, KP, 16 * b, 32 * kk, lane);
            issue_fence();
#pragma unroll
            for (int b = 0; b < 4; ++b) d[b] = mfma16(kf[b], kf[b], d[b]);
        }
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
        solve_diag_blocks(Lf, lane, x);
    } else if (wave == 1) {
        if constexpr (!HALVES) {  // L (32..63, 0..31) only feeds the 32-row level
            f32x16 acc = {};
    #pragma unroll
            for (int half = 0; half < DK / 64; ++half) {
                bf16x8 fa[4], fb[4];
    #pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    fa[kk] = frag(Kc, KP, 32, 64 * half + 16 * kk, lane);
                    fb[kk] = frag(Kc, KP, 0, 64 * half + 16 * kk, lane);
                }
                issue_fence();
    #pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma(fa[kk], fb[kk], acc);
            }
            f32x4 b4[4];
    #pragma unroll
            for (int rb = 0; rb < 4; ++rb) b4[rb] = *reinterpret_cast<const f32x4*>(bs + 32 + 8 * rb + 4 * (lane >> 5));
    #pragma unroll
            for (int r = 0; r < 16; ++r) Lf[(32 + acc_row(r, lane)) * LP + (lane & 31)] = b4[r >> 2][r & 3] * acc[r];
        }
    } else {
        const int R = wave == 2 ? 16 : 48, Cc = R - 16;
        f32x4 d = {};
        bf16x8 fa[DK / 32], fb[DK / 32];
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            fa[kk] = frag16(Kc, KP, R, 32 * kk, lane);
            fb[kk] = frag16(Kc, KP, Cc, 32 * kk, lane);
        }
        issue_fence();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) d = mfma16(fa[kk], fb[kk], d);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(bs + R + 4 * g16);
#pragma unroll
        for (int r = 0; r < 4; ++r) Lf[(R + 4 * g16 + r) * LP + Cc + m16] = b4[r] * d[r];
    }
    assemble_inverse<HALVES>(Xs, Lf, Rtmp, x, wave, lane);

    // ---- A = X diag(beta) -> the record (STORE_T: X itself -> the second record)
    const int64_t rec_off = (static_cast<int64_t>(gc) * n_heads + h) * (A_RECORD_BYTES / 2);
    write_solve_record<true, HALVES>(arec + rec_off, Xs, bs, tid);
    if constexpr (STORE_T) write_solve_record<false, HALVES>(trec + rec_off, Xs, bs, tid);
    block_sync();  // X, read above, shares its space with the next item's K
    }
}

// ============================================================================
// scan_kernel: the S-dependent chunk products, one workgroup of 8 waves (two per
// SIMD) per (sequence, head, block of 64 value rows).
//
// Waves 0, 1, the chain waves, each own 32 value rows i of the state -- S^T[j][i]
// for every key channel j, as fp32 MFMA accumulators in 16x16 tiles -- and run
// the chunk's S-dependent chain for those rows in registers:
//   Y = X - K S^T            (X = V 2^{-G}, formed by the loader waves)
//   U = A Y
//   S^T <- diag(gamma) (S^T + K^T U)
// A 16x16 accumulator tile holds, in lane (column n = l % 16, group g = l / 16),
// rows 4g..4g+3.  Two tiles stacked along the row index give a lane the 8 rows
// {4g..4g+3, 16+4g..16+4g+3}; taken as the 8 reduction indices of a
// v_mfma_f32_16x16x32_bf16 B operand (the A operand reads the same indices,
// two 8-byte pieces per lane), Y, U and S feed the next product straight from
// the accumulators.
// Waves 2, 3, the out waves, form the outputs O^T = 2^{G} (S Q^T + U^T P^T) of
// the same 32-row blocks from the bf16 copies of S and U that the chain waves
// leave in LDS.  Waves 4-7, the loader waves, load each chunk one chunk ahead,
// stage it and form G and X; waves 6, 7 also form P = tril(Q K^T).
// Three barriers per chunk: staging | Y, U; P, S Q^T | S update; U^T P^T.
// ============================================================================
template <int DK>
struct ScanSmem {
    // Row pitches (bf16) are chosen per access pattern: with the pitch in dwords
    // = 4 (mod 8), the 16-row 8-byte operand reads and the 32-row 16-byte reads
    // are free of bank conflicts; with 0 (mod 8), the transposing reads and the
    // 16-row 16-byte reads are.  K is read both ways; Q and the S copy are read
    // by 16-row 16-byte loads.
    static constexpr int KP = DK + PAD;         // pitch of K rows
    static constexpr int QP = DK + 2 * PAD;     // pitch of Q and S rows
    static constexpr int GP = BV + 4;           // pitch of G rows (fp32)
    static constexpr int OP = BV + PAD;         // pitch of V and O rows (bf16)
    static constexpr int HILO = 2 * C * CP * 2;
    // each region is its own __shared__ array, so the compiler knows accesses to
    // different regions never alias and can move loads ahead of unrelated stores
    static constexpr int RK = C * KP * 2;       // K [t][j]
    static constexpr int RQ = C * QP * 2;       // Q [t][j]
    static constexpr int RS = BV * QP * 2;      // S bf16 [i][j], the state entering the chunk
    static constexpr int RA = HILO;             // A hi/lo [t][s]
    static constexpr int RP = HILO;             // P hi/lo [t][s]
    static constexpr int RU = 2 * BV * CP * 2;  // U^T hi/lo [i][t]
    static constexpr int XP = C + 4;            // pitch of X^T rows (fp32; 4 mod 64 dwords: the
                                                // loaders' row-per-lane writes are conflict-free)
    static constexpr int RX = BV * XP * 4;      // X^T [i][t] = V 2^{-G}, transposed
    static constexpr int RO = C * OP * 2;       // O [t][i], staged for the store
    static constexpr int RG = C * GP * 4;       // G [t][i] (log2 units)
    static constexpr int RB = BV * 4;           // gamma = 2^{G[C-1, :]}
    static constexpr int RT = 2 * 4 * BV * 4;   // loader-wave totals of log2 alpha, two chunks
    static constexpr int TOTAL = RK + RQ + RS + RA + RP + RU + RX + RO + RG + RB + RT;
};

// SPLIT_S: the state enters K S^T as hi + lo bf16 (two MFMAs per step) instead of
// one bf16 copy; used where no decay damps that rounding (the segment transitions
// of the sequence-parallel path, which start from S0 = I).
//
// Range: X = V 2^{-G} and U grow like 2^{-G} inside a chunk, so the factored form
// holds only while every row's log2-decay over a chunk stays above -RANGE_LOG2
// (G is monotone for alpha in [0, 1], so the chunk total is its minimum).  Wave 7
// checks each chunk's totals; a unit with any chunk beyond the range (alpha = 0
// gives -inf) is marked in range_flags[unit] and does not write S_T, so that S0
// is intact when S_T aliases it, and a token-recurrent pass recomputes exactly
// the marked units afterwards.  Below the limit 2^{-G} stays below 2^{100}:
// fp32 and bf16 (same exponent range) keep it, and the products with A, P and K
// add at most a few powers of two.
constexpr float RANGE_LOG2 = 100.f;

template <int DK, int DV, int GATE, bool SPLIT_S = false>
__global__ __launch_bounds__(512) void scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, const int32_t* __restrict__ chunk_off,
    const uint16_t* __restrict__ arec, int n_seq, int n_tok, int n_heads,
    uint16_t* __restrict__ o, float* __restrict__ S_T, int flags, float* __restrict__ glog_out,
    int32_t* __restrict__ range_flags) {
    using SM = ScanSmem<DK>;
    static_assert(SM::TOTAL <= 160 * 1024, "LDS budget");
    static_assert(DK == 64 || DK == 128, "d_k");
    constexpr int NVB = DV / BV;
    constexpr int KP = SM::KP, QP = SM::QP, GP = SM::GP, OP = SM::OP, XP = SM::XP;
    constexpr int NJ = DK / 16;   // 16-row tiles of S^T along j
    constexpr int NM = DK / 32;   // 32-wide reduction steps over j
    constexpr int PPR = DK / 8;   // 16-byte pieces per row of q or k

    __shared__ __align__(16) unsigned char rk_[SM::RK];
    __shared__ __align__(16) unsigned char rq_[SM::RQ];
    __shared__ __align__(16) unsigned char rs_[SM::RS];
    __shared__ __align__(16) unsigned char ra_[SM::RA];
    __shared__ __align__(16) unsigned char rp_[SM::RP];
    __shared__ __align__(16) unsigned char ru_[SM::RU];
    __shared__ __align__(16) unsigned char rx_[SM::RX];
    __shared__ __align__(16) unsigned char ro_[SM::RO];
    __shared__ __align__(16) unsigned char rg_[SM::RG];
    __shared__ __align__(16) unsigned char rb_[SM::RB];
    __shared__ __align__(16) unsigned char rt_[SM::RT];
    uint16_t* Kc = reinterpret_cast<uint16_t*>(rk_);
    uint16_t* Qc = reinterpret_cast<uint16_t*>(rq_);
    uint16_t* Sx = reinterpret_cast<uint16_t*>(rs_);
    uint16_t* A_hi = reinterpret_cast<uint16_t*>(ra_);
    uint16_t* A_lo = A_hi + C * CP;
    uint16_t* P_hi = reinterpret_cast<uint16_t*>(rp_);
    uint16_t* P_lo = P_hi + C * CP;
    uint16_t* Ux_hi = reinterpret_cast<uint16_t*>(ru_);
    uint16_t* Ux_lo = Ux_hi + BV * CP;
    float* XT = reinterpret_cast<float*>(rx_);
    uint16_t* Os = reinterpret_cast<uint16_t*>(ro_);
    float* Gs = reinterpret_cast<float*>(rg_);
    float* gam = reinterpret_cast<float*>(rb_);
    float* Tot = reinterpret_cast<float*>(rt_);  // [2][4][BV]

    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, NVB, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform: keep it (and every tile offset derived from it) scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wave < 2;                 // chain waves 0, 1
    const bool outw = wave == 2 || wave == 3;    // out waves 2, 3
    const int rb = 32 * (wave & 1);  // first of the 32 value rows of a chain or out wave
    const int64_t H = n_heads;
    const int h = u.head;
    const int i0 = u.vblk * BV;
    const int64_t row_qk = H * DK, row_v = H * DV;  // element strides between tokens
    const int chunk0 = first_chunk(u.seq, n_seq, n_tok, chunk_off);

    // ---- state of the chain waves: R[(ib) * NJ + (jt)] = S^T rows 16 jt .. 16 jt + 15 (key
    // channels), columns = value rows rb + 16 ib .. +15
    const int64_t s_base = ((static_cast<int64_t>(u.seq) * H + h) * DV + i0) * DK;
    // One register array holds each role's long-lived values, so the register
    // allocator (which cannot know that a wave keeps one role) does not keep every
    // role's set live at once: chain waves keep S^T at [NJ ib + jt] and the U^T
    // packs at CARRY0 + ..; out waves the O^T accumulators at CARRY0 + ..; loader
    // waves the loaded pieces of K, Q, V, the A record and alpha.
    constexpr int CARRY0 = 2 * NJ;
    constexpr int NKQ = C * PPR / 256;   // 16-byte pieces of K (and of Q) per loader thread
    constexpr int NA = A_RECORD_PIECES / 256;
    constexpr int PK0 = 0, PQ0 = NKQ, PV0 = 2 * NKQ, PA0 = PV0 + 4, PL0 = PA0 + NA;
    constexpr int RN = (CARRY0 + 8 > PL0 + 4) ? CARRY0 + 8 : PL0 + 4;
    f32x4 R[RN];
#pragma unroll
    for (int x = 0; x < RN; ++x) R[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (chain && (flags & SCAN_S0_IDENTITY)) {
        // S0 = I (d_v = d_k): row i holds 1 at key channel i
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int row = i0 + rb + 16 * ib + (lane & 15);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) R[(ib) * NJ + (jt)][e] = row == 16 * jt + 4 * (lane >> 4) + e ? 1.f : 0.f;
        }
    } else if (chain && S0) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const float* src =
                S0 + s_base + static_cast<int64_t>(rb + 16 * ib + (lane & 15)) * DK + 4 * (lane >> 4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) R[(ib) * NJ + (jt)] = *reinterpret_cast<const f32x4*>(src + 16 * jt);
        }
    }
    // negated bf16 copy of S as the B operand of K (-S)^T for the 32-wide j step m
    auto neg_state = [&](int ib, int m) {
        u32x4 w;
        w[0] = pack_bf16(-R[(ib) * NJ + (2 * m)][0], -R[(ib) * NJ + (2 * m)][1]);
        w[1] = pack_bf16(-R[(ib) * NJ + (2 * m)][2], -R[(ib) * NJ + (2 * m)][3]);
        w[2] = pack_bf16(-R[(ib) * NJ + (2 * m + 1)][0], -R[(ib) * NJ + (2 * m + 1)][1]);
        w[3] = pack_bf16(-R[(ib) * NJ + (2 * m + 1)][2], -R[(ib) * NJ + (2 * m + 1)][3]);
        return __builtin_bit_cast(bf16x8, w);
    };
    // the low half of the hi + lo split of -S (the high half is neg_state)
    auto neg_state_lo = [&](int ib, int m) {
        u32x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const f32x4& t = R[(ib) * NJ + (2 * m + (x >> 1))];
            uint32_t hi, lo;
            split_bf16x2(-t[2 * (x & 1)], -t[2 * (x & 1) + 1], hi, lo);
            w[x] = lo;
        }
        return __builtin_bit_cast(bf16x8, w);
    };
    auto pack_state = [&](int ln) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            // S [i][j] for the out waves: lane holds j = 16 jt + 4g .. +3 of row i
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

    // ---- loads of the next chunk's inputs by the loader waves (4-7), issued while
    // the chain and out waves compute; every load reads whole rows.  Loader
    // thread ht = tid - 256 holds 16-byte pieces ht + 256 p of K, Q (row-major)
    // and the A record; V and alpha: loader wave w holds token rows 16 (w - 4) ..
    // +15, lane = value row (one token row of the block per load).
    // The loads (and the O store below) are issued unconditionally: a chunk past
    // the end gets an empty buffer range, so nothing is accessed.  Uniform control
    // flow lets the compiler count outstanding memory operations exactly.
    const bool loader = wave >= 4;
    auto prefetch = [&](int64_t tc, int n, int gc) {
        const int ht = tid - 256;
        const int64_t tok0 = tc * H + h;  // (token tc, head h) row index
        const bool any = n > 0;
        const int64_t bytes = any ? ((n - 1) * row_qk + DK) * 2 : 0;
        const auto rk = make_rsrc(k + tok0 * DK, bytes);
        const auto rq = make_rsrc(q + tok0 * DK, bytes);
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int idx = ht + 256 * p;
            const int off = static_cast<int>((idx / PPR) * row_qk + 8 * (idx % PPR)) * 2;
            R[PK0 + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
            R[PQ0 + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        }
        const uint16_t* recp = arec + (static_cast<int64_t>(gc) * n_heads + h) * (A_RECORD_BYTES / 2);
        const auto rr = make_rsrc(recp, any ? A_RECORD_BYTES : 0);
#pragma unroll
        for (int p = 0; p < NA; ++p)
            R[PA0 + p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (ht + 256 * p) * 16, 0, 0));
        // v reads as zero when the flag asks for it (an empty range)
        const auto rv = make_rsrc(v + tok0 * DV + i0, any && !(flags & SCAN_ZERO_V) ? ((n - 1) * row_v + BV) * 2 : 0);
        // alpha: a value row per lane (per-channel gate), or the token's one gate,
        // the same address in every lane (scalar gate); nothing without a gate
        const auto ra = GATE == GATE_CHANNEL ? make_rsrc(alpha + tok0 * DV + i0, any ? ((n - 1) * row_v + BV) * 4 : 0)
                        : GATE == GATE_SCALAR ? make_rsrc(alpha + tok0, any ? ((n - 1) * H + 1) * 4 : 0)
                                              : make_rsrc(alpha, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = static_cast<int>((16 * (wave - 4) + r) * row_v + lane);
            R[PV0 + r / 4][r % 4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b16(rv, e * 2, 0, 0));
            if constexpr (GATE != GATE_NONE) {
                const int ea = GATE == GATE_CHANNEL ? e : static_cast<int>((16 * (wave - 4) + r) * H);
                R[PL0 + r / 4][r % 4] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, ea * 4, 0, 0));
            }
        }
    };

    auto chunk_len = [&](int64_t tc) { return static_cast<int>(max<int64_t>(0, min<int64_t>(C, u.t1 - tc))); };

    // staged O rows of a finished chunk -> global by the out waves (2, 3), four
    // 16-byte pieces per thread (n = 0: nothing is stored)
    auto store_o = [&](int64_t tc, int n, int ln) {
        const auto ro = make_rsrc(o + (tc * H + h) * DV + i0, n > 0 ? ((n - 1) * row_v + BV) * 2 : 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int idx = ln + 64 * (wave - 2) + 128 * p, t = idx >> 3, c = idx & 7;
            const u32x4 val = *reinterpret_cast<const u32x4*>(Os + t * OP + 8 * c);
            __builtin_amdgcn_raw_buffer_store_b128(val, ro, static_cast<int>(t * row_v + 8 * c) * 2, 0, 0);
        }
    };

    // one 16-byte piece of an A record -> A hi/lo [t][s]
    auto stage_a = [&](u32x4 val, int piece) {
        const int b = piece >> 8, half = (piece >> 7) & 1, row = (piece >> 2) & 31, c8 = 8 * (piece & 3);
        uint16_t* dst = (half ? A_lo : A_hi) + ((b == 0 ? 0 : 32) + row) * CP + (b == 2 ? 32 : 0) + c8;
        *reinterpret_cast<u32x4*>(dst) = val;
    };

    // G is kept in base-2 units (log2 alpha summed; e^{G} = 2^{G}), so every log
    // and exp below is one hardware instruction (v_log_f32 / v_exp_f32).  alpha
    // is in [0, 1]; alpha = 0 gives G = -inf, which the range check (wave 7, in
    // finalize) sends to the token-recurrent recomputation.
    // The log-decay cumsum G of a chunk is formed in two steps one phase apart,
    // so the prefix across waves never needs a barrier of its own:
    // local_scan -- each loader wave's inclusive prefix over its 16 token rows (in
    //   registers: a lane holds one value row), kept in the alpha registers, and
    //   V 2^{-prefix}, kept in the V registers; the wave's totals go to
    //   Tot[parity][wave - 4];
    // finalize   -- after a barrier, add the totals of the loader waves before
    //   (the rows before this wave's), write G [t][i] and X^T [i][t] = V 2^{-G}
    //   = (V 2^{-prefix}) 2^{-carry} (the chain waves' initial Y: one exponential
    //   per lane in this phase, which the chain waves wait for); wave 7 writes
    //   gamma.
    // Rows past the sequence end contribute log alpha = 0.
    bool beyond = false;  // loader waves: some chunk of some row of the unit is beyond the range
    auto local_scan = [&](int n, int par, int ln) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (GATE != GATE_NONE) {
                const float l = 16 * (wave - 4) + r < n ? __builtin_amdgcn_logf(R[PL0 + r / 4][r % 4]) : 0.f;
                run += l;
            }
            R[PL0 + r / 4][r % 4] = run;
            // V 2^{-prefix}: the part of X = V 2^{-G} this wave knows before the carry
            R[PV0 + r / 4][r % 4] = bf16_bits_to_f32(static_cast<uint16_t>(__float_as_uint(R[PV0 + r / 4][r % 4]))) *
                                    __builtin_amdgcn_exp2f(-run);
        }
        Tot[(par * 4 + wave - 4) * BV + ln] = run;
    };
    float glog = 0.f;  // wave 7: this row's total log2-decay over the unit's chunks
    auto finalize = [&](int par, int ln) {
        float carry = 0.f;
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            const float tb = Tot[(par * 4 + b) * BV + ln];
            carry += b < wave - 4 ? tb : 0.f;
        }
        float* xt = XT + ln * XP + 16 * (wave - 4);
        const float ec = __builtin_amdgcn_exp2f(-carry);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Gs[(16 * (wave - 4) + 4 * p + e) * GP + ln] = R[PL0 + p][e] + carry;
            *reinterpret_cast<f32x4*>(xt + 4 * p) = R[PV0 + p] * ec;
        }
        if (wave == 7) {
            const float tot = R[PL0 + 3][3] + carry;
            gam[ln] = __builtin_amdgcn_exp2f(tot);
            glog += tot;
            // (also true for a NaN total)
            beyond = beyond || __builtin_amdgcn_ballot_w64(!(tot >= -RANGE_LOG2)) != 0;
        }
    };
    // loaded pieces -> LDS
    auto stage = [&](int ln) {
        const int ht = ln + 64 * (wave - 4);
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int idx = ht + 256 * p;
            *reinterpret_cast<u32x4*>(Kc + (idx / PPR) * KP + 8 * (idx % PPR)) = __builtin_bit_cast(u32x4, R[PK0 + p]);
            *reinterpret_cast<u32x4*>(Qc + (idx / PPR) * QP + 8 * (idx % PPR)) = __builtin_bit_cast(u32x4, R[PQ0 + p]);
        }
#pragma unroll
        for (int p = 0; p < NA; ++p) stage_a(__builtin_bit_cast(u32x4, R[PA0 + p]), ht + 256 * p);
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
        // Lane-derived values are recomputed every chunk from an opaque copy of
        // the lane id, so the compiler does not hoist dozens of loop-invariant
        // LDS addresses into registers (which spills).
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int ln = lane_o;
        const int g = ln >> 4, m16 = ln & 15;
        block_sync();  // the previous chunk is done with every buffer

        // ======== the loaders stage this chunk and finish its G; the out waves
        // store the previous chunk's O
        if (loader) {
            stage(ln);
            finalize(c & 1, ln);
        } else if (outw) {
            store_o(prev_tc, prev_n, ln);
        }
        block_sync();

        // carried across the middle barrier in one register array: the U^T packs of
        // a chain wave (hi at 2 ib + m, lo at 4 + 2 ib + m) or the O^T accumulators of
        // an out wave (4 ib + tt)
        if (chain) {
            // ======== Y = X - K S^T, then U = A Y, for value rows i = rb + 16 ib + m16
            // (lane column); rows t = 16 tt + 4g + r of tile tt.  Every K and A
            // fragment serves both 16-row blocks ib.
            // Y starts as X (four consecutive t of one value row per read); K
            // fragments are loaded one step ahead of their use.
            f32x4 Y[2][4];
            bf16x8 kf[2][4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) kf[0][tt] = frag_st(Kc, KP, 16 * tt, 0, ln);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    Y[ib][tt] = *reinterpret_cast<const f32x4*>(XT + (rb + 16 * ib + m16) * XP + 16 * tt + 4 * g);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + 1 < NM) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) kf[(m + 1) & 1][tt] = frag_st(Kc, KP, 16 * tt, 32 * (m + 1), ln);
                }
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const bf16x8 sb = neg_state(ib, m);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) Y[ib][tt] = mfma16(kf[m & 1][tt], sb, Y[ib][tt]);
                    if constexpr (SPLIT_S) {
                        const bf16x8 sl = neg_state_lo(ib, m);
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) Y[ib][tt] = mfma16(kf[m & 1][tt], sl, Y[ib][tt]);
                    }
                }
            }
            bf16x8 af[2][4];
            af[0][0] = frag_st(A_hi, CP, 0, 0, ln);
            af[0][1] = frag_st(A_lo, CP, 0, 0, ln);
            issue_fence();
            bf16x8 Yh[2][2], Yl[2][2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                split_stack(Y[ib][0], Y[ib][1], Yh[ib][0], Yl[ib][0]);
                split_stack(Y[ib][2], Y[ib][3], Yh[ib][1], Yl[ib][1]);
            }
            // U = A Y.  A is lower triangular: t-tiles 0, 1 need s < 32 only.  The
            // fragments of t-tile tt + 1 are loaded while tile tt computes.
            f32x4 U[2][4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x8* cur = af[tt & 1];
                bf16x8* nxt = af[(tt + 1) & 1];
                if (tt + 1 < 4) {
                    nxt[0] = frag_st(A_hi, CP, 16 * (tt + 1), 0, ln);
                    nxt[1] = frag_st(A_lo, CP, 16 * (tt + 1), 0, ln);
                    if (tt + 1 >= 2) {
                        nxt[2] = frag_st(A_hi, CP, 16 * (tt + 1), 32, ln);
                        nxt[3] = frag_st(A_lo, CP, 16 * (tt + 1), 32, ln);
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
            // U^T hi/lo [i][t] for the out waves: the stacked packs hold t = 32 m +
            // 4g .. +3 (words 0, 1) and 32 m + 16 + 4g .. +3 (words 2, 3)
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
            // ======== O^T = S Q^T for value rows rb + 16 ib + 4g + r (tile rows) and
            // tokens t = 16 tt + m16 (tile column); every Q fragment serves both blocks
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
                for (int tt = 0; tt < 4; ++tt) qf[tt] = frag16(Qc, QP, 16 * tt, 32 * m, ln);
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
            if (wave >= 6) {
            // ======== P = tril(Q K^T) hi/lo [t][s], formed transposed (32x32 tile
            // D[s][t], so each lane holds 4 consecutive s of one t).  P^T tiles
            // (s-tile, t-tile): wave 6 takes (0,0) and (1,1), wave 7 (0,1); (1,0) is
            // all zero.
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                if (wave == 7 && pt == 1) break;
                const int sb = (wave == 6 && pt == 1) ? 1 : 0, tb = wave == 7 ? 1 : sb;
                f32x16 acc = {};
#pragma unroll
                for (int half = 0; half < DK / 64; ++half) {
                    bf16x8 fa[4], fb[4];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        fa[kk] = frag(Kc, KP, 32 * sb, 64 * half + 16 * kk, ln);
                        fb[kk] = frag(Qc, QP, 32 * tb, 64 * half + 16 * kk, ln);
                    }
                    issue_fence();
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) acc = mfma(fa[kk], fb[kk], acc);
                }
                const int t = 32 * tb + (ln & 31);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int s0 = 32 * sb + 8 * q4 + 4 * (ln >> 5);
                    float pv4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) pv4[e] = s0 + e <= t ? acc[4 * q4 + e] : 0.f;
                    uint2 wh, wl;
                    split_bf16x2(pv4[0], pv4[1], wh.x, wl.x);
                    split_bf16x2(pv4[2], pv4[3], wh.y, wl.y);
                    *reinterpret_cast<uint2*>(P_hi + t * CP + s0) = wh;
                    *reinterpret_cast<uint2*>(P_lo + t * CP + s0) = wl;
                }
            }
            }
            // ======== the loaders (4, 5 at once, 6, 7 after P) issue the next
            // chunk's loads, off the chain waves' path
            prefetch(tc + C, chunk_len(tc + C), gc + 1);
        }
        block_sync();

        if (chain) {
            // ======== S^T += K^T U, then the decay: the K^T operand (rows j,
            // reduction t) comes from row-major K through the transposing read
            // (fragments of tile jt + 1 are read while tile jt computes)
            bf16x8 kt[2][2];
#pragma unroll
            for (int m = 0; m < 2; ++m) kt[0][m] = frag_tr_st(Kc, KP, 0, 32 * m, ln);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                if (jt + 1 < NJ) {
#pragma unroll
                    for (int m = 0; m < 2; ++m) kt[(jt + 1) & 1][m] = frag_tr_st(Kc, KP, 16 * (jt + 1), 32 * m, ln);
                }
                issue_fence();
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const bf16x8 uh = __builtin_bit_cast(bf16x8, R[CARRY0 + 2 * ib + m]);
                        const bf16x8 ul = __builtin_bit_cast(bf16x8, R[CARRY0 + 4 + 2 * ib + m]);
                        R[(ib) * NJ + (jt)] = mfma16(kt[jt & 1][m], uh, R[(ib) * NJ + (jt)]);
                        R[(ib) * NJ + (jt)] = mfma16(kt[jt & 1][m], ul, R[(ib) * NJ + (jt)]);
                    }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const float gm = gam[rb + 16 * ib + m16];
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) R[(ib) * NJ + (jt)] *= gm;
            }
            pack_state(ln);
        } else if (outw) {
            // ======== O^T += U^T P^T (P is lower triangular: t-tiles 0, 1 need s < 32),
            // then O = 2^{G} O, staged as bf16 [t][i]
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
                const bf16x8 ph0 = frag16(P_hi, CP, 16 * tt, 0, ln), pl0 = frag16(P_lo, CP, 16 * tt, 0, ln);
                bf16x8 ph1 = {}, pl1 = {};
                if (tt >= 2) {
                    ph1 = frag16(P_hi, CP, 16 * tt, 32, ln);
                    pl1 = frag16(P_lo, CP, 16 * tt, 32, ln);
                }
                issue_fence();
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    Oacc[ib][tt] = mfma16(uh[ib][0], ph0, Oacc[ib][tt]);
                    Oacc[ib][tt] = mfma16(ul[ib][0], ph0, Oacc[ib][tt]);
                    Oacc[ib][tt] = mfma16(uh[ib][0], pl0, Oacc[ib][tt]);
                    if (tt >= 2) {
                        Oacc[ib][tt] = mfma16(uh[ib][1], ph1, Oacc[ib][tt]);
                        Oacc[ib][tt] = mfma16(ul[ib][1], ph1, Oacc[ib][tt]);
                        Oacc[ib][tt] = mfma16(uh[ib][1], pl1, Oacc[ib][tt]);
                    }
                }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int t = 16 * tt + m16, i = rb + 16 * ib + 4 * g;
                    const f32x4 g4 = *reinterpret_cast<const f32x4*>(Gs + t * GP + i);
                    uint2 w;
                    w.x = pack_bf16(__builtin_amdgcn_exp2f(g4[0]) * Oacc[ib][tt][0],
                                    __builtin_amdgcn_exp2f(g4[1]) * Oacc[ib][tt][1]);
                    w.y = pack_bf16(__builtin_amdgcn_exp2f(g4[2]) * Oacc[ib][tt][2],
                                    __builtin_amdgcn_exp2f(g4[3]) * Oacc[ib][tt][3]);
                    *reinterpret_cast<uint2*>(Os + t * OP + i) = w;
                }
        }
        if (loader) local_scan(chunk_len(tc + C), (c + 1) & 1, ln);
        prev_tc = tc;
        prev_n = n;
    }
    __shared__ int beyond_s[4];
    if (loader && lane == 0) beyond_s[wave - 4] = beyond ? 1 : 0;
    block_sync();
    const bool unit_beyond = (beyond_s[0] | beyond_s[1] | beyond_s[2] | beyond_s[3]) != 0;
    if (outw) store_o(prev_tc, prev_n, lane);  // (n = 0: nothing is stored)
    if (range_flags && tid == 0)
        range_flags[(static_cast<int64_t>(u.seq) * H + h) * NVB + u.vblk] = unit_beyond ? 1 : 0;

    // the unit's total log2-decay per value row, when asked for (the sequence-parallel
    // path composes segments with it)
    if (glog_out && wave == 7) glog_out[(static_cast<int64_t>(u.seq) * H + h) * DV + i0 + lane] = glog;

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
// A records: (n_tok / C + n_seq) bounds the number of chunks of any split of
// n_tok tokens into n_seq sequences.
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int64_t chunk_bound(int32_t n_seq, int32_t n_tok) { return static_cast<int64_t>(n_tok) / C + n_seq; }

// Segment states of the sequence-parallel path: dS and S_start
// [n_seq G, H, d_v, d_k] and M [n_seq G, H, d_k, d_k], fp32 (d_k = d_v), then the
// segments' log2-decays [n_seq G, H, d_v].
static size_t segment_state_bytes(int32_t n_seq, int32_t n_heads, int32_t d_k, int32_t d_v, int G) {
    return static_cast<size_t>(n_seq) * G * n_heads * static_cast<size_t>(d_v) * d_k * 4;
}
static size_t segment_log_bytes(int32_t n_seq, int32_t n_heads, int32_t d_v, int G) {
    return align256(static_cast<size_t>(n_seq) * G * n_heads * static_cast<size_t>(d_v) * 4);
}

// Workspace layout of the bf16 path (each part 256-byte aligned; NS = n_seq G
// sequences when the call is split into G segments per sequence, else n_seq):
//   order      NS int32      longest-first schedule (packed input)
//   chunk_off  NS + 1 int32  first chunk of every sequence (packed input)
//   cu_seg     NS + 1 int32  segment token offsets (split calls only)
//   flags      NS x n_heads x (d_v / 64) int32: units beyond the decay range
//   A records  (n_tok / C + n_seq) x n_heads x A_RECORD_BYTES
//   dS, M, S_start, glog     segment states (split calls only)
struct Bf16Layout {
    size_t order, chunk_off, cu_seg, flags, rec, seg, total;
};

static Bf16Layout bf16_layout(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    const int G = prefill_segments(n_seq, n_tok, n_heads, d_k, d_v);
    const size_t ns = static_cast<size_t>(n_seq) * G;
    Bf16Layout L;
    L.order = 0;
    L.chunk_off = L.order + align256(ns * 4);
    L.cu_seg = L.chunk_off + align256((ns + 1) * 4);
    L.flags = L.cu_seg + (G > 1 ? align256((ns + 1) * 4) : 0);
    L.rec = L.flags + align256(ns * n_heads * static_cast<size_t>(d_v / BV) * 4);
    L.seg = L.rec + align256(static_cast<size_t>(chunk_bound(n_seq, n_tok)) * n_heads * A_RECORD_BYTES);
    L.total = L.seg;
    if (G > 1) L.total += 3 * segment_state_bytes(n_seq, n_heads, d_k, d_v, G) + segment_log_bytes(n_seq, n_heads, d_v, G);
    return L;
}

size_t prefill_bf16_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    return bf16_layout(n_seq, n_tok, n_heads, d_k, d_v).total;
}

template <int DK, int DV, int GATE>
static hipError_t launch_bf16_t(const PrefillArgs& a, hipStream_t stream) {
    constexpr int NVB = DV / BV;
    const Bf16Layout L = bf16_layout(a.n_seq, a.n_tok, a.n_heads, DK, DV);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* order = reinterpret_cast<int32_t*>(ws + L.order);
    int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
    int32_t* rflags = reinterpret_cast<int32_t*>(ws + L.flags);
    uint16_t* arec = reinterpret_cast<uint16_t*>(ws + L.rec);
    const int64_t mc = chunk_bound(a.n_seq, a.n_tok);
    hipError_t e;

    // How the sequences are cut (G = 1: one scan per sequence).  A split call whose
    // sequences all have the same length, a multiple of G chunks, keeps the dense
    // form: n_seq G sequences of len / G tokens, offsets computed in the kernels.
    // Any other split call describes its segments by token offsets built on the
    // device (cu_seg), so packed input and ragged lengths are split the same way.
    // Segments end on chunk boundaries, so in both forms the chunks -- and the A
    // records solved below -- are those of the whole sequences, in the same order.
    const int G = prefill_segments(a.n_seq, a.n_tok, a.n_heads, DK, DV);
    const int ns = a.n_seq * G;
    const bool dense = !a.cu_seqlens && (G == 1 || (a.n_tok / a.n_seq) % (C * G) == 0);
    const int32_t* cu = a.cu_seqlens;
    if (G > 1 && !dense) {
        int32_t* cu_seg = reinterpret_cast<int32_t*>(ws + L.cu_seg);
        hipLaunchKernelGGL(segment_cu_kernel, dim3((a.n_seq + 255) / 256), dim3(256), 0, stream, a.cu_seqlens,
                           a.n_seq, a.n_tok, G, cu_seg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        cu = cu_seg;
    }
    const int nseq_eff = cu && G > 1 ? ns : a.n_seq;  // sequences as the kernels see them
    if (cu) {
        if ((e = launch_schedule(cu, nseq_eff, order, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, stream, cu, nseq_eff, a.n_tok, chunk_off);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        chunk_off = nullptr;  // equal lengths: the kernels compute the offsets
    }
    if (a.n_tok > 0) {
        // as many workgroups as stay resident (four per CU); each loops over items
        int dev = 0, n_cu = 0;
        if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        const int64_t grid = std::min<int64_t>(mc * a.n_heads, 4 * static_cast<int64_t>(n_cu));
        // one scan per sequence (the 32-token scan) needs only the records' diagonal blocks
        if (G == 1)
            hipLaunchKernelGGL((chunk_solve_kernel<DK, false, true>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                               stream, static_cast<const uint16_t*>(a.k), a.beta, cu, chunk_off, nseq_eff, a.n_tok,
                               a.n_heads, static_cast<int>(mc), arec, nullptr, nullptr, 0);
        else
            hipLaunchKernelGGL((chunk_solve_kernel<DK>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                               static_cast<const uint16_t*>(a.k), a.beta, cu, chunk_off, nseq_eff, a.n_tok, a.n_heads,
                               static_cast<int>(mc), arec, nullptr, nullptr, 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    auto scan = [&](auto kern, int nvb, const void* vv, const float* al, const float* s0, int nsq, float* st,
                    int flags, float* glog, int32_t* rf) {
        const int64_t grid = prefill_grid(static_cast<int64_t>(nsq) * a.n_heads, nvb);
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(vv), al, s0, cu, cu ? order : nullptr, chunk_off, arec, nsq,
                           a.n_tok, a.n_heads, static_cast<uint16_t*>(a.o), st, flags, glog, rf);
        return hipGetLastError();
    };
    // Units with a chunk beyond the decay range (marked in rflags by the scan, S_T left
    // unwritten) are recomputed token by token; the pass returns at once for the others.
    // Without a gate nothing decays, so nothing can be marked.
    if (G == 1) {
        if ((e = launch_scan32<DK, DV, GATE>(a, cu, order, chunk_off, arec, GATE == GATE_NONE ? nullptr : rflags,
                                             stream)) != hipSuccess)
            return e;
        return GATE == GATE_NONE ? hipSuccess : launch_prefill_range_fixup(a, rflags, 1, stream);
    }

    // Sequence-parallel path (d_k = d_v, few units, long sequences):
    //   1. dS: each segment's end state from a zero start, and its total log2-decay
    //      per value row;
    //   2. M: each segment's key-side transition, from S0 = I with v = 0 and no gate,
    //      the state split hi + lo in K S^T (nothing decays, so its rounding would
    //      otherwise reach the composed states in full);
    //   3. the segments' true starting states (and S_T), in order per (sequence, head);
    //   4. every segment again from its starting state, writing o.
    // Passes 1 and 2 write o as well; pass 4 overwrites it.  An empty segment has
    // dS = 0, M = I and no decay.
    const size_t sb = segment_state_bytes(a.n_seq, a.n_heads, DK, DV, G);
    float* dS = reinterpret_cast<float*>(ws + L.seg);
    float* Mt = reinterpret_cast<float*>(ws + L.seg + sb);
    float* Sst = reinterpret_cast<float*>(ws + L.seg + 2 * sb);
    float* glog = reinterpret_cast<float*>(ws + L.seg + 3 * sb);
    int32_t* rf = GATE == GATE_NONE ? nullptr : rflags;
    if ((e = scan(scan_kernel<DK, DV, GATE>, NVB, a.v, a.alpha, nullptr, ns, dS, 0, glog, rf)) != hipSuccess)
        return e;
    if ((e = scan(scan_kernel<DK, DK, GATE_NONE, true>, DK / BV, a.v, nullptr, nullptr, ns, Mt,
                  SCAN_ZERO_V | SCAN_S0_IDENTITY, nullptr, nullptr)) != hipSuccess)
        return e;
    if ((e = launch_combine_segments<DK, DV>(glog, a.S0, dS, Mt, rf, a.n_seq, G, a.n_heads, Sst, a.S_T,
                                             stream)) != hipSuccess)
        return e;
    if ((e = scan(scan_kernel<DK, DV, GATE>, NVB, a.v, a.alpha, Sst, ns, nullptr, 0, nullptr, nullptr)) !=
        hipSuccess)
        return e;
    return rf ? launch_prefill_range_fixup(a, rf, G, stream) : hipSuccess;
}

// The chunked backward's forward pass (see kda_backward_chunk.hip).
template <int DK, int DV, int GATE>
static hipError_t bwd_forward_t(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream) {
    constexpr int NVB = DV / BV;
    hipError_t e;
    const int32_t* cu = a.cu_seqlens;
    if (cu) {
        if ((e = launch_schedule(cu, a.n_seq, b.order, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, stream, cu, a.n_seq, a.n_tok, b.chunk_off);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    int dev = 0, n_cu = 0;
    if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t sgrid = std::min<int64_t>(b.max_chunks * a.n_heads, 4 * static_cast<int64_t>(n_cu));
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    // one solve writes both records: A (for the checkpoint scan) into the space of the state
    // gradients, which only the reverse scan writes, after this pass; T into rec
    uint16_t* arec = reinterpret_cast<uint16_t*>(b.gck);
    hipLaunchKernelGGL((chunk_solve_kernel<DK, true>), dim3(static_cast<unsigned>(sgrid)), dim3(256), 0, stream, k,
                       a.beta, cu, b.chunk_off, a.n_seq, a.n_tok, a.n_heads, static_cast<int>(b.max_chunks), arec,
                       b.rec, b.flags, NVB);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the checkpoint scan in 32-token steps (the diagonal blocks of the A records)
    return launch_scan32_ckpt<DK, DV, GATE>(a, b.order, b.chunk_off, arec, b.flags, b.sck, stream);
}

template <int GATE>
static hipError_t bwd_forward_g(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return bwd_forward_t<128, 128, GATE>(a, b, stream);
    if (a.d_k == 64 && a.d_v == 64) return bwd_forward_t<64, 64, GATE>(a, b, stream);
    if (a.d_k == 128 && a.d_v == 64) return bwd_forward_t<128, 64, GATE>(a, b, stream);
    if (a.d_k == 64 && a.d_v == 128) return bwd_forward_t<64, 128, GATE>(a, b, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_backward_forward_pass(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream) {
    switch (a.gate) {
        case GATE_CHANNEL: return bwd_forward_g<GATE_CHANNEL>(a, b, stream);
        case GATE_SCALAR: return bwd_forward_g<GATE_SCALAR>(a, b, stream);
        case GATE_NONE: return bwd_forward_g<GATE_NONE>(a, b, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int GATE>
static hipError_t launch_bf16_g(const PrefillArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_bf16_t<128, 128, GATE>(a, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_bf16_t<64, 64, GATE>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_bf16_t<128, 64, GATE>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_bf16_t<64, 128, GATE>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    // a few tokens per sequence (multi-token decode): token by token, each state read
    // and written once; with cu_seqlens the lengths are unknown on the host, so packed
    // calls keep the chunked path
    if (!a.cu_seqlens && a.n_tok > 0 && a.n_tok <= static_cast<int64_t>(RECURRENT_MAX_TOKENS) * a.n_seq)
        return launch_prefill_recurrent(a, stream);
    // the key-channel gate has its own chunk algebra (its decay falls inside K K^T):
    // kda_prefill_keygate.hip
    switch (a.gate) {
        case GATE_CHANNEL: return launch_bf16_g<GATE_CHANNEL>(a, stream);
        case GATE_SCALAR: return launch_bf16_g<GATE_SCALAR>(a, stream);
        case GATE_NONE: return launch_bf16_g<GATE_NONE>(a, stream);
        case GATE_KEY: return launch_prefill_keygate(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
