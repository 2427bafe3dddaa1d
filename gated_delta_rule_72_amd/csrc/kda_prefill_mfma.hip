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
// (this file) solves it for every (chunk, head) at once and hands it to the scan
// through the workspace as hi/lo bf16.  The scan (kda_prefill_scan32.hip) walks
// each sequence in steps of 32 tokens with only the S-dependent products on its
// critical path: one workgroup of 8 waves per (sequence, head, block of 64 value
// rows) holds S^T in fp32 MFMA accumulators for the whole scan.  Calls with few
// (sequence, head) units cut every sequence into segments that the same scan runs
// in parallel, composed in between (kda_segments.hip; the launcher at the end of
// this file).
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
// solved systems of the chunk's two halves, packed (A_TRI_RECORD_BYTES a record); block
// 1 is neither formed nor written.
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
    const int64_t rec_off = (static_cast<int64_t>(gc) * n_heads + h) * ((HALVES ? A_TRI_RECORD_BYTES : A_RECORD_BYTES) / 2);
    write_solve_record<true, HALVES>(arec + rec_off, Xs, bs, tid);
    if constexpr (STORE_T) write_solve_record<false, HALVES>(trec + rec_off, Xs, bs, tid);
    block_sync();  // X, read above, shares its space with the next item's K
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
static size_t segment_decay_bytes(int32_t n_seq, int32_t n_heads, int32_t d_v, int G) {
    return align256(static_cast<size_t>(n_seq) * G * n_heads * static_cast<size_t>(d_v) * 4);
}

// Workspace layout of the bf16 path (each part 256-byte aligned; NS = n_seq G
// sequences when the call is split into G segments per sequence, else n_seq):
//   order      NS int32      longest-first schedule (packed input)
//   chunk_off  NS + 1 int32  first chunk of every sequence (packed input)
//   cu_seg     NS + 1 int32  segment token offsets (split calls only)
//   flags      NS x n_heads x (d_v / 64) int32: units beyond the decay range
//   A records  (n_tok / C + n_seq) x n_heads x A_RECORD_BYTES
//   dS, M, S_start, gdecay   segment states (split calls only)
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
    if (G > 1) L.total += 3 * segment_state_bytes(n_seq, n_heads, d_k, d_v, G) + segment_decay_bytes(n_seq, n_heads, d_v, G);
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
        // the 32-token scan needs only the records' diagonal blocks
        hipLaunchKernelGGL((chunk_solve_kernel<DK, false, true>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(a.k), a.beta, cu, chunk_off, nseq_eff, a.n_tok,
                           a.n_heads, static_cast<int>(mc), arec, nullptr, nullptr, 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // Units with a step beyond the decay range (marked in rflags by the scan, S_T left
    // unwritten) are recomputed token by token; the pass returns at once for the others.
    // Without a gate nothing decays, so nothing can be marked.
    int32_t* rf = GATE == GATE_NONE ? nullptr : rflags;
    if (G == 1) {
        if ((e = launch_scan32_pass<DK, DV, GATE, false, false>(a, a.n_seq, cu, order, chunk_off, arec, a.S0, a.S_T, 0,
                                                                nullptr, rf, stream)) != hipSuccess)
            return e;
        return rf ? launch_prefill_range_fixup(a, rf, 1, stream) : hipSuccess;
    }

    // Sequence-parallel path (d_k = d_v, few units, long sequences), on the 32-token scan:
    //   1. dS: each segment's end state from a zero start (in accumulator fragment
    //      order), and its total decay per value row (no outputs);
    //   2. M: each segment's key-side transition, from S0 = I with v = 0 and no gate,
    //      the state split hi + lo in K S^T (nothing decays, so its rounding would
    //      otherwise reach the composed states in full; no outputs), stored as the
    //      A operands of M^T (fragment order, hi and lo bf16);
    //   3. the segments' true starting states (and S_T), in order per (sequence, head),
    //      and the token-recurrent recomputation of units marked beyond the decay range;
    //   4. every segment again from its starting state, writing o (marked units skipped).
    // An empty segment has dS = 0, M = I and no decay.
    const size_t sb = segment_state_bytes(a.n_seq, a.n_heads, DK, DV, G);
    float* dS = reinterpret_cast<float*>(ws + L.seg);
    float* Mf = reinterpret_cast<float*>(ws + L.seg + sb);
    float* Sst = reinterpret_cast<float*>(ws + L.seg + 2 * sb);
    float* gdec = reinterpret_cast<float*>(ws + L.seg + 3 * sb);
    if ((e = launch_scan32_pair<DK, DV, GATE>(a, ns, cu, order, chunk_off, arec, dS, gdec, rf, Mf, stream)) !=
        hipSuccess)
        return e;
    // marked units are recomputed token by token inside the composition's launch, and the
    // output pass skips them
    SegmentFixupArgs fx;
    fx.q = static_cast<const uint16_t*>(a.q);
    fx.k = static_cast<const uint16_t*>(a.k);
    fx.v = static_cast<const uint16_t*>(a.v);
    fx.alpha = a.alpha;
    fx.beta = a.beta;
    fx.cu_seqlens = a.cu_seqlens;
    fx.n_tok = a.n_tok;
    fx.o = static_cast<uint16_t*>(a.o);
    if ((e = launch_combine_segments<DK, DV, GATE>(gdec, a.S0, dS, Mf, rf, a.n_seq, G, a.n_heads, Sst, a.S_T, fx,
                                                   stream)) != hipSuccess)
        return e;
    return launch_scan32_pass<DK, DV, GATE, false, false>(a, ns, cu, order, chunk_off, arec, Sst, nullptr, 0, nullptr,
                                                          nullptr, stream, rf, G);
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
