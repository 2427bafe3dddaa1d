// kda_segments.hip -- composition of segment states for sequence-parallel
// prefill of long sequences.
//
// Within a chunk the state update is affine in the entering state S (page
// "Kimi (AI)", section "Kimi Delta Attention (KDA)": the forget gate scales
// rows, and the predict / update steps act on S from the right):
//     S' = diag(gamma) S (I - K^T A^T K) + (terms that do not involve S),
// so over a segment of whole chunks
//     S_end = diag(Gamma) S_start M + dS,
// with Gamma the product of the segment's gates (per value row), M the product
// of the chunks' key-side factors (d_k x d_k, the same for every row), and dS
// the segment's end state from a zero start.  The prefill computes dS and M for
// every segment in parallel (two scans), this kernel walks the segments of
// each (sequence, head) in order to get every segment's true starting state,
// and a last scan reruns each segment from it.
#include "kda_mfma.h"
#include "kda_staged.h"

namespace kda {

// One workgroup per (sequence, head, block of 16 value rows r): d_k / 16 composing waves,
// one per 16 key columns c, and as many loader waves.  For segment g = 0 .. G-1 of
// sequence n:
//     S_start[n G + g] = S                      (S = S0[n], or zeros, for g = 0)
//     S = diag(gamma_g) S M_g + dS_g
// and S_T[n] = S after the last segment (G even).  gamma_g is the segment's total
// decay per value row (the product of its gates), written by the scan that produced dS.
// Each step runs transposed, (S M)^T = M^T S^T, on v_mfma_f32_16x16x32_bf16 with
// both fp32 operands split into hi + lo bf16 parts (hi hi + hi lo + lo hi, so a
// term is off by about 2^-16 of its size, against 2^-8 for plain bf16):
//   A = M^T [c][k]: the scan that produced M stored these operands, hi and lo parts
//       already split, in fragment order (Mf below).  The loader waves copy each
//       segment's 1 KB fragments into one of two LDS buffers two steps ahead (every
//       load 1 KB contiguous), and a composing wave reads its operands from there.
//       (A CU issues a transition's 64 loads per step slowly enough that a composing
//       wave issuing them itself stalls its MFMA chain behind them.)
//   B = S^T [k][r]: the accumulator tiles of the state.  Wave w holds rows
//       16w .. 16w + 15 of S^T, i.e. lane (g, i) holds S[r0 + i][16w + 4g + j] in
//       register j; two such tiles are exactly one stacked B operand, so each wave
//       splits its tile, leaves it in LDS, and reads every tile back.
// dS comes in accumulator order (dSf), one 16-byte load per lane; dS and gamma of the
// next two segments are in the composing waves' registers.  One barrier per step: before
// it, the step's state tiles and transition fragments are written (state exchange and
// fragment buffer both by step parity); after it, read.
// Layouts, per (segment n G + g, head h) block of d_v d_k floats: Mf in the A-operand
// fragment order of the transposed state, dSf in the accumulator fragment order (both
// as the 32-token scan writes them with SCAN_STATE_AFRAG / SCAN_STATE_DFRAG); S_start
// [n_seq G, H, d_v, d_k] row-major;
// gdecay [n_seq G, H, d_v]; S0, S_T [n_seq, H, d_v, d_k].
// range_flags [n_seq G, H, d_v / 64] (or null): segments whose scan met a chunk
// beyond the decay range of the factored form; their dS is not valid, so a
// workgroup whose rows belong to such a segment leaves S_T unwritten.  The
// workgroups past the composing ones are the token-recurrent recomputation of such
// units (the staged form, kda_staged.h, over the whole sequence from S0, writing o
// and S_T; a workgroup returns at once for an unmarked unit), run here rather than
// after the output pass, which skips the marked units.  Their S_start is never read,
// so the composing workgroups' read of S0 there does not matter when S_T aliases S0.
template <int DK>
struct CombineShape {
    static constexpr int NW = DK / 16;          // composing waves (and loader waves)
    static constexpr int NT = 2 * 64 * NW;      // threads
    static constexpr int KB = DK / 32;          // stacked reduction blocks
    static constexpr int NF = NW * KB * 2;      // 1 KB fragments of one transition
    static constexpr int FPL = NF / NW;         // fragments per loader wave
    static constexpr int FR = 64, FL = NT / FR; // the fixup's rows and lanes per row
    static constexpr int COMB_BYTES = (2 * NF + 2 * NW) * 1024;
};

template <int DK, int DV, int GATE>
__global__ __launch_bounds__(CombineShape<DK>::NT) void combine_segments_kernel(
    const float* __restrict__ gdecay, const float* __restrict__ S0, const float* __restrict__ dSf,
    const float* __restrict__ Mf, const int32_t* __restrict__ range_flags, int n_seq, int G, int n_heads,
    float* __restrict__ S_start, float* __restrict__ S_T, SegmentFixupArgs fx) {
    static_assert(DK == DV, "the transition M acts on the state's key side and has d_k rows");
    using SH = CombineShape<DK>;
    constexpr int NW = SH::NW, KB = SH::KB, NF = SH::NF, FPL = SH::FPL, FR = SH::FR, FL = SH::FL;
    constexpr int NRB = DV / 16;
    using FixBuf = StageBuf<DK, GATE, FR>;
    constexpr int SMEM = SH::COMB_BYTES > 2 * static_cast<int>(sizeof(FixBuf)) ? SH::COMB_BYTES
                                                                              : 2 * static_cast<int>(sizeof(FixBuf));
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    __shared__ __align__(16) unsigned char smem[SMEM];
    u32x4(*MB)[NF][64] = reinterpret_cast<u32x4(*)[NF][64]>(smem);                 // [parity][fragment][lane]
    u32x4(*X)[NW][64] = reinterpret_cast<u32x4(*)[NW][64]>(smem + 2 * NF * 1024);  // [parity][tile][lane]

    // Workgroups go round-robin to the 8 XCDs (block b to XCD b % 8), and each XCD has
    // its own L2: the NRB row blocks of a (sequence, head) read the same transitions,
    // so they are given blocks of one residue mod 8 and share that XCD's L2 copy.
    const int b = blockIdx.x;
    const int n_comp = (n_seq * n_heads + 7) / 8 * 8 * NRB;
    if (b >= n_comp) {
        // the fixup, 64 rows per workgroup with this kernel's threads as the lanes per row
        prefill_staged_body<uint16_t, DK, DV, GATE, FR, FL, false>(
            reinterpret_cast<FixBuf*>(smem), b - n_comp, fx.q, fx.k, fx.v, fx.alpha, fx.beta, S0, fx.cu_seqlens,
            nullptr, n_seq, fx.n_tok, n_heads, fx.o, S_T, nullptr, range_flags, G);
        return;
    }
    const int rblk = (b / 8) % NRB, unit = (b / (8 * NRB)) * 8 + b % 8;
    const int h = unit % n_heads, n = unit / n_heads;
    if (n >= n_seq) return;  // (the grid is rounded up to whole groups of 8 units)
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t H = n_heads;
    auto seg_of = [&](int g) { return static_cast<int64_t>(n) * G + g; };

    // Both roles run G barriers, one per step, at the same points: a role's loop body is
    // unrolled over the two parities and its first pass only loads (one load site per
    // register set, so the wait counts are the same on every pass).  The loads are
    // unconditional (the last ones reread segment G - 1), so the sets stay in their
    // registers instead of being copied, which would wait for them; the scheduling
    // barriers keep each reload after the code that reads the set.
    if (w >= NW) {
        // ---- loader wave: fragments lw FPL .. + FPL - 1 of every transition
        const int lw = w - NW;
        struct LSet {
            u32x4 m[FPL];
        };
        auto lload = [&](LSet& x, int g) {
            const u32x4* Mg = reinterpret_cast<const u32x4*>(Mf + (seg_of(g) * H + h) * DK * DK) + lw * FPL * 64;
#pragma unroll
            for (int p = 0; p < FPL; ++p) x.m[p] = Mg[p * 64 + lane];
        };
        auto lwrite = [&](const LSet& x, int par) {
#pragma unroll
            for (int p = 0; p < FPL; ++p) MB[par][lw * FPL + p][lane] = x.m[p];
        };
        // segment j's fragments go into buffer j & 1 before barrier j (which the composing
        // step j waits for); that buffer was last read in step j - 2, before barrier j - 1
        LSet la, lb;
        for (int j = -2; j < G; j += 2) {
            if (j >= 0) {
                lwrite(la, 0);
                __syncthreads();
            }
            __builtin_amdgcn_sched_barrier(0);
            lload(la, min(j + 2, G - 1));
            __builtin_amdgcn_sched_barrier(0);
            if (j >= 0) {
                lwrite(lb, 1);
                __syncthreads();
            }
            __builtin_amdgcn_sched_barrier(0);
            lload(lb, min(j + 3, G - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }

    // ---- composing wave w: key columns 16 w .. +15
    const int i = lane & 15, gq = lane >> 4;
    const int r = rblk * 16 + i;     // value row of this lane
    const int c4 = 16 * w + 4 * gq;  // first of its four key columns
    const int64_t row_off = static_cast<int64_t>(r) * DK + c4;
    struct Next {
        f32x4 d;    // dS[r][c4 .. c4 + 3]
        float gam;  // gamma[r]
    };
    auto load = [&](Next& x, int g) {
        const int64_t sg = seg_of(g);
        x.d = reinterpret_cast<const f32x4*>(dSf + (sg * H + h) * DV * DK)[dfrag_index(rblk, w, lane, NW)];
        x.gam = gdecay[(sg * H + h) * DV + r];
    };
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](const Next& x, int g) {
        if (g > 0) *reinterpret_cast<f32x4*>(S_start + (seg_of(g) * H + h) * DV * DK + row_off) = s;
        uint32_t h01, l01, h23, l23;
        split_bf16x2(s[0], s[1], h01, l01);
        split_bf16x2(s[2], s[3], h23, l23);
        X[g & 1][w][lane] = u32x4{h01, h23, l01, l23};
        __syncthreads();
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const u32x4 t0 = X[g & 1][2 * kb][lane], t1 = X[g & 1][2 * kb + 1][lane];
            const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{t0[0], t0[1], t1[0], t1[1]});
            const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{t0[2], t0[3], t1[2], t1[3]});
            const bf16x8 a_hi = __builtin_bit_cast(bf16x8, MB[g & 1][(kb * 2 + 0) * NW + w][lane]);
            const bf16x8 a_lo = __builtin_bit_cast(bf16x8, MB[g & 1][(kb * 2 + 1) * NW + w][lane]);
            acc = mfma16(a_lo, bh, acc);
            acc = mfma16(a_hi, bl, acc);
            acc = mfma16(a_hi, bh, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = x.gam * acc[j] + x.d[j];
    };
    Next xa, xb;
    bool beyond = false;  // a segment of these rows is marked beyond the decay range
    for (int g = -2; g < G; g += 2) {
        if (g >= 0) step(xa, g);
        __builtin_amdgcn_sched_barrier(0);
        load(xa, min(g + 2, G - 1));
        __builtin_amdgcn_sched_barrier(0);
        if (g >= 0) step(xb, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        load(xb, min(g + 3, G - 1));
        __builtin_amdgcn_sched_barrier(0);
        if (g < 0) {
            // the segments' range marks, one per lane (read together, not one after another),
            // and the entering state (the store waits for both here, not at a later pass)
            bool mark = false;
            if (range_flags) {
                const int vb = (rblk * 16) / 64;  // the scan's block of 64 rows that holds these rows
                for (int gg = lane; gg < G; gg += 64) mark |= range_flags[(seg_of(gg) * H + h) * (DV / 64) + vb] != 0;
            }
            if (S0) s = *reinterpret_cast<const f32x4*>(S0 + (static_cast<int64_t>(n) * H + h) * DV * DK + row_off);
            *reinterpret_cast<f32x4*>(S_start + (seg_of(0) * H + h) * DV * DK + row_off) = s;
            beyond = __ballot(mark) != 0;
        }
    }
    if (S_T && !beyond)
        *reinterpret_cast<f32x4*>(S_T + (static_cast<int64_t>(n) * H + h) * DV * DK + row_off) = s;
}

template <int DK, int DV, int GATE>
hipError_t launch_combine_segments(const float* gdecay, const float* S0, const float* dSf, const float* Mf,
                                   const int32_t* range_flags, int n_seq, int G, int n_heads, float* S_start,
                                   float* S_T, const SegmentFixupArgs& fx, hipStream_t stream) {
    if (G < 2 || G % 2) return hipErrorInvalidValue;
    using SH = CombineShape<DK>;
    const int64_t n_comp = (static_cast<int64_t>(n_seq) * n_heads + 7) / 8 * 8 * (DV / 16);
    const int64_t n_fix = range_flags ? prefill_grid(static_cast<int64_t>(n_seq) * n_heads, DV / SH::FR) : 0;
    hipLaunchKernelGGL((combine_segments_kernel<DK, DV, GATE>), dim3(static_cast<unsigned>(n_comp + n_fix)),
                       dim3(SH::NT), 0, stream, gdecay, S0, dSf, Mf, range_flags, n_seq, G, n_heads, S_start, S_T,
                       fx);
    return hipGetLastError();
}

#define KDA_COMBINE(DK, GATE)                                                                                      \
    template hipError_t launch_combine_segments<DK, DK, GATE>(const float*, const float*, const float*,           \
                                                              const float*, const int32_t*, int, int, int, float*, \
                                                              float*, const SegmentFixupArgs&, hipStream_t);
KDA_COMBINE(128, GATE_CHANNEL)
KDA_COMBINE(128, GATE_SCALAR)
KDA_COMBINE(128, GATE_NONE)
KDA_COMBINE(64, GATE_CHANNEL)
KDA_COMBINE(64, GATE_SCALAR)
KDA_COMBINE(64, GATE_NONE)
#undef KDA_COMBINE

}  // namespace kda
