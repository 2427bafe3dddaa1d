// kda_staged.h -- the token-recurrent prefill in its staged form (tokens staged in LDS
// by blocks), as a device function: the body of prefill_staged_kernel
// (kda_prefill_valu.hip) and of the range fixup that the sequence-parallel prefill runs
// inside its segment composition (kda_segments.hip).  Private to the library.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_schedule.h"

namespace kda {

// ------------------------------------------------------------ staged form --
// Long calls: tokens staged in LDS by blocks.  The ring form (prefill_valu_kernel)
// has every wave fetch each token's q and k (and the key-channel gates) for itself,
// only three tokens ahead, and it waits on those loads.  Here a workgroup owns R
// value rows of one (sequence, head), one row per 8 lanes as there (16 for the
// smaller calls); its
// threads together load a block of 16 tokens' q, k, v, gates and beta
// (widened to fp32) into one of two LDS buffers while the block before is
// computed from the other, so a block's loads have a whole block of compute to
// arrive in and a single barrier per block orders the buffers.  Within a block
// each wave reads the next token's operands from LDS while it computes the
// current one.  R = 64 when that gives a workgroup per CU or more, else 32 or
// 16, so that small calls still spread over many CUs.  The read-out is
// o_i = s_i . q_t taken on the updated row, which needs no k . q term.
// Measured against the ring form (ms per call): the key-channel gate on the
// batched prefill workload (4 x 8192 tokens, H = 32, d = 128, bf16) 13.3 ->
// 4.0; fp32 4 x 2048 tokens, H = 32, d = 128: 1.41 -> 0.99.  Holding two rows
// per lane (half the LDS reads, twice the instructions per wave) was slower.
constexpr int STAGE_TOKENS = 16;  // tokens per staged block

template <typename T> struct Raw4;  // four elements as loaded, widened when staged
template <> struct Raw4<float> {
    using type = f32x4;
    static __device__ __forceinline__ type load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ f32x4 widen(type x) { return x; }
};
template <> struct Raw4<uint16_t> {
    using type = u16x4;
    static __device__ __forceinline__ type load(const uint16_t* p) { return *reinterpret_cast<const u16x4*>(p); }
    static __device__ __forceinline__ f32x4 widen(type x) {
        return f32x4{bf16_bits_to_f32(x[0]), bf16_bits_to_f32(x[1]), bf16_bits_to_f32(x[2]), bf16_bits_to_f32(x[3])};
    }
};

template <int DK, int GATE, int R>
struct StageBuf {
    f32x4 k[STAGE_TOKENS][DK / 4], q[STAGE_TOKENS][DK / 4];
    f32x4 ak[GATE == GATE_KEY ? STAGE_TOKENS : 1][DK / 4];  // key-channel gates
    float v[STAGE_TOKENS][R];
    float a[GATE == GATE_CHANNEL ? STAGE_TOKENS : 1][R];    // value-channel gates
    float g[STAGE_TOKENS];  // scalar gate
    float b[STAGE_TOKENS];
};

// One token's operands for one lane (L lanes per row), read from LDS.
template <int DK, int GATE, int L>
struct StageOps {
    f32x4 k[DK / (4 * L)], q[DK / (4 * L)];
    f32x4 ak[GATE == GATE_KEY ? DK / (4 * L) : 1];
    float v, g, b;
};

template <int DK, int GATE, int R, int L>
__device__ __forceinline__ void read_ops(StageOps<DK, GATE, L>& x, const StageBuf<DK, GATE, R>& B, int tl, int j,
                                         int r) {
#pragma unroll
    for (int m = 0; m < DK / (4 * L); ++m) {
        x.k[m] = B.k[tl][j + L * m];
        x.q[m] = B.q[tl][j + L * m];
        if constexpr (GATE == GATE_KEY) x.ak[m] = B.ak[tl][j + L * m];
    }
    x.v = B.v[tl][r];
    x.g = GATE == GATE_CHANNEL ? B.a[tl][r] : GATE == GATE_SCALAR ? B.g[tl] : 1.f;
    x.b = B.b[tl];
}

// Sum over each aligned group of L (8 or 16) lanes.
template <int L>
__device__ __forceinline__ float sum_lanes(float x) {
    return L == 16 ? sum16(x) : sum8(x);
}

// CKPT: the backward's forward pass -- no o, and the state entering every block
// stored into ckpt.
// range_flags (or null): only the units marked there are computed (the
// recomputation after the chunked bf16 scan, launch_prefill_range_fixup); a
// workgroup returns at once unless one of the flag_segs segments of its
// sequence is marked for its block of 64 value rows.
// buf: the two LDS staging buffers (the caller's, so that a kernel with other work can
// share its LDS with them).
template <typename T, int DK, int DV, int GATE, int R, int L, bool CKPT>
__device__ __forceinline__ void prefill_staged_body(
    StageBuf<DK, GATE, R>* buf, int64_t block, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int n_seq, int n_tok, int n_heads,
    T* __restrict__ o, float* __restrict__ S_T, float* __restrict__ ckpt,
    const int32_t* __restrict__ range_flags, int flag_segs) {
    constexpr int TB = STAGE_TOKENS;
    constexpr int NT = L * R;                // threads: L lanes per row
    constexpr int M = DK / (4 * L);          // float4 chunks of a row per lane
    constexpr int KN = TB * DK / 4;          // float4 groups of k (q, key gates) per block
    constexpr int KG = (KN + NT - 1) / NT;   // ... per thread
    constexpr int VN = TB * R / 4;           // float4 groups of v (value-channel gates) per block
    constexpr int VG = (VN + NT - 1) / NT;
    static_assert(2 * TB <= NT && DV % R == 0, "staging shape");

    const Unit u = map_unit(block, n_seq, n_heads, DV / R, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    const int tid = threadIdx.x;
    const int j = tid % L;     // which chunks of the row
    const int r = tid / L;     // local row of this lane
    const int row0 = u.vblk * R;
    const int64_t H = n_heads;
    const int h = u.head;
    if (range_flags) {
        static_assert(R <= 64 && 64 % R == 0 && NT % 64 == 0, "a workgroup's rows lie in one block of 64; whole waves");
        // one segment's flag per lane, so the flags are loaded together, not one after
        // another; every wave reaches the same answer
        bool marked = false;
        for (int g = tid % 64; g < flag_segs; g += 64)
            marked |= range_flags[((static_cast<int64_t>(u.seq) * flag_segs + g) * H + h) * (DV / 64) + row0 / 64] != 0;
        if (__ballot(marked) == 0) return;
    }

    const int64_t s_row = ((static_cast<int64_t>(u.seq) * H + h) * DV + row0 + r) * DK;
    f32x4 s[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        s[m] = S0 ? *reinterpret_cast<const f32x4*>(S0 + s_row + 4 * (j + L * m)) : f32x4{0.f, 0.f, 0.f, 0.f};

    // this thread's share of one block, held in registers between load and store
    using Rw = Raw4<T>;
    typename Rw::type rk[KG], rq[KG], rv[VG];
    f32x4 rak[GATE == GATE_KEY ? KG : 1], ra[GATE == GATE_CHANNEL ? VG : 1];
    float rs = 0.f;  // beta (threads 0 .. TB-1) or the scalar gate (threads TB .. 2 TB - 1)
    auto tok = [&](int64_t tb, int tl) { return tb + tl < u.t1 ? tb + tl : u.t1 - 1; };  // past the end: repeat
    auto fetch = [&](int64_t tb) {
#pragma unroll
        for (int p = 0; p < KG; ++p) {
            const int gi = tid + NT * p;
            if (KN % NT == 0 || gi < KN) {
                const int64_t t = tok(tb, gi / (DK / 4));
                const int c = 4 * (gi % (DK / 4));
                rk[p] = Rw::load(k + (t * H + h) * DK + c);
                if constexpr (!CKPT) rq[p] = Rw::load(q + (t * H + h) * DK + c);  // no read-out without o
                if constexpr (GATE == GATE_KEY) rak[p] = *reinterpret_cast<const f32x4*>(alpha + (t * H + h) * DK + c);
            }
        }
#pragma unroll
        for (int p = 0; p < VG; ++p) {
            const int gi = tid + NT * p;
            if (VN % NT == 0 || gi < VN) {
                const int64_t t = tok(tb, gi / (R / 4));
                const int c = row0 + 4 * (gi % (R / 4));
                rv[p] = Rw::load(v + (t * H + h) * DV + c);
                if constexpr (GATE == GATE_CHANNEL) ra[p] = *reinterpret_cast<const f32x4*>(alpha + (t * H + h) * DV + c);
            }
        }
        if (tid < 2 * TB) {
            const int64_t t = tok(tb, tid % TB);
            if (tid < TB) rs = beta[t * H + h];
            else if constexpr (GATE == GATE_SCALAR) rs = alpha[t * H + h];
        }
    };
    auto stage = [&](StageBuf<DK, GATE, R>& B) {
#pragma unroll
        for (int p = 0; p < KG; ++p) {
            const int gi = tid + NT * p;
            if (KN % NT == 0 || gi < KN) {
                const int tl = gi / (DK / 4), c = gi % (DK / 4);
                B.k[tl][c] = Rw::widen(rk[p]);
                if constexpr (!CKPT) B.q[tl][c] = Rw::widen(rq[p]);
                if constexpr (GATE == GATE_KEY) B.ak[tl][c] = rak[p];
            }
        }
#pragma unroll
        for (int p = 0; p < VG; ++p) {
            const int gi = tid + NT * p;
            if (VN % NT == 0 || gi < VN) {
                const int tl = gi / (R / 4), c = 4 * (gi % (R / 4));
                *reinterpret_cast<f32x4*>(&B.v[tl][c]) = Rw::widen(rv[p]);
                if constexpr (GATE == GATE_CHANNEL) *reinterpret_cast<f32x4*>(&B.a[tl][c]) = ra[p];
            }
        }
        if (tid < TB) B.b[tid] = rs;
        else if (GATE == GATE_SCALAR && tid < 2 * TB) B.g[tid - TB] = rs;
    };

    // one token for this lane's row
    auto step = [&](const StageOps<DK, GATE, L>& x, int64_t t) {
        if constexpr (GATE == GATE_KEY) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[m][e] *= x.ak[m][e];
        }
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            a0 += s[m][0] * x.k[m][0] + s[m][2] * x.k[m][2];
            a1 += s[m][1] * x.k[m][1] + s[m][3] * x.k[m][3];
        }
        const float uu = x.b * (x.v - x.g * sum_lanes<L>(a0 + a1));
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (GATE == GATE_CHANNEL || GATE == GATE_SCALAR)
                    s[m][e] = x.g * s[m][e] + uu * x.k[m][e];
                else
                    s[m][e] += uu * x.k[m][e];
            }
        if constexpr (!CKPT) {
            float c0 = 0.f, c1 = 0.f;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                c0 += s[m][0] * x.q[m][0] + s[m][2] * x.q[m][2];
                c1 += s[m][1] * x.q[m][1] + s[m][3] * x.q[m][3];
            }
            const float oo = sum_lanes<L>(c0 + c1);
            if (j == 0) Elem<T>::store(o + (t * H + h) * DV + row0 + r, oo);
        }
    };

    const int64_t len = u.t1 - u.t0;
    const int nblk = static_cast<int>((len + TB - 1) / TB);
    if (nblk > 0) {
        fetch(u.t0);
        stage(buf[0]);
    }
    block_sync();
    StageOps<DK, GATE, L> xa, xb;  // ping-pong: one token's operands in use, the next one's in flight
    for (int bi = 0; bi < nblk; ++bi) {
        const int64_t tb = u.t0 + static_cast<int64_t>(bi) * TB;
        if (bi + 1 < nblk) fetch(tb + TB);  // in flight while this block is computed
        if constexpr (CKPT) {
            // the state entering the block, for the backward (slot: sequence index + first
            // token / 16 + block, which never collide between sequences)
            float* c = ckpt + (((u.seq + u.t0 / TB + bi) * H + h) * DV + row0 + r) * DK;
#pragma unroll
            for (int m = 0; m < M; ++m) *reinterpret_cast<f32x4*>(c + 4 * (j + L * m)) = s[m];
        }
        const StageBuf<DK, GATE, R>& B = buf[bi & 1];
        const int nb = static_cast<int>(u.t1 - tb < TB ? u.t1 - tb : TB);
        read_ops(xa, B, 0, j, r);
        for (int tl = 0; tl < nb; tl += 2) {
            if (tl + 1 < nb) read_ops(xb, B, tl + 1, j, r);
            step(xa, tb + tl);
            if (tl + 1 < nb) {
                if (tl + 2 < nb) read_ops(xa, B, tl + 2, j, r);
                step(xb, tb + tl + 1);
            }
        }
        if (bi + 1 < nblk) stage(buf[(bi + 1) & 1]);
        block_sync();  // the next block is staged; this block's buffer may be refilled
    }
    if (S_T) {
#pragma unroll
        for (int m = 0; m < M; ++m) *reinterpret_cast<f32x4*>(S_T + s_row + 4 * (j + L * m)) = s[m];
    }
}

}  // namespace kda
