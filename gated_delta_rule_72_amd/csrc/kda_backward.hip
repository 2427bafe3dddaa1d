// kda_backward.hip -- gradients of the KDA recurrence (token-recurrent form).
//
// Page "Kimi (AI)", section "Kimi Delta Attention (KDA)" gives the per-token
// steps (forget S~ = diag(alpha_t) S, predict v~ = S~ k_t, update
// S_t = S~ + beta_t (v_t - v~) k_t^T, read-out o_t = S_t q_t); the
// transcript page ("Per dins de Kimi K3 ..."), where it turns to training,
// says the model is trained with the chunk-wise parallel algorithm, which
// needs these gradients.  With a_t = S_{t-1} k_t,
// u_t = beta_t (v_t - alpha_t a_t) and G_t = dL/dS_t, walking the tokens in
// reverse:
//     G_t     += dO_t q_t^T
//     dq_t     = S_t^T dO_t              du_t = G_t k_t
//     da_t     = -beta_t alpha_t du_t    dk_t = G_t^T u_t + S_{t-1}^T da_t
//     dv_t     = beta_t du_t             dbeta_t = du_t . (v_t - alpha_t a_t)
//     dalpha_t = rowsum(G_t (.) S_{t-1}) - beta_t a_t du_t
//     G_{t-1}  = diag(alpha_t) G_t + da_t k_t^T
// With the gate on key channels, S~ = S_{t-1} diag(alpha_t), a_t = S~ k_t,
// u_t = beta_t (v_t - a_t): da_t = -beta_t du_t, dk_t = G_t^T u_t + S~^T da_t,
// dalpha_t = column sums of (G_t + da_t k_t^T) (.) S_{t-1} and
// G_{t-1} = (G_t + da_t k_t^T) diag(alpha_t).
// Rows of the state are independent (every gate form updates each row on its
// own), so one wave owns
// 8 value rows of one (sequence, head), 8 lanes per row as in the forward
// kernel: dv and a value-channel dalpha are per row and stored directly; dq,
// dk, dbeta and a scalar dalpha are sums over rows, reduced over the wave's
// rows and added into zeroed outputs with float atomics (so their last bits
// depend on the order of the waves).
// States: a forward pass (the staged forward kernel, run first, with no o)
// stores the state every 16 tokens; the backward pass walks the blocks in
// reverse, recomputes the 16 states of a block from its checkpoint into the
// wave's own scratch, and walks those tokens in reverse.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_schedule.h"

namespace kda {

constexpr int BWD_BLOCK = STATE_CHECKPOINT_TOKENS;  // tokens between state checkpoints
constexpr int BWD_ROWS = 64;     // value rows per workgroup
constexpr int BWD_THREADS = 512; // eight waves of 8 rows

// Checkpoint slot of block b of a sequence that starts at token t0 and is the
// n-th: n + t0 / 16 + b.  Consecutive sequences never share a slot (a sequence
// of L tokens has ceil(L / 16) blocks) and every slot is below
// n_seq + n_tok / 16 + 1.
__host__ __device__ inline int64_t bwd_slots(int32_t n_seq, int32_t n_tok) {
    return static_cast<int64_t>(n_seq) + n_tok / BWD_BLOCK + 1;
}

// gfx950 lane-half swaps: permlane32 exchanges the upper 32 lanes of its first
// operand with the lower 32 lanes of its second; permlane16 exchanges the odd
// 16-lane rows of the first with the even rows of the second.  Summing the two
// results adds lanes 32 (or 16) apart without a trip through LDS.
__device__ __forceinline__ void swap32(float x, float y, float& a, float& b) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void swap16(float x, float y, float& a, float& b) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}

// DPP row_ror:8: within each 16-lane row, lane i reads lane i ^ 8.
constexpr int DPP_ROW_ROR8 = 0x128;

// Sum over the 8 lanes that hold the same key channels of the wave's 8 rows.
__device__ __forceinline__ float sum_rows8(float x) {
    float a, b;
    swap32(x, x, a, b);
    x = a + b;
    swap16(x, x, a, b);
    x = a + b;
    x += dpp_mov<DPP_ROW_ROR8>(x);
    return x;
}

// Reduce-scatter over the wave's 8 rows: x holds V = 4 M values (value c of chunk
// m = c / 4, element c % 4) summed over the lane's row; on return lane group g
// (lane / 8) holds in r[0 .. V/8) the sums over all 8 rows of values
// c = g V / 8 + i.  Three butterfly steps, each keeping half of the values and
// exchanging the other half with the partner group (lanes 32, 16, 8 apart): the
// first two are lane-half swaps of value pairs (i, i + V/2), then (i, i + V/4),
// after which the lower lanes hold the lower index of the pair; the last a DPP
// move within 16-lane rows.
template <int V>
__device__ __forceinline__ void reduce_scatter_rows8(const float (&x)[V], float (&r)[V / 8], int lane) {
    float a[V / 2], b[V / 4];
    const bool h0 = lane & 8;
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        float p, q;
        swap32(x[i], x[i + V / 2], p, q);
        a[i] = p + q;
    }
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
        float p, q;
        swap16(a[i], a[i + V / 4], p, q);
        b[i] = p + q;
    }
#pragma unroll
    for (int i = 0; i < V / 8; ++i) {
        const float send = h0 ? b[i] : b[i + V / 8];
        r[i] = (h0 ? b[i + V / 8] : b[i]) + dpp_mov<DPP_ROW_ROR8>(send);
    }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0.f;
}

template <typename T, int DK, int DV, int GATE>
__global__ __launch_bounds__(BWD_THREADS) void backward_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, const float* __restrict__ dO, const float* __restrict__ dS_T,
    int n_seq, int n_tok, int n_heads, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta,
    float* __restrict__ dS0, float* __restrict__ ckpt, float* __restrict__ sbuf,
    const int32_t* __restrict__ range_flags) {
    constexpr int M = DK / 32;
    constexpr int NW = BWD_THREADS / 64;   // waves per workgroup, 8 rows each
    constexpr bool KEY = GATE == GATE_KEY;
    // one wave's row sums of a token: dq, dk, (key-channel dalpha,) dbeta, scalar dalpha; padded
    constexpr int OFF_DB = KEY ? 3 * DK : 2 * DK;
    constexpr int RW = OFF_DB + 4;
    constexpr int NSUM = OFF_DB + (GATE == GATE_SCALAR ? 2 : 1);
    __shared__ float red[2][NW][RW];       // double-buffered by token
    const Unit u = map_unit(blockIdx.x, n_seq, n_heads, DV / BWD_ROWS, n_tok, cu_seqlens, order);
    if (!u.valid) return;
    // only the units marked by the chunked path, when it ran first
    if (range_flags && range_flags[(static_cast<int64_t>(u.seq) * n_heads + u.head) * (DV / BWD_ROWS) + u.vblk] == 0)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int j = lane & 7;
    const int row = u.vblk * BWD_ROWS + w * 8 + (lane >> 3);
    const int64_t H = n_heads;
    const int h = u.head;
    const int64_t len = u.t1 - u.t0;
    const int nblk = static_cast<int>((len + BWD_BLOCK - 1) / BWD_BLOCK);
    const int64_t slot0 = u.seq + u.t0 / BWD_BLOCK;
    auto ck = [&](int b) { return ckpt + (((slot0 + b) * H + h) * DV + row) * DK; };
    float* my = sbuf + (static_cast<int64_t>(blockIdx.x) * NW + w) * BWD_BLOCK * 8 * DK + (lane >> 3) * DK;
    auto col = [&](int m) { return 4 * (j + 8 * m); };
    // key channel of value c = (lane / 8) M / 2 + i after reduce_scatter_rows8
    auto vcol = [&](int i) {
        const int c = (lane >> 3) * (M / 2) + i;
        return 4 * (j + 8 * (c / 4)) + c % 4;
    };

    struct Tok { f32x4 k[M], q[M], ak[KEY ? M : 1]; float v, a, b, go; };
    // a token's operands; the forward passes (full = false) need no q and no dO
    auto load = [&](Tok& x, int64_t t, bool full) {
        const int64_t th = t * H + h;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            x.k[m] = Elem<T>::load4(k + th * DK + col(m));
            if (full) x.q[m] = Elem<T>::load4(q + th * DK + col(m));
            if constexpr (KEY) x.ak[m] = *reinterpret_cast<const f32x4*>(alpha + th * DK + col(m));
        }
        x.v = Elem<T>::load(v + th * DV + row);
        x.a = GATE == GATE_CHANNEL ? alpha[th * DV + row] : GATE == GATE_SCALAR ? alpha[th] : 1.f;
        x.b = beta[th];
        if (full) x.go = dO[th * DV + row];
    };
    // a = s . k for this lane's row (all 8 lanes of the row get it)
    auto dot_k = [&](const f32x4* s, const Tok& x) {
        float p = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) p += s[m][e] * x.k[m][e];
        return sum8(p);
    };
    auto advance = [&](f32x4* s, const Tok& x) {
        if constexpr (KEY) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[m][e] *= x.ak[m][e];
        }
        const float uu = x.b * (x.v - x.a * dot_k(s, x));
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[m][e] = x.a * s[m][e] + uu * x.k[m][e];
    };

    // the checkpoints come from the staged forward, run before this kernel
    f32x4 s[M];
    const int64_t s_row = ((static_cast<int64_t>(u.seq) * H + h) * DV + row) * DK;
    Tok x, xn;

    // backward
    f32x4 G[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        G[m] = dS_T ? *reinterpret_cast<const f32x4*>(dS_T + s_row + col(m)) : f32x4{0.f, 0.f, 0.f, 0.f};
    int par = 0;
    for (int b = nblk - 1; b >= 0; --b) {
        const int64_t tb = u.t0 + static_cast<int64_t>(b) * BWD_BLOCK;
        const int nb = static_cast<int>(u.t1 - tb < BWD_BLOCK ? u.t1 - tb : BWD_BLOCK);
        // the block's states S_{t-1}, t = tb .. tb + nb - 1, into this wave's scratch
        const float* c = ck(b);
#pragma unroll
        for (int m = 0; m < M; ++m) s[m] = *reinterpret_cast<const f32x4*>(c + col(m));
        load(x, tb, false);
        for (int i = 0; i < nb; ++i) {
            if (i + 1 < nb) load(xn, tb + i + 1, false);
#pragma unroll
            for (int m = 0; m < M; ++m) *reinterpret_cast<f32x4*>(my + i * 8 * DK + col(m)) = s[m];
            advance(s, x);
            x = xn;
        }
        f32x4 sp[M], spn[M];
        load(x, tb + nb - 1, true);
#pragma unroll
        for (int m = 0; m < M; ++m) sp[m] = *reinterpret_cast<const f32x4*>(my + (nb - 1) * 8 * DK + col(m));
        for (int i = nb - 1; i >= 0; --i) {
            const int64_t t = tb + i;
            const int64_t th = t * H + h;
            if (i > 0) {
                load(xn, t - 1, true);
#pragma unroll
                for (int m = 0; m < M; ++m) spn[m] = *reinterpret_cast<const f32x4*>(my + (i - 1) * 8 * DK + col(m));
            }
            // the gated state: S~ = S_{t-1} diag(alpha) for the gate on key channels; for the
            // others S_{t-1} itself, with the row gate applied through x.a below
            f32x4 st[M];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[m][e] = KEY ? sp[m][e] * x.ak[m][e] : sp[m][e];
            const float a = dot_k(st, x);
            const float uu = x.b * (x.v - x.a * a);
            float* rw = red[par][w];
            // dq_t = S_t^T dO_t, with S_t = alpha S_{t-1} + u k^T (S~ + u k^T); G_t += dO_t q_t^T
            float pq[4 * M], rq[M / 2];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pq[4 * m + e] = x.go * (x.a * st[m][e] + uu * x.k[m][e]);
                    G[m][e] += x.go * x.q[m][e];
                }
            reduce_scatter_rows8<4 * M>(pq, rq, lane);
#pragma unroll
            for (int i = 0; i < M / 2; ++i) rw[vcol(i)] = rq[i];
            float pdu = 0.f, pga = 0.f;
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pdu += G[m][e] * x.k[m][e];
                    pga += G[m][e] * sp[m][e];
                }
            const float du = sum8(pdu);
            const float da = -x.b * x.a * du;
            const float dal = sum8(pga) - x.b * a * du;
            // dk_t = G^T u + S_{t-1}^T da (S~^T da)
            float pk[4 * M], rk[M / 2];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[4 * m + e] = uu * G[m][e] + da * st[m][e];
            reduce_scatter_rows8<4 * M>(pk, rk, lane);
#pragma unroll
            for (int i = 0; i < M / 2; ++i) rw[DK + vcol(i)] = rk[i];
            // the row's own gradients (every lane of the row holds them; lane 0 of the eight writes)
            if (j == 0) {
                dv[th * DV + row] = x.b * du;
                if constexpr (GATE == GATE_CHANNEL) dalpha[th * DV + row] = dal;
            }
            const float dbs = sum_rows8(du * (x.v - x.a * a));
            const float das = GATE == GATE_SCALAR ? sum_rows8(dal) : 0.f;
            if (lane == 0) {
                rw[OFF_DB] = dbs;
                rw[OFF_DB + 1] = das;
            }
            if constexpr (KEY) {
                // dS~ = G_t + da k^T; dalpha_t = column sums of dS~ (.) S_{t-1}; G_{t-1} = dS~ diag(alpha)
                float pa[4 * M], ra[M / 2];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ds = G[m][e] + da * x.k[m][e];
                        pa[4 * m + e] = ds * sp[m][e];
                        G[m][e] = ds * x.ak[m][e];
                    }
                reduce_scatter_rows8<4 * M>(pa, ra, lane);
#pragma unroll
                for (int i = 0; i < M / 2; ++i) rw[2 * DK + vcol(i)] = ra[i];
            } else {
                // G_{t-1} = alpha G_t + da k^T
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) G[m][e] = x.a * G[m][e] + da * x.k[m][e];
            }
            // the workgroup's row sums of this token: one atomic add per value
            block_sync();
            if (tid < NSUM) {
                float acc = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) acc += red[par][ww][tid];
                float* dst = tid < DK                ? dq + th * DK + tid
                             : tid < 2 * DK          ? dk + th * DK + (tid - DK)
                             : tid < OFF_DB          ? dalpha + th * DK + (tid - 2 * DK)
                             : tid == OFF_DB         ? dbeta + th
                                                     : dalpha + th;
                atomicAdd(dst, acc);
            }
            par ^= 1;  // the next token's sums go to the other buffer; this one is read before the next barrier
            x = xn;
#pragma unroll
            for (int m = 0; m < M; ++m) sp[m] = spn[m];
        }
    }
    if (dS0) {
#pragma unroll
        for (int m = 0; m < M; ++m) *reinterpret_cast<f32x4*>(dS0 + s_row + col(m)) = G[m];
    }
}

namespace {

constexpr size_t kWsAlign = 256;
size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace: order, chunk offsets and unit marks, then one region used either by the
// chunked path (solved records, the states entering and the gradients leaving every
// chunk) or by the token-recurrent path (state checkpoints every 16 tokens, each
// wave's states within a block) -- the latter also after the chunked passes, for the
// units they marked, when the chunked region is no longer needed.
struct BwdLayout {
    size_t order, chunk_off, flags, un;  // un: start of the shared region
    size_t rec, sck, gck;                // chunked, relative to un
    size_t ckpt, sbuf;                   // token-recurrent, relative to un
    size_t total;
};

BwdLayout bwd_layout(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    BwdLayout L;
    L.order = 0;
    L.chunk_off = align_up(static_cast<size_t>(n_seq) * 4);
    L.flags = L.chunk_off + align_up((static_cast<size_t>(n_seq) + 1) * 4);
    L.un = L.flags + align_up(static_cast<size_t>(n_seq) * n_heads * (d_v / BWD_ROWS) * 4);
    const size_t mc = static_cast<size_t>(n_tok) / PREFILL_CHUNK_BF16 + n_seq;
    const size_t st_bytes = mc * n_heads * d_v * d_k * 4;
    L.rec = 0;
    L.sck = align_up(mc * n_heads * 12288);  // 12 KiB solved record per (chunk, head)
    L.gck = L.sck + align_up(st_bytes);
    const size_t chunked = L.gck + align_up(st_bytes);
    L.ckpt = 0;
    const size_t ck_bytes = static_cast<size_t>(bwd_slots(n_seq, n_tok)) * n_heads * d_v * d_k * 4;
    L.sbuf = align_up(ck_bytes);
    const int64_t waves = prefill_grid(static_cast<int64_t>(n_seq) * n_heads, d_v / 8);
    const size_t recurrent = align_up(L.sbuf + static_cast<size_t>(waves) * BWD_BLOCK * 8 * d_k * 4);
    L.total = L.un + (chunked > recurrent ? chunked : recurrent);
    return L;
}

hipError_t fill_zero(float* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

template <typename T, int DK, int DV, int GATE>
hipError_t launch_bwd_t(const BackwardArgs& a, const int32_t* order, float* ckpt, float* sbuf, const int32_t* rf,
                        hipStream_t stream) {
    const int64_t grid = prefill_grid(static_cast<int64_t>(a.n_seq) * a.n_heads, DV / BWD_ROWS);
    hipLaunchKernelGGL((backward_kernel<T, DK, DV, GATE>), dim3(static_cast<unsigned>(grid)), dim3(BWD_THREADS), 0,
                       stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.alpha,
                       a.beta, a.S0, a.cu_seqlens, order, a.dO, a.dS_T, a.n_seq, a.n_tok, a.n_heads, a.dq, a.dk,
                       a.dv, a.dalpha, a.dbeta, a.dS0, ckpt, sbuf, rf);
    return hipGetLastError();
}

template <typename T, int GATE>
hipError_t launch_bwd_g(const BackwardArgs& a, const int32_t* order, float* ckpt, float* sbuf, const int32_t* rf,
                        hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_bwd_t<T, 128, 128, GATE>(a, order, ckpt, sbuf, rf, stream);
    if (a.d_k == 64 && a.d_v == 64) return launch_bwd_t<T, 64, 64, GATE>(a, order, ckpt, sbuf, rf, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_bwd_t<T, 128, 64, GATE>(a, order, ckpt, sbuf, rf, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_bwd_t<T, 64, 128, GATE>(a, order, ckpt, sbuf, rf, stream);
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_bwd_type(const BackwardArgs& a, const int32_t* order, float* ckpt, float* sbuf, const int32_t* rf,
                           hipStream_t stream) {
    switch (a.gate) {
        case GATE_CHANNEL: return launch_bwd_g<T, GATE_CHANNEL>(a, order, ckpt, sbuf, rf, stream);
        case GATE_SCALAR: return launch_bwd_g<T, GATE_SCALAR>(a, order, ckpt, sbuf, rf, stream);
        case GATE_NONE: return launch_bwd_g<T, GATE_NONE>(a, order, ckpt, sbuf, rf, stream);
        case GATE_KEY: return launch_bwd_g<T, GATE_KEY>(a, order, ckpt, sbuf, rf, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_backward_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    return bwd_layout(n_seq, n_tok, n_heads, d_k, d_v).total;
}

// The token-recurrent backward: a forward pass storing the state every 16 tokens, then the
// reverse walk; with flags, only the marked units (whole (sequence, head) pairs).
hipError_t launch_backward_recurrent(const BackwardArgs& a, const int32_t* order, const int32_t* flags, char* un,
                                     hipStream_t stream) {
    const BwdLayout L = bwd_layout(a.n_seq, a.n_tok, a.n_heads, a.d_k, a.d_v);
    float* ckpt = reinterpret_cast<float*>(un + L.ckpt);
    float* sbuf = reinterpret_cast<float*>(un + L.sbuf);
    hipError_t e;
    if (a.n_tok > 0) {
        const PrefillArgs fa{a.q, a.k, a.v, a.alpha, a.beta, a.S0, a.cu_seqlens, a.n_seq, a.n_tok, a.n_heads,
                             a.d_k, a.d_v, a.bf16, nullptr, nullptr, nullptr, 0, a.gate};
        if ((e = launch_prefill_checkpoints(fa, order, ckpt, stream, flags)) != hipSuccess) return e;
    }
    return a.bf16 ? launch_bwd_type<uint16_t>(a, order, ckpt, sbuf, flags, stream)
                  : launch_bwd_type<float>(a, order, ckpt, sbuf, flags, stream);
}

hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t stream) {
    const BwdLayout L = bwd_layout(a.n_seq, a.n_tok, a.n_heads, a.d_k, a.d_v);
    char* ws = static_cast<char*>(a.workspace);
    const int64_t nt = static_cast<int64_t>(a.n_tok) * a.n_heads;
    hipError_t e;
    if (a.bf16 && a.gate != GATE_KEY && a.n_tok > 0) {
        // the chunked path; the units it marks are left to the token-recurrent pass
        BwdChunkBufs b;
        b.order = a.cu_seqlens ? reinterpret_cast<int32_t*>(ws + L.order) : nullptr;
        b.chunk_off = a.cu_seqlens ? reinterpret_cast<int32_t*>(ws + L.chunk_off) : nullptr;
        b.flags = reinterpret_cast<int32_t*>(ws + L.flags);
        b.rec = reinterpret_cast<uint16_t*>(ws + L.un + L.rec);
        b.sck = reinterpret_cast<float*>(ws + L.un + L.sck);
        b.gck = reinterpret_cast<float*>(ws + L.un + L.gck);
        b.max_chunks = static_cast<int64_t>(a.n_tok) / PREFILL_CHUNK_BF16 + a.n_seq;
        // the marks start clear: the forward pass's solve and scan only set them
        if ((e = fill_zero(reinterpret_cast<float*>(b.flags),
                           static_cast<int64_t>(a.n_seq) * a.n_heads * (a.d_v / BWD_ROWS), stream)) != hipSuccess)
            return e;
        if ((e = launch_backward_forward_pass(a, b, stream)) != hipSuccess) return e;
        if ((e = launch_backward_chunk_passes(a, b, stream)) != hipSuccess) return e;
        return launch_backward_recurrent(a, b.order, b.flags, ws + L.un, stream);
    }
    // the summed gradients are accumulated with atomics into zeroed outputs
    e = fill_zero(a.dq, nt * a.d_k, stream);
    if (e == hipSuccess) e = fill_zero(a.dk, nt * a.d_k, stream);
    if (e == hipSuccess) e = fill_zero(a.dbeta, nt, stream);
    if (e == hipSuccess && a.gate == GATE_SCALAR) e = fill_zero(a.dalpha, nt, stream);
    if (e == hipSuccess && a.gate == GATE_KEY) e = fill_zero(a.dalpha, nt * a.d_k, stream);
    if (e != hipSuccess) return e;
    const int32_t* order = nullptr;
    if (a.cu_seqlens) {
        int32_t* ord = reinterpret_cast<int32_t*>(ws + L.order);
        e = launch_schedule(a.cu_seqlens, a.n_seq, ord, stream);
        if (e != hipSuccess) return e;
        order = ord;
    }
    return launch_backward_recurrent(a, order, nullptr, ws + L.un, stream);
}

}  // namespace kda
