// kda_mfma.h -- constants and device helpers shared by the chunkwise bf16
// kernels (the forward prefill in kda_prefill_mfma.hip, the chunked backward in
// kda_backward_chunk.hip): chunk geometry, the solved-record layout, MFMA
// fragment loaders for CDNA4 (wave64) matrix instructions, buffer resources
// and chunk addressing.  Private to the library.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = PREFILL_CHUNK_BF16;  // 64 tokens per chunk
// scan flags: v read as zero; S0 taken as the identity (d_v = d_k); S_T stored in the
// order of 16x16x32 MFMA fragments, as the A operand of S^T (hi and lo bf16 parts) or as
// a 16x16 accumulator (fp32) -- the layouts the segment composition reads
constexpr int SCAN_ZERO_V = 1;
constexpr int SCAN_S0_IDENTITY = 2;
constexpr int SCAN_STATE_AFRAG = 4;
constexpr int SCAN_STATE_DFRAG = 8;

// Fragment layouts of a d_v x d_k state S of one (sequence, head), 16-row blocks rb and
// 16-column tiles w (NW = d_k / 16 of them), lane l = 16 g + i of a wave, 16 bytes per
// lane, so that a wave reads 1 KB contiguous at a time:
//  - accumulator (DFRAG), fp32: the f32x4 at index (rb NW + w) 64 + l holds
//    S[16 rb + i][16 w + 4 g + e];
//  - A operand of S^T (AFRAG, d_v = d_k), bf16: the 8 values at index ((kb 2 + part) NW
//    + w) 64 + l (part 0 = hi, 1 = lo) hold that part of S[32 kb + 4 g + (e & 3) + 16 (e
//    >> 2)][16 w + i], e = 0 .. 7: lane l's reduction values in the stacked order of a
//    16x16x32 MFMA, ready to use.
__device__ __forceinline__ int64_t dfrag_index(int rb, int w, int lane, int nw) {
    return (static_cast<int64_t>(rb) * nw + w) * 64 + lane;
}
__device__ __forceinline__ int64_t afrag_index(int w, int kb, int part, int lane, int nw) {
    return ((static_cast<int64_t>(kb) * 2 + part) * nw + w) * 64 + lane;
}
constexpr int BV = 64;                 // value rows per scan workgroup
constexpr int PAD = 8;                 // bf16 row padding (16 bytes) against bank conflicts
constexpr int CP = C + PAD;            // pitch of bf16 rows of length C
constexpr int LP = C + 4;              // pitch of fp32 rows of length C
// A of one (chunk, head): the three nonzero 32x32 blocks (rows 0-31 x cols 0-31,
// rows 32-63 x cols 0-31, rows 32-63 x cols 32-63), each as hi then lo bf16,
// row-major; entries above the diagonal are zero.
constexpr int A_BLOCK_ELEMS = 32 * 32;
constexpr int A_RECORD_BYTES = 3 * 2 * A_BLOCK_ELEMS * 2;
constexpr int A_RECORD_PIECES = A_RECORD_BYTES / 16;  // 16-byte pieces
// The records of the 32-token scan hold blocks 0 and 2 only, each packed: of a block's
// 32 rows x 4 pieces of 8 columns, the 80 pieces that reach the diagonal (8 c <= row), in
// bands of 8 rows (band r / 8 has r / 8 + 1 pieces a row), the hi pieces then the lo
// pieces.  The all-zero pieces above the diagonal are neither written nor read.
constexpr int A_TRI_PIECES = 80;
constexpr int A_TRI_BLOCK_ELEMS = 2 * A_TRI_PIECES * 8;            // hi + lo, bf16
constexpr int A_TRI_RECORD_BYTES = 2 * A_TRI_BLOCK_ELEMS * 2;      // blocks 0 and 2
// Piece p of a whole record (block p / 256, hi or lo, row (p / 4) % 32, 8 columns
// 8 (p % 4) ..) lies entirely above the diagonal of a diagonal block: always zero.
__host__ __device__ constexpr bool record_piece_zero(int p) {
    return (p >> 8) != 1 && (p & 3) > (((p >> 2) & 31) >> 3);
}
__host__ __device__ constexpr int tri_piece(int row, int c) {
    return 8 * ((row >> 3) * ((row >> 3) + 1) / 2) + (row & 7) * ((row >> 3) + 1) + c;
}
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

// v_mfma_f32_16x16x4_f32: lane l supplies A[l & 15][l >> 4] and B[l >> 4][l & 15].
__device__ __forceinline__ f32x4 mfma16f(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Accumulator layout of a 32x32 tile: register r of lane l holds
// D[row = 8*(r/4) + 4*(l>>5) + (r&3)][col = l & 31]; of a 16x16 tile: register
// r holds D[4*(l>>4) + r][l & 15].
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Compiler-only fence: the LDS operand loads above it are issued before the
// matrix instructions below it, so their latencies overlap instead of each
// MFMA waiting for its own freshly issued load.  The asm keeps the loads above
// it; the scheduling barrier keeps the machine scheduler from sinking them
// back between the MFMAs (which it otherwise does to save registers).
__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Order this wave's own LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Buffer resource over [p, p + bytes): loads past the end return 0 and stores
// past the end are dropped, so a chunk's rows beyond its sequence need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kBufferWord3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives element (i % 4) of the 8 bytes addressed by lane 4e + i / 4, as its
// element e.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ inline int64_t seq_start(int seq, int n_seq, int n_tok, const int32_t* cu) {
    return cu ? static_cast<int64_t>(cu[seq]) : static_cast<int64_t>(seq) * (n_tok / n_seq);
}

// First global chunk of sequence m (m = n_seq gives the number of chunks):
// chunk_off[m] for packed sequences of any lengths; for n_seq sequences of
// n_tok / n_seq tokens each (chunk_off == nullptr) it is m ceil(len / C).
__device__ inline int first_chunk(int m, int n_seq, int n_tok, const int32_t* chunk_off) {
    if (chunk_off) return chunk_off[m];
    return m * ((n_tok / n_seq + C - 1) / C);
}

// Token range [t0, t0 + n) of global chunk gc.
struct ChunkRef {
    int64_t t0;
    int n;
    int seq;  // the sequence that holds the chunk
};

__device__ inline ChunkRef chunk_ref(int gc, int n_seq, int n_tok, const int32_t* cu,
                                     const int32_t* chunk_off) {
    int lo = 0;
    if (chunk_off) {
        int hi = n_seq;  // chunk_off[lo] <= gc < chunk_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_off[mid] <= gc) lo = mid;
            else hi = mid;
        }
    } else {
        lo = gc / first_chunk(1, n_seq, n_tok, nullptr);  // only called while chunks exist
    }
    const int64_t s0 = seq_start(lo, n_seq, n_tok, cu), s1 = seq_start(lo + 1, n_seq, n_tok, cu);
    ChunkRef r;
    r.t0 = s0 + static_cast<int64_t>(gc - first_chunk(lo, n_seq, n_tok, chunk_off)) * C;
    r.n = static_cast<int>(min<int64_t>(C, s1 - r.t0));
    r.seq = lo;
    return r;
}

// 16x16x32 operand whose 8 reduction values per lane are the stacked-tile
// indices {4g..4g+3, 16+4g..16+4g+3} (g = lane / 16) past k0, from a row-major
// [row][k] buffer: row row0 + lane % 16.
__device__ __forceinline__ bf16x8 frag_st(const uint16_t* base, int pitch, int row0, int k0, int lane) {
    const uint16_t* p = base + (row0 + (lane & 15)) * pitch + k0 + 4 * (lane >> 4);
    const u16x4 lo = *reinterpret_cast<const u16x4*>(p);
    const u16x4 hi = *reinterpret_cast<const u16x4*>(p + 16);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The stacked-tile B operand of two 16x16 accumulator tiles a (first 16 rows)
// and b (next 16), rounded to bf16 as hi + lo parts.
__device__ __forceinline__ void split_stack(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_bf16x2(a[0], a[1], h0, l0);
    split_bf16x2(a[2], a[3], h1, l1);
    split_bf16x2(b[0], b[1], h2, l2);
    split_bf16x2(b[2], b[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

// The same stacked operand from a buffer stored transposed, [k][row] (k = the
// reduction index): rows row0 + lane % 16, reduction indices {k0 + 4g .. +3,
// k0 + 16 + 4g .. +3}, through two transposing LDS reads.  In each 16-lane group
// lane i addresses row k0 + 4g + i / 4 at columns row0 + 4 (i % 4) .. +3 and
// receives element e of its operand from lane 4e + i / 4, i.e. [k0 + 4g + e][row0 + i].
__device__ __forceinline__ bf16x8 frag_tr_st(const uint16_t* base, int pitch, int row0, int k0, int lane) {
    const int g = lane >> 4, m16 = lane & 15;
    const uint16_t* p = base + (k0 + 4 * g + (m16 >> 2)) * pitch + row0 + 4 * (m16 & 3);
    const s16x4 t0 = lds_read_tr16(p);
    const s16x4 t1 = lds_read_tr16(p + 16 * pitch);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 4 x 4 transpose within each quad of lanes: quad lane j holds row j of the quad's block
// in a[0 .. 3] before, and column j (a[e] = the former a[j] of quad lane e) after.  Two
// butterfly stages -- DPP exchanges with the lane 1 and then 2 apart, selects on that lane
// bit -- so no register is indexed by a lane-dependent value (the compiler turns such an
// index into branches).
__device__ __forceinline__ void quad_transpose4(u32x4& a, int lane) {
    const bool b0 = lane & 1, b1 = lane & 2;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint32_t rcv =
            __builtin_amdgcn_mov_dpp(b0 ? a[2 * c] : a[2 * c + 1], 0xB1, 0xF, 0xF, true);  // quad lanes 1,0,3,2
        a[2 * c] = b0 ? rcv : a[2 * c];
        a[2 * c + 1] = b0 ? a[2 * c + 1] : rcv;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint32_t rcv = __builtin_amdgcn_mov_dpp(b1 ? a[c] : a[c + 2], 0x4E, 0xF, 0xF, true);  // quad lanes 2,3,0,1
        a[c] = b1 ? rcv : a[c];
        a[c + 2] = b1 ? a[c + 2] : rcv;
    }
}

// Where 16-byte piece `piece` of a solved record goes in a [t][s] hi/lo pair of
// C x CP buffers: block b (rows 0-31 x cols 0-31, rows 32-63 x cols 0-31, rows
// 32-63 x cols 32-63), half (hi, lo), row, 8-column group.
__device__ __forceinline__ uint16_t* record_piece_dst(uint16_t* hi, uint16_t* lo, int piece) {
    const int b = piece >> 8, half = (piece >> 7) & 1, row = (piece >> 2) & 31, c8 = 8 * (piece & 3);
    return (half ? lo : hi) + ((b == 0 ? 0 : 32) + row) * CP + (b == 2 ? 32 : 0) + c8;
}

}  // namespace
}  // namespace kda
