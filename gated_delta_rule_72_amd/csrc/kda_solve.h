// kda_solve.h -- the unit-lower triangular solve of one chunk, shared by the
// solve kernels of the chunked prefill (kda_prefill_mfma.hip: the decay-free
// Gram of the value-row and scalar gates; kda_prefill_keygate.hip: the decayed
// Gram of the key-channel gate).
//
// Given L (C x C, strictly lower, fp32 in LDS with pitch LP), the inverse
// X = (I + L)^{-1} is built by blocks in a workgroup of four waves: the four
// 16x16 diagonal blocks by forward substitution (wave 0), then
// X21 = -X22 L21 X11 at 16 rows and at 32 rows on fp32 MFMA.  The result is
// written as a solved record (three 32x32 blocks, hi + lo bf16).
// Private to the library.
#pragma once

#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int SOLVE_RP = 36;  // pitch of the 32x32 fp32 temporary of the 32-row level

// The inverse of one 16x16 unit-lower block I + Lb (strictly lower part read from
// Lb, fp32 rows of pitch PITCH), one column per lane: on return x[r] = row r of
// column c of the inverse (zero above the diagonal).
template <int PITCH>
__device__ __forceinline__ void solve_block16(const float* Lb, int c, float (&x)[16]) {
    // Each strictly lower row is loaded one row ahead of its use, so no LDS
    // round trip sits inside the dependent substitution chain.  Piece p
    // enumerates (row r = 1..15, columns s4..s4+3 < r + 3).
    f32x4 lrow[36];
    auto first_piece = [](int r) {
        int p = 0;
        for (int rr = 1; rr < r; ++rr) p += (rr + 3) / 4;
        return p;
    };
    auto load_row = [&](int r) {
#pragma unroll
        for (int s4 = 0, p = first_piece(r); s4 < r; s4 += 4, ++p)
            lrow[p] = *reinterpret_cast<const f32x4*>(Lb + r * PITCH + s4);
    };
    auto solve_row = [&](int r) {
        float acc0 = (r == c) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
        for (int s4 = 0, p = first_piece(r); s4 < r; s4 += 4, ++p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (s4 + e < r) {
                    if (e & 1) acc1 -= lrow[p][e] * x[s4 + e];
                    else acc0 -= lrow[p][e] * x[s4 + e];
                }
            }
        }
        x[r] = acc0 + acc1;  // zero for r < c
    };
    x[0] = c == 0 ? 1.f : 0.f;
    load_row(1);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
        if (r + 1 < 16) load_row(r + 1);
        issue_fence();
        solve_row(r);
    }
}

// Wave 0: the inverses of the four 16x16 unit-lower diagonal blocks of I + L.
// Lane = (block b = lane / 16, column c = lane % 16); on return x[r] = row r of
// column c of block b's inverse.  Reads only the diagonal blocks of Lf.
__device__ __forceinline__ void solve_diag_blocks(const float* Lf, int lane, float (&x)[16]) {
    const int b = lane >> 4, c = lane & 15;
    solve_block16<LP>(Lf + (16 * b) * LP + 16 * b, c, x);
}

// All four waves, once L is complete in Lf (the call begins with the barrier that
// makes it so): X = (I + L)^{-1} into Xs (pitch LP), from wave 0's diagonal-block
// inverses x.  Xs may alias storage that is dead once L is formed; Rtmp (32 rows
// of pitch SOLVE_RP) may alias rows 0-16 of Lf, which only the 16-row level reads.
// HALVES: only the two diagonal 32x32 blocks (the inverses of the two 32-token halves'
// systems); the 32-row level, and L's block (32..63, 0..31) it reads, are left out.
// Ends with a barrier.
template <bool HALVES = false>
__device__ __forceinline__ void assemble_inverse(float* Xs, const float* Lf, float* Rtmp, const float (&x)[16],
                                                 int wave, int lane) {
    const int g16 = lane >> 4, m16 = lane & 15;
    block_sync();
    if (wave == 0) {
        const int b = g16, c = m16;
#pragma unroll
        for (int r = 0; r < 16; ++r) Xs[(16 * b + r) * LP + 16 * b + c] = x[r];
    }
    block_sync();

    // ---- 16-row level (waves 0, 1): X[R, Cc] = -T_R L[R, Cc] T_Cc for the 16x16
    // blocks (16, 0) and (48, 32)
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
    }
    block_sync();
    if constexpr (HALVES) return;

    // ---- 32-row level, first half: Y2 = L[32:64, 0:32] X[0:32, 0:32], one 16x16
    // quadrant per wave
    const int qr = wave >> 1, qc = wave & 1;
    {
        float la[8], xa[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            la[kk] = Lf[(32 + 16 * qr + m16) * LP + 4 * kk + g16];
            xa[kk] = Xs[(4 * kk + g16) * LP + 16 * qc + m16];
        }
        issue_fence();
        f32x4 y = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            if (kk >= 4 * qc) y = mfma16f(la[kk], xa[kk], y);  // X[0:32, 0:32] is block-lower
#pragma unroll
        for (int r = 0; r < 4; ++r) Rtmp[(16 * qr + 4 * g16 + r) * SOLVE_RP + 16 * qc + m16] = y[r];
    }
    block_sync();

    // ---- second half: X[32:64, 0:32] = -X[32:64, 32:64] Y2
    {
        float xa[8], ra[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            xa[kk] = Xs[(32 + 16 * qr + m16) * LP + 32 + 4 * kk + g16];
            ra[kk] = Rtmp[(4 * kk + g16) * SOLVE_RP + 16 * qc + m16];
        }
        issue_fence();
        f32x4 z = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            if (kk < 4 * (qr + 1)) z = mfma16f(xa[kk], ra[kk], z);  // X[32:64, 32:64] is block-lower
#pragma unroll
        for (int r = 0; r < 4; ++r) Xs[(32 + 16 * qr + 4 * g16 + r) * LP + 16 * qc + m16] = -z[r];
    }
    block_sync();
}

// X (SCALE_BETA: X diag(beta)) -> the solved record at rec, by all 256 threads.
// Item = (block, row, 8-column piece); entries above the diagonal (never
// written in Xs) are selected away.  HALVES: blocks 0 and 2 only, in the packed
// form of the 32-token scan's records (pieces above the diagonal left out).
template <bool SCALE_BETA, bool HALVES = false>
__device__ __forceinline__ void write_solve_record(uint16_t* rec, const float* Xs, const float* bs, int tid) {
    constexpr int NB = HALVES ? 2 : 3;
    for (int item = tid; item < NB * 32 * 4; item += 256) {
        const int blk = HALVES ? 2 * (item >> 7) : item >> 7, row = (item >> 2) & 31, c8 = 8 * (item & 3);
        if (HALVES && (item & 3) > (row >> 3)) continue;  // all zero, not stored
        const int t = (blk == 0 ? 0 : 32) + row, s0 = (blk == 2 ? 32 : 0) + c8;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(Xs + t * LP + s0);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(Xs + t * LP + s0 + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bs + s0);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(bs + s0 + 4);
        float av[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = e < 4 ? x0[e] : x1[e - 4];
            av[e] = s0 + e <= t ? (SCALE_BETA ? xv * (e < 4 ? b0[e] : b1[e - 4]) : xv) : 0.f;
        }
        u32x4 wh, wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t a, b;
            split_bf16x2(av[2 * e], av[2 * e + 1], a, b);
            wh[e] = a;
            wl[e] = b;
        }
        if constexpr (HALVES) {
            uint16_t* dst = rec + (item >> 7) * A_TRI_BLOCK_ELEMS + tri_piece(row, item & 3) * 8;
            *reinterpret_cast<u32x4*>(dst) = wh;
            *reinterpret_cast<u32x4*>(dst + A_TRI_PIECES * 8) = wl;
        } else {
            uint16_t* dst = rec + blk * 2 * A_BLOCK_ELEMS + row * 32 + c8;
            *reinterpret_cast<u32x4*>(dst) = wh;
            *reinterpret_cast<u32x4*>(dst + A_BLOCK_ELEMS) = wl;
        }
    }
}

}  // namespace
}  // namespace kda
