// kda_internal.h -- argument bundles and launcher declarations between the
// C ABI layer (kda_api.hip) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Layout of the forget gate alpha.
//   GATE_CHANNEL  [.., H, d_v]: one gate per value channel (KDA, page "Kimi (AI)",
//                 section "Kimi Delta Attention (KDA)")
//   GATE_SCALAR   [.., H]: one gate per (token, head) for every row -- the
//                 scalar-gated delta rule (Gated DeltaNet) that KDA refines
//   GATE_NONE     no gate (alpha = 1): the plain delta rule; alpha is NULL
//   GATE_KEY      [.., H, d_k]: one gate per key channel, applied from the right
//                 (S~ = S diag(alpha)); token-recurrent kernels only
enum Gate : int { GATE_CHANNEL = 0, GATE_SCALAR = 1, GATE_NONE = 2, GATE_KEY = 3 };

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    float* S;
    void* o;
    int32_t batch, n_heads, d_k, d_v;
    bool bf16;
    Gate gate;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* S0;           // may be null (zeros)
    const int32_t* cu_seqlens;  // may be null (equal lengths)
    int32_t n_seq, n_tok, n_heads, d_k, d_v;
    bool bf16;
    void* o;
    float* S_T;                // may be null
    void* workspace;
    size_t workspace_bytes;
    Gate gate;
};

// Chunk length of the chunkwise bf16 prefill (tokens solved together).  The
// fp32 prefill runs token by token.
constexpr int PREFILL_CHUNK_BF16 = 64;

// Segments per sequence for the sequence-parallel bf16 prefill (1 = one scan
// per sequence).  Calls whose (sequence, head, 64-row block) units would leave
// most of the 256 CUs idle have each sequence cut into G segments of whole
// 64-token chunks (G a power of two, units x G at most 256 workgroups, on
// average at least two chunks per segment).  Each segment is scanned twice more
// than one scan would (its end state and transition, in one launch), so the split
// pays from G = 4 on (measured, ms per call: 2 x 8192 tokens, 32 heads, G = 2:
// 0.549 against 0.404 for one scan; G = 4: 1 x 8192, 32 heads, 0.308 against
// 0.372; 2 x 4096, 16 heads, 0.154 against 0.194; 1 x 2048, 32 heads, 0.091
// against 0.102).  Needs d_k = d_v.  Decided from the sizes alone (the host never
// reads cu_seqlens).
inline int prefill_segments(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    if (d_k != d_v || n_tok <= 0 || n_seq < 1) return 1;
    const int64_t units = static_cast<int64_t>(n_seq) * n_heads * (d_v / 64);
    const int64_t avg = n_tok / n_seq;
    int g = 1;
    while (units * 2 * g <= 256 && avg / (2 * g) >= 2 * 64) g *= 2;
    return g >= 4 ? g : 1;
}

// One pass of the bf16 prefill's scan in 32-token steps (kda_prefill_scan32.hip) over
// n_units_seq sequences (or segments, through cu and the dense split), with the
// diagonal blocks of the chunk solve's A records, the schedule (packed input) and the
// range marks.  NOOUT: no outputs (o is not written); SPLIT: the state enters K S^T as
// hi + lo bf16.  flags: SCAN_ZERO_V (v read as zero), SCAN_S0_IDENTITY (S0 = I, d_v = d_k),
// SCAN_STATE_AFRAG / SCAN_STATE_DFRAG (S_T stored in MFMA fragment order, kda_mfma.h).
// gdecay (or null): every unit's total decay per value row, [n_units_seq, H, d_v].
// skip_flags (or null): range marks [n_units_seq, H, d_v / 64] of segments, skip_segs
// consecutive units to a sequence; a unit is skipped (nothing written) when any segment
// of its sequence is marked for its block of rows.
template <int DK, int DV, int GATE, bool NOOUT, bool SPLIT>
hipError_t launch_scan32_pass(const PrefillArgs& a, int n_units_seq, const int32_t* cu, const int32_t* order,
                              const int32_t* chunk_off, const uint16_t* arec, const float* S0, float* S_T, int flags,
                              float* gdecay, int32_t* range_flags, hipStream_t stream,
                              const int32_t* skip_flags = nullptr, int skip_segs = 1);

// The sequence-parallel prefill's two output-free passes in one launch (kda_prefill_scan32.hip):
// every segment's end state from zero (dS, accumulator fragment order), its total decay per
// value row (gdecay) and range marks, and its transition from S0 = I with v = 0 and no gate
// (Mf, A-operand fragment order); d_v = d_k.
template <int DK, int DV, int GATE>
hipError_t launch_scan32_pair(const PrefillArgs& a, int n_units_seq, const int32_t* cu, const int32_t* order,
                              const int32_t* chunk_off, const uint16_t* arec, float* dS, float* gdecay,
                              int32_t* range_flags, float* Mf, hipStream_t stream);

// The inputs and outputs of the token-recurrent recomputation that the segment
// composition runs for units marked beyond the decay range (the call's own, not the
// segments').
struct SegmentFixupArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* alpha;
    const float* beta;
    const int32_t* cu_seqlens;
    int n_tok;
    uint16_t* o;
};
// Composes the segment states of the sequence-parallel prefill (kda_segments.hip) from
// every segment's transition (Mf) and end state from zero (dSf), both in MFMA fragment
// order; G even.  With range_flags it also recomputes the marked units token by token.
template <int DK, int DV, int GATE>
hipError_t launch_combine_segments(const float* gdecay, const float* S0, const float* dSf, const float* Mf,
                                   const int32_t* range_flags, int n_seq, int G, int n_heads, float* S_start,
                                   float* S_T, const SegmentFixupArgs& fx, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
// Token-recurrent prefill (kda_prefill_valu.hip): float32 inputs, the
// key-channel gate for either input type, and short bf16 calls.
hipError_t launch_prefill_recurrent(const PrefillArgs& a, hipStream_t stream);
// The token-recurrent recomputation, from S0, of the (sequence, head, block of 64
// value rows) units that the chunked bf16 scan marked as beyond the decay range
// of its factored form: range_flags [n_seq G, H, d_v / 64], G segments per
// sequence (1 without the sequence-parallel split); a unit is recomputed if any
// of its segments is marked.  Workgroups of unmarked units return at once.
hipError_t launch_prefill_range_fixup(const PrefillArgs& a, const int32_t* range_flags, int G, hipStream_t stream);

// bf16 prefill calls this short (equal lengths of at most this many tokens per
// sequence, no cu_seqlens) run token by token: multi-token decode.
constexpr int RECURRENT_MAX_TOKENS = 16;
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// The chunked bf16 prefill with the gate on key channels (kda_prefill_keygate.hip).
hipError_t launch_prefill_keygate(const PrefillArgs& a, hipStream_t stream);
// chunk_off[m] = number of 64-token chunks of sequences 0 .. m-1 (m = 0 .. n_seq), from
// cu_seqlens on the device (kda_prefill_mfma.hip).
hipError_t launch_chunk_offsets(const int32_t* cu_seqlens, int n_seq, int n_tok, int32_t* chunk_off,
                                hipStream_t stream);

// Workspace bytes of the fp32 prefill (the varlen schedule) and of the bf16
// prefill (schedule, chunk offsets, the per-(chunk, head) solved A blocks, and
// for the sequence-parallel path the segment states).
size_t prefill_workspace_bytes(int32_t n_seq, bool varlen);
size_t prefill_bf16_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v);
// The same for the bf16 prefill with the gate on key channels: schedule, chunk
// offsets, unit flags, chunk marks, and two solved records (A and the decayed
// Q K^T) per (chunk, head).
size_t prefill_keygate_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v);

// Backward of the token-recurrent prefill (kda_backward.hip): the gradients of
// q, k, v, alpha, beta and S0 given those of o and S_T, for every gate.
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* S0;            // may be null (zeros)
    const int32_t* cu_seqlens;  // may be null (equal lengths)
    const float* dO;
    const float* dS_T;          // may be null (zeros)
    int32_t n_seq, n_tok, n_heads, d_k, d_v;
    bool bf16;
    float* dq;
    float* dk;
    float* dv;
    float* dalpha;              // null for GATE_NONE
    float* dbeta;
    float* dS0;                 // may be null (not wanted)
    void* workspace;
    Gate gate;
};
hipError_t launch_prefill_backward(const BackwardArgs& a, hipStream_t stream);

// Buffers of the chunked backward (bf16 inputs; value-channel, scalar or no gate),
// carved from the backward's workspace.
struct BwdChunkBufs {
    int32_t* order;      // longest-first schedule (packed input) or null
    int32_t* chunk_off;  // first chunk of every sequence (packed input) or null
    int32_t* flags;      // [n_seq, H, d_v / 64]: units left to the token-recurrent pass
    uint16_t* rec;       // solved T record of every (chunk, head)
    float* sck;          // [chunks, H, d_v, d_k] state entering every chunk
    float* gck;          // [chunks, H, d_v, d_k] gradient of the state leaving every chunk
    int64_t max_chunks;  // n_tok / 64 + n_seq: bound on the number of chunks
};
// The backward's forward pass (kda_prefill_mfma.hip): schedule and chunk offsets for
// packed input, the chunk solve (A records into the space of gck, which nothing
// writes before the reverse scan; T records into rec; marks for tiny beta), and the
// checkpoint scan (states into sck, range marks into flags).  The caller clears flags.
hipError_t launch_backward_forward_pass(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream);
// Its checkpoint scan (kda_prefill_scan32.hip, 32-token steps): the state entering every
// 64-token chunk into ckpt, range marks set in range_flags, the diagonal blocks of the
// chunk solve's A records.
template <int DK, int DV, int GATE>
hipError_t launch_scan32_ckpt(const BackwardArgs& a, const int32_t* order, const int32_t* chunk_off,
                              const uint16_t* arec, int32_t* range_flags, float* ckpt, hipStream_t stream);
// The chunked passes proper (kda_backward_chunk.hip): the reverse state-gradient scan
// (gck, dS0) and the per-(chunk, head) gradients.
hipError_t launch_backward_chunk_passes(const BackwardArgs& a, const BwdChunkBufs& b, hipStream_t stream);
// The token-recurrent backward (kda_backward.hip) of the units marked in flags only
// (null: every unit), accumulating into outputs zeroed by the caller where summed.
hipError_t launch_backward_recurrent(const BackwardArgs& a, const int32_t* order, const int32_t* flags, char* ws,
                                     hipStream_t stream);
// Tokens between the state checkpoints the backward keeps; the staged forward
// (kda_prefill_valu.hip) writes them for it: slot n + t0 / 16 + b holds the state
// entering block b of sequence n (first token t0), [slot, H, d_v, d_k] fp32.
constexpr int STATE_CHECKPOINT_TOKENS = 16;
hipError_t launch_prefill_checkpoints(const PrefillArgs& a, const int32_t* order, float* ckpt, hipStream_t stream,
                                      const int32_t* range_flags = nullptr);
// Workspace bytes: the longest-first schedule, a state checkpoint every 16
// tokens of every (sequence, head), and each wave's states within one block.
size_t prefill_backward_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v);

}  // namespace kda
