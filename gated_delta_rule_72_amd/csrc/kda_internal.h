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
enum Gate : int { GATE_CHANNEL = 0, GATE_SCALAR = 1, GATE_NONE = 2 };

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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);

// Workspace bytes of the fp32 prefill (the varlen schedule) and of the bf16
// prefill (schedule, chunk offsets and the per-(chunk, head) solved A blocks).
size_t prefill_workspace_bytes(int32_t n_seq, bool varlen);
size_t prefill_bf16_workspace_bytes(int32_t n_seq, int32_t n_tok, int32_t n_heads);

}  // namespace kda
