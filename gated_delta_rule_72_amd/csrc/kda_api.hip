// kda_api.hip -- the C ABI of libkda: host-side validation and dispatch.
//
// Every argument is checked here before any HIP call, so invalid calls return
// a status without touching the device (and the checks run on machines with
// no GPU).  See include/kda.h for the contract of each entry point.
#include "kda.h"
#include "kda_internal.h"

namespace {

// Vector-loaded tensors need 16-byte alignment; beta, cu_seqlens and a scalar
// gate are read as scalars and need only their element alignment.
constexpr size_t kAlign = 16;

bool aligned(const void* p, size_t a = kAlign) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

size_t elem_bytes(kda_dtype dt) { return dt == KDA_DTYPE_BF16 ? 2 : 4; }

bool valid_dtype(kda_dtype dt) { return dt == KDA_DTYPE_F32 || dt == KDA_DTYPE_BF16; }

size_t workspace_need(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v, kda_dtype dt,
                      kda::Gate gate = kda::GATE_CHANNEL) {
    if (dt != KDA_DTYPE_BF16) return kda::prefill_workspace_bytes(n_seq, true);
    return gate == kda::GATE_KEY ? kda::prefill_keygate_workspace_bytes(n_seq, n_tok, n_heads, d_k, d_v)
                                 : kda::prefill_bf16_workspace_bytes(n_seq, n_tok, n_heads, d_k, d_v);
}

// Shared body of kda_prefill and kda_prefill_scalar_gate.
kda_status prefill_impl(const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const float* S0, const int32_t* cu_seqlens,
                        int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v,
                        kda_dtype dt, void* o, float* S_T, void* workspace,
                        size_t workspace_bytes, void* stream, kda::Gate gate) {
    if (!valid_dtype(dt)) return KDA_ERR_INVALID_ARGUMENT;
    if (n_seq < 1 || n_tok < 0 || n_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (!cu_seqlens && (n_tok % n_seq) != 0) return KDA_ERR_INVALID_ARGUMENT;
    const bool has_tokens = n_tok > 0;
    if (has_tokens && (!q || !k || !v || !beta || !o)) return KDA_ERR_INVALID_ARGUMENT;
    if (has_tokens && gate != kda::GATE_NONE && !alpha) return KDA_ERR_INVALID_ARGUMENT;
    if (gate == kda::GATE_NONE) alpha = nullptr;
    const void* ptrs[] = {q, k, v, S0, o, S_T, workspace};
    for (const void* p : ptrs)
        if (p && !aligned(p)) return KDA_ERR_INVALID_ARGUMENT;
    if (alpha && !aligned(alpha, gate == kda::GATE_SCALAR ? 4 : kAlign)) return KDA_ERR_INVALID_ARGUMENT;
    if ((beta && !aligned(beta, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return KDA_ERR_INVALID_ARGUMENT;
    // outputs may not overlap inputs, except S_T == S0 exactly
    const size_t eb = elem_bytes(dt);
    const size_t nt = static_cast<size_t>(n_tok), nh = static_cast<size_t>(n_heads);
    const size_t qk_bytes = nt * nh * d_k * eb, v_bytes = nt * nh * d_v * eb;
    const size_t a_bytes = gate == kda::GATE_CHANNEL ? nt * nh * d_v * 4
                           : gate == kda::GATE_KEY   ? nt * nh * d_k * 4
                           : gate == kda::GATE_SCALAR ? nt * nh * 4
                                                      : 0;
    const size_t b_bytes = nt * nh * 4;
    const size_t s_bytes = static_cast<size_t>(n_seq) * nh * d_v * d_k * 4;
    const size_t cu_bytes = cu_seqlens ? (static_cast<size_t>(n_seq) + 1) * 4 : 0;
    struct Region { const void* p; size_t n; };
    const Region ins[] = {{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {alpha, a_bytes},
                          {beta, b_bytes}, {cu_seqlens, cu_bytes}};
    const Region outs[] = {{o, v_bytes}, {S_T, S_T ? s_bytes : 0}};
    for (const Region& out : outs)
        for (const Region& in : ins)
            if (ranges_overlap(out.p, out.n, in.p, in.n)) return KDA_ERR_INVALID_ARGUMENT;
    if (ranges_overlap(o, v_bytes, S_T, S_T ? s_bytes : 0)) return KDA_ERR_INVALID_ARGUMENT;
    if (S_T && S0 && S_T != S0 && ranges_overlap(S_T, s_bytes, S0, s_bytes))
        return KDA_ERR_INVALID_ARGUMENT;
    if (S0 && ranges_overlap(o, v_bytes, S0, s_bytes)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t need = workspace_need(n_seq, n_tok, n_heads, d_k, d_v, dt, gate);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    // the workspace is written by the call: it may overlap no other argument
    const Region all[] = {{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {alpha, a_bytes}, {beta, b_bytes},
                          {cu_seqlens, cu_bytes}, {o, v_bytes}, {S0, S0 ? s_bytes : 0},
                          {S_T, S_T ? s_bytes : 0}};
    for (const Region& r : all)
        if (ranges_overlap(workspace, need, r.p, r.n)) return KDA_ERR_INVALID_ARGUMENT;

    kda::PrefillArgs a{q, k, v, alpha, beta, S0, cu_seqlens, n_seq, n_tok, n_heads, d_k, d_v,
                       dt == KDA_DTYPE_BF16, o, S_T, workspace, workspace_bytes, gate};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = a.bf16 ? kda::launch_prefill_bf16(a, s) : kda::launch_prefill_f32(a, s);
    return err == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

// Shared body of kda_decode_step and kda_decode_step_scalar_gate.
kda_status decode_impl(const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, float* S, void* o, int32_t batch, int32_t n_heads,
                       int32_t d_k, int32_t d_v, kda_dtype dt, void* stream, kda::Gate gate) {
    if (!valid_dtype(dt)) return KDA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || n_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (batch == 0) return KDA_OK;
    if (!q || !k || !v || !beta || !S || !o) return KDA_ERR_INVALID_ARGUMENT;
    if (gate != kda::GATE_NONE && !alpha) return KDA_ERR_INVALID_ARGUMENT;
    if (gate == kda::GATE_NONE) alpha = nullptr;
    const void* ptrs[] = {q, k, v, S, o};
    for (const void* p : ptrs)
        if (!aligned(p)) return KDA_ERR_INVALID_ARGUMENT;
    if (alpha && !aligned(alpha, gate == kda::GATE_SCALAR ? 4 : kAlign)) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned(beta, 4)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t eb = elem_bytes(dt);
    const size_t heads = static_cast<size_t>(batch) * n_heads;
    const size_t s_bytes = heads * d_v * d_k * 4, o_bytes = heads * d_v * eb;
    const size_t a_bytes = gate == kda::GATE_CHANNEL ? heads * d_v * 4
                           : gate == kda::GATE_KEY   ? heads * d_k * 4
                           : gate == kda::GATE_SCALAR ? heads * 4
                                                      : 0;
    struct Region { const void* p; size_t n; };
    const Region others[] = {{q, heads * d_k * eb}, {k, heads * d_k * eb}, {v, o_bytes},
                             {alpha, a_bytes}, {beta, heads * 4}};
    for (const Region& r : others)
        if (ranges_overlap(S, s_bytes, r.p, r.n) || ranges_overlap(o, o_bytes, r.p, r.n))
            return KDA_ERR_INVALID_ARGUMENT;
    if (ranges_overlap(S, s_bytes, o, o_bytes)) return KDA_ERR_INVALID_ARGUMENT;

    kda::DecodeArgs a{q, k, v, alpha, beta, S, o, batch, n_heads, d_k, d_v, dt == KDA_DTYPE_BF16, gate};
    const hipError_t err = kda::launch_decode(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}


// Shared body of kda_prefill_backward and its scalar-gate and key-gate forms.
kda_status backward_impl(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                         const float* S0, const int32_t* cu_seqlens, const float* dO, const float* dS_T,
                         int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v, kda_dtype dt,
                         float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dS0, void* workspace,
                         size_t workspace_bytes, void* stream, kda::Gate gate) {
    if (!valid_dtype(dt)) return KDA_ERR_INVALID_ARGUMENT;
    if (n_seq < 1 || n_tok < 0 || n_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (!cu_seqlens && (n_tok % n_seq) != 0) return KDA_ERR_INVALID_ARGUMENT;
    if (n_tok > 0 && (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta)) return KDA_ERR_INVALID_ARGUMENT;
    if (n_tok > 0 && gate != kda::GATE_NONE && (!alpha || !dalpha)) return KDA_ERR_INVALID_ARGUMENT;
    if (gate == kda::GATE_NONE) alpha = nullptr, dalpha = nullptr;
    const void* vec[] = {q, k, v, S0, dS_T, dq, dk, dS0, workspace};
    for (const void* p : vec)
        if (p && !aligned(p)) return KDA_ERR_INVALID_ARGUMENT;
    const void* scal[] = {alpha, beta, cu_seqlens, dO, dv, dalpha, dbeta};
    for (const void* p : scal)
        if (p && !aligned(p, 4)) return KDA_ERR_INVALID_ARGUMENT;
    if (gate == kda::GATE_KEY && alpha && !aligned(alpha)) return KDA_ERR_INVALID_ARGUMENT;  // float4 loads
    const size_t eb = elem_bytes(dt);
    const size_t nt = static_cast<size_t>(n_tok), nh = static_cast<size_t>(n_heads);
    const size_t qk_bytes = nt * nh * d_k * eb, v_bytes = nt * nh * d_v * eb;
    const size_t a_bytes = gate == kda::GATE_CHANNEL  ? nt * nh * d_v * 4
                           : gate == kda::GATE_KEY    ? nt * nh * d_k * 4
                           : gate == kda::GATE_SCALAR ? nt * nh * 4
                                                      : 0;
    const size_t b_bytes = nt * nh * 4, s_bytes = static_cast<size_t>(n_seq) * nh * d_v * d_k * 4;
    const size_t cu_bytes = cu_seqlens ? (static_cast<size_t>(n_seq) + 1) * 4 : 0;
    const size_t need = kda::prefill_backward_workspace_bytes(n_seq, n_tok, n_heads, d_k, d_v);
    if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
    struct Region { const void* p; size_t n; };
    const Region ins[] = {{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {alpha, a_bytes}, {beta, b_bytes},
                          {S0, S0 ? s_bytes : 0}, {cu_seqlens, cu_bytes}, {dO, nt * nh * d_v * 4},
                          {dS_T, dS_T ? s_bytes : 0}};
    const Region outs[] = {{dq, nt * nh * d_k * 4}, {dk, nt * nh * d_k * 4}, {dv, nt * nh * d_v * 4},
                           {dalpha, a_bytes}, {dbeta, b_bytes}, {dS0, dS0 ? s_bytes : 0}, {workspace, need}};
    // outputs (and the workspace) overlap neither the inputs nor each other
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Region& in : ins)
            if (ranges_overlap(outs[i].p, outs[i].n, in.p, in.n)) return KDA_ERR_INVALID_ARGUMENT;
        for (size_t j2 = i + 1; j2 < sizeof(outs) / sizeof(outs[0]); ++j2)
            if (ranges_overlap(outs[i].p, outs[i].n, outs[j2].p, outs[j2].n)) return KDA_ERR_INVALID_ARGUMENT;
    }
    kda::BackwardArgs a{q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq, n_tok, n_heads, d_k, d_v,
                        dt == KDA_DTYPE_BF16, dq, dk, dv, dalpha, dbeta, dS0, workspace, gate};
    const hipError_t err = kda::launch_prefill_backward(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    }
    return "KDA_ERR_UNKNOWN";
}

size_t kda_prefill_workspace_size(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k,
                                  int32_t d_v, kda_dtype dt) {
    if (n_seq < 1 || n_tok < 0 || n_heads < 1 || !supported_dim(d_k) || !supported_dim(d_v) ||
        !valid_dtype(dt))
        return 0;
    return workspace_need(n_seq, n_tok, n_heads, d_k, d_v, dt);
}

size_t kda_prefill_key_gate_workspace_size(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k,
                                           int32_t d_v, kda_dtype dt) {
    if (n_seq < 1 || n_tok < 0 || n_heads < 1 || !supported_dim(d_k) || !supported_dim(d_v) ||
        !valid_dtype(dt))
        return 0;
    return workspace_need(n_seq, n_tok, n_heads, d_k, d_v, dt, kda::GATE_KEY);
}

kda_status kda_prefill(const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const float* S0, const int32_t* cu_seqlens,
                       int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v,
                       kda_dtype dt, void* o, float* S_T, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, alpha, beta, S0, cu_seqlens, n_seq, n_tok, n_heads, d_k, d_v, dt, o,
                        S_T, workspace, workspace_bytes, stream, kda::GATE_CHANNEL);
}

kda_status kda_prefill_scalar_gate(const void* q, const void* k, const void* v, const float* alpha,
                                   const float* beta, const float* S0, const int32_t* cu_seqlens,
                                   int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k,
                                   int32_t d_v, kda_dtype dt, void* o, float* S_T, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, alpha, beta, S0, cu_seqlens, n_seq, n_tok, n_heads, d_k, d_v, dt, o,
                        S_T, workspace, workspace_bytes, stream,
                        alpha ? kda::GATE_SCALAR : kda::GATE_NONE);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, float* S, void* o, int32_t batch, int32_t n_heads,
                           int32_t d_k, int32_t d_v, kda_dtype dt, void* stream) {
    return decode_impl(q, k, v, alpha, beta, S, o, batch, n_heads, d_k, d_v, dt, stream, kda::GATE_CHANNEL);
}

kda_status kda_decode_step_scalar_gate(const void* q, const void* k, const void* v, const float* alpha,
                                       const float* beta, float* S, void* o, int32_t batch,
                                       int32_t n_heads, int32_t d_k, int32_t d_v, kda_dtype dt,
                                       void* stream) {
    return decode_impl(q, k, v, alpha, beta, S, o, batch, n_heads, d_k, d_v, dt, stream,
                       alpha ? kda::GATE_SCALAR : kda::GATE_NONE);
}

kda_status kda_prefill_key_gate(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t n_seq,
                                int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v, kda_dtype dt, void* o,
                                float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, alpha, beta, S0, cu_seqlens, n_seq, n_tok, n_heads, d_k, d_v, dt, o, S_T,
                        workspace, workspace_bytes, stream, kda::GATE_KEY);
}

kda_status kda_decode_step_key_gate(const void* q, const void* k, const void* v, const float* alpha,
                                    const float* beta, float* S, void* o, int32_t batch, int32_t n_heads,
                                    int32_t d_k, int32_t d_v, kda_dtype dt, void* stream) {
    return decode_impl(q, k, v, alpha, beta, S, o, batch, n_heads, d_k, d_v, dt, stream, kda::GATE_KEY);
}

size_t kda_prefill_backward_workspace_size(int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v) {
    if (n_seq < 1 || n_tok < 0 || n_heads < 1 || !supported_dim(d_k) || !supported_dim(d_v)) return 0;
    return kda::prefill_backward_workspace_bytes(n_seq, n_tok, n_heads, d_k, d_v);
}

kda_status kda_prefill_backward(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                                const float* S0, const int32_t* cu_seqlens, const float* dO, const float* dS_T,
                                int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k, int32_t d_v,
                                kda_dtype dt, float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                                float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq, n_tok, n_heads, d_k, d_v, dt, dq, dk,
                         dv, dalpha, dbeta, dS0, workspace, workspace_bytes, stream, kda::GATE_CHANNEL);
}

kda_status kda_prefill_backward_scalar_gate(const void* q, const void* k, const void* v, const float* alpha,
                                            const float* beta, const float* S0, const int32_t* cu_seqlens,
                                            const float* dO, const float* dS_T, int32_t n_seq, int32_t n_tok,
                                            int32_t n_heads, int32_t d_k, int32_t d_v, kda_dtype dt, float* dq,
                                            float* dk, float* dv, float* dalpha, float* dbeta, float* dS0,
                                            void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq, n_tok, n_heads, d_k, d_v, dt, dq, dk,
                         dv, dalpha, dbeta, dS0, workspace, workspace_bytes, stream,
                         alpha ? kda::GATE_SCALAR : kda::GATE_NONE);
}

kda_status kda_prefill_backward_key_gate(const void* q, const void* k, const void* v, const float* alpha,
                                         const float* beta, const float* S0, const int32_t* cu_seqlens,
                                         const float* dO, const float* dS_T, int32_t n_seq, int32_t n_tok,
                                         int32_t n_heads, int32_t d_k, int32_t d_v, kda_dtype dt, float* dq,
                                         float* dk, float* dv, float* dalpha, float* dbeta, float* dS0,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(q, k, v, alpha, beta, S0, cu_seqlens, dO, dS_T, n_seq, n_tok, n_heads, d_k, d_v, dt, dq, dk,
                         dv, dalpha, dbeta, dS0, workspace, workspace_bytes, stream, kda::GATE_KEY);
}

}  // extern "C"
