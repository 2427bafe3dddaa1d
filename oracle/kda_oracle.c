/*
 * kda_oracle.c -- fp64 CPU oracle of the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library.  The GPU
 * library never links it, never includes it, and shares no source with it.
 *
 * What it computes (page "Kimi (AI)", section "Kimi Delta Attention (KDA)"):
 *   - the memory matrix S is d_v x d_k: the naive linear-attention equation
 *     writes S_t as the sum of v_i k_i^T, so rows index value channels and
 *     columns index key channels;
 *   - the three-step update of that section, in its order:
 *       forget gating    S~ = diag(alpha_t) S_{t-1}   (alpha_t scales rows)
 *       predict          v~ = S~ k_t
 *       memory updating  S_t = S~ + beta_t (v_t - v~) k_t^T
 *   - the read-out of the linear-attention equation, o_t = S_t q_t, taken
 *     with the post-update state (the state that already holds token t).
 *
 * A second form, the key-channel variant, gates the state from the right,
 * S~ = S diag(alpha_t) with alpha_t in R^{d_k} (column j scaled by
 * alpha_t[j]); predict, update and read-out are the same.  It is the reading of
 * the forget-gating step with the gate acting on the key side; the row form
 * above is the one the section's equations write.
 *
 * Everything is a plain sequential loop over tokens in double precision.
 * Independent (sequence, head) pairs are the only thing run in parallel
 * (OpenMP); within a pair nothing is blocked, fused or reordered.
 *
 * Inputs arrive as float32 arrays: every bf16 and every fp32 value the GPU
 * library receives is exactly a float32 value, and it is widened to double
 * without change.  Outputs are double.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_BAD_ARG 1
#define KDA_ORACLE_NO_MEMORY 2

int kda_oracle_abi_version(void) { return 1; }

/*
 * One (sequence, head) unit: runs tokens [t0, t0+len) of the packed token
 * axis through the recurrence, starting from S (d_v x d_k, row-major, double),
 * which is updated in place.  Token t of the unit has
 *   q at q + t*q_stride, k at k + t*k_stride   (d_k floats each),
 *   v at v + t*v_stride (d_v floats), alpha at a + t*a_stride (d_v floats, or
 *   d_k floats when key_gate is set),
 *   beta at beta[t*b_stride], output o + t*o_stride (d_v doubles).
 */
static void kda_unit(int key_gate, int64_t len, int64_t dk, int64_t dv,
                     const float* q, int64_t q_stride,
                     const float* k, int64_t k_stride,
                     const float* v, int64_t v_stride,
                     const float* a, int64_t a_stride,
                     const float* beta, int64_t b_stride,
                     double* S, double* o, int64_t o_stride,
                     double* vp /* d_v scratch */, double* e /* d_v scratch */)
{
    for (int64_t t = 0; t < len; ++t) {
        const float* qt = q + t * q_stride;
        const float* kt = k + t * k_stride;
        const float* vt = v + t * v_stride;
        const float* at = a + t * a_stride;
        const double bt = (double)beta[t * b_stride];
        double* ot = o ? o + t * o_stride : NULL;

        if (key_gate) {
            /* forget gating, key-channel form: S~ = S_{t-1} diag(alpha_t) -- column j scaled by alpha_t[j] */
            for (int64_t i = 0; i < dv; ++i) {
                double* Si = S + i * dk;
                for (int64_t j = 0; j < dk; ++j) Si[j] *= (double)at[j];
            }
        } else {
            /* forget gating: S~ = diag(alpha_t) S_{t-1} -- row i scaled by alpha_t[i] */
            for (int64_t i = 0; i < dv; ++i) {
                const double ai = (double)at[i];
                double* Si = S + i * dk;
                for (int64_t j = 0; j < dk; ++j) Si[j] *= ai;
            }
        }
        /* predict: v~ = S~ k_t */
        for (int64_t i = 0; i < dv; ++i) {
            const double* Si = S + i * dk;
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j) acc += Si[j] * (double)kt[j];
            vp[i] = acc;
        }
        /* error scaled by beta_t: beta_t (v_t - v~) */
        for (int64_t i = 0; i < dv; ++i) e[i] = bt * ((double)vt[i] - vp[i]);
        /* memory updating: S_t = S~ + e k_t^T */
        for (int64_t i = 0; i < dv; ++i) {
            double* Si = S + i * dk;
            const double ei = e[i];
            for (int64_t j = 0; j < dk; ++j) Si[j] += ei * (double)kt[j];
        }
        /* read-out: o_t = S_t q_t */
        if (ot) {
            for (int64_t i = 0; i < dv; ++i) {
                const double* Si = S + i * dk;
                double acc = 0.0;
                for (int64_t j = 0; j < dk; ++j) acc += Si[j] * (double)qt[j];
                ot[i] = acc;
            }
        }
    }
}

/*
 * Prefill over packed sequences.
 *   q, k      [n_tok, H, d_k]  float32 (values exactly as the GPU receives them)
 *   v, alpha  [n_tok, H, d_v]  float32
 *   beta      [n_tok, H]       float32
 *   S0        [n_seq, H, d_v, d_k] double, or NULL for zeros (double so that
 *             a state returned by an earlier call continues without rounding)
 *   cu_seqlens host int64 [n_seq+1], nondecreasing, cu_seqlens[0] = 0;
 *             sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
 *   o         [n_tok, H, d_v]  double (may be NULL: state only)
 *   S_T       [n_seq, H, d_v, d_k] double
 * An empty sequence leaves S_T = S0 (or zeros).  Returns 0 on success.
 */
static int prefill_f64(int key_gate, const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta,
                       const double* S0, const int64_t* cu_seqlens,
                       int64_t n_seq, int64_t H, int64_t dk, int64_t dv,
                       double* o, double* S_T)
{
    const int64_t da = key_gate ? dk : dv; /* gate values per (token, head) */
    if (!q || !k || !v || !alpha || !beta || !cu_seqlens || !S_T) return KDA_ORACLE_BAD_ARG;
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ORACLE_BAD_ARG;
    if (cu_seqlens[0] != 0) return KDA_ORACLE_BAD_ARG;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return KDA_ORACLE_BAD_ARG;

    int failed = 0;
    const int64_t units = n_seq * H;
#pragma omp parallel
    {
        double* vp = (double*)malloc((size_t)dv * sizeof(double));
        double* e = (double*)malloc((size_t)dv * sizeof(double));
        /* every thread reaches the worksharing loop; a thread without
           scratch memory only records the failure */
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!vp || !e) {
#pragma omp atomic write
                failed = 1;
            } else {
                const int64_t n = u / H, h = u % H;
                const int64_t t0 = cu_seqlens[n], len = cu_seqlens[n + 1] - t0;
                double* S = S_T + u * dv * dk;
                if (S0) {
                    memcpy(S, S0 + u * dv * dk, (size_t)(dv * dk) * sizeof(double));
                } else {
                    memset(S, 0, (size_t)(dv * dk) * sizeof(double));
                }
                kda_unit(key_gate, len, dk, dv,
                         q + (t0 * H + h) * dk, H * dk,
                         k + (t0 * H + h) * dk, H * dk,
                         v + (t0 * H + h) * dv, H * dv,
                         alpha + (t0 * H + h) * da, H * da,
                         beta + t0 * H + h, H,
                         S, o ? o + (t0 * H + h) * dv : NULL, H * dv, vp, e);
            }
        }
        free(vp);
        free(e);
    }
    return failed ? KDA_ORACLE_NO_MEMORY : KDA_ORACLE_OK;
}

int kda_oracle_prefill_f64(const float* q, const float* k, const float* v,
                           const float* alpha, const float* beta,
                           const double* S0, const int64_t* cu_seqlens,
                           int64_t n_seq, int64_t H, int64_t dk, int64_t dv,
                           double* o, double* S_T)
{
    return prefill_f64(0, q, k, v, alpha, beta, S0, cu_seqlens, n_seq, H, dk, dv, o, S_T);
}

/* The key-channel form: alpha is [n_tok, H, d_k]; everything else as above. */
int kda_oracle_prefill_keygate_f64(const float* q, const float* k, const float* v,
                                   const float* alpha, const float* beta,
                                   const double* S0, const int64_t* cu_seqlens,
                                   int64_t n_seq, int64_t H, int64_t dk, int64_t dv,
                                   double* o, double* S_T)
{
    return prefill_f64(1, q, k, v, alpha, beta, S0, cu_seqlens, n_seq, H, dk, dv, o, S_T);
}

/*
 * Decode: n_steps successive single-token steps for B sequences, each with
 * H heads -- the same recurrence, one token per step.  Inputs are step-major:
 *   q, k     [n_steps, B, H, d_k]   float32
 *   v, alpha [n_steps, B, H, d_v]   float32
 *   beta     [n_steps, B, H]        float32
 *   S        [B, H, d_v, d_k]       double, in/out (the persistent state)
 *   o        [n_steps, B, H, d_v]   double (may be NULL)
 * Steps run innermost per (b, h), so each head's state stays in cache.
 */
static int decode_f64(int key_gate, const float* q, const float* k, const float* v,
                      const float* alpha, const float* beta,
                      int64_t n_steps, int64_t B, int64_t H, int64_t dk, int64_t dv,
                      double* S, double* o)
{
    const int64_t da = key_gate ? dk : dv;
    if (!q || !k || !v || !alpha || !beta || !S) return KDA_ORACLE_BAD_ARG;
    if (n_steps < 0 || B < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ORACLE_BAD_ARG;
    int failed = 0;
    const int64_t units = B * H;
#pragma omp parallel
    {
        double* vp = (double*)malloc((size_t)dv * sizeof(double));
        double* e = (double*)malloc((size_t)dv * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!vp || !e) {
#pragma omp atomic write
                failed = 1;
            } else {
                const int64_t step_tok = B * H; /* stride between steps, in (b,h) units */
                kda_unit(key_gate, n_steps, dk, dv,
                         q + u * dk, step_tok * dk,
                         k + u * dk, step_tok * dk,
                         v + u * dv, step_tok * dv,
                         alpha + u * da, step_tok * da,
                         beta + u, step_tok,
                         S + u * dv * dk, o ? o + u * dv : NULL, step_tok * dv, vp, e);
            }
        }
        free(vp);
        free(e);
    }
    return failed ? KDA_ORACLE_NO_MEMORY : KDA_ORACLE_OK;
}

int kda_oracle_decode_f64(const float* q, const float* k, const float* v,
                          const float* alpha, const float* beta,
                          int64_t n_steps, int64_t B, int64_t H, int64_t dk, int64_t dv,
                          double* S, double* o)
{
    return decode_f64(0, q, k, v, alpha, beta, n_steps, B, H, dk, dv, S, o);
}

/* The key-channel form: alpha is [n_steps, B, H, d_k]. */
int kda_oracle_decode_keygate_f64(const float* q, const float* k, const float* v,
                                  const float* alpha, const float* beta,
                                  int64_t n_steps, int64_t B, int64_t H, int64_t dk, int64_t dv,
                                  double* S, double* o)
{
    return decode_f64(1, q, k, v, alpha, beta, n_steps, B, H, dk, dv, S, o);
}
