/*
 * CPU fp64 oracle for decayed recurrent (Lightning) attention: forward pass and
 * its gradients (backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  It shares
 * no code, header, table or helper with the GPU library and must never be
 * used as a fallback for it.
 *
 * What it computes (ejkernel "recurrent" interface page, docstring "The core
 * update is"): for every sequence n and query head h, a state S of shape
 * [dk, dv] is carried token by token,
 *
 *     S_t = exp(g_gamma[h]) * S_{t-1} + k_t^T v_t          (outer product)
 *     o_t = scale * (q_t S_t)                              (contract over dk)
 *
 * with S_{-1} = initial_state (or zeros) and final_state = S after the last
 * token.  Readings taken where the pages are silent or garbled:
 *   - g_gamma is a log-decay: the per-step factor is exp(g_gamma[h]); all-zero
 *     g_gamma is "no decay" (recurrent page, defaults of the forward rule).
 *   - decay first, then add token t, then read out: token t reaches o_t with
 *     weight 1.
 *   - the printed "o_t = h_t @ q_t" is read as q_t^T S_t (a dv-vector), the
 *     only orientation whose shapes agree when dk != dv.
 *   - scale multiplies q (lightning_attn page, softmax_scale argument), so it
 *     scales o and never the state.
 *   - GQA: query head h reads kv head h / (H / Hkv) (grouped, contiguous);
 *     decay and state are per query head.  The pages fix no grouping, so this
 *     convention is parity unpinned against them: the pins check it only
 *     against an independent statement of the same convention.
 *   - reverse: the same recurrence run from the last position to the first;
 *     o_t stays at index t; initial_state enters at the last position.
 *   - packed varlen (cu_seqlens): the state restarts at every boundary and
 *     each sequence has its own initial/final state.
 *
 * All arithmetic is IEEE fp64.  Inputs are the exact values of the bf16 or
 * fp32 words the GPU receives.  Loops are written in the order of the
 * recurrence, with no blocking or reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_IN_BF16 0
#define ORACLE_IN_F32 1

/* Exact value of element i of an input array stored as bf16 words or fp32. */
static double in_value(const void* base, int dtype, int64_t i) {
    if (dtype == ORACLE_IN_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Lightning per-head log-decay (ejkernel lightning_attn page, module docstring
 * "Key innovation" and the wrapper body):
 *     g_gamma[h] = -(8 / H) * (1 - layer_idx / num_layers) * h,  h = 0..H-1.
 * The wrapper builds the coefficient as a Python float (fp64) and multiplies
 * it into a float32 arange; under JAX's weak typing the coefficient is first
 * rounded to float32, then the product is taken in float32.
 */
int oracle_lightning_g_gamma(int num_heads, int layer_idx, int num_layers, float* out) {
    if (num_heads <= 0 || num_layers <= 0 || out == NULL) return -1;
    double coef = -(8.0 / (double)num_heads * (1.0 - (double)layer_idx / (double)num_layers));
    float coef32 = (float)coef;
    for (int h = 0; h < num_heads; ++h) {
        volatile float hv = (float)h; /* float32 arange element */
        out[h] = coef32 * hv;         /* float32 product */
    }
    return 0;
}

int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * Forward recurrence (ejkernel "recurrent" page, update equation; lightning_attn
 * page for the argument meanings).
 *
 *   q [B, T, H, dk], k [B, T, Hkv, dk], v [B, T, Hkv, dv]   (in_dtype)
 *   g_gamma [H] float32, scale (fp64 value of the float32 scale)
 *   initial_state [N_seq, H, dk, dv] float32, or NULL for zeros
 *   cu_seqlens [N_seq + 1] int64, or NULL: then N_seq = B and sequence n is
 *     batch row n; else B must be 1 and sequence n is rows [cu[n], cu[n+1]).
 *   pair_mask [N_seq * H] or NULL: when given, only (n, h) pairs with a
 *     non-zero entry are computed (the others are left untouched).
 *   o [B, T, H, dv] fp64, final_state [N_seq, H, dk, dv] fp64 (outputs)
 * Returns 0, or -1 on inconsistent arguments.
 */
int oracle_recurrent_fwd(int batch, int seqlen, int num_heads, int num_kv_heads,
                         int dk, int dv, int in_dtype,
                         const void* q, const void* k, const void* v,
                         const float* g_gamma, double scale,
                         const float* initial_state, int reverse,
                         const int64_t* cu_seqlens, int num_seqs,
                         const uint8_t* pair_mask,
                         double* o, double* final_state) {
    if (batch <= 0 || seqlen < 0 || num_heads <= 0 || num_kv_heads <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (num_heads % num_kv_heads != 0) return -1;
    if (cu_seqlens != NULL && batch != 1) return -1;
    const int n_seq = cu_seqlens ? num_seqs : batch;
    const int group = num_heads / num_kv_heads;
    const int64_t n_pairs = (int64_t)n_seq * num_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pair = 0; pair < n_pairs; ++pair) {
        if (pair_mask && !pair_mask[pair]) continue;
        const int n = (int)(pair / num_heads);
        const int h = (int)(pair % num_heads);
        const int kvh = h / group;
        int64_t row0, len; /* rows row0 .. row0+len-1 of the flattened [B*T] axis */
        if (cu_seqlens) {
            row0 = cu_seqlens[n];
            len = cu_seqlens[n + 1] - cu_seqlens[n];
        } else {
            row0 = (int64_t)n * seqlen;
            len = seqlen;
        }
        const double lam = exp((double)g_gamma[h]);

        double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
        double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
        double* out_row = (double*)malloc(sizeof(double) * (size_t)dv);
        const int64_t st_base = ((int64_t)n * num_heads + h) * dk * dv;
        for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
            S[i] = initial_state ? (double)initial_state[st_base + i] : 0.0;

        for (int64_t step = 0; step < len; ++step) {
            const int64_t row = reverse ? row0 + len - 1 - step : row0 + step;
            const int64_t qo = (row * num_heads + h) * dk;
            const int64_t ko = (row * num_kv_heads + kvh) * dk;
            const int64_t vo = (row * num_kv_heads + kvh) * dv;
            for (int a = 0; a < dk; ++a) qt[a] = in_value(q, in_dtype, qo + a);
            for (int a = 0; a < dk; ++a) kt[a] = in_value(k, in_dtype, ko + a);
            for (int c = 0; c < dv; ++c) vt[c] = in_value(v, in_dtype, vo + c);
            /* S <- lam * S + k_t^T v_t */
            for (int a = 0; a < dk; ++a)
                for (int c = 0; c < dv; ++c)
                    S[(int64_t)a * dv + c] = lam * S[(int64_t)a * dv + c] + kt[a] * vt[c];
            /* o_t = scale * (q_t S) */
            for (int c = 0; c < dv; ++c) out_row[c] = 0.0;
            for (int a = 0; a < dk; ++a)
                for (int c = 0; c < dv; ++c) out_row[c] += qt[a] * S[(int64_t)a * dv + c];
            for (int c = 0; c < dv; ++c) o[(row * num_heads + h) * dv + c] = scale * out_row[c];
        }
        for (int64_t i = 0; i < (int64_t)dk * dv; ++i) final_state[st_base + i] = S[i];
        free(qt);
        free(kt);
        free(vt);
        free(out_row);
        free(S);
    }
    return 0;
}

/*
 * Gradients of the forward recurrence above (the recurrent page's custom-VJP
 * backward: given dO and d final_state it returns dq, dk, dv and d
 * initial_state; g_gamma is not differentiated, as in the lightning wrapper).
 *
 * Derivation by the chain rule through S_t = lam S_{t-1} + k_t^T v_t and
 * o_t = scale q_t S_t.  Write D_t for the total gradient that reaches S_t:
 *
 *     D_t  = scale q_t^T dO_t + lam D_{t+1}     (D after the last token = d_final / lam,
 *                                                i.e. the last step adds d_final undecayed)
 *     dq_t = scale dO_t S_t^T                   (dk-vector)
 *     dk_t = D_t v_t                            (contract over dv)
 *     dv_t = k_t D_t                            (contract over dk)
 *     d_initial_state = lam D_first
 *
 * "first" and "last" follow the direction of the forward pass (reverse runs
 * from the last position to the first).  Under GQA, dk and dv of kv head j
 * sum the contributions of every query head that reads j.
 *
 *   d_o [B, T, H, dv] in_dtype (like q, k, v);  d_final [N_seq, H, dk, dv] float32 or NULL (zeros)
 *   dq [B, T, H, dk], dk_out [B, T, Hkv, dk], dv_out [B, T, Hkv, dv] fp64 (outputs;
 *     rows outside every sequence are left untouched)
 *   d_init [N_seq, H, dk, dv] fp64 or NULL (then not computed)
 * Two sweeps per (sequence, query head): forward for S_t and dq_t, then backward
 * for D_t, dk_t and dv_t.  Returns 0, or -1 on inconsistent arguments.
 */
int oracle_recurrent_bwd(int batch, int seqlen, int num_heads, int num_kv_heads,
                         int dk, int dv, int in_dtype,
                         const void* q, const void* k, const void* v,
                         const float* g_gamma, double scale,
                         const float* initial_state, int reverse,
                         const int64_t* cu_seqlens, int num_seqs,
                         const void* d_o, const float* d_final,
                         double* dq, double* dk_out, double* dv_out, double* d_init) {
    if (batch <= 0 || seqlen < 0 || num_heads <= 0 || num_kv_heads <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (num_heads % num_kv_heads != 0) return -1;
    if (cu_seqlens != NULL && batch != 1) return -1;
    const int n_seq = cu_seqlens ? num_seqs : batch;
    const int group = num_heads / num_kv_heads;
    const int64_t n_groups = (int64_t)n_seq * num_kv_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t gi = 0; gi < n_groups; ++gi) {
        const int n = (int)(gi / num_kv_heads);
        const int kvh = (int)(gi % num_kv_heads);
        int64_t row0, len;
        if (cu_seqlens) {
            row0 = cu_seqlens[n];
            len = cu_seqlens[n + 1] - cu_seqlens[n];
        } else {
            row0 = (int64_t)n * seqlen;
            len = seqlen;
        }
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
        double* D = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
        double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
        double* dot = (double*)malloc(sizeof(double) * (size_t)dv);

        /* the group's rows of dk and dv start from zero and collect every head */
        for (int64_t step = 0; step < len; ++step) {
            const int64_t row = row0 + step;
            for (int a = 0; a < dk; ++a) dk_out[(row * num_kv_heads + kvh) * dk + a] = 0.0;
            for (int c = 0; c < dv; ++c) dv_out[(row * num_kv_heads + kvh) * dv + c] = 0.0;
        }
        for (int h = kvh * group; h < (kvh + 1) * group; ++h) {
            const double lam = exp((double)g_gamma[h]);
            const int64_t st_base = ((int64_t)n * num_heads + h) * dk * dv;

            /* sweep 1, in the forward direction: S_t, then dq_t = scale dO_t S_t^T */
            for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
                S[i] = initial_state ? (double)initial_state[st_base + i] : 0.0;
            for (int64_t step = 0; step < len; ++step) {
                const int64_t row = reverse ? row0 + len - 1 - step : row0 + step;
                const int64_t ko = (row * num_kv_heads + kvh) * dk;
                const int64_t vo = (row * num_kv_heads + kvh) * dv;
                for (int a = 0; a < dk; ++a) kt[a] = in_value(k, in_dtype, ko + a);
                for (int c = 0; c < dv; ++c) vt[c] = in_value(v, in_dtype, vo + c);
                for (int c = 0; c < dv; ++c) dot[c] = in_value(d_o, in_dtype, (row * num_heads + h) * dv + c);
                for (int a = 0; a < dk; ++a)
                    for (int c = 0; c < dv; ++c)
                        S[(int64_t)a * dv + c] = lam * S[(int64_t)a * dv + c] + kt[a] * vt[c];
                for (int a = 0; a < dk; ++a) {
                    double acc = 0.0;
                    for (int c = 0; c < dv; ++c) acc += dot[c] * S[(int64_t)a * dv + c];
                    dq[(row * num_heads + h) * dk + a] = scale * acc;
                }
            }

            /* sweep 2, against the forward direction: D_t, dk_t, dv_t */
            for (int64_t i = 0; i < (int64_t)dk * dv; ++i) D[i] = d_final ? (double)d_final[st_base + i] : 0.0;
            for (int64_t step = 0; step < len; ++step) {
                const int64_t row = reverse ? row0 + step : row0 + len - 1 - step;
                const int64_t qo = (row * num_heads + h) * dk;
                const int64_t ko = (row * num_kv_heads + kvh) * dk;
                const int64_t vo = (row * num_kv_heads + kvh) * dv;
                for (int a = 0; a < dk; ++a) qt[a] = in_value(q, in_dtype, qo + a);
                for (int a = 0; a < dk; ++a) kt[a] = in_value(k, in_dtype, ko + a);
                for (int c = 0; c < dv; ++c) vt[c] = in_value(v, in_dtype, vo + c);
                for (int c = 0; c < dv; ++c) dot[c] = in_value(d_o, in_dtype, (row * num_heads + h) * dv + c);
                const double carry = step == 0 ? 1.0 : lam; /* d_final enters undecayed */
                for (int a = 0; a < dk; ++a)
                    for (int c = 0; c < dv; ++c)
                        D[(int64_t)a * dv + c] = carry * D[(int64_t)a * dv + c] + scale * qt[a] * dot[c];
                for (int a = 0; a < dk; ++a) {
                    double acc = 0.0;
                    for (int c = 0; c < dv; ++c) acc += D[(int64_t)a * dv + c] * vt[c];
                    dk_out[ko + a] += acc;
                }
                for (int c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int a = 0; a < dk; ++a) acc += kt[a] * D[(int64_t)a * dv + c];
                    dv_out[vo + c] += acc;
                }
            }
            if (d_init) {
                /* S_first = lam S_init + ..., so the state handed in receives lam D_first */
                for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
                    d_init[st_base + i] = (len > 0 ? lam * D[i] : (d_final ? (double)d_final[st_base + i] : 0.0));
            }
        }
        free(dot);
        free(vt);
        free(kt);
        free(qt);
        free(D);
        free(S);
    }
    return 0;
}

/*
 * Gated forward recurrence (recurrent page: the g, gk and gv gate arguments of
 * recurrent(), "GLA-style gating"; recurrent_gla page: the GLA wrapper passes g).
 * The pages give only the shapes of the gates and the update with a decay_t
 * factor; the reading taken here is that every gate is a log-decay like g_gamma,
 * acting on the state axis its last dimension names:
 *
 *     S_t[a][c] = exp(g_gamma[h] + g_t[a] + gk_t[a] + gv_t[c]) * S_{t-1}[a][c] + k_t[a] v_t[c]
 *     o_t       = scale * (q_t S_t)
 *
 * g and gk are [B, T, H, dk] (per query head and key channel), gv is [B, T, H, dv]
 * (per value channel); each may be NULL (zero).  They are stored in in_dtype, like
 * q, k and v; g_gamma [H] float32 may be NULL.  Everything else (GQA, reverse,
 * packed sequences, initial and final states) is as in oracle_recurrent_fwd.
 */
int oracle_recurrent_gated_fwd(int batch, int seqlen, int num_heads, int num_kv_heads,
                               int dk, int dv, int in_dtype,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* gk, const void* gv,
                               const float* g_gamma, double scale,
                               const float* initial_state, int reverse,
                               const int64_t* cu_seqlens, int num_seqs,
                               double* o, double* final_state) {
    if (batch <= 0 || seqlen < 0 || num_heads <= 0 || num_kv_heads <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (num_heads % num_kv_heads != 0) return -1;
    if (cu_seqlens != NULL && batch != 1) return -1;
    const int n_seq = cu_seqlens ? num_seqs : batch;
    const int group = num_heads / num_kv_heads;
    const int64_t n_pairs = (int64_t)n_seq * num_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pair = 0; pair < n_pairs; ++pair) {
        const int n = (int)(pair / num_heads);
        const int h = (int)(pair % num_heads);
        const int kvh = h / group;
        int64_t row0, len;
        if (cu_seqlens) {
            row0 = cu_seqlens[n];
            len = cu_seqlens[n + 1] - cu_seqlens[n];
        } else {
            row0 = (int64_t)n * seqlen;
            len = seqlen;
        }
        const double base = g_gamma ? (double)g_gamma[h] : 0.0;
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
        double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* la = (double*)malloc(sizeof(double) * (size_t)dk); /* log-decay per key channel */
        double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
        double* lb = (double*)malloc(sizeof(double) * (size_t)dv); /* log-decay per value channel */
        double* out_row = (double*)malloc(sizeof(double) * (size_t)dv);
        const int64_t st_base = ((int64_t)n * num_heads + h) * dk * dv;
        for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
            S[i] = initial_state ? (double)initial_state[st_base + i] : 0.0;

        for (int64_t step = 0; step < len; ++step) {
            const int64_t row = reverse ? row0 + len - 1 - step : row0 + step;
            const int64_t qo = (row * num_heads + h) * dk;
            const int64_t ko = (row * num_kv_heads + kvh) * dk;
            const int64_t vo = (row * num_kv_heads + kvh) * dv;
            const int64_t go = (row * num_heads + h) * dk;
            const int64_t gvo = (row * num_heads + h) * dv;
            for (int a = 0; a < dk; ++a) {
                qt[a] = in_value(q, in_dtype, qo + a);
                kt[a] = in_value(k, in_dtype, ko + a);
                la[a] = base + (g ? in_value(g, in_dtype, go + a) : 0.0) + (gk ? in_value(gk, in_dtype, go + a) : 0.0);
            }
            for (int c = 0; c < dv; ++c) {
                vt[c] = in_value(v, in_dtype, vo + c);
                lb[c] = gv ? in_value(gv, in_dtype, gvo + c) : 0.0;
            }
            /* S <- exp(la + lb) .* S + k_t^T v_t */
            for (int a = 0; a < dk; ++a)
                for (int c = 0; c < dv; ++c)
                    S[(int64_t)a * dv + c] = exp(la[a] + lb[c]) * S[(int64_t)a * dv + c] + kt[a] * vt[c];
            /* o_t = scale * (q_t S) */
            for (int c = 0; c < dv; ++c) out_row[c] = 0.0;
            for (int a = 0; a < dk; ++a)
                for (int c = 0; c < dv; ++c) out_row[c] += qt[a] * S[(int64_t)a * dv + c];
            for (int c = 0; c < dv; ++c) o[(row * num_heads + h) * dv + c] = scale * out_row[c];
        }
        for (int64_t i = 0; i < (int64_t)dk * dv; ++i) final_state[st_base + i] = S[i];
        free(out_row);
        free(lb);
        free(vt);
        free(la);
        free(kt);
        free(qt);
        free(S);
    }
    return 0;
}
