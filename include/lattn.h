/*
 * lattn — Lightning (decayed recurrent) attention, forward and backward, on AMD MI355X (gfx950).
 *
 * Public C ABI of liblattn.so.  Plain C types only: device buffers are passed as
 * untyped pointers, the HIP stream as `void*` (a hipStream_t; NULL = the default
 * stream).  No function allocates device memory, synchronises, or keeps a pointer
 * after it returns.  Every function is thread-safe.
 *
 * The operation (ejkernel "recurrent" interface page, docstring of recurrent():
 * "The core update is"; lightning_attn interface page for the argument meanings):
 * for each sequence n and query head h, with lam = exp(g_gamma[h]),
 *
 *     S_t = lam * S_{t-1} + k_t^T v_t        S_{-1} = initial_state[n, h] or 0
 *     o_t = scale * (q_t S_t)                final_state[n, h] = S after the last token
 *
 * where k_t, v_t are the rows of kv head h / (H / Hkv) (grouped-query attention).
 * With `reverse` the positions are visited from last to first (o_t stays at t).
 * With `cu_seqlens` the input is packed: sequence n is rows [cu[n], cu[n+1]) of a
 * batch-1 input and the state restarts at every boundary.
 */
#ifndef LATTN_H
#define LATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
    LATTN_BF16 = 0, /* bfloat16 words */
    LATTN_F32 = 1   /* IEEE float32 */
} lattn_dtype;

/* Status codes: 0 on success, negative on error.  Nothing is launched on error. */
enum {
    LATTN_OK = 0,
    LATTN_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, bad alignment */
    LATTN_ERR_VARLEN_BATCH = -2, /* cu_seqlens given with batch != 1 (lightning_attn page, Raises) */
    LATTN_ERR_HEADS = -3,        /* num_heads not a multiple of num_kv_heads */
    LATTN_ERR_UNSUPPORTED = -4,  /* head dims or dtypes without a compiled kernel */
    LATTN_ERR_WORKSPACE = -5,    /* workspace missing or smaller than lattn_fwd_workspace_size */
    LATTN_ERR_LAUNCH = -6,       /* the HIP runtime rejected a launch */
    LATTN_ERR_DEVICE = -7        /* no usable device, or the current device is not gfx950 */
};

/*
 * Problem description (shapes of the lightning_attn / recurrent signatures).
 *   q  [batch, seqlen, num_heads,    head_dim_qk]
 *   k  [batch, seqlen, num_kv_heads, head_dim_qk]
 *   v  [batch, seqlen, num_kv_heads, head_dim_v]
 *   o  [batch, seqlen, num_heads,    head_dim_v]           (out_dtype)
 *   initial_state / final_state [num_seqs, num_heads, head_dim_qk, head_dim_v] float32
 * All arrays are dense, row-major, in that axis order.
 */
typedef struct {
    int32_t batch;        /* B >= 1; must be 1 when cu_seqlens is given */
    int32_t seqlen;       /* T >= 0 tokens per batch row (total packed tokens when varlen) */
    int32_t num_heads;    /* H >= 1: query heads; o, g_gamma and the states use H */
    int32_t num_kv_heads; /* Hkv >= 1, H % Hkv == 0; head h reads kv head h / (H / Hkv) */
    int32_t head_dim_qk;  /* dk */
    int32_t head_dim_v;   /* dv */
    int32_t num_seqs;     /* packed sequences: > 0 exactly when cu_seqlens is given, else 0 (then N_seq = B) */
    int32_t in_dtype;     /* lattn_dtype of q, k, v: LATTN_BF16 or LATTN_F32 */
    int32_t out_dtype;    /* lattn_dtype of o: LATTN_F32, or LATTN_BF16 for lattn_fwd
                             with bf16 input (every other call takes LATTN_F32) */
} lattn_problem;

/*
 * Device workspace (bytes) that lattn_fwd needs for problem *p.  Sequences may be cut
 * into segments that run in parallel, chained through their states (a state-only
 * pass gives each segment's own contribution; the main pass, or a scan before it when
 * a row has more than sixteen segments, chains them), when that fills the GPU better:
 *  - fixed-length bf16 input with too few (batch row, head) pairs to fill the GPU:
 *    every row in P segments, one float32 state per segment but the last:
 *    B * (P - 1) * H * dk * dv * 4 bytes;
 *  - packed bf16 input (at most 1024 sequences, fewer than 256 workgroups per
 *    sequence): a plan made on the device from cu_seqlens cuts the sequences longer
 *    than the balanced load per compute unit; the workspace holds the plan and at
 *    most 2 * ceil(256 / J) + 2 float32 states per head (J = workgroups per segment).
 * Other packed input needs room for the longest-first sequence order; other
 * fixed-length input needs none.  The knob LATTN_KNOB_SPLIT (lattn_set_knob)
 * changes the segment count.  Returns 0 also for an invalid problem (lattn_fwd then
 * reports it).
 */
size_t lattn_fwd_workspace_size(const lattn_problem* p);

/*
 * Forward pass, enqueued on `stream`; returns without waiting for the GPU.
 *   q, k, v        device, in_dtype, 16-byte aligned, layout above.
 *   g_gamma        device float32 [H]: per-head log-decay, finite and <= 0.
 *   scale          multiplies q (so o), never the state.
 *   initial_state  device float32 [N_seq, H, dk, dv], or NULL for zeros.
 *   reverse        0: positions ascending; 1: descending.
 *   cu_seqlens     device int32 [N_seq + 1], or NULL.  Must start at 0, be
 *                  non-decreasing and end at seqlen; values outside [0, seqlen]
 *                  are clamped into it so that no access leaves the buffers.
 *   o              device output in out_dtype: float32, or (bf16 input only) bf16,
 *                  each element the round-to-nearest-even of the float32 result.
 *   final_state    device float32 output [N_seq, H, dk, dv].
 *   workspace      device buffer of >= lattn_fwd_workspace_size(p) bytes, 16-byte
 *                  aligned (may be NULL when that is 0).  Owned by the caller;
 *                  contents on entry are ignored; must not be shared by calls that
 *                  overlap in time.
 * Supported: in_dtype BF16 with dk in {32, 64, 128, 192, 256}; in_dtype F32 with
 * dk in {16, 32, 64, 128}; dv a multiple of 16 up to 256; out_dtype F32, or BF16
 * with in_dtype BF16 (o in the input dtype, half the output bytes; the state stays
 * float32); num_heads * max(dk, dv) * 256 < 2^31 (the kernels address the 64 rows
 * of a chunk with 32-bit byte offsets); else LATTN_ERR_UNSUPPORTED.
 * Returns LATTN_OK or a negative status; buffers are untouched on error.
 */
int lattn_fwd(const lattn_problem* p, const void* q, const void* k, const void* v,
              const float* g_gamma, float scale, const float* initial_state, int reverse,
              const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * lattn_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  The arguments
 * and results are those of lattn_fwd; the workspace comes from a device array that
 * the library owns, LATTN_NOALLOC_SCRATCH_BYTES (32 MiB) on each device it runs on,
 * held from the first call on that device until the process ends.  The call itself
 * allocates nothing.
 *   Limit: problems with lattn_fwd_workspace_size(p) > LATTN_NOALLOC_SCRATCH_BYTES are
 *          refused with LATTN_ERR_WORKSPACE before any device call (use lattn_fwd with
 *          a caller-owned workspace for them).
 *   Races: every call on one device uses the same array, so calls that may overlap in
 *          time on one device (other streams, other threads) must be serialized by the
 *          caller; calls on different devices are independent.
 * Returns LATTN_OK or a negative status as lattn_fwd does; LATTN_ERR_DEVICE if the
 * array's device address cannot be obtained.
 */
#define LATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int lattn_fwd_noalloc(const lattn_problem* p, const void* q, const void* k, const void* v,
                      const float* g_gamma, float scale, const float* initial_state, int reverse,
                      const int32_t* cu_seqlens, void* o, float* final_state, void* stream);

/*
 * Device workspace (bytes) that lattn_bwd needs for problem *p: room for the
 * per-query-head gradients before their sum into kv heads (num_heads >
 * num_kv_heads) and for the sequence order of packed input; 0 when neither
 * applies.  Returns 0 also for an invalid problem.
 */
size_t lattn_bwd_workspace_size(const lattn_problem* p);

/*
 * Backward pass, enqueued on `stream` (recurrent interface page, the custom-VJP
 * backward rule: from dO and d final_state to dq, dk, dv and d initial_state;
 * g_gamma is not differentiated, as in the lightning_attn wrapper).  With
 * lam = exp(g_gamma[h]) and D_t the gradient reaching S_t,
 *
 *     D_t  = scale q_t^T dO_t + lam D_{t+1}      (d_final_state enters at the last
 *                                                 position without decay)
 *     dq_t = scale dO_t S_t^T,   dk_t = D_t v_t,   dv_t = k_t D_t,
 *     d_initial_state = lam D_first,
 *
 * "first"/"last" in the direction of the forward pass; dk and dv of a kv head sum
 * over its query heads.  Computed as three chunked sweeps: dq in the forward
 * direction, dk and dv in the opposite one (bf16 with dk = dv and no grouped heads:
 * the dk and dv sweeps share one launch; the knob LATTN_KNOB_BWD_PAIR = 0 keeps them
 * apart).
 *   q, k, v, g_gamma, scale, initial_state, reverse, cu_seqlens: as for lattn_fwd
 *                  (the forward inputs; initial_state may be NULL).  scale must be a
 *                  finite normal float (the sweeps carry D / scale).
 *   d_o            device [B, T, H, dv] in in_dtype (like q, k, v), 16-byte aligned:
 *                  the gradient of o.  A caller holding an fp32 gradient of a bf16
 *                  problem rounds it first; the sweeps compute on bf16 operands.
 *   d_final_state  device float32 [N_seq, H, dk, dv] or NULL (zeros).
 *   dq             device float32 [B, T, H, dk]   (written)
 *   dk, dv         device float32 [B, T, Hkv, dk], [B, T, Hkv, dv]   (written)
 *   d_initial_state device float32 [N_seq, H, dk, dv] or NULL (not computed).
 *   workspace      device buffer of >= lattn_bwd_workspace_size(p) bytes, 16-byte
 *                  aligned, owned by the caller; must not be shared by calls that
 *                  overlap in time.
 * Rows of packed input outside every sequence are unspecified in dq, dk and dv.
 * Supported: every problem lattn_fwd supports whose transposed head dims
 * (dk' = dv, dv' = dk) it also supports.  Returns LATTN_OK or a negative status;
 * nothing is launched on error.
 */
int lattn_bwd(const lattn_problem* p, const void* q, const void* k, const void* v,
              const float* g_gamma, float scale, const float* initial_state, int reverse,
              const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, float* dq,
              float* dk, float* dv, float* d_initial_state, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * Forward pass with per-token log-decay gates (recurrent interface page: the g, gk
 * and gv arguments, "GLA-style gating"; the recurrent_gla page passes g).  Every gate
 * is a log-decay on the state axis its last dimension names:
 *
 *     S_t[a][c] = exp(g_gamma[h] + g_t[a] + gk_t[a] + gv_t[c]) * S_{t-1}[a][c] + k_t[a] v_t[c]
 *     o_t       = scale * (q_t S_t)
 *
 *   g, gk          device [B, T, H, dk] in in_dtype (per query head and key channel), or NULL.
 *   gv             device [B, T, H, dv] in in_dtype (per value channel), or NULL.
 *   g_gamma        device float32 [H] or NULL (zeros).  All gates must be finite and <= 0.
 *   the rest       as for lattn_fwd (GQA, reverse, packed input, states).
 * Chunks of 16 tokens; fp32 inputs are computed in fp32 (fp32 MFMA), bf16 inputs on
 * bf16 MFMA with every decayed operand split into bf16 hi + lo parts (fp32
 * accumulation; about 1e-4 relative to the output RMS).  Supported: in_dtype BF16 or
 * F32, dk in {32, 64, 128}, dv a multiple of 16 up to 256, out_dtype F32, and
 * H * max(dk, dv) < 2^25.  Workspace:
 * lattn_fwd_gated_workspace_size(p, gates) with gates the LATTN_GATE_* bits of the
 * gates that will be passed: the sequence order of packed input, and an fp32
 * [B, T, H, dk] sum when both g and gk are given; else 0.
 * Returns LATTN_OK or a negative status; nothing is launched on error.
 */
enum { LATTN_GATE_G = 1, LATTN_GATE_GK = 2, LATTN_GATE_GV = 4 };
size_t lattn_fwd_gated_workspace_size(const lattn_problem* p, int gates);
int lattn_fwd_gated(const lattn_problem* p, const void* q, const void* k, const void* v, const void* g,
                    const void* gk, const void* gv, const float* g_gamma, float scale,
                    const float* initial_state, int reverse, const int32_t* cu_seqlens, void* o,
                    float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decoding step for a batch of sequences: the recurrence of lattn_fwd advanced
 * by one new token per sequence (the GLA interface page notes that the recurrent
 * form suits autoregressive decoding).  For every batch row n and query head h,
 *
 *     state[n, h] <- lam * state[n, h] + k_n^T v_n,    o[n, h] = scale * (q_n state[n, h]),
 *
 * i.e. lattn_fwd with seqlen 1, initial_state = state_in and final_state = state_out.
 *   p              seqlen must be 1 and num_seqs 0; batch = number of sequences; dk and
 *                  dv multiples of 16 up to 256; in_dtype BF16 or F32; out_dtype F32.
 *   q, k, v        device [B, 1, H|Hkv, dk|dv] in in_dtype, 16-byte aligned.
 *   state_in       device float32 [B, H, dk, dv], or NULL for zeros (a first token).
 *   state_out      device float32 [B, H, dk, dv]; may be state_in (update in place).
 *   o              device float32 [B, 1, H, dv].
 * Returns LATTN_OK or a negative status; nothing is launched on error.
 */
int lattn_decode(const lattn_problem* p, const void* q, const void* k, const void* v,
                 const float* g_gamma, float scale, const float* state_in, float* state_out, void* o,
                 void* stream);

/*
 * Lightning decay schedule (lightning_attn interface page, module docstring "Key
 * innovation" and wrapper body): out_host[h] = -(8/H) * (1 - layer_idx/num_layers) * h,
 * coefficient computed in double, rounded to float32, then multiplied by the
 * float32 head index in float32.  out_host is host memory of num_heads floats.
 * Returns LATTN_OK, or LATTN_ERR_INVALID_ARG (num_heads < 1, num_layers < 1,
 * layer_idx outside [0, num_layers], out_host NULL).
 */
int lattn_lightning_g_gamma(int num_heads, int layer_idx, int num_layers, float* out_host);

/* Static description of a status code (never NULL). */
const char* lattn_status_string(int status);

/*
 * Testing and measurement hook: force a kernel choice that the library otherwise
 * makes from the problem's shape.  The setting is process-wide (every thread and
 * device) and stays until changed; the results of every choice meet the same
 * tolerance, only the summation order and the speed differ.  It exists so that
 * tests can reach every kernel variant on small problems and so that the speed of
 * one variant can be measured against another; production code leaves every knob at
 * LATTN_KNOB_AUTO.  Set a knob only while no call that reads it is being made, and
 * query workspace sizes after setting it (the split changes them).
 *   which     one of the LATTN_KNOB_* values below
 *   value     LATTN_KNOB_AUTO, or the forced value (>= 0) described there
 *   previous  host int receiving the knob's previous value, or NULL
 * Returns LATTN_OK, or LATTN_ERR_INVALID_ARG for an unknown knob or a negative value
 * other than LATTN_KNOB_AUTO.  Forced values that the problem cannot use (a width
 * that does not divide dv, say) fall back to the automatic choice.
 */
enum {
    LATTN_KNOB_AUTO = -1,
    LATTN_KNOB_WAVES = 0,    /* waves per value block of lattn_fwd / lattn_bwd: 1, 2 or 4 */
    LATTN_KNOB_SPLIT = 1,    /* lattn_fwd: segments per sequence; 0 or 1 = never split */
    LATTN_KNOB_BWD_PAIR = 2  /* lattn_bwd: 0 = the dk and dv sweeps as two launches */
};
int lattn_set_knob(int which, int value, int* previous);

/* ABI version of this header: 5 (1 had no backward, 2 no decoding step, 3 no gates,
   4 no knobs). */
int lattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LATTN_H */
