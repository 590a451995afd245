// Internal interface between the C ABI layer (lattn_api.cpp) and the HIP kernels
// (lattn_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lattn {

// Tokens per chunk of the chunked recurrence.
constexpr int kChunk = 64;
// Accelerator complex dies on MI355X; consecutive workgroup ids are dealt to them
// round-robin, so the work decode groups siblings by (id mod kNumXcd).
constexpr int kNumXcd = 8;
// Largest packed sequence count that the longest-first ordering kernel handles
// (its lengths live in LDS); above it sequences run in their given order.
constexpr int kMaxOrderedSeqs = 16384;
// Compute units of MI355X: the intra-sequence split balances its work over them.
constexpr int kNumCu = 256;
// Largest packed sequence count that the split planner handles (one workgroup, a
// thread per sequence, its tables in LDS), and the most segments it can list; above
// either, packed input is not split.
constexpr int kMaxPlanSeqs = 1024;
constexpr int kMaxPlanSegs = 2048;
// Packed-split plan in the workspace (int32 words): a header (main-pass count,
// state-only count), then the main pass's segments (longest first), then the
// state-only pass's segments.  An entry is kPlanEntry words:
//   [0] first row  [1] length  [2] sequence
//   [3] first state slot to chain into the initial state, or -1
//   [4] slots to chain (the segment's index k in its sequence)
//   [5] 1 if the segment writes the sequence's final state
//   [6] length of the sequence's full segments (tokens)
//   [7] state slot written by the state-only pass (state-only list)
constexpr int kPlanHeader = 8;
constexpr int kPlanEntry = 8;

// Everything one forward launch needs.  Sizes are element counts.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g_gamma;
    const float* init;      // [N_seq, H, dk, dv] or nullptr (zeros)
    const int32_t* cu;      // [N_seq + 1] or nullptr (fixed length)
    const int32_t* order;   // longest-first sequence order [N_seq] or nullptr (identity)
    float* o;
    float* final_state;
    int batch;
    int seqlen;
    int num_heads;
    int num_kv_heads;
    int dk;
    int dv;
    int num_seqs;     // sequences (= batch when fixed length)
    int nvb;          // dv / BV value blocks per head
    int num_groups;   // num_seqs * num_kv_heads
    int group_size;   // (num_heads / num_kv_heads) * nvb workgroups per group
    float scale;
    // Generalisations used by the gradient sweeps; the forward pass sets the
    // defaults noted on each field.
    int swap_heads;   // 1: q is read at kv head h / group and k, v at query head h (default 0)
    int64_t init_rs;  // element stride of a state row (dk index) inside one init block (default dv)
    int64_t init_cs;  // element stride of a state column (dv index) (default 1)
    float init_mul;   // init is multiplied by this when loaded (default 1)
    int init_at_end;  // 1: init already sits at the first processed position, so it
                      //    reaches that token undecayed (default 0: one decay step)
    float final_mul;  // final_state = final_mul * S (default 1) ...
    int final_lam;    // ... times exp(g_gamma[h]) when set and the sequence is not empty
                      //    (default 0); final_state may be null
    // Intra-sequence split (default 0 / null: off).  Segments are numbered in
    // processing order: segment k of a sequence of length L covers positions
    // [k * seg_len, min((k + 1) * seg_len, L)) forward, the mirror image in reverse,
    // so only the last processed segment can be short.  The state-only pass writes
    // segment k's own contribution dS_k (from a zero state) to state slot k of its
    // sequence (k < P - 1).  Fixed length with many segments: a scan then turns slot
    // k into the state entering segment k + 1, in place, and the main pass starts
    // segment k > 0 from slot k - 1.  Packed input, and fixed length with seg_chain
    // set: the main pass chains the slots itself: segment k starts from lam^seg_len
    // ... applied k times to the sequence's initial state plus dS_0 .. dS_{k-1}.
    // Segment 0 starts from the sequence's initial state, and the last segment writes
    // the final state.
    int seg_phase;    // 1: the state-only pass; 2: the main pass (with seg_count or plan)
    int seg_count;    // fixed length: P segments per batch row (every row alike)
    int seg_len;      // fixed length: segment length in tokens (a multiple of the chunk)
    int seg_chain;    // fixed length: 1 = the main pass chains the slots (no scan)
    const int32_t* plan;  // packed input: the plan (kPlanHeader ... above)
    int plan_main;        // capacity of the plan's main-pass list (entries)
    int plan_slots;       // capacity of its state-only list and of the state slots
    float* slots;         // state slots [slots][H][dk][dv]
    int o_bf16;       // 1: o holds bf16, each the round-to-nearest-even of the fp32 result
                      //    (bf16-input chunked kernel only; default 0: fp32)
    // Gated recurrence only (gated kernels): the key log-decay gate g [B, T, H, dk] and
    // the value gate gv [B, T, H, dv], in the input dtype (g in fp32 when gk_is_f32:
    // the sum of two key gates), or null.
    const void* g;
    const void* gv;
    int gk_is_f32;
    int reverse;  // 1: positions descending (the gated kernels and the fixed-length split read it)
};

// Kernel arguments of the forward kernels: one problem, or two of the same shape
// run by one launch (launch_fwd_pair).
struct FwdArgs {
    FwdParams p[2];
};

// Forward defaults of the fields above.
inline void set_forward_defaults(FwdParams& p) {
    p.swap_heads = 0;
    p.init_rs = p.dv;
    p.init_cs = 1;
    p.init_mul = 1.f;
    p.init_at_end = 0;
    p.final_mul = 1.f;
    p.final_lam = 0;
    p.seg_phase = 0;
    p.seg_count = 0;
    p.seg_len = 0;
    p.seg_chain = 0;
    p.plan = nullptr;
    p.plan_main = 0;
    p.plan_slots = 0;
    p.slots = nullptr;
    p.g = p.gv = nullptr;
    p.gk_is_f32 = 0;
    p.reverse = 0;
}

// Workgroups of 64 * nw threads own BV = 16 * nw value columns each.
bool have_fwd_kernel(int in_dtype, int dk, int nw);
// Grid size for the decode used by the forward kernels.
int fwd_grid_size(const FwdParams& p);
// Enqueue the forward kernel; returns the HIP error of the launch.  state_only (bf16
// only) runs just the state recurrence: final_state from K and V, no Q, no output.
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int nw, bool reverse, hipStream_t stream,
                      bool state_only = false);
// Two bf16 problems of the same shape (dims, work decode) in one launch; the work
// of a and b with the same id shares a die and runs together (the backward's dk and
// dv sweeps read the same Q and dO).
hipError_t launch_fwd_pair(const FwdParams& a, const FwdParams& b, int nw, bool reverse, hipStream_t stream);
// Gated recurrence (GLA gates), 64 * nw threads for BV = 16 * nw value columns.
bool have_gated_kernel(int dk, int nw);
// out = g + gk in fp32 (n elements, a multiple of 4; inputs in in_dtype).
hipError_t launch_gate_sum(const void* g, const void* gk, float* out, int64_t n, int in_dtype, hipStream_t stream);
hipError_t launch_gated(const FwdParams& p, int in_dtype, int nw, hipStream_t stream);
// Intra-sequence split of fixed-length input, chaining step: turn the state slots of
// B rows of P segments of seg_len tokens (row b's slots b * (P - 1) + k, each
// segment's own contribution) into the states entering the segments, in place; see
// seg_scan_kernel.
hipError_t launch_seg_scan(float* slots, const float* init, const float* g_gamma, int B, int H, int P, int seg_len,
                           int64_t elems, hipStream_t stream);
// Packed split plan: cut the sequences of cu_seqlens into segments (see
// split_plan_kernel) and write the plan.  wgs_per_seq: workgroups per segment;
// forced > 1: cut every sequence into that many segments (tests); else balance.
hipError_t launch_split_plan(const int32_t* cu, int num_seqs, int seqlen, int wgs_per_seq, int min_seg_chunks,
                             int forced, bool reverse, int max_main, int max_slots, int32_t* plan, hipStream_t stream);
// out[r, j, :] = sum over g < G of part[r, j * G + g, :] for rows r < rows, j < Hkv,
// with G = H / Hkv and d a multiple of 4.
hipError_t launch_group_sum(const float* part, float* out, int64_t rows, int H, int Hkv, int d,
                            hipStream_t stream);
// One decoding step over a batch of states (one new token per sequence).
struct DecodeParams {
    const void* q;         // [B, H, dk]   (in_dtype)
    const void* k;         // [B, Hkv, dk]
    const void* v;         // [B, Hkv, dv]
    const float* g_gamma;  // [H]
    const float* state_in; // [B, H, dk, dv] or nullptr (zeros); may equal state_out
    float* state_out;      // [B, H, dk, dv]
    float* o;              // [B, H, dv]
    int batch;
    int num_heads;
    int num_kv_heads;
    int dk;                // multiple of 16, at most 256
    int dv;                // multiple of 16, at most 256
    float scale;
};
// Value-block width (16, 32 or 64 columns) the decode kernel uses for dv.
int decode_block(int dv);
hipError_t launch_decode(const DecodeParams& p, int in_dtype, hipStream_t stream);

// Enqueue the longest-first ordering of packed sequences into `order`.
hipError_t launch_seq_order(const int32_t* cu, int num_seqs, int seqlen, int32_t* order,
                            hipStream_t stream);

}  // namespace lattn
