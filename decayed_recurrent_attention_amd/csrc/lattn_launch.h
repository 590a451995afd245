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
};

// Workgroups of 64 * nw threads own BV = 16 * nw value columns each.
bool have_fwd_kernel(int in_dtype, int dk, int nw);
// Grid size for the decode used by the forward kernels.
int fwd_grid_size(const FwdParams& p);
// Enqueue the forward kernel; returns the HIP error of the launch.
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int nw, bool reverse, hipStream_t stream);
// Enqueue the longest-first ordering of packed sequences into `order`.
hipError_t launch_seq_order(const int32_t* cu, int num_seqs, int seqlen, int32_t* order,
                            hipStream_t stream);

}  // namespace lattn
