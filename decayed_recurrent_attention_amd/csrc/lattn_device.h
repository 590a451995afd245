// Device helpers shared by the kernel sources (not installed; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lattn_launch.h"

namespace lattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsBudget = 160 * 1024;

// One unit of work, decoded from the workgroup id.
struct Work {
    int n;          // sequence (batch row, packed sequence, or fixed-length segment)
    int h;          // query head
    int kvh;        // kv head read by h
    int vb;         // value block
    int64_t start;  // first token row of the work in the flattened [B*T] axis
    int64_t len;    // tokens in the work
    const float* init_blk;  // this head's initial state block [dk][dv], or null (zeros)
    float* fin_blk;         // where this head's final state block goes, or null (nowhere)
    // Split with the chain in the main pass: the initial state is lam^chain_len applied
    // to the state above plus the `chain` state blocks at chain_blk, chain_blk + H dk dv,
    // ... in turn.
    const float* chain_blk;
    int chain;
    int chain_len;
};

// Work id (normally the workgroup id) -> work.  Groups are (sequence rank, kv head); the workgroups of one
// group (its query heads x value blocks, which re-read the same K and V, and per
// head the same Q) get ids that are equal mod kNumXcd, so they share one L2.
// Consecutive groups go to consecutive dies; with sequences ranked longest first,
// each die receives its longest work first.
__device__ inline bool decode_work(const FwdParams& p, int id, Work& w) {
    const int x = id % kNumXcd;
    const int slot = id / kNumXcd;
    const int g = (slot / p.group_size) * kNumXcd + x;
    if (g >= p.num_groups) return false;
    const int j = slot % p.group_size;
    const int rank = g / p.num_kv_heads;
    w.kvh = g % p.num_kv_heads;
    w.h = w.kvh * (p.num_heads / p.num_kv_heads) + j / p.nvb;
    w.vb = j % p.nvb;
    const int H = p.num_heads;
    const int64_t blk = (int64_t)p.dk * p.dv;  // elements of one head's state block
    w.chain_blk = nullptr;
    w.chain = 0;
    w.chain_len = 0;
    if (p.plan) {  // packed split: the plan's entry of this rank
        const int count = p.plan[p.seg_phase == 1 ? 1 : 0];
        if (rank >= count) return false;
        const int32_t* e = p.plan + kPlanHeader + kPlanEntry * (p.seg_phase == 1 ? p.plan_main + rank : rank);
        w.n = e[2];
        w.start = e[0];
        w.len = e[1];
        if (p.seg_phase == 1) {
            w.init_blk = nullptr;
            w.fin_blk = p.slots + ((int64_t)e[7] * H + w.h) * blk;
        } else {
            w.init_blk = p.init ? p.init + ((int64_t)w.n * H + w.h) * blk : nullptr;
            w.fin_blk = (e[5] && p.final_state) ? p.final_state + ((int64_t)w.n * H + w.h) * blk : nullptr;
            if (e[3] >= 0 && e[4] > 0) {
                w.chain_blk = p.slots + ((int64_t)e[3] * H + w.h) * blk;
                w.chain = e[4];
                w.chain_len = e[6];
            }
        }
        return true;
    }
    if (p.seg_count > 0) {  // fixed length: segments of seg_len tokens, in processing order
        const int P = p.seg_count;
        const int per = p.seg_phase == 1 ? P - 1 : P;  // the state-only pass skips the last
        const int b = rank / per, k = rank % per;
        const int64_t a = (int64_t)k * p.seg_len;
        const int64_t e = min(a + p.seg_len, (int64_t)p.seqlen);
        const int64_t seg_len = e > a ? e - a : 0;
        // reverse: segment k ends k * seg_len before the row's end
        w.start = (int64_t)b * p.seqlen + (p.reverse ? (int64_t)p.seqlen - a - seg_len : a);
        w.len = seg_len;
        w.n = b;
        const int64_t slot0 = (int64_t)b * (P - 1);
        if (p.seg_phase == 1) {
            w.init_blk = nullptr;
            w.fin_blk = p.slots + ((slot0 + k) * H + w.h) * blk;
        } else {
            const float* row_init = p.init ? p.init + ((int64_t)b * H + w.h) * blk : nullptr;
            if (p.seg_chain) {  // the slots hold dS_0 .. dS_{P-2}: chain the earlier ones
                w.init_blk = row_init;
                if (k > 0) {
                    w.chain_blk = p.slots + (slot0 * H + w.h) * blk;
                    w.chain = k;
                    w.chain_len = p.seg_len;
                }
            } else {  // the scan left the state entering segment k in slot k - 1
                w.init_blk = k > 0 ? p.slots + ((slot0 + k - 1) * H + w.h) * blk : row_init;
            }
            w.fin_blk = (k == P - 1 && p.final_state) ? p.final_state + ((int64_t)b * H + w.h) * blk : nullptr;
        }
        return true;
    }
    w.n = p.order ? p.order[rank] : rank;
    if (p.cu) {
        int64_t a = p.cu[w.n];
        int64_t e = p.cu[w.n + 1];
        a = min(max(a, (int64_t)0), (int64_t)p.seqlen);
        e = min(max(e, a), (int64_t)p.seqlen);
        w.start = a;
        w.len = e - a;
    } else {
        w.start = (int64_t)w.n * p.seqlen;
        w.len = p.seqlen;
    }
    w.init_blk = p.init ? p.init + ((int64_t)w.n * H + w.h) * blk : nullptr;
    w.fin_blk = p.final_state ? p.final_state + ((int64_t)w.n * H + w.h) * blk : nullptr;
    return true;
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline float bf16_half(uint32_t w, int hi) { return hi ? bf16_hi(w) : bf16_lo(w); }
__device__ inline uint32_t half16(uint32_t w, int hi) { return hi ? (w >> 16) : (w & 0xffffu); }

// ---------------------------------------------------------------------------
// Direct global -> LDS copies (buffer_load_dwordx4 ... lds).  One instruction moves
// 16 bytes per lane to LDS address M0 + 16 * lane, so a wave fills one contiguous
// kilobyte while each lane picks its own source.  The copies are issued from
// inline assembly: the compiler would otherwise make every later LDS access wait
// for all of them.  Their completion is awaited explicitly (vmcnt) before the
// barrier that publishes a stage, and every barrier in the chunk loop waits for
// LDS operations only.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferDword3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

struct RawBuf {
    i32x4 d;  // raw buffer descriptor (base, stride 0, size in bytes, gfx9 raw format)
};
__device__ inline RawBuf raw_buf(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    RawBuf r;
    r.d = i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, kRawBufferDword3};
    return r;
}
__device__ inline uint32_t lds_addr(const void* p) {
    typedef __attribute__((address_space(3))) const void* lds_ptr;
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)p);
}
__device__ inline void copy16_to_lds(uint32_t lds_base, const RawBuf& r, int voffset) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voffset), "s"(r.d)
                 : "memory", "m0");
}
template <int N>
__device__ inline void wait_vmem() {  // at most N vector-memory operations outstanding
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane s
// supplies the address of four consecutive 16-bit elements; lane i receives
// element (i & 3) of the piece addressed by lane 4e + (i >> 2), as its element e.
// With lane s pointing at row (r0 + (s >> 2)), columns c(s & 3) .. c(s & 3) + 3 of
// a row-major tile, lane i therefore receives column c(i >> 2) + (i & 3) of rows
// r0 .. r0 + 3: one column per lane, four consecutive rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x2 lds_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}
__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ inline T lds_load(const void* p) {
    return *reinterpret_cast<const T*>(p);
}
template <typename T>
__device__ inline void lds_store(void* p, T v) {
    *reinterpret_cast<T*>(p) = v;
}

__device__ inline void lds_barrier() {  // this wave's LDS accesses done, then workgroup barrier
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Workgroups for a grid-stride streaming kernel over n4 16-byte pieces.
inline int stream_blocks(int64_t n4) {
    const int64_t b = (n4 + 255) / 256;
    return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace lattn
