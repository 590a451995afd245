// Chunked forward kernels for Lightning (decayed recurrent) attention on gfx950.
//
// The recurrence (ejkernel "recurrent" interface page, docstring "The core update
// is"), per sequence and query head with lam = exp(g):
//     S_t = lam S_{t-1} + k_t^T v_t,      o_t = scale * q_t S_t.
// Unrolled over a chunk of C tokens with local rows i, j = 0..Lc-1 and S the state
// entering the chunk, it is exactly
//     O   = scale * [ ((Q K^T) .* M) V  +  diag(lam^(i+1)) (Q S) ],  M_ij = lam^(i-j) (j <= i)
//     S'  = lam^Lc S + (diag(lam^(Lc-1-j)) K)^T V.
// The intra-chunk term and both state products are dense contractions and run on
// MFMA; only non-negative powers of lam are ever formed, so fast decays underflow
// to zero instead of overflowing, and lam = 1 (g = 0, no decay) is exact.
//
// Work decomposition: one workgroup per (sequence, query head, block of BV = 16*NW
// value columns).  Value columns are independent (column c of S only sees column c
// of V), so the state block S[:, BV] lives in MFMA accumulator registers for the
// whole sequence: wave w owns columns [16w, 16w+16).  Each chunk of Q, K, V is
// staged through LDS: Q and K row-major for the QK^T and Q S products, K
// (pre-multiplied by its decay) and V transposed, so the token index is contiguous
// for the products that contract over tokens.  Global loads of chunk c+1 are in
// flight while chunk c is computed.
//
// Two layout facts of the 16x16 MFMA shapes make accumulators reusable as
// operands without an LDS round trip: an output tile gives lane l column l%16 and
// rows 4*(l/16)+{0..3}, while an A (B) operand gives lane l row (column) l%16 and
// eight k values that only have to be paired the same way in A and B.  Hence
//   * the state tile pair (2kb, 2kb+1), converted to bf16 hi + lo, is directly the
//     B operand of Q S for dk block kb, provided the state's dk rows are mapped by
//     dmap() below so that they line up with Q's natural 8 consecutive dk values;
//   * a (K Q^T) output tile pair, masked and converted, is directly the A operand
//     of P V, with V read in the matching token order.
// The state is kept in fp32 and fed to the Q S product as bf16 hi + lo (two MFMAs),
// and so is the masked intra-chunk matrix P in P V, so that neither rounding reaches
// the output; o and the states are fp32.
#include <type_traits>

#include "lattn_launch.h"

namespace lattn {
namespace {

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
    int n;          // sequence (batch row, or packed sequence)
    int h;          // query head
    int kvh;        // kv head read by h
    int vb;         // value block
    int64_t start;  // first token row of the sequence in the flattened [B*T] axis
    int64_t len;    // tokens in the sequence
};

// Workgroup id -> work.  Groups are (sequence rank, kv head); the workgroups of one
// group (its query heads x value blocks, which re-read the same K and V, and per
// head the same Q) get ids that are equal mod kNumXcd, so they share one L2.
// Consecutive groups go to consecutive dies; with sequences ranked longest first,
// each die receives its longest work first.
__device__ inline bool decode_work(const FwdParams& p, Work& w) {
    const int id = blockIdx.x;
    const int x = id % kNumXcd;
    const int slot = id / kNumXcd;
    const int g = (slot / p.group_size) * kNumXcd + x;
    if (g >= p.num_groups) return false;
    const int j = slot % p.group_size;
    const int rank = g / p.num_kv_heads;
    w.kvh = g % p.num_kv_heads;
    w.n = p.order ? p.order[rank] : rank;
    w.h = w.kvh * (p.num_heads / p.num_kv_heads) + j / p.nvb;
    w.vb = j % p.nvb;
    if (p.seg_count > 0) {  // sequence n = segment n % seg_count of batch row n / seg_count
        const int b = w.n / p.seg_count, sg = w.n % p.seg_count;
        const int64_t a = (int64_t)sg * p.seg_len;
        const int64_t e = min(a + p.seg_len, (int64_t)p.seqlen);
        w.start = (int64_t)b * p.seqlen + a;
        w.len = e > a ? e - a : 0;
    } else if (p.cu) {
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

// Index of (K Q^T) tile (a, b), a <= b, among the 10 lower-triangle tiles of a chunk.
__host__ __device__ constexpr int tidx(int a, int b) { return b * (b + 1) / 2 + a; }
__host__ __device__ constexpr int tile_b(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }

// dk index of row m of state tile mt (bf16 path): tiles 2kb and 2kb+1 interleave in
// groups of four so that lane group g of the tile pair holds dk 32kb + 8g + 0..7.
__host__ __device__ constexpr int dmap(int mt, int m) {
    return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

// Per-lane decay factors that do not depend on the chunk: the causal mask of the
// ten (K Q^T) tiles and lam^(i+1) for this lane's output rows.
struct LaneDecay {
    float mask[10][4];
    float lamq[4][4];
};

__device__ inline void make_lane_decay(float g2, int lr, int lg, LaneDecay& d) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int a = 0; a <= b; ++a) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int j = 16 * a + 4 * lg + ii;
                const int i = 16 * b + lr;
                d.mask[tidx(a, b)][ii] = (j <= i) ? exp2f(g2 * (float)(i - j)) : 0.f;
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) d.lamq[b][ii] = exp2f(g2 * (float)(16 * b + 4 * lg + ii + 1));
    }
}

// ---------------------------------------------------------------------------
// Global memory through raw buffer descriptors.  A descriptor covers exactly the
// valid token rows of one chunk, so out-of-range loads return zero and
// out-of-range stores are dropped by the hardware: partial chunks and the rows of
// neighbouring packed sequences need no branches.  Offsets stay 32-bit because
// every descriptor is rebased at its chunk.
// ---------------------------------------------------------------------------
constexpr int kRawBufferDword3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferDword3);
}
__device__ inline u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float buf_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void buf_store_f32(float v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
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
__device__ inline bf16x8 cat_bf16(u32x2 a, u32x2 b) {
    const u32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
}

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
__device__ inline void lds_barrier() {  // this wave's LDS accesses done, then workgroup barrier
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// ---------------------------------------------------------------------------
// bf16 inputs: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
// ---------------------------------------------------------------------------
// XOR swizzles of the 16-byte blocks of a row (rows are unpadded), chosen with the
// measured gfx950 bank behaviour (a half-wave's 16-byte reads conflict-free when
// their blocks differ mod 32; 8-byte reads when their 8-byte slots differ mod 32):
// Q/K rows serve 16-byte operand reads conflict-free and the transposing K^T reads
// at the two-way floor; V rows serve both transposing read patterns conflict-free.
template <int PP>
__host__ __device__ constexpr int qk_swz(int r) {
    if constexpr (PP == 4) return ((r >> 3) & 1) << 1;
    else if constexpr (PP == 8) return (r & 1) ^ ((r >> 1) & 7);
    else if constexpr (PP == 16) return ((r & 1) << 2) ^ (r & 15);
    else if constexpr (PP == 24) return (r >> 1) & 7;
    else return ((r & 1) << 3) ^ ((r & 15) << 1);
}
template <int PVB>
__host__ __device__ constexpr int v_swz(int r) {
    if constexpr (PVB == 8) return (r & 7) ^ ((r >> 1) & 7);
    else if constexpr (PVB == 4) return ((r >> 1) & 3) ^ ((r >> 2) & 3);
    else return 0;
}

template <int DK, int NW>
struct Bf16Cfg {
    static constexpr int BV = 16 * NW;
    static constexpr int PP = DK / 8;    // 16-byte blocks per Q / K row
    static constexpr int PVB = BV / 8;   // 16-byte blocks per V row (this value block)
    static constexpr int Q_BYTES = kChunk * DK * 2;
    static constexpr int V_BYTES = kChunk * BV * 2;
    static constexpr int STAGE_BYTES = 2 * Q_BYTES + V_BYTES;
    // Masked intra-chunk matrix P, exchanged between waves in MFMA A-operand layout:
    // 6 operand blocks (row tile b, token block kb) x {hi, lo} x 64 lanes x 16 bytes.
    static constexpr int P_BYTES = 6 * 2 * 64 * 16;
    static constexpr int FIT = (kLdsBudget - P_BYTES) / STAGE_BYTES;
    static constexpr int STAGES = FIT >= 3 ? 3 : FIT;  // ring of chunk stages
    static constexpr int DEPTH = STAGES - 1;           // chunks copied ahead of the one computed
    static constexpr int QCOPIES = PP / NW;            // copy instructions per wave per Q (or K) tile
    static constexpr int VCOPIES = PVB / NW;           // ... per V tile
    static constexpr int NCOPY = 2 * QCOPIES + VCOPIES;
    static constexpr int NSTORE = 16;                  // output stores per wave per chunk
    static constexpr int KB = DK / 32;                 // dk blocks of one MFMA
    static constexpr int MT = DK / 16;                 // state row tiles
    static_assert(DK % 32 == 0 && DK <= 256, "dk must be a multiple of 32 up to 256");
    static_assert(STAGES >= 2, "need at least two stages");
    static_assert(PP % NW == 0 && PVB % NW == 0, "copies divide evenly between waves");
    static_assert(STAGES * STAGE_BYTES + P_BYTES <= kLdsBudget, "LDS budget");
};

// Operand block of P for row tile b and token block kb (2kb <= b): 0..5.
__host__ __device__ constexpr int pidx(int b, int kb) { return b < 2 ? b : 2 + 2 * (b - 2) + kb; }
// Column tile a of lower-triangle (K Q^T) tile t = tidx(a, b).
__host__ __device__ constexpr int tile_a(int t) { return t - tile_b(t) * (tile_b(t) + 1) / 2; }

template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int KB>
__device__ inline void split_state(const f32x4* S, bf16x8* hi, bf16x8* lo) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const float s[8] = {S[2 * kb][0],     S[2 * kb][1],     S[2 * kb][2],     S[2 * kb][3],
                            S[2 * kb + 1][0], S[2 * kb + 1][1], S[2 * kb + 1][2], S[2 * kb + 1][3]};
        u32x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = pack_bf16x2(s[2 * e], s[2 * e + 1]);
            h[e] = w;
            l[e] = pack_bf16x2(s[2 * e] - bf16_lo(w), s[2 * e + 1] - bf16_hi(w));
        }
        hi[kb] = __builtin_bit_cast(bf16x8, h);
        lo[kb] = __builtin_bit_cast(bf16x8, l);
    }
}

// SONLY: only the state recurrence (no Q, no output): the final state of every
// sequence from K and V alone.
template <int DK, int NW, bool REV, bool SONLY>
__global__ __launch_bounds__(64 * NW, 1) void fwd_bf16_kernel(const FwdParams p) {
    using Cfg = Bf16Cfg<DK, NW>;
    constexpr int BV = Cfg::BV, PP = Cfg::PP, PVB = Cfg::PVB, KB = Cfg::KB, MT = Cfg::MT;
    constexpr int NST = Cfg::STAGES, DEPTH = Cfg::DEPTH;
    constexpr int QROW = DK * 2, VROW = BV * 2;  // LDS row bytes
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * Cfg::STAGE_BYTES + Cfg::P_BYTES];
    uint8_t* Pbuf = smem + NST * Cfg::STAGE_BYTES;

    Work wk;
    if (!decode_work(p, wk)) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const float g2 = p.g_gamma[wk.h] * kLog2e;  // log2 of the per-step decay
    const int L = (int)wk.len;
    const int nch = (L + kChunk - 1) / kChunk;
    const int H = p.num_heads, dv = p.dv;
    const int col = 16 * wv + lr;  // this lane's value column inside the block
    // Operand heads: q at h and k, v at the kv head, or the other way round.
    const int qh = p.swap_heads ? wk.kvh : wk.h, kh = p.swap_heads ? wk.h : wk.kvh;
    const int QH = p.swap_heads ? p.num_kv_heads : H, KH = p.swap_heads ? H : p.num_kv_heads;
    const uint32_t qrow_b = (uint32_t)QH * DK * 2, krow_b = (uint32_t)KH * DK * 2;
    const uint32_t vrow_b = (uint32_t)KH * dv * 2, orow_b = (uint32_t)H * dv * 4;
    const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)qh * DK;
    const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)kh * DK;
    const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)kh * dv + wk.vb * BV;
    const uint32_t smem_base = lds_addr(smem);

    // Tiles (1, 0) and (3, 2) lie above the diagonal: their halves of P stay zero.
    if (tid < 64) {
        const u32x2 z2 = {0u, 0u};
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
            lds_store<u32x2>(Pbuf + ((pidx(0, 0) * 2 + hl) * 64 + tid) * 16 + 8, z2);
            lds_store<u32x2>(Pbuf + ((pidx(2, 1) * 2 + hl) * 64 + tid) * 16 + 8, z2);
        }
    }

    // Decay factors, all with non-negative exponents and with `scale` folded in.
    // Mask of (K Q^T) tile (a, b): diagonal tiles use dg[ii] = lam^(lr - 4lg - ii)
    // (0 above the diagonal); tile b - a = d > 0 uses od[d-1][ii] = lam^(16d + lr - 4lg - ii).
    const float sc = p.scale;
    float dg[4], od[3][4], lamq[4][4], vw[2][8];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int e = lr - 4 * lg - ii;
        dg[ii] = e >= 0 ? sc * exp2f(g2 * (float)e) : 0.f;
#pragma unroll
        for (int d = 1; d <= 3; ++d) od[d - 1][ii] = sc * exp2f(g2 * (float)(16 * d + e));
#pragma unroll
        for (int b = 0; b < 4; ++b) lamq[b][ii] = sc * exp2f(g2 * (float)(16 * b + 4 * lg + ii + 1));
    }
    // Decay of value token j = 32kb + 8lg + e to the end of a full chunk: lam^(C-1-j).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) vw[kb][e] = exp2f(g2 * (float)(kChunk - 1 - (32 * kb + 8 * lg + e)));
    const float lamC = exp2f(g2 * (float)kChunk);

    // State block: tile mt holds rows dmap(mt, 4*lg + ii) at column `col`.
    f32x4 S[MT];
    const int64_t st_blk = ((int64_t)wk.n * H + wk.h) * DK * dv;  // this head's state block
    const int64_t st_off = st_blk + (int64_t)wk.vb * BV;
    {
        // Without an initial state the descriptor is empty and every load returns 0.
        const auto ri = make_rsrc(p.init ? p.init + st_blk : p.g_gamma, p.init ? (uint32_t)(DK * dv * 4) : 0u);
        const int rs = (int)p.init_rs, cs = (int)p.init_cs, gcol = wk.vb * BV + col;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[mt][ii] = p.init_mul * buf_load_f32(ri, (dmap(mt, 4 * lg + ii) * rs + gcol * cs) * 4);
    }
    bf16x8 Shi[KB], Slo[KB];
    split_state<KB>(S, Shi, Slo);

    auto first_row = [&](int p0, int Lc) -> int64_t { return REV ? wk.start + L - p0 - Lc : wk.start + p0; };
    auto qk_off = [](int row, int blk) { return row * QROW + 16 * (blk ^ qk_swz<PP>(row)); };
    auto v_off = [](int row, int blk) { return row * VROW + 16 * (blk ^ v_swz<PVB>(row)); };

    // Copy chunk c into stage c % NST.  Past the last chunk the descriptors are
    // empty, so the copies only write zeros (keeping the per-chunk operation count
    // fixed for the waits below) into the stage the previous chunk used.
    auto issue_chunk = [&](int c) {
        const uint32_t stage = smem_base + (uint32_t)((c % NST) * Cfg::STAGE_BYTES);
        const int p0 = c * kChunk;
        const bool real = c < nch;
        const int Lc = real ? min(kChunk, L - p0) : 1;
        const int64_t r0 = real ? first_row(p0, Lc) : 0;
        const RawBuf rq = raw_buf(qg + r0 * QH * DK, real ? (uint32_t)(Lc - 1) * qrow_b + DK * 2 : 0u);
        const RawBuf rk = raw_buf(kg + r0 * KH * DK, real ? (uint32_t)(Lc - 1) * krow_b + DK * 2 : 0u);
        const RawBuf rv = raw_buf(vg + r0 * KH * dv, real ? (uint32_t)(Lc - 1) * vrow_b + BV * 2 : 0u);
#pragma unroll
        for (int j = 0; j < Cfg::QCOPIES; ++j) {
            const int kbyte = j * NW + wv;  // this wave's kilobyte of the tile
            const int B = kbyte * 64 + lane, row = B / PP;
            const int blk = (B % PP) ^ qk_swz<PP>(row);
            const int rs = REV ? Lc - 1 - row : row;  // out of range past the end
            if constexpr (!SONLY) copy16_to_lds(stage + kbyte * 1024, rq, rs * (int)qrow_b + blk * 16);
            copy16_to_lds(stage + Cfg::Q_BYTES + kbyte * 1024, rk, rs * (int)krow_b + blk * 16);
        }
#pragma unroll
        for (int j = 0; j < Cfg::VCOPIES; ++j) {
            const int kbyte = j * NW + wv;
            const int B = kbyte * 64 + lane, row = B / PVB;
            const int blk = (B % PVB) ^ v_swz<PVB>(row);
            const int rs = REV ? Lc - 1 - row : row;
            copy16_to_lds(stage + 2 * Cfg::Q_BYTES + kbyte * 1024, rv, rs * (int)vrow_b + blk * 16);
        }
    };
    // Wait until this wave's copies of chunk c are in LDS.  Issued after them, in
    // order: the copies of DEPTH-1 later chunks and the output stores of the
    // min(c, DEPTH) chunks computed since.
    constexpr int NCOPY = SONLY ? Cfg::QCOPIES + Cfg::VCOPIES : Cfg::NCOPY;
    constexpr int NSTORE = SONLY ? 0 : Cfg::NSTORE;
    constexpr int W0 = (DEPTH - 1) * NCOPY;
    constexpr int WC = W0 + DEPTH * NSTORE;
    auto wait_chunk = [&](int c) {
        if (c >= DEPTH) {
            wait_vmem<(WC < 63 ? WC : 63)>();
        } else if (c == 0) {
            wait_vmem<(W0 < 63 ? W0 : 63)>();
        } else {
            constexpr int W1 = W0 + NSTORE;
            wait_vmem<(W1 < 63 ? W1 : 63)>();
        }
    };

    auto compute_chunk = [&](int c, const uint8_t* st) {
        const uint8_t* Qs = st;
        const uint8_t* Ks = st + Cfg::Q_BYTES;
        const uint8_t* Vs = st + 2 * Cfg::Q_BYTES;
        const int p0 = c * kChunk, Lc = min(kChunk, L - p0);
        const int vblk = 2 * wv + ((lr & 3) >> 1), vhalf = 8 * (lr & 1);  // this lane's V piece

        // S <- lam^Lc S + K^T (decayed V).  Operands by transposing reads: lane group
        // lg takes tokens 32kb + 8lg + 0..7; the A operand row of lane lr is dk
        // dmap(mt, lr); the B operand (column `col`) is decayed in registers.
        // A state handed in at the first processed position (gradient sweeps) reaches
        // the first chunk one decay step less far.
        const bool at_end = p.init_at_end && c == 0;
        float lamL = at_end ? exp2f(g2 * (float)(Lc - 1)) : lamC;
        if (Lc != kChunk) {  // the last chunk of a sequence: decays to its own end
            lamL = exp2f(g2 * (float)(at_end ? Lc - 1 : Lc));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * kb + 8 * lg + e;
                    vw[kb][e] = j < Lc ? exp2f(g2 * (float)(Lc - 1 - j)) : 0.f;
                }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) S[mt] *= lamL;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int jr = 32 * kb + 8 * lg + (lr >> 2);  // token row this lane addresses
            u32x4 vw4 = __builtin_bit_cast(u32x4, cat_bf16(lds_tr16((const uint16_t*)(Vs + v_off(jr, vblk) + vhalf)),
                                                         lds_tr16((const uint16_t*)(Vs + v_off(jr + 4, vblk) + vhalf))));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                vw4[e] = pack_bf16x2(bf16_lo(vw4[e]) * vw[kb][2 * e], bf16_hi(vw4[e]) * vw[kb][2 * e + 1]);
            const bf16x8 vop = __builtin_bit_cast(bf16x8, vw4);
            bf16x8 kop[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int kblk = 4 * (mt >> 1) + (lr & 3), khalf = 8 * (mt & 1);
                kop[mt] = cat_bf16(lds_tr16((const uint16_t*)(Ks + qk_off(jr, kblk) + khalf)),
                                   lds_tr16((const uint16_t*)(Ks + qk_off(jr + 4, kblk) + khalf)));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) S[mt] = mfma_bf16(kop[mt], vop, S[mt]);
        }
        if constexpr (SONLY) return;

        // Q S_prev for all 64 rows of this wave's columns, and this wave's share of
        // the ten lower-triangle (K Q^T) tiles: tiles t = wv, wv + NW, ... (round
        // robin).  Each wave masks its tiles and publishes P = scale (A .* M) in
        // bf16 hi + lo to LDS in A-operand layout; all waves then read all of P.
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 O[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) O[b] = z;
        auto qs_and_tiles = [&](auto wconst) {
            constexpr int W = decltype(wconst)::value;
            constexpr int NTILE = (10 - W + NW - 1) / NW;
            f32x4 At[NTILE];
#pragma unroll
            for (int s = 0; s < NTILE; ++s) At[s] = z;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                bf16x8 qa[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) qa[r] = lds_load<bf16x8>(Qs + qk_off(16 * r + lr, 4 * kb + lg));
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    O[b] = mfma_bf16(qa[b], Shi[kb], O[b]);
                    O[b] = mfma_bf16(qa[b], Slo[kb], O[b]);
                }
#pragma unroll
                for (int s = 0; s < NTILE; ++s) {
                    const int t = W + s * NW;
                    const int a = tile_a(t), b = tile_b(t);
                    const bf16x8 ka = lds_load<bf16x8>(Ks + qk_off(16 * a + lr, 4 * kb + lg));
                    At[s] = mfma_bf16(ka, qa[b], At[s]);
                }
            }
#pragma unroll
            for (int s = 0; s < NTILE; ++s) {
                const int t = W + s * NW;
                const int a = tile_a(t), b = tile_b(t);
                float pv4[4];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) pv4[ii] = At[s][ii] * (a == b ? dg[ii] : od[a < b ? b - a - 1 : 0][ii]);
                const uint32_t h0 = pack_bf16x2(pv4[0], pv4[1]), h1 = pack_bf16x2(pv4[2], pv4[3]);
                const uint32_t l0 = pack_bf16x2(pv4[0] - bf16_lo(h0), pv4[1] - bf16_hi(h0));
                const uint32_t l1 = pack_bf16x2(pv4[2] - bf16_lo(h1), pv4[3] - bf16_hi(h1));
                uint8_t* dst = Pbuf + (pidx(b, a >> 1) * 2 * 64 + lane) * 16 + 8 * (a & 1);
                const u32x2 hv = {h0, h1}, lv = {l0, l1};
                lds_store<u32x2>(dst, hv);
                lds_store<u32x2>(dst + 64 * 16, lv);
            }
        };
        if constexpr (NW == 1) {
            qs_and_tiles(IntC<0>{});
        } else if constexpr (NW == 2) {
            if (wv == 0) qs_and_tiles(IntC<0>{});
            else qs_and_tiles(IntC<1>{});
        } else {
            switch (wv) {
                case 0: qs_and_tiles(IntC<0>{}); break;
                case 1: qs_and_tiles(IntC<1>{}); break;
                case 2: qs_and_tiles(IntC<2>{}); break;
                default: qs_and_tiles(IntC<3>{}); break;
            }
        }
        // The inter-chunk part decays by lam^(i+1) (times scale); lam^i for a state
        // handed in at the first position.
        if (at_end) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) O[b][ii] *= sc * exp2f(g2 * (float)(16 * b + 4 * lg + ii));
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) O[b][ii] *= lamq[b][ii];
        }
        lds_barrier();  // P complete

        // O += P V.  For row tile b and token block kb, P elements 0..3 are tokens
        // 32kb + 4lg + 0..3 and 4..7 are 32kb + 16 + 4lg + 0..3; V is read in the
        // same token order.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int jr = 32 * kb + 4 * lg + (lr >> 2);
            const bf16x8 vop = cat_bf16(lds_tr16((const uint16_t*)(Vs + v_off(jr, vblk) + vhalf)),
                                        lds_tr16((const uint16_t*)(Vs + v_off(jr + 16, vblk) + vhalf)));
#pragma unroll
            for (int b = 2 * kb; b < 4; ++b) {
                const uint8_t* pp = Pbuf + (pidx(b, kb) * 2 * 64 + lane) * 16;
                O[b] = mfma_bf16(lds_load<bf16x8>(pp), vop, O[b]);
                O[b] = mfma_bf16(lds_load<bf16x8>(pp + 64 * 16), vop, O[b]);
            }
        }

        // Store the chunk's outputs; rows past the end fall outside the descriptor.
        const int64_t r0 = first_row(p0, Lc);
        const auto ro = make_rsrc(p.o + (r0 * H + wk.h) * dv + wk.vb * BV, (uint32_t)(Lc - 1) * orow_b + BV * 4);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * b + 4 * lg + ii;
                const int rs = REV ? Lc - 1 - i : i;
                buf_store_f32(O[b][ii], ro, rs * (int)orow_b + col * 4);
            }

        split_state<KB>(S, Shi, Slo);
    };

    if (nch > 0) {
#pragma unroll
        for (int c = 0; c < DEPTH; ++c) issue_chunk(c);
        for (int c = 0; c < nch; ++c) {
            wait_chunk(c);
            lds_barrier();  // chunk c is in LDS; every wave is done with chunk c - 1
            issue_chunk(c + DEPTH);
            compute_chunk(c, smem + (c % NST) * Cfg::STAGE_BYTES);
        }
        wait_vmem<0>();  // no copy may still be writing LDS when the workgroup ends
    }

    if (p.final_state) {
        const float fm = (p.final_lam && nch > 0) ? p.final_mul * exp2f(g2) : p.final_mul;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.final_state[st_off + (int64_t)dmap(mt, 4 * lg + ii) * dv + col] = fm * S[mt][ii];
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_16x16x4_f32, no rounding of any operand.
// ---------------------------------------------------------------------------
template <int DK, int NW>
struct F32Cfg {
    static constexpr int BV = 16 * NW;
    static constexpr int NT = 64 * NW;
    static constexpr int QLD = DK + 4;       // floats
    static constexpr int TLD = kChunk + 4;   // floats
    static constexpr int Q_ELEMS = kChunk * QLD;
    static constexpr int KT_ELEMS = DK * TLD;
    static constexpr int VT_ELEMS = BV * TLD;
    static constexpr int STAGE_ELEMS = 2 * Q_ELEMS + KT_ELEMS + VT_ELEMS;
    static constexpr int STAGES = (2 * STAGE_ELEMS * 4 <= kLdsBudget) ? 2 : 1;
    static constexpr int MT = DK / 16;
    static constexpr int QITEMS = kChunk * DK / 4;          // 16-byte pieces of a Q chunk
    static constexpr int KITEMS = (kChunk / 4) * (DK / 4);  // 4-token x 4-dk blocks of K
    static constexpr int VITEMS = (kChunk / 4) * (BV / 4);
    static constexpr int QPER = (QITEMS + NT - 1) / NT;
    static constexpr int KPER = (KITEMS + NT - 1) / NT;
    static constexpr int VPER = (VITEMS + NT - 1) / NT;
    static_assert(DK % 16 == 0 && DK <= 128, "dk must be a multiple of 16 up to 128");
    static_assert(STAGES * STAGE_ELEMS * 4 <= kLdsBudget, "LDS budget");
};

template <int DK, int NW, bool REV>
__global__ __launch_bounds__(64 * NW, 1) void fwd_f32_kernel(const FwdParams p) {
    using Cfg = F32Cfg<DK, NW>;
    constexpr int BV = Cfg::BV, NT = Cfg::NT, QLD = Cfg::QLD, TLD = Cfg::TLD, MT = Cfg::MT;
    __shared__ __attribute__((aligned(16))) float smem[Cfg::STAGES * Cfg::STAGE_ELEMS];

    Work wk;
    if (!decode_work(p, wk)) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const float g2 = p.g_gamma[wk.h] * kLog2e;
    const int64_t L = wk.len;
    const int nch = (int)((L + kChunk - 1) / kChunk);
    const int H = p.num_heads, dv = p.dv;
    const int vcol = wk.vb * BV + 16 * wv + lr;

    // Operand heads: q at h and k, v at the kv head, or the other way round.
    const int qh = p.swap_heads ? wk.kvh : wk.h, kh = p.swap_heads ? wk.h : wk.kvh;
    const int QH = p.swap_heads ? p.num_kv_heads : H, KH = p.swap_heads ? H : p.num_kv_heads;
    const float* qbase = static_cast<const float*>(p.q) + (int64_t)qh * DK;
    const float* kbase = static_cast<const float*>(p.k) + (int64_t)kh * DK;
    const float* vbase = static_cast<const float*>(p.v) + (int64_t)kh * dv + wk.vb * BV;
    const int64_t qstride = (int64_t)QH * DK;
    const int64_t kstride = (int64_t)KH * DK;
    const int64_t vstride = (int64_t)KH * dv;
    auto tok_row = [&](int64_t pos) -> int64_t { return REV ? wk.start + L - 1 - pos : wk.start + pos; };

    LaneDecay dec;
    make_lane_decay(g2, lr, lg, dec);
    const float lamC = exp2f(g2 * (float)kChunk);

    // State tile mt holds rows 16*mt + 4*lg + ii, column vcol.
    f32x4 S[MT];
    const int64_t st_off = ((int64_t)wk.n * H + wk.h) * DK * dv;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            S[mt][ii] = p.init ? p.init_mul * p.init[st_off + (int64_t)(16 * mt + 4 * lg + ii) * p.init_rs +
                                                      (int64_t)vcol * p.init_cs]
                               : 0.f;

    f32x4 pq[Cfg::QPER];
    f32x4 pk[Cfg::KPER][4];
    f32x4 pv[Cfg::VPER][4];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    auto load_chunk = [&](int c) {
        const int64_t p0 = (int64_t)c * kChunk;
#pragma unroll
        for (int s = 0; s < Cfg::QPER; ++s) {
            const int item = tid + s * NT;
            pq[s] = zero4;
            if (item < Cfg::QITEMS) {
                const int r = item / (DK / 4), c4 = item % (DK / 4);
                if (p0 + r < L) pq[s] = *reinterpret_cast<const f32x4*>(qbase + tok_row(p0 + r) * qstride + c4 * 4);
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::KPER; ++s) {
            const int item = tid + s * NT;
            const int tg = item / (DK / 4), c4 = item % (DK / 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pk[s][u] = zero4;
                if (item < Cfg::KITEMS && p0 + 4 * tg + u < L)
                    pk[s][u] = *reinterpret_cast<const f32x4*>(kbase + tok_row(p0 + 4 * tg + u) * kstride + c4 * 4);
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = tid + s * NT;
            const int tg = item / (BV / 4), c4 = item % (BV / 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pv[s][u] = zero4;
                if (item < Cfg::VITEMS && p0 + 4 * tg + u < L)
                    pv[s][u] = *reinterpret_cast<const f32x4*>(vbase + tok_row(p0 + 4 * tg + u) * vstride + c4 * 4);
            }
        }
    };

    auto store_chunk = [&](int c, float* st) {
        float* Qs = st;
        float* Ks = st + Cfg::Q_ELEMS;
        float* Kt = Ks + Cfg::Q_ELEMS;
        float* Vt = Kt + Cfg::KT_ELEMS;
        const int Lc = (int)min((int64_t)kChunk, L - (int64_t)c * kChunk);
#pragma unroll
        for (int s = 0; s < Cfg::QPER; ++s) {
            const int item = tid + s * NT;
            if (item < Cfg::QITEMS) {
                const int r = item / (DK / 4), c4 = item % (DK / 4);
                lds_store<f32x4>(Qs + r * QLD + c4 * 4, pq[s]);
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::KPER; ++s) {
            const int item = tid + s * NT;
            if (item < Cfg::KITEMS) {
                const int tg = item / (DK / 4), c4 = item % (DK / 4);
                float wgt[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    lds_store<f32x4>(Ks + (4 * tg + u) * QLD + c4 * 4, pk[s][u]);
                    const int tok = 4 * tg + u;
                    wgt[u] = tok < Lc ? exp2f(g2 * (float)(Lc - 1 - tok)) : 0.f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x4 col = {pk[s][0][e] * wgt[0], pk[s][1][e] * wgt[1], pk[s][2][e] * wgt[2],
                                       pk[s][3][e] * wgt[3]};
                    lds_store<f32x4>(Kt + (c4 * 4 + e) * TLD + 4 * tg, col);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = tid + s * NT;
            if (item < Cfg::VITEMS) {
                const int tg = item / (BV / 4), c4 = item % (BV / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x4 col = {pv[s][0][e], pv[s][1][e], pv[s][2][e], pv[s][3][e]};
                    lds_store<f32x4>(Vt + (c4 * 4 + e) * TLD + 4 * tg, col);
                }
            }
        }
    };

    auto compute_chunk = [&](int c, const float* st) {
        const float* Qs = st;
        const float* Ks = st + Cfg::Q_ELEMS;
        const float* Kt = Ks + Cfg::Q_ELEMS;
        const float* Vt = Kt + Cfg::KT_ELEMS;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 O[4], At[10];
#pragma unroll
        for (int b = 0; b < 4; ++b) O[b] = z;
#pragma unroll
        for (int t = 0; t < 10; ++t) At[t] = z;
        // Step (t, ii) pairs lane group lg with dk = 16t + 4lg + ii in every operand.
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 qa[4], ka[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                qa[r] = lds_load<f32x4>(Qs + (16 * r + lr) * QLD + 16 * t + 4 * lg);
                ka[r] = lds_load<f32x4>(Ks + (16 * r + lr) * QLD + 16 * t + 4 * lg);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
#pragma unroll
                    for (int a = 0; a <= b; ++a) At[tidx(a, b)] = mfma_f32(ka[a][ii], qa[b][ii], At[tidx(a, b)]);
                    O[b] = mfma_f32(qa[b][ii], S[t][ii], O[b]);
                }
        }
        // A state handed in at the first processed position (gradient sweeps) reaches
        // the first chunk one decay step less far.
        const bool at_end = p.init_at_end && c == 0;
        if (at_end) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) O[b][ii] *= exp2f(g2 * (float)(16 * b + 4 * lg + ii));
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) O[b][ii] *= dec.lamq[b][ii];
        }
        // O += (A .* M) V; token step (a, ii) pairs lane group lg with j = 16a + 4lg + ii.
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 vop = lds_load<f32x4>(Vt + (16 * wv + lr) * TLD + 16 * a + 4 * lg);
#pragma unroll
            for (int b = a; b < 4; ++b)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    O[b] = mfma_f32(At[tidx(a, b)][ii] * dec.mask[tidx(a, b)][ii], vop[ii], O[b]);
        }
        const int64_t p0 = (int64_t)c * kChunk;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * b + 4 * lg + ii;
                if (p0 + i < L) p.o[(tok_row(p0 + i) * H + wk.h) * dv + vcol] = p.scale * O[b][ii];
            }
        const int Lc = (int)min((int64_t)kChunk, L - p0);
        const float lamL = at_end ? exp2f(g2 * (float)(Lc - 1)) : (Lc == kChunk) ? lamC : exp2f(g2 * (float)Lc);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) S[mt] *= lamL;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 vop = lds_load<f32x4>(Vt + (16 * wv + lr) * TLD + 16 * a + 4 * lg);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 kop = lds_load<f32x4>(Kt + (16 * mt + lr) * TLD + 16 * a + 4 * lg);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) S[mt] = mfma_f32(kop[ii], vop[ii], S[mt]);
            }
        }
    };

    if (nch > 0) load_chunk(0);
    for (int c = 0; c < nch; ++c) {
        float* st = smem + (Cfg::STAGES == 2 ? (c & 1) * Cfg::STAGE_ELEMS : 0);
        if (Cfg::STAGES == 1) __syncthreads();
        store_chunk(c, st);
        if (c + 1 < nch) load_chunk(c + 1);
        __syncthreads();
        compute_chunk(c, st);
    }

    if (p.final_state) {
        const float fm = (p.final_lam && nch > 0) ? p.final_mul * exp2f(g2) : p.final_mul;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.final_state[st_off + (int64_t)(16 * mt + 4 * lg + ii) * dv + vcol] = fm * S[mt][ii];
    }
}

// ---------------------------------------------------------------------------
// Gated recurrence (GLA gates): log-decays per key channel, g_gamma[h] + g_t + gk_t,
// and per value channel, gv_t, each token.  Chunks of 16 tokens in fp32
// (v_mfma_f32_16x16x4_f32).  With A_t and B_t the log-decays summed from the chunk
// start through token t, every exponent below is <= 0, so nothing overflows:
//   o_t  = scale [ ((q_t .* e^{A_t}) S) .* e^{B_t} + sum_{u<=t} W_tu (v_u .* e^{B_t - B_u}) ]
//   W_tu = sum_i q_t[i] k_u[i] e^{A_t[i] - A_u[i]}                        (u <= t)
//   S'   = (e^{A_15} e^{B_15}^T) .* S + (k .* e^{A_15 - A_u})^T (v .* e^{B_15 - B_u})
// W has a per-channel exponent inside its sum.  When the chunk's decay spans stay
// below 2^kGSpan, W and the intra term run on MFMA after rescaling about the mid
// token m (q .* 2^{A_t - A_m} against k .* 2^{A_m - A_u}, v .* 2^{B_m - B_u}, then the
// rows times 2^{B_t - B_m}): every factor stays below 2^kGSpan, so nothing overflows.
// Otherwise W is built exactly on the VALU, one entry per thread.  Q S and the state
// update always run on MFMA.  Wave w owns value columns 16w .. 16w+15 of the block;
// its state tiles hold rows 16mt + 4lg + ii at column lr (accumulator layout, as in
// the fp32 kernel).
// ---------------------------------------------------------------------------
constexpr int kGChunk = 16;
constexpr int kGMid = 7;        // reference token of the fast path
constexpr float kGSpan = 64.f;  // largest |summed log2-decay| of a chunk on the fast path

// Hardware 2^x (v_exp_f32).  Results below the smallest normal float flush to zero,
// which only drops terms weighted below 2^-126 against a unit-weight term.
__device__ inline float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DK, int NW>
struct GatedCfg {
    static constexpr int BV = 16 * NW;
    static constexpr int NT = 64 * NW;
    static constexpr int KS = DK + 4;  // row stride (floats) of the dk-wide arrays
    static constexpr int VS = BV + 4;  // row stride of the BV-wide arrays
    static constexpr int MT = DK / 16;
    static constexpr int TS = kGChunk + 4;  // row stride of the token-minor arrays
    // Staged chunk (from registers): q, k, la = key log2-decay per token; v, lb =
    // value log2-decay per token (the prep phase turns la, lb into their sums A, B
    // from the chunk start, in place).  Derived for the matrix phase: qh = q .* 2^A,
    // qm = q .* 2^{A - A_m}, km = k .* 2^{A_m - A} (token-major); kt = k .* 2^{A_15 - A},
    // vt = v .* 2^{B_15 - B}, vm = v .* 2^{B_m - B} (token-minor: one 16-byte read gives
    // an MFMA lane its four tokens); bt = 2^B, bm = 2^{B - B_m}; ea = 2^{A_15},
    // eb = 2^{B_15}; W and oi for the exact path.
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + kGChunk * KS;
    static constexpr int OFF_A = OFF_K + kGChunk * KS;
    static constexpr int OFF_QH = OFF_A + kGChunk * KS;
    static constexpr int OFF_KT = OFF_QH + kGChunk * KS;
    static constexpr int OFF_QM = OFF_KT + DK * TS;
    static constexpr int OFF_KM = OFF_QM + kGChunk * KS;
    static constexpr int OFF_V = OFF_KM + kGChunk * KS;
    static constexpr int OFF_B = OFF_V + kGChunk * VS;
    static constexpr int OFF_VT = OFF_B + kGChunk * VS;
    static constexpr int OFF_VM = OFF_VT + BV * TS;
    static constexpr int OFF_BT = OFF_VM + BV * TS;
    static constexpr int OFF_BM = OFF_BT + kGChunk * VS;
    static constexpr int OFF_OI = OFF_BM + kGChunk * VS;
    static constexpr int OFF_W = OFF_OI + kGChunk * VS;
    static constexpr int OFF_EA = OFF_W + kGChunk * 17;
    static constexpr int OFF_EB = OFF_EA + DK;
    static constexpr int FLOATS = OFF_EB + BV;
    // Staging: 4-element pieces of a chunk, spread over all threads.
    static constexpr int KITEMS = kGChunk * DK / 4, VITEMS = kGChunk * BV / 4;
    static constexpr int KPER = (KITEMS + NT - 1) / NT, VPER = (VITEMS + NT - 1) / NT;
    static_assert(DK % 16 == 0 && DK <= 128, "dk must be a multiple of 16 up to 128");
    static_assert(FLOATS * 4 <= kLdsBudget, "LDS budget");
};

// Four consecutive elements as raw words (bf16: words x, y hold them; fp32: all four).
template <bool F32>
__device__ inline u32x4 load4_raw(const void* base, int64_t i) {
    if constexpr (F32) {
        return *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + i);
    } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + i);
        u32x4 r;
        r[0] = w[0];
        r[1] = w[1];
        return r;
    }
}
__device__ inline f32x4 raw_to_f32(u32x4 w, bool f32) {
    return f32 ? __builtin_bit_cast(f32x4, w) : f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
}

// One chunk per loop trip, two barriers: (1) the staged chunk is in LDS and the
// previous matrix phase is done; each thread then owns state channels (columns)
// and derives, from the decays summed over the chunk in registers, the decayed
// operands; (2) they are in LDS; the next chunk is staged from registers (its loads
// were issued a loop trip earlier; raw words are converted only here, so no load is
// waited for where it is issued) while the waves run the matrix phase.  The
// barriers wait for LDS operations only, so the prefetch loads stay in flight.
template <int DK, int NW, bool BF16, bool GF32>
__global__ __launch_bounds__(64 * NW, 1) void gated_kernel(const FwdParams p) {
    using Cfg = GatedCfg<DK, NW>;
    constexpr int BV = Cfg::BV, NT = Cfg::NT, KS = Cfg::KS, VS = Cfg::VS, MT = Cfg::MT, TS = Cfg::TS;
    __shared__ __attribute__((aligned(16))) float sm[Cfg::FLOATS];
    __shared__ int wide_span[2];  // per chunk parity: take the exact VALU path
    float* Qs = sm + Cfg::OFF_Q;
    float* Ks = sm + Cfg::OFF_K;
    float* As = sm + Cfg::OFF_A;
    float* QHs = sm + Cfg::OFF_QH;
    float* KTs = sm + Cfg::OFF_KT;
    float* QMs = sm + Cfg::OFF_QM;
    float* KMs = sm + Cfg::OFF_KM;
    float* Vs = sm + Cfg::OFF_V;
    float* Bs = sm + Cfg::OFF_B;
    float* VTs = sm + Cfg::OFF_VT;
    float* VMs = sm + Cfg::OFF_VM;
    float* BTs = sm + Cfg::OFF_BT;
    float* BMs = sm + Cfg::OFF_BM;
    float* OIs = sm + Cfg::OFF_OI;
    float* Ws = sm + Cfg::OFF_W;
    float* EAs = sm + Cfg::OFF_EA;
    float* EBs = sm + Cfg::OFF_EB;

    Work wk;
    if (!decode_work(p, wk)) return;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.num_heads, dv = p.dv;
    const int64_t L = wk.len;
    const int nch = (int)((L + kGChunk - 1) / kGChunk);
    const bool rev = p.reverse_gated != 0;
    const bool has_g = p.g != nullptr, has_gv = p.gv != nullptr;
    constexpr bool g_f32 = !BF16 || GF32;  // dtype of the key gate
    const float gg2 = p.g_gamma ? p.g_gamma[wk.h] * kLog2e : 0.f;
    const int j = 16 * wv + lr;       // this lane's column inside the block
    const int vcol = wk.vb * BV + j;  // ... of v and o
    auto tok_row = [&](int64_t pos) -> int64_t { return rev ? wk.start + L - 1 - pos : wk.start + pos; };
    const int64_t qrow = (int64_t)H * DK, krow = (int64_t)p.num_kv_heads * DK;
    const int64_t vrow = (int64_t)p.num_kv_heads * dv, gvrow = (int64_t)H * dv;
    const int64_t qoff = (int64_t)wk.h * DK, koff = (int64_t)wk.kvh * DK;
    const int64_t voff = (int64_t)wk.kvh * dv + wk.vb * BV, gvoff = (int64_t)wk.h * dv + wk.vb * BV;
    // Absent gates read an element of an array with the same layout (q for the key
    // gate, v itself for the value gate) and are written as zero.
    const void* gbase = has_g ? p.g : p.q;
    const void* gvbase = has_gv ? p.gv : p.v;
    const int64_t gvrow_r = has_gv ? gvrow : vrow, gvoff_r = has_gv ? gvoff : voff;

    f32x4 S[MT];
    const int64_t st_off = ((int64_t)wk.n * H + wk.h) * DK * dv;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            S[mt][ii] = p.init ? p.init[st_off + (int64_t)(16 * mt + 4 * lg + ii) * dv + vcol] : 0.f;
    // The state is in registers before the loop: inside it, the only loads in flight
    // are the staging prefetches, which the matrix phase then never waits for.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // Staging registers: raw words of this thread's pieces of q, k, the key gate, v
    // and the value gate; rows past the end read a valid row and are written as zero.
    u32x4 rq[Cfg::KPER], rk[Cfg::KPER], ra[Cfg::KPER], rv[Cfg::VPER], rb[Cfg::VPER];
    uint32_t kok = 0, vok = 0;  // bit s: piece s lies inside the sequence
    auto load_chunk = [&](int c) {
        const int64_t p0 = (int64_t)c * kGChunk;
        kok = vok = 0;
#pragma unroll
        for (int s = 0; s < Cfg::KPER; ++s) {
            const int item = tid + s * NT;
            const int t = item / (DK / 4), c4 = item % (DK / 4);
            const bool ok = item < Cfg::KITEMS && p0 + t < L;
            kok |= (ok ? 1u : 0u) << s;
            const int64_t row = tok_row(ok ? p0 + t : p0);
            rq[s] = load4_raw<!BF16>(p.q, row * qrow + qoff + 4 * c4);
            rk[s] = load4_raw<!BF16>(p.k, row * krow + koff + 4 * c4);
            ra[s] = load4_raw<g_f32>(gbase, row * qrow + qoff + 4 * c4);
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = tid + s * NT;
            const int t = item / (BV / 4), c4 = item % (BV / 4);
            const bool ok = item < Cfg::VITEMS && p0 + t < L;
            vok |= (ok ? 1u : 0u) << s;
            const int64_t row = tok_row(ok ? p0 + t : p0);
            rv[s] = load4_raw<!BF16>(p.v, row * vrow + voff + 4 * c4);
            rb[s] = load4_raw<!BF16>(gvbase, row * gvrow_r + gvoff_r + 4 * c4);
        }
    };
    // Write the staged pieces to LDS as floats: la = log2-decay of the key channels
    // (g_gamma plus the gate), lb of the value channels; zero past the end.
    auto store_chunk = [&]() {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < Cfg::KPER; ++s) {
            const int item = tid + s * NT;
            if (item < Cfg::KITEMS) {
                const int t = item / (DK / 4), c4 = item % (DK / 4);
                const bool ok = (kok >> s) & 1u;
                const f32x4 a = has_g ? kLog2e * raw_to_f32(ra[s], g_f32) : z;
                lds_store<f32x4>(Qs + t * KS + 4 * c4, ok ? raw_to_f32(rq[s], !BF16) : z);
                lds_store<f32x4>(Ks + t * KS + 4 * c4, ok ? raw_to_f32(rk[s], !BF16) : z);
                lds_store<f32x4>(As + t * KS + 4 * c4, ok ? a + gg2 : z);
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = tid + s * NT;
            if (item < Cfg::VITEMS) {
                const int t = item / (BV / 4), c4 = item % (BV / 4);
                const bool ok = (vok >> s) & 1u;
                const f32x4 b = has_gv ? kLog2e * raw_to_f32(rb[s], !BF16) : z;
                lds_store<f32x4>(Vs + t * VS + 4 * c4, ok ? raw_to_f32(rv[s], !BF16) : z);
                lds_store<f32x4>(Bs + t * VS + 4 * c4, ok ? b : z);
            }
        }
    };

    if (tid == 0) wide_span[0] = wide_span[1] = 0;
    if (nch > 0) {
        load_chunk(0);
        store_chunk();
    }
    if (nch > 1) load_chunk(1);
    for (int c = 0; c < nch; ++c) {
        lds_barrier();  // (1) chunk c staged; the previous matrix phase is done
        if (tid == 0) wide_span[(c + 1) & 1] = 0;  // the next chunk's flag, set in its prep
        // Prep: a thread owns a key channel (or a value channel) for all 16 tokens:
        // it sums the decays in registers and writes the decayed operands.
        for (int ch = tid; ch < DK + BV; ch += NT) {
            if (ch < DK) {
                const int i = ch;
                float A[kGChunk];
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < kGChunk; ++t) {
                    acc += As[t * KS + i];
                    A[t] = acc;
                }
                if (!(fabsf(acc) <= kGSpan)) wide_span[c & 1] = 1;
                const float aend = A[kGChunk - 1], amid = A[kGMid];
                EAs[i] = hw_exp2(aend);
#pragma unroll
                for (int t = 0; t < kGChunk; ++t) {
                    const float qv = Qs[t * KS + i], kv = Ks[t * KS + i];
                    As[t * KS + i] = A[t];
                    QHs[t * KS + i] = qv * hw_exp2(A[t]);
                    KTs[i * TS + t] = kv * hw_exp2(aend - A[t]);
                    QMs[t * KS + i] = qv * hw_exp2(A[t] - amid);
                    KMs[t * KS + i] = kv * hw_exp2(amid - A[t]);
                }
            } else {
                const int jj = ch - DK;
                float Bc[kGChunk];
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < kGChunk; ++t) {
                    acc += Bs[t * VS + jj];
                    Bc[t] = acc;
                }
                if (!(fabsf(acc) <= kGSpan)) wide_span[c & 1] = 1;
                const float bend = Bc[kGChunk - 1], bmid = Bc[kGMid];
                EBs[jj] = hw_exp2(bend);
#pragma unroll
                for (int t = 0; t < kGChunk; ++t) {
                    const float vv = Vs[t * VS + jj];
                    Bs[t * VS + jj] = Bc[t];
                    VTs[jj * TS + t] = vv * hw_exp2(bend - Bc[t]);
                    VMs[jj * TS + t] = vv * hw_exp2(bmid - Bc[t]);
                    BTs[t * VS + jj] = hw_exp2(Bc[t]);
                    BMs[t * VS + jj] = hw_exp2(Bc[t] - bmid);
                }
            }
        }
        lds_barrier();  // (2) derived operands are in LDS
        const bool fast = wide_span[c & 1] == 0;
        if (!fast) {  // exact intra term on the VALU (uniform branch): W, then W (v .* 2^{B_t - B_u})
            for (int e = tid; e < kGChunk * kGChunk; e += NT) {
                const int t = e >> 4, u = e & 15;
                float w = 0.f;
                if (u <= t) {
                    const float* qt = Qs + t * KS;
                    const float* ku = Ks + u * KS;
                    const float* at = As + t * KS;
                    const float* au = As + u * KS;
#pragma unroll 4
                    for (int i = 0; i < DK; i += 4) {
                        const f32x4 q4 = lds_load<f32x4>(qt + i), k4 = lds_load<f32x4>(ku + i);
                        const f32x4 a4 = lds_load<f32x4>(at + i), b4 = lds_load<f32x4>(au + i);
#pragma unroll
                        for (int x = 0; x < 4; ++x) w += q4[x] * k4[x] * hw_exp2(a4[x] - b4[x]);
                    }
                }
                Ws[t * 17 + u] = w;
            }
            lds_barrier();
            for (int e = tid; e < kGChunk * BV; e += NT) {
                const int t = e / BV, jj = e % BV;
                const float bt = Bs[t * VS + jj];
                float acc = 0.f;
                for (int u = 0; u <= t; ++u) acc += Ws[t * 17 + u] * Vs[u * VS + jj] * hw_exp2(bt - Bs[u * VS + jj]);
                OIs[t * VS + jj] = acc;
            }
            lds_barrier();
        }
        if (c + 1 < nch) {
            store_chunk();  // chunk c + 1; q, k, v and the decay arrays are read only before (2)
            if (c + 2 < nch) load_chunk(c + 2);
        }

        // Inter-chunk part: (q .* 2^A) S on four independent accumulators.
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 Oq[4] = {z, z, z, z};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 qh = lds_load<f32x4>(QHs + lr * KS + 16 * mt + 4 * lg);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) Oq[ii] = mfma_f32(qh[ii], S[mt][ii], Oq[ii]);
        }
        f32x4 O = (Oq[0] + Oq[1]) + (Oq[2] + Oq[3]);
        if (has_gv) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) O[ii] *= BTs[(4 * lg + ii) * VS + j];
        }
        if (fast) {
            // W^T = (k .* 2^{A_m - A}) (q .* 2^{A - A_m})^T: lane holds W[t = lr][u = 4lg + ii].
            // The contraction runs over dk = (DK/4) lg + sq, so each lane reads runs of
            // its own row.
            f32x4 Wa[4] = {z, z, z, z};
#pragma unroll
            for (int s4 = 0; s4 < DK / 16; ++s4) {
                const f32x4 km = lds_load<f32x4>(KMs + lr * KS + (DK / 4) * lg + 4 * s4);
                const f32x4 qm = lds_load<f32x4>(QMs + lr * KS + (DK / 4) * lg + 4 * s4);
#pragma unroll
                for (int x = 0; x < 4; ++x) Wa[x] = mfma_f32(km[x], qm[x], Wa[x]);
            }
            const f32x4 W = (Wa[0] + Wa[1]) + (Wa[2] + Wa[3]);
            const f32x4 vm = lds_load<f32x4>(VMs + j * TS + 4 * lg);
            f32x4 Oi = z;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int u = 4 * lg + ii;
                Oi = mfma_f32(u <= lr ? W[ii] : 0.f, vm[ii], Oi);  // causal: u <= t
            }
            if (has_gv) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) Oi[ii] *= BMs[(4 * lg + ii) * VS + j];
            }
            O += Oi;
        } else {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) O[ii] += OIs[(4 * lg + ii) * VS + j];
        }
        const int64_t p0 = (int64_t)c * kGChunk;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = 4 * lg + ii;
            if (p0 + t < L) p.o[(tok_row(p0 + t) * H + wk.h) * dv + vcol] = p.scale * O[ii];
        }

        // State update: S <- (2^{A_15} 2^{B_15}^T) .* S + kt^T vt.
        const float eb = has_gv ? EBs[j] : 1.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 ea = lds_load<f32x4>(EAs + 16 * mt + 4 * lg);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) S[mt][ii] *= ea[ii] * eb;
        }
        // Contraction over the 16 tokens u = 4lg + sq: kt and vt are token-minor.
        const f32x4 vt = lds_load<f32x4>(VTs + j * TS + 4 * lg);
        f32x4 kt[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) kt[mt] = lds_load<f32x4>(KTs + (16 * mt + lr) * TS + 4 * lg);
#pragma unroll
        for (int sq = 0; sq < 4; ++sq)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) S[mt] = mfma_f32(kt[mt][sq], vt[sq], S[mt]);
    }

    if (p.final_state) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.final_state[st_off + (int64_t)(16 * mt + 4 * lg + ii) * dv + vcol] = S[mt][ii];
    }
}

// ---------------------------------------------------------------------------
// Gated recurrence, bf16 inputs: the chunk algebra of gated_kernel with every
// product on bf16 MFMA.  A decayed fp32 operand X is split X = hi + lo, hi its bf16
// truncation and lo the bf16 rounding of the exact remainder; a product takes
// hi*hi + hi*lo + lo*hi with fp32 accumulation (about 2^-14 relative error per
// term).  Raw bf16 v needs no split.  Where a contraction runs over the 16 tokens,
// hi and lo share one 16x16x32 MFMA: its k index covers the tokens twice, with the
// hi and then the lo parts of one operand against the other operand repeated.
// With e_t = 2^{A_t} per key channel, the fast path (every channel's summed decay
// over the chunk within 2^-kGSpan) takes one exponential pair per element:
//   o_t  = scale 2^{B_t} .* [ (q_t .* e_t) S + sum_{u<=t} W_tu (v_u .* 2^{-B_u}) ]
//   W_tu = (q_t .* e_t) . (k_u ./ e_u)
//   S'   = 2^{A_15} .* [ 2^{B_15}^T .* S + (k ./ e)^T (v .* 2^{B_15 - B_u}) ]
// so k ./ e serves both W and the state update; masked pairs u > t and the bracket
// stay below 2^kGSpan times their operands.  A key channel pair with a wider span
// stores k .* 2^{A_15 - A_u} instead and moves its factor 2^{A_15} in front of S
// (per-row factors pre and post); a chunk holding one takes the exact VALU path of
// gated_kernel for W and the intra term.
//
// Roles: a workgroup of 2 NW waves.  Waves 0 .. NW-1 (matrix waves) own 16 value
// columns each and the state in accumulator registers; waves NW .. 2NW-1 (producer
// waves) stage the chunks from global memory and derive the decayed operands.  With
// one wave of each role per SIMD, the prep of chunk c+1 runs while the matrix waves
// compute chunk c.  LDS holds two staged raw chunks and two sets of decayed
// operands; one barrier per chunk hands both over.
// Prep: one item (channel pair, quarter of the chunk) per producer lane, the four
// quarters of a pair in one lane quad; each quarter sums its four decays and the quad
// exchanges the partial sums (DPP), so every lane has its tokens' A_t and A_15.
// ---------------------------------------------------------------------------
template <int DK, int NW>
struct GatedBCfg {
    static constexpr int BV = 16 * NW;
    static constexpr int PT = 64 * NW;  // producer threads
    static constexpr int NT = 2 * PT;   // all threads
    static constexpr int MT = DK / 16;
    static constexpr int KB = DK / 32;  // 32-deep blocks of the dk contraction
    // Dwords per row.  Staged raw chunk (token-major): q, k and a bf16 key gate;
    // an fp32 key gate; v and the value gate.  Padded so that the prep reads of a
    // half-wave (8 pairs x 4 quarters) hit distinct banks.
    static constexpr int SQ = DK / 2 + 2;
    static constexpr int SG32 = DK + 4;
    static constexpr int SV = BV / 2 + 2;
    // Decayed operands read along dk (token-major): bf16 hi half, lo half, 8 dwords
    // of pad (16-byte blocks per row = 2 mod 32: conflict-free operand reads).
    static constexpr int OPR = DK + 8;
    // Token-minor rows (a row per channel): four 16-byte blocks of four tokens,
    // [hi x4 | lo x4] in bf16 or four fp32.  Key rows carry two blocks of pad; value
    // rows swizzle their blocks instead (vblk).
    static constexpr int TMR = 24;
    static constexpr int VMR = 16;
    // fp32 summed decays for the exact path (token-major).
    static constexpr int AR = DK + 4, BR = BV + 4;
    // One staged raw chunk.
    static constexpr int ST_Q = 0;
    static constexpr int ST_K = ST_Q + kGChunk * SQ;
    static constexpr int ST_G = ST_K + kGChunk * SQ;  // bf16 or fp32 key gate
    static constexpr int ST_V = ST_G + kGChunk * SG32;
    static constexpr int ST_GV = ST_V + kGChunk * SV;
    static constexpr int ST_SIZE = ST_GV + kGChunk * SV;
    // One set of decayed operands.
    static constexpr int D_QH = 0;
    static constexpr int D_KP = D_QH + kGChunk * OPR;
    static constexpr int D_KT = D_KP + kGChunk * OPR;
    static constexpr int D_VP = D_KT + DK * TMR;
    static constexpr int D_VT = D_VP + BV * VMR;
    static constexpr int D_BT = D_VT + BV * VMR;
    static constexpr int D_PRE = D_BT + BV * VMR;
    static constexpr int D_POST = D_PRE + DK;
    static constexpr int D_EB = D_POST + DK;
    static constexpr int D_SIZE = D_EB + BV;
    static constexpr int OFF_ST = 0;
    static constexpr int OFF_D = OFF_ST + 2 * ST_SIZE;
    static constexpr int OFF_A = OFF_D + 2 * D_SIZE;
    static constexpr int OFF_B = OFF_A + kGChunk * AR;
    static constexpr int OFF_OI = OFF_B + kGChunk * BR;
    static constexpr int OFF_W = OFF_OI + kGChunk * BR;
    static constexpr int DWORDS = OFF_W + kGChunk * 17;
    // Staging: 4-element pieces of a chunk, spread over the producer threads.
    static constexpr int KITEMS = kGChunk * DK / 4, VITEMS = kGChunk * BV / 4;
    static constexpr int KPER = (KITEMS + PT - 1) / PT, VPER = (VITEMS + PT - 1) / PT;
    // Prep items: channel pairs x quarters.
    static constexpr int KPREP = 2 * DK, VPREP = 2 * BV;
    static_assert(DK % 32 == 0 && DK <= 128, "dk must be 32, 64 or 128");
    static_assert(ST_SIZE % 4 == 0 && D_SIZE % 4 == 0 && OFF_A % 4 == 0 && OFF_OI % 4 == 0 && D_PRE % 4 == 0,
                  "16-byte alignment");
    static_assert(DWORDS * 4 <= kLdsBudget, "LDS budget");
};

// A vector of raw words at a byte offset from a workgroup-uniform base (the offset
// fits 32 bits, so the load takes the scalar-base form).
template <typename T>
__device__ inline T load_at(const void* base, uint32_t byte_off) {
    return *reinterpret_cast<const T*>(static_cast<const char*>(base) + byte_off);
}

__device__ inline f32x4 mfma_bf16_w(u32x4 a, u32x4 b, f32x4 c) {
    return mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c);
}
// hi * lo term of a 16-token contraction as a 16x16x32 MFMA with the upper half of
// k zeroed.  (A 16x16x16 MFMA accumulating onto a 16x16x32 result read part of the
// accumulator stale in testing: no wait states were placed between the two
// opcodes.  Same-opcode chains are fine.)
__device__ inline f32x4 mfma_bf16_half(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
    return mfma_bf16_w(u32x4{a0, a1, 0u, 0u}, u32x4{b0, b1, 0u, 0u}, c);
}
// bf16 truncations of a and b in one word (a in the low half).
__device__ inline uint32_t hi_pack(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ inline float lo_part(float x) { return x - __uint_as_float(__float_as_uint(x) & 0xffff0000u); }
// bf16 roundings of what the truncations of a and b leave (exact in fp32).
__device__ inline uint32_t lo_pack(float a, float b) { return pack_bf16x2(lo_part(a), lo_part(b)); }
// Lane k of this lane's quad.
template <int K>
__device__ inline float quad_get(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), K * 0x55, 0xF, 0xF, false));
}
// Dword of a token-major operand row that holds channels 2pp, 2pp+1.  Channel
// 32s + 16h + 4g + r sits at position 32s + 8g + 4h + r, so that the eight
// positions an MFMA lane group reads for block s are the channels whose state rows
// that lane group holds in tiles 2s and 2s+1 (accumulator layout).
__host__ __device__ constexpr int gpos_dword(int pp) {
    return 16 * (pp >> 4) + 4 * ((pp >> 1) & 3) + 2 * ((pp >> 3) & 1) + (pp & 1);
}
// Dword offset of block b (tokens 4b .. 4b+3) of value row r: the blocks of rows
// 8 .. 15 mod 16 are swapped in pairs, so the 32 lanes of a half-wave reading
// (row, block lg) hit distinct banks.
__host__ __device__ constexpr int vblk(int r, int b) { return 16 * r + 4 * (b ^ ((r >> 2) & 2)); }
// Inclusive sums of a quarter's log2-decays (la, per token and channel) over the
// chunk: the lane quad holds the four quarters of a channel pair.  a = A_t of this
// quarter's tokens, tot = A_15.
__device__ inline void quarter_sums(const float (&la)[4][2], int tq, float (&a)[4][2], float (&tot)[2]) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        float cs[4];
        float acc = 0.f;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            acc += la[tau][x];
            cs[tau] = acc;
        }
        const float s0 = quad_get<0>(acc), s1 = quad_get<1>(acc), s2 = quad_get<2>(acc), s3 = quad_get<3>(acc);
        const float s01 = s0 + s1, s012 = s01 + s2;
        // sum of the earlier quarters, in the order that gives s012 for tq = 3
        const float pre = ((tq > 0 ? s0 : 0.f) + (tq > 1 ? s1 : 0.f)) + (tq > 2 ? s2 : 0.f);
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) a[tau][x] = pre + cs[tau];
        tot[x] = s012 + s3;
    }
}

template <int DK, int NW, bool GF32>
__global__ __launch_bounds__(128 * NW, 1) void gated_bf16_kernel(const FwdParams p) {
    using Cfg = GatedBCfg<DK, NW>;
    constexpr int BV = Cfg::BV, NT = Cfg::NT, PT = Cfg::PT, MT = Cfg::MT, KB = Cfg::KB;
    constexpr int SQ = Cfg::SQ, SV = Cfg::SV, OPR = Cfg::OPR, TMR = Cfg::TMR, AR = Cfg::AR, BR = Cfg::BR;
    constexpr int SGR = GF32 ? Cfg::SG32 : SQ;  // row stride of the staged key gate
    __shared__ __attribute__((aligned(16))) uint32_t sm[Cfg::DWORDS];
    __shared__ int wide_flag[3];  // per chunk mod 3: take the exact VALU path
    float* Af = reinterpret_cast<float*>(sm + Cfg::OFF_A);
    float* Bf = reinterpret_cast<float*>(sm + Cfg::OFF_B);
    float* OIf = reinterpret_cast<float*>(sm + Cfg::OFF_OI);
    float* Wf = reinterpret_cast<float*>(sm + Cfg::OFF_W);
    auto staged = [&](int c) __attribute__((always_inline)) -> uint32_t* { return sm + Cfg::OFF_ST + (c & 1) * Cfg::ST_SIZE; };
    auto derived = [&](int c) __attribute__((always_inline)) -> uint32_t* { return sm + Cfg::OFF_D + (c & 1) * Cfg::D_SIZE; };

    Work wk;
    if (!decode_work(p, wk)) return;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wv >= NW;
    const int ptid = tid - PT;  // producer thread index
    const int H = p.num_heads, dv = p.dv;
    const int64_t L = wk.len;
    const int nch = (int)((L + kGChunk - 1) / kGChunk);
    const bool rev = p.reverse_gated != 0;
    const bool has_g = p.g != nullptr, has_gv = p.gv != nullptr;
    const float gg2 = p.g_gamma ? p.g_gamma[wk.h] * kLog2e : 0.f;
    const int j = 16 * wv + lr;       // matrix waves: this lane's column inside the block
    const int vcol = wk.vb * BV + j;  // ... of v and o
    const int64_t qrow = (int64_t)H * DK, krow = (int64_t)p.num_kv_heads * DK;
    const int64_t vrow = (int64_t)p.num_kv_heads * dv, gvrow = (int64_t)H * dv;
    const int64_t qoff = (int64_t)wk.h * DK, koff = (int64_t)wk.kvh * DK;
    const int64_t voff = (int64_t)wk.kvh * dv + wk.vb * BV, gvoff = (int64_t)wk.h * dv + wk.vb * BV;
    // Chunk c holds the rows [low, low + nv) of the flattened token axis (in either
    // direction); token t of the chunk is row low + lrow(t).  Offsets inside a chunk
    // stay 32-bit (the host bounds 16 rows of every array below 2^31 bytes).
    auto chunk_nv = [&](int c) __attribute__((always_inline)) -> int { return (int)min((int64_t)kGChunk, L - (int64_t)c * kGChunk); };
    auto chunk_low = [&](int c, int nv) __attribute__((always_inline)) -> int64_t {
        const int64_t p0 = (int64_t)c * kGChunk;
        return rev ? wk.start + L - p0 - nv : wk.start + p0;
    };
    auto lrow = [&](int t, int nv) __attribute__((always_inline)) -> uint32_t { return (uint32_t)(rev ? nv - 1 - t : t); };

    f32x4 S[MT];
    const int64_t st_off = ((int64_t)wk.n * H + wk.h) * DK * dv;
    if (!producer) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[mt][ii] = p.init ? p.init[st_off + (int64_t)(16 * mt + 4 * lg + ii) * dv + vcol] : 0.f;
    }

    // Producer staging registers: raw words of this thread's pieces (bf16: words 0
    // and 1).  Two sets: chunk m goes through set m & 1, loaded two chunks ahead of
    // its store to LDS.  Absent gates are staged as zeros.
    using GateW = typename std::conditional<GF32, u32x4, u32x2>::type;  // four gate values
    struct StageRegs {
        u32x2 q[Cfg::KPER], k[Cfg::KPER], v[Cfg::VPER], b[Cfg::VPER];
        GateW a[Cfg::KPER];
        uint32_t kok, vok;  // bit s: piece s lies inside the sequence
    };
    StageRegs R0, R1;
    auto load_chunk = [&](int c, StageRegs& r) __attribute__((always_inline)) {
        u32x2(&rq)[Cfg::KPER] = r.q;
        u32x2(&rk)[Cfg::KPER] = r.k;
        GateW(&ra)[Cfg::KPER] = r.a;
        u32x2(&rv)[Cfg::VPER] = r.v;
        u32x2(&rb)[Cfg::VPER] = r.b;
        uint32_t& kok = r.kok;
        uint32_t& vok = r.vok;
        const int nv = chunk_nv(c);
        const int64_t low = chunk_low(c, nv);
        const uint16_t* qb = static_cast<const uint16_t*>(p.q) + (low * qrow + qoff);
        const uint16_t* kb = static_cast<const uint16_t*>(p.k) + (low * krow + koff);
        const uint16_t* vb = static_cast<const uint16_t*>(p.v) + (low * vrow + voff);
        // An absent gate re-reads q (v) at the same offsets: the same number of loads
        // every chunk keeps the waits on the earlier register set exact.
        constexpr uint32_t gsz = GF32 ? 4 : 2;
        const char* gb = has_g ? static_cast<const char*>(p.g) + (low * qrow + qoff) * gsz
                               : reinterpret_cast<const char*>(qb);
        const char* gvb = has_gv ? reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.gv) + (low * gvrow + gvoff))
                                 : reinterpret_cast<const char*>(vb);
        const uint32_t gvstride = (uint32_t)(has_gv ? gvrow : vrow);
        kok = vok = 0;
#pragma unroll
        for (int s = 0; s < Cfg::KPER; ++s) {
            const int item = ptid + s * PT;
            const int t = item / (DK / 4), c4 = item % (DK / 4);
            const bool ok = item < Cfg::KITEMS && t < nv;
            kok |= (ok ? 1u : 0u) << s;
            const uint32_t rr = ok ? lrow(t, nv) : 0u;  // rows past the end read row 0
            rq[s] = load_at<u32x2>(qb, 2 * (rr * (uint32_t)qrow + 4 * c4));
            rk[s] = load_at<u32x2>(kb, 2 * (rr * (uint32_t)krow + 4 * c4));
            ra[s] = load_at<GateW>(gb, gsz * (rr * (uint32_t)qrow + 4 * c4));
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = ptid + s * PT;
            const int t = item / (BV / 4), c4 = item % (BV / 4);
            const bool ok = item < Cfg::VITEMS && t < nv;
            vok |= (ok ? 1u : 0u) << s;
            const uint32_t rr = ok ? lrow(t, nv) : 0u;
            rv[s] = load_at<u32x2>(vb, 2 * (rr * (uint32_t)vrow + 4 * c4));
            rb[s] = load_at<u32x2>(gvb, 2 * (rr * gvstride + 4 * c4));
        }
    };
    // Raw words to LDS (zero past the end); nothing is converted here.
    auto store_chunk = [&](int c, const StageRegs& r) __attribute__((always_inline)) {
        const u32x2(&rq)[Cfg::KPER] = r.q;
        const u32x2(&rk)[Cfg::KPER] = r.k;
        const GateW(&ra)[Cfg::KPER] = r.a;
        const u32x2(&rv)[Cfg::VPER] = r.v;
        const u32x2(&rb)[Cfg::VPER] = r.b;
        const uint32_t kok = r.kok, vok = r.vok;
        uint32_t* st = staged(c);
        const u32x2 z2 = {0u, 0u};
        const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < Cfg::KPER; ++s) {
            const int item = ptid + s * PT;
            if (item < Cfg::KITEMS) {
                const int t = item / (DK / 4), c4 = item % (DK / 4);
                const bool ok = (kok >> s) & 1u;
                lds_store<u32x2>(st + Cfg::ST_Q + t * SQ + 2 * c4, ok ? rq[s] : z2);
                lds_store<u32x2>(st + Cfg::ST_K + t * SQ + 2 * c4, ok ? rk[s] : z2);
                const bool gok = ok && has_g;
                if constexpr (GF32) lds_store<u32x4>(st + Cfg::ST_G + t * SGR + 4 * c4, gok ? ra[s] : z4);
                else lds_store<u32x2>(st + Cfg::ST_G + t * SGR + 2 * c4, gok ? ra[s] : z2);
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = ptid + s * PT;
            if (item < Cfg::VITEMS) {
                const int t = item / (BV / 4), c4 = item % (BV / 4);
                const bool ok = (vok >> s) & 1u;
                lds_store<u32x2>(st + Cfg::ST_V + t * SV + 2 * c4, ok ? rv[s] : z2);
                if (has_gv) lds_store<u32x2>(st + Cfg::ST_GV + t * SV + 2 * c4, ok ? rb[s] : z2);
            }
        }
    };

    // Prep of chunk c (producer waves): staged(c) -> derived(c), the summed decays
    // (exact path) and the chunk's flag.
    auto prep_chunk = [&](int c) __attribute__((always_inline)) {
        const uint32_t* st = staged(c);
        uint32_t* d = derived(c);
        const int nv = chunk_nv(c);
        int* flag = &wide_flag[c % 3];
        // Key channels 2pp, 2pp+1, tokens 4tq .. 4tq+3.
#pragma unroll
        for (int r = 0; r < (Cfg::KPREP + PT - 1) / PT; ++r) {
            const int it = ptid + r * PT;
            if (Cfg::KPREP % PT != 0 && it >= Cfg::KPREP) break;
            const int pp = it >> 2, tq = it & 3;
            float la[4][2];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const int t = 4 * tq + tau;
                float g0, g1;
                if constexpr (GF32) {
                    const f32x2 g = lds_load<f32x2>(st + Cfg::ST_G + t * SGR + 2 * pp);
                    g0 = g[0];
                    g1 = g[1];
                } else {
                    const uint32_t w = st[Cfg::ST_G + t * SGR + pp];
                    g0 = bf16_lo(w);
                    g1 = bf16_hi(w);
                }
                const bool tv = t < nv;
                la[tau][0] = tv ? kLog2e * g0 + gg2 : 0.f;
                la[tau][1] = tv ? kLog2e * g1 + gg2 : 0.f;
            }
            float a[4][2], tot[2];
            quarter_sums(la, tq, a, tot);
            const bool wl = !(tot[0] >= -kGSpan) || !(tot[1] >= -kGSpan);
            if (wl) *flag = 1;
            if (tq == 3) {
                const f32x2 e15 = {hw_exp2(tot[0]), hw_exp2(tot[1])}, one = {1.f, 1.f};
                lds_store<f32x2>(d + Cfg::D_PRE + 2 * pp, wl ? e15 : one);
                lds_store<f32x2>(d + Cfg::D_POST + 2 * pp, wl ? one : e15);
            }
            // kp = k ./ e (narrow pair) or k .* 2^{A_15 - A} (wide pair)
            const float off[2] = {wl ? tot[0] : 0.f, wl ? tot[1] : 0.f};
            float qh[4][2], kp[4][2], kl[4][2];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const int t = 4 * tq + tau;
                lds_store<f32x2>(Af + t * AR + 2 * pp, f32x2{a[tau][0], a[tau][1]});
                const uint32_t qw = st[Cfg::ST_Q + t * SQ + pp], kw = st[Cfg::ST_K + t * SQ + pp];
                const float qv[2] = {bf16_lo(qw), bf16_hi(qw)}, kv[2] = {bf16_lo(kw), bf16_hi(kw)};
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    qh[tau][x] = qv[x] * hw_exp2(a[tau][x]);
                    kp[tau][x] = kv[x] * hw_exp2(off[x] - a[tau][x]);
                    kl[tau][x] = lo_part(kp[tau][x]);
                }
            }
            const int pd = gpos_dword(pp);
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                uint32_t* qr = d + Cfg::D_QH + (4 * tq + tau) * OPR + pd;
                uint32_t* kr = d + Cfg::D_KP + (4 * tq + tau) * OPR + pd;
                qr[0] = hi_pack(qh[tau][0], qh[tau][1]);
                qr[DK / 2] = lo_pack(qh[tau][0], qh[tau][1]);
                kr[0] = hi_pack(kp[tau][0], kp[tau][1]);
                kr[DK / 2] = pack_bf16x2(kl[tau][0], kl[tau][1]);
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
                lds_store<u32x4>(d + Cfg::D_KT + (2 * pp + x) * TMR + 4 * tq,
                                 u32x4{hi_pack(kp[0][x], kp[1][x]), hi_pack(kp[2][x], kp[3][x]),
                                       pack_bf16x2(kl[0][x], kl[1][x]), pack_bf16x2(kl[2][x], kl[3][x])});
        }
        // Value columns 2qq, 2qq+1 of the block, tokens 4tq .. 4tq+3; the last
        // producer threads take these items (the key prep fills the first ones when
        // the item counts do not divide evenly).
#pragma unroll
        for (int r = 0; r < (Cfg::VPREP + PT - 1) / PT; ++r) {
            const int it = (PT - 1 - ptid) + r * PT;
            if (Cfg::VPREP % PT != 0 && it >= Cfg::VPREP) break;
            const int qq = it >> 2, tq = 3 - (it & 3);
            if (has_gv) {
                float la[4][2];
#pragma unroll
                for (int tau = 0; tau < 4; ++tau) {
                    const int t = 4 * tq + tau;
                    const uint32_t w = st[Cfg::ST_GV + t * SV + qq];
                    const bool tv = t < nv;
                    la[tau][0] = tv ? kLog2e * bf16_lo(w) : 0.f;
                    la[tau][1] = tv ? kLog2e * bf16_hi(w) : 0.f;
                }
                float b[4][2], tot[2];
                quarter_sums(la, tq, b, tot);
                const bool wl = !(tot[0] >= -kGSpan) || !(tot[1] >= -kGSpan);
                if (wl) *flag = 1;
                const float e15[2] = {hw_exp2(tot[0]), hw_exp2(tot[1])};
                if (tq == 3) lds_store<f32x2>(d + Cfg::D_EB + 2 * qq, f32x2{e15[0], e15[1]});
                float bt[4][2], vp[4][2], vt[4][2];
#pragma unroll
                for (int tau = 0; tau < 4; ++tau) {
                    const int t = 4 * tq + tau;
                    lds_store<f32x2>(Bf + t * BR + 2 * qq, f32x2{b[tau][0], b[tau][1]});
                    const uint32_t vw = st[Cfg::ST_V + t * SV + qq];
                    const float vv[2] = {bf16_lo(vw), bf16_hi(vw)};
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        // wide: v .* 2^{-B} is not needed (and may overflow)
                        const float e = hw_exp2(b[tau][x]), y = hw_exp2(wl ? tot[x] - b[tau][x] : -b[tau][x]);
                        bt[tau][x] = e;
                        vp[tau][x] = wl ? 0.f : vv[x] * y;
                        vt[tau][x] = wl ? vv[x] * y : vp[tau][x] * e15[x];
                    }
                }
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int row = vblk(2 * qq + x, tq);
                    lds_store<f32x4>(reinterpret_cast<float*>(d + Cfg::D_BT) + row,
                                     f32x4{bt[0][x], bt[1][x], bt[2][x], bt[3][x]});
                    lds_store<u32x4>(d + Cfg::D_VP + row, u32x4{hi_pack(vp[0][x], vp[1][x]), hi_pack(vp[2][x], vp[3][x]),
                                                               lo_pack(vp[0][x], vp[1][x]), lo_pack(vp[2][x], vp[3][x])});
                    lds_store<u32x4>(d + Cfg::D_VT + row, u32x4{hi_pack(vt[0][x], vt[1][x]), hi_pack(vt[2][x], vt[3][x]),
                                                               lo_pack(vt[0][x], vt[1][x]), lo_pack(vt[2][x], vt[3][x])});
                }
            } else {  // v is exact in bf16: copy it token-minor, hi only
                uint32_t w[4];
#pragma unroll
                for (int tau = 0; tau < 4; ++tau) w[tau] = st[Cfg::ST_V + (4 * tq + tau) * SV + qq];
                lds_store<u32x2>(d + Cfg::D_VT + vblk(2 * qq, tq), u32x2{__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                                                                       __builtin_amdgcn_perm(w[3], w[2], 0x05040100u)});
                lds_store<u32x2>(d + Cfg::D_VT + vblk(2 * qq + 1, tq),
                                 u32x2{__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                                       __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)});
            }
        }
    };

    // Exact intra term of a wide chunk (all threads, between barriers): W, then
    // OI = W (v .* 2^{B_t - B_u}), from the raw staged chunk and the summed decays.
    auto exact_chunk = [&](int c) __attribute__((always_inline)) {
        const uint32_t* st = staged(c);
        for (int e = tid; e < kGChunk * kGChunk; e += NT) {
            const int t = e >> 4, u = e & 15;
            float w = 0.f;
            if (u <= t) {
                const uint32_t* qt = st + Cfg::ST_Q + t * SQ;
                const uint32_t* ku = st + Cfg::ST_K + u * SQ;
                const float* at = Af + t * AR;
                const float* au = Af + u * AR;
#pragma unroll 4
                for (int i = 0; i < DK; i += 4) {
                    const u32x2 q2 = lds_load<u32x2>(qt + i / 2), k2 = lds_load<u32x2>(ku + i / 2);
                    const f32x4 a4 = lds_load<f32x4>(at + i), b4 = lds_load<f32x4>(au + i);
                    const float q4[4] = {bf16_lo(q2[0]), bf16_hi(q2[0]), bf16_lo(q2[1]), bf16_hi(q2[1])};
                    const float k4[4] = {bf16_lo(k2[0]), bf16_hi(k2[0]), bf16_lo(k2[1]), bf16_hi(k2[1])};
#pragma unroll
                    for (int x = 0; x < 4; ++x) w += q4[x] * k4[x] * hw_exp2(a4[x] - b4[x]);
                }
            }
            Wf[t * 17 + u] = w;
        }
        lds_barrier();
        for (int e = tid; e < kGChunk * BV; e += NT) {
            const int t = e / BV, jj = e % BV;
            const float bt = has_gv ? Bf[t * BR + jj] : 0.f;
            float acc = 0.f;
            for (int u = 0; u <= t; ++u) {
                const float vu = bf16_half(st[Cfg::ST_V + u * SV + (jj >> 1)], jj & 1);
                const float dd = has_gv ? hw_exp2(bt - Bf[u * BR + jj]) : 1.f;
                acc += Wf[t * 17 + u] * vu * dd;
            }
            OIf[t * BR + jj] = acc;
        }
        lds_barrier();
    };

    // Matrix phase of chunk c (matrix waves).
    auto matrix_chunk = [&](int c, bool fast) __attribute__((always_inline)) {
        const uint32_t* d = derived(c);
        const uint32_t* QHw = d + Cfg::D_QH;
        const uint32_t* KPw = d + Cfg::D_KP;
        const float* BTf = reinterpret_cast<const float*>(d + Cfg::D_BT);
        const int nv = chunk_nv(c);
        // Inter-chunk part (q .* 2^A) S: the state tile pair (2s, 2s+1), split into
        // bf16 hi + lo, is the B operand of dk block s.  Fast path: W^T = (k ./ e)
        // (q .* e)^T in the same loop (q .* e is its B operand too); lane holds
        // W[t = lr][u = 4lg + ii].
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 O;
        const int vrow_j = vblk(j, lg);
        if (fast) {
            f32x4 Oa = z, Ob = z, Oc = z, Wa = z, Wb = z, Wc = z;
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const uint32_t* qr = QHw + lr * OPR + 16 * s + 4 * lg;
                const uint32_t* kr = KPw + lr * OPR + 16 * s + 4 * lg;
                const u32x4 qh = lds_load<u32x4>(qr), ql = lds_load<u32x4>(qr + DK / 2);
                const u32x4 kh = lds_load<u32x4>(kr), kl = lds_load<u32x4>(kr + DK / 2);
                const f32x4 s0 = S[2 * s], s1 = S[2 * s + 1];
                const u32x4 sh = {hi_pack(s0[0], s0[1]), hi_pack(s0[2], s0[3]), hi_pack(s1[0], s1[1]),
                                  hi_pack(s1[2], s1[3])};
                const u32x4 sl = {lo_pack(s0[0], s0[1]), lo_pack(s0[2], s0[3]), lo_pack(s1[0], s1[1]),
                                  lo_pack(s1[2], s1[3])};
                Oa = mfma_bf16_w(qh, sh, Oa);
                Wa = mfma_bf16_w(kh, qh, Wa);
                Ob = mfma_bf16_w(qh, sl, Ob);
                Wb = mfma_bf16_w(kh, ql, Wb);
                Oc = mfma_bf16_w(ql, sh, Oc);
                Wc = mfma_bf16_w(kl, qh, Wc);
            }
            O = (Oa + Ob) + Oc;
            f32x4 W = (Wa + Wb) + Wc;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                if (4 * lg + ii > lr) W[ii] = 0.f;  // causal: u <= t
            // Intra term W (v .* 2^{-B}): k = 8lg + e covers the tokens 4lg + (e & 3)
            // with W's hi (e < 4) and lo (e >= 4) parts, against v's hi part twice.
            const u32x4 vpx = lds_load<u32x4>(d + (has_gv ? Cfg::D_VP : Cfg::D_VT) + vrow_j);
            const u32x4 wa = {hi_pack(W[0], W[1]), hi_pack(W[2], W[3]), lo_pack(W[0], W[1]), lo_pack(W[2], W[3])};
            f32x4 Oi = mfma_bf16_w(wa, u32x4{vpx[0], vpx[1], vpx[0], vpx[1]}, z);
            if (has_gv) Oi = mfma_bf16_half(wa[0], wa[1], vpx[2], vpx[3], Oi);
            O += Oi;
            if (has_gv) O *= lds_load<f32x4>(BTf + vrow_j);
        } else {
            f32x4 Oa = z, Ob = z, Oc = z;
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const uint32_t* qr = QHw + lr * OPR + 16 * s + 4 * lg;
                const u32x4 qh = lds_load<u32x4>(qr), ql = lds_load<u32x4>(qr + DK / 2);
                const f32x4 s0 = S[2 * s], s1 = S[2 * s + 1];
                const u32x4 sh = {hi_pack(s0[0], s0[1]), hi_pack(s0[2], s0[3]), hi_pack(s1[0], s1[1]),
                                  hi_pack(s1[2], s1[3])};
                const u32x4 sl = {lo_pack(s0[0], s0[1]), lo_pack(s0[2], s0[3]), lo_pack(s1[0], s1[1]),
                                  lo_pack(s1[2], s1[3])};
                Oa = mfma_bf16_w(qh, sh, Oa);
                Ob = mfma_bf16_w(qh, sl, Ob);
                Oc = mfma_bf16_w(ql, sh, Oc);
            }
            O = (Oa + Ob) + Oc;
            if (has_gv) O *= lds_load<f32x4>(BTf + vrow_j);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) O[ii] += OIf[(4 * lg + ii) * BR + j];
        }
        {
            const int64_t orow = (int64_t)H * dv;
            char* ob = reinterpret_cast<char*>(p.o + (chunk_low(c, nv) * orow + (int64_t)wk.h * dv + wk.vb * BV));
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int t = 4 * lg + ii;
                if (t < nv) *reinterpret_cast<float*>(ob + 4 * (lrow(t, nv) * (uint32_t)orow + j)) = p.scale * O[ii];
            }
        }

        // State update: S <- post .* (pre .* 2^{B_15}^T .* S + kp^T vt), contracting
        // over the 16 tokens with kp's hi and lo parts in one k range (token-minor
        // operands: lane group lg reads tokens 4lg .. 4lg+3).
        const float* PREf = reinterpret_cast<const float*>(d + Cfg::D_PRE);
        const float* POSTf = reinterpret_cast<const float*>(d + Cfg::D_POST);
        const float eb = has_gv ? reinterpret_cast<const float*>(d + Cfg::D_EB)[j] : 1.f;
        if (!fast) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 pre = lds_load<f32x4>(PREf + 16 * mt + 4 * lg);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) S[mt][ii] *= pre[ii] * eb;
            }
        } else if (has_gv) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) S[mt] *= eb;
        }
        const u32x4 vtx = lds_load<u32x4>(d + Cfg::D_VT + vrow_j);
        const u32x4 vt2 = {vtx[0], vtx[1], vtx[0], vtx[1]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x4 ktx = lds_load<u32x4>(d + Cfg::D_KT + (16 * mt + lr) * TMR + 4 * lg);
            S[mt] = mfma_bf16_w(ktx, vt2, S[mt]);
            if (has_gv) S[mt] = mfma_bf16_half(ktx[0], ktx[1], vtx[2], vtx[3], S[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 post = lds_load<f32x4>(POSTf + 16 * mt + 4 * lg);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) S[mt][ii] *= post[ii];
        }
    };

    // Pipeline: before the barrier that opens step c, the producers have staged
    // chunk c+1 and derived chunk c.  During step c the matrix waves compute chunk c
    // while the producers derive chunk c+1, stage chunk c+2 (into the buffer chunk c
    // used) and load chunk c+4 (chunks c+3 and c+4 are in flight).  A wide chunk
    // first takes the exact path with all waves, before its staged buffer is
    // reused.  Chunk flags cycle through three slots: slot (c+2) mod 3 is cleared
    // during step c, after every read of chunk c-1's flag and before chunk c+2's
    // prep.  The two roles run separate loops with the same barriers in the same
    // order; the producers' steps run in pairs so that each register set has a
    // fixed name.
    if (producer) {
        if (ptid == 0) wide_flag[0] = wide_flag[1] = wide_flag[2] = 0;
        // Every step stores and loads one chunk (past the end: the last chunk again,
        // into a buffer no prep reads), so the loads in flight are always the two
        // register sets in order and the waits before each store are exact.
        auto clampc = [&](int m) __attribute__((always_inline)) -> int { return min(m, nch - 1); };
        if (nch > 0) {
            load_chunk(0, R0);
            load_chunk(clampc(1), R1);
            store_chunk(0, R0);
            load_chunk(clampc(2), R0);
        }
        lds_barrier();
        if (nch > 0) {
            prep_chunk(0);
            store_chunk(1, R1);
            load_chunk(clampc(3), R1);
            auto step = [&](int c, StageRegs& r) __attribute__((always_inline)) {  // r: chunks c+2, c+4
                if (c < nch) {
                    lds_barrier();  // chunk c derived, chunk c+1 staged, chunk c's flag final
                    if (wide_flag[c % 3] != 0) exact_chunk(c);
                }
                if (c + 1 < nch) {
                    if (ptid == 0) wide_flag[(c + 2) % 3] = 0;
                    prep_chunk(c + 1);
                }
                store_chunk(c + 2, r);
                load_chunk(clampc(c + 4), r);
            };
            for (int c = 0; c < nch; c += 2) {
                step(c, R0);
                step(c + 1, R1);
            }
        }
    } else {
        lds_barrier();
        for (int c = 0; c < nch; ++c) {
            lds_barrier();
            const bool fast = wide_flag[c % 3] == 0;
            if (!fast) exact_chunk(c);
            matrix_chunk(c, fast);
        }
    }

    if (!producer && p.final_state) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.final_state[st_off + (int64_t)(16 * mt + 4 * lg + ii) * dv + vcol] = S[mt][ii];
    }
}

// Four consecutive input elements as floats (bf16 words or fp32).
template <bool BF16>
__device__ inline f32x4 load4(const void* base, int64_t i) {
    return raw_to_f32(load4_raw<!BF16>(base, i), !BF16);
}

// Sum of the two key gates into one fp32 gate (the gated kernel reads one).
template <bool BF16>
__global__ __launch_bounds__(256) void gate_sum_kernel(const void* __restrict__ g, const void* __restrict__ gk,
                                                       float* __restrict__ out, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        *reinterpret_cast<f32x4*>(out + 4 * i) = load4<BF16>(g, 4 * i) + load4<BF16>(gk, 4 * i);
}

// ---------------------------------------------------------------------------
// Gradient sweeps under grouped-query attention: the sum of per-query-head
// gradients into their kv head, streamed in 16-byte pieces.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void group_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                        int64_t n4, int G, int d4) {
    // n4 = rows * Hkv * d4 output pieces; piece i is (row * Hkv + j, x4) and reads
    // the G query heads j*G .. j*G+G-1 of the same row, which are contiguous.
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const int64_t rj = i / d4, x4 = i % d4;
        const float* src = part + (rj * G * d4 + x4) * 4;
        f32x4 acc = *reinterpret_cast<const f32x4*>(src);
        for (int g = 1; g < G; ++g) acc += *reinterpret_cast<const f32x4*>(src + (int64_t)g * d4 * 4);
        *reinterpret_cast<f32x4*>(out + i * 4) = acc;
    }
}

// ---------------------------------------------------------------------------
// Decoding step: state <- lam * state + k^T v, o = scale * q state, for one new
// token per sequence.  The state is streamed once (read, updated, written back),
// so the kernel is bound by HBM: a workgroup owns the state block of one
// (sequence, head, BV columns); thread t updates column quad t % (BV/4) of rows
// t / (BV/4) + i * RG, each row a coalesced run of BV floats, and accumulates its
// share of q state; the row groups are then summed in LDS.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ inline float in_elem(const void* base, int64_t i) {
    if constexpr (BF16) return bf16_lo((uint32_t) static_cast<const uint16_t*>(base)[i]);
    else return static_cast<const float*>(base)[i];
}

template <int BV, bool BF16>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    constexpr int TPR = BV / 4;      // threads per state row (one float4 each)
    constexpr int RG = 256 / TPR;    // rows handled per pass of the workgroup
    constexpr int MAXR = (256 + RG - 1) / RG;  // passes for the widest head (dk = 256)
    __shared__ f32x4 red[256];
    const int tid = threadIdx.x, cq = tid % TPR, rg = tid / TPR;
    const int H = p.num_heads, dk = p.dk, dv = p.dv;
    const int nvb = dv / BV;
    const int64_t nh = blockIdx.x / nvb;  // n * H + h
    const int vb = blockIdx.x % nvb;
    const int h = (int)(nh % H);
    const int64_t n = nh / H;
    const int kvh = h / (H / p.num_kv_heads);
    const int c = vb * BV + 4 * cq;
    const float lam = exp2f(p.g_gamma[h] * kLog2e);
    const int64_t kvrow = n * p.num_kv_heads + kvh;
    f32x4 vq;
#pragma unroll
    for (int e = 0; e < 4; ++e) vq[e] = in_elem<BF16>(p.v, kvrow * dv + c + e);

    const int64_t blk = nh * dk * dv + c;
    f32x4 s[MAXR];
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {  // all loads first: MAXR independent 16-byte reads in flight
        const int r = rg + i * RG;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        s[i] = (r < dk && p.state_in) ? *reinterpret_cast<const f32x4*>(p.state_in + blk + (int64_t)r * dv) : z;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
        const int r = rg + i * RG;
        if (r < dk) {
            const float kr = in_elem<BF16>(p.k, kvrow * dk + r);
            const float qr = in_elem<BF16>(p.q, nh * dk + r);
            const f32x4 u = lam * s[i] + kr * vq;
            *reinterpret_cast<f32x4*>(p.state_out + blk + (int64_t)r * dv) = u;
            acc += qr * u;
        }
    }
    red[tid] = acc;
    __syncthreads();
#pragma unroll
    for (int stride = RG / 2; stride > 0; stride /= 2) {
        if (rg < stride) red[tid] += red[tid + stride * TPR];
        __syncthreads();
    }
    if (rg == 0) *reinterpret_cast<f32x4*>(p.o + nh * dv + c) = p.scale * red[cq];
}

// ---------------------------------------------------------------------------
// Intra-sequence split: chain the segments' own state contributions dS (from a
// state-only pass) into the state entering each segment and the final state.
// Per (row b, head h) and 4 state elements, in processing order:
//     S_in[seg] = S;   S = lam^len(seg) * S + dS[seg];   final = S.
// dS and S_in are [B * P, H, dk, dv] with segment index b * P + seg.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ dS, const float* __restrict__ init,
                                                       float* __restrict__ s_in, float* __restrict__ final_state,
                                                       const float* __restrict__ g_gamma, int H, int P, int seg_len,
                                                       int seqlen, int elems4, int rev) {
    const int e4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (e4 >= elems4) return;
    const int64_t bh = blockIdx.y;  // b * H + h
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const float g2 = g_gamma[h] * kLog2e;
    const int64_t elems = (int64_t)elems4 * 4;
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (init) S = *reinterpret_cast<const f32x4*>(init + bh * elems + 4 * e4);
    for (int j = 0; j < P; ++j) {
        const int sg = rev ? P - 1 - j : j;
        const int len = min(seg_len, seqlen - sg * seg_len);
        const int64_t at = ((b * P + sg) * H + h) * elems + 4 * e4;
        *reinterpret_cast<f32x4*>(s_in + at) = S;
        S = exp2f(g2 * (float)len) * S + *reinterpret_cast<const f32x4*>(dS + at);
    }
    if (final_state) *reinterpret_cast<f32x4*>(final_state + bh * elems + 4 * e4) = S;
}

// ---------------------------------------------------------------------------
// Longest-first order of packed sequences (ties by index): order[rank] = sequence.
// Lengths are clamped exactly as decode_work clamps them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void seq_order_kernel(const int32_t* cu, int num_seqs, int seqlen,
                                                        int32_t* order) {
    extern __shared__ int32_t lens[];
    for (int i = threadIdx.x; i < num_seqs; i += blockDim.x) {
        int64_t a = cu[i], e = cu[i + 1];
        a = min(max(a, (int64_t)0), (int64_t)seqlen);
        e = min(max(e, a), (int64_t)seqlen);
        lens[i] = (int32_t)(e - a);
    }
    __syncthreads();
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= num_seqs) return;
    const int li = lens[i];
    int rank = 0;
    for (int j = 0; j < num_seqs; ++j) {
        const int lj = lens[j];
        rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
}

template <int DK, int NW>
hipError_t launch_bf16(const FwdParams& p, bool rev, bool sonly, hipStream_t s) {
    const dim3 grid(fwd_grid_size(p)), block(64 * NW);
    if (sonly) {
        if (rev)
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, true, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, false, true>), grid, block, 0, s, p);
    } else {
        if (rev)
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, true, false>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, false, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

template <int DK, int NW>
hipError_t launch_f32(const FwdParams& p, bool rev, hipStream_t s) {
    const dim3 grid(fwd_grid_size(p)), block(64 * NW);
    if (rev)
        hipLaunchKernelGGL((fwd_f32_kernel<DK, NW, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((fwd_f32_kernel<DK, NW, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

// Compiled variants.  Narrow workgroups (fewer waves) stage more data per thread;
// with a wide head that exceeds the register file, so wide heads use 4 waves.
__host__ __device__ constexpr bool bf16_variant(int dk, int nw) {
    return (dk == 32 || dk == 64) ? (nw == 1 || nw == 2 || nw == 4)
           : dk == 128            ? (nw == 2 || nw == 4)
           : (dk == 192 || dk == 256) ? nw == 4
                                      : false;
}
__host__ __device__ constexpr bool f32_variant(int dk, int nw) {
    return (dk == 16 || dk == 32) ? (nw == 1 || nw == 2 || nw == 4)
           : dk == 64             ? (nw == 2 || nw == 4)
           : dk == 128            ? nw == 4
                                  : false;
}

template <int DK>
hipError_t launch_bf16_nw(const FwdParams& p, int nw, bool rev, bool sonly, hipStream_t s) {
    if constexpr (bf16_variant(DK, 1)) {
        if (nw == 1) return launch_bf16<DK, 1>(p, rev, sonly, s);
    }
    if constexpr (bf16_variant(DK, 2)) {
        if (nw == 2) return launch_bf16<DK, 2>(p, rev, sonly, s);
    }
    if constexpr (bf16_variant(DK, 4)) {
        if (nw == 4) return launch_bf16<DK, 4>(p, rev, sonly, s);
    }
    return hipErrorInvalidValue;
}

template <int DK>
hipError_t launch_f32_nw(const FwdParams& p, int nw, bool rev, hipStream_t s) {
    if constexpr (f32_variant(DK, 1)) {
        if (nw == 1) return launch_f32<DK, 1>(p, rev, s);
    }
    if constexpr (f32_variant(DK, 2)) {
        if (nw == 2) return launch_f32<DK, 2>(p, rev, s);
    }
    if constexpr (f32_variant(DK, 4)) {
        if (nw == 4) return launch_f32<DK, 4>(p, rev, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// dtype codes follow lattn_dtype: 0 = bf16, 1 = f32.
bool have_fwd_kernel(int in_dtype, int dk, int nw) {
    if (in_dtype == 0) return bf16_variant(dk, nw);
    if (in_dtype == 1) return f32_variant(dk, nw);
    return false;
}

int fwd_grid_size(const FwdParams& p) {
    const int per_xcd = (p.num_groups + kNumXcd - 1) / kNumXcd;
    return kNumXcd * per_xcd * p.group_size;
}

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int nw, bool reverse, hipStream_t s, bool state_only) {
    if (in_dtype == 0) {
        switch (p.dk) {
            case 32: return launch_bf16_nw<32>(p, nw, reverse, state_only, s);
            case 64: return launch_bf16_nw<64>(p, nw, reverse, state_only, s);
            case 128: return launch_bf16_nw<128>(p, nw, reverse, state_only, s);
            case 192: return launch_bf16_nw<192>(p, nw, reverse, state_only, s);
            case 256: return launch_bf16_nw<256>(p, nw, reverse, state_only, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (state_only) return hipErrorInvalidValue;  // the split runs bf16 problems only
    if (in_dtype == 1) {
        switch (p.dk) {
            case 16: return launch_f32_nw<16>(p, nw, reverse, s);
            case 32: return launch_f32_nw<32>(p, nw, reverse, s);
            case 64: return launch_f32_nw<64>(p, nw, reverse, s);
            case 128: return launch_f32_nw<128>(p, nw, reverse, s);
            default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

namespace {
int stream_blocks(int64_t n4) {
    const int64_t b = (n4 + 255) / 256;
    return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}
}  // namespace

hipError_t launch_group_sum(const float* part, float* out, int64_t rows, int H, int Hkv, int d, hipStream_t s) {
    const int64_t n4 = rows * Hkv * (d / 4);
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(group_sum_kernel, dim3(stream_blocks(n4)), dim3(256), 0, s, part, out, n4, H / Hkv, d / 4);
    return hipGetLastError();
}

int decode_block(int dv) { return dv % 64 == 0 ? 64 : dv % 32 == 0 ? 32 : 16; }

namespace {
template <int BV>
hipError_t launch_decode_bv(const DecodeParams& p, int in_dtype, hipStream_t s) {
    const int64_t blocks = (int64_t)p.batch * p.num_heads * (p.dv / BV);
    if (blocks == 0) return hipSuccess;
    if (in_dtype == 0)
        hipLaunchKernelGGL((decode_kernel<BV, true>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<BV, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_decode(const DecodeParams& p, int in_dtype, hipStream_t s) {
    switch (decode_block(p.dv)) {
        case 64: return launch_decode_bv<64>(p, in_dtype, s);
        case 32: return launch_decode_bv<32>(p, in_dtype, s);
        default: return launch_decode_bv<16>(p, in_dtype, s);
    }
}

hipError_t launch_seg_scan(const float* dS, const float* init, float* s_in, float* final_state, const float* g_gamma,
                           int B, int H, int P, int seg_len, int seqlen, int64_t elems, bool rev, hipStream_t s) {
    const int elems4 = (int)(elems / 4);
    const dim3 grid((elems4 + 255) / 256, (unsigned)(B * H));
    hipLaunchKernelGGL(seg_scan_kernel, grid, dim3(256), 0, s, dS, init, s_in, final_state, g_gamma, H, P, seg_len,
                       seqlen, elems4, rev ? 1 : 0);
    return hipGetLastError();
}

namespace {
template <int DK, int NW>
hipError_t launch_gated_t(const FwdParams& p, bool bf16, hipStream_t s) {
    const dim3 grid(fwd_grid_size(p));
    // bf16: NW matrix waves plus NW producer waves; fp32: NW waves
    const dim3 block_bf16(GatedBCfg<DK, NW>::NT), block_f32(64 * NW);
    if (bf16 && p.gk_is_f32)
        hipLaunchKernelGGL((gated_bf16_kernel<DK, NW, true>), grid, block_bf16, 0, s, p);
    else if (bf16)
        hipLaunchKernelGGL((gated_bf16_kernel<DK, NW, false>), grid, block_bf16, 0, s, p);
    else
        hipLaunchKernelGGL((gated_kernel<DK, NW, false, true>), grid, block_f32, 0, s, p);
    return hipGetLastError();
}
template <int DK>
hipError_t launch_gated_dk(const FwdParams& p, int nw, bool bf16, hipStream_t s) {
    if (nw == 4) return launch_gated_t<DK, 4>(p, bf16, s);
    if (nw == 1) return launch_gated_t<DK, 1>(p, bf16, s);
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_gate_sum(const void* g, const void* gk, float* out, int64_t n, int in_dtype, hipStream_t s) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    if (in_dtype == 0)
        hipLaunchKernelGGL((gate_sum_kernel<true>), dim3(stream_blocks(n4)), dim3(256), 0, s, g, gk, out, n4);
    else
        hipLaunchKernelGGL((gate_sum_kernel<false>), dim3(stream_blocks(n4)), dim3(256), 0, s, g, gk, out, n4);
    return hipGetLastError();
}

bool have_gated_kernel(int dk, int nw) { return (dk == 32 || dk == 64 || dk == 128) && (nw == 1 || nw == 4); }

hipError_t launch_gated(const FwdParams& p, int in_dtype, int nw, hipStream_t s) {
    const bool bf16 = in_dtype == 0;
    switch (p.dk) {
        case 32: return launch_gated_dk<32>(p, nw, bf16, s);
        case 64: return launch_gated_dk<64>(p, nw, bf16, s);
        case 128: return launch_gated_dk<128>(p, nw, bf16, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_seq_order(const int32_t* cu, int num_seqs, int seqlen, int32_t* order, hipStream_t s) {
    const int blocks = (num_seqs + 255) / 256;
    hipLaunchKernelGGL(seq_order_kernel, dim3(blocks), dim3(256), (size_t)num_seqs * sizeof(int32_t), s, cu,
                       num_seqs, seqlen, order);
    return hipGetLastError();
}

}  // namespace lattn
