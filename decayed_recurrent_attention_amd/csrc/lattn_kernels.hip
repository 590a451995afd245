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
// whole sequence: column block w (16 columns) belongs to one wave, or, with the dk
// split, to two waves that each hold half of its dk rows and exchange partial Q S
// sums through LDS (eight waves per workgroup, two per SIMD).  Each chunk of Q, K, V
// goes from HBM straight into LDS, row-major; the products that contract over tokens
// read K and V with transposing LDS reads.  The copies of the next DEPTH chunks are
// in flight while a chunk is computed.
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
#include <algorithm>

#include "lattn_device.h"

namespace lattn {
namespace {

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

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferDword3);
}
__device__ inline u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float buf_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// Output stores carry the streaming hint at device scope (cache-policy bits nt and sc1):
// o is written once and never read back by the kernel, and with the hint the chunk loop
// ran 1.4 % faster than with default stores (same results).
constexpr int kStreamStore = 2 | 16;
__device__ inline void buf_store_f32(float v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kStreamStore);
}
// Two bf16 (round to nearest even), a at the lower address.  Default cache policy: a
// wave writes only 32 bytes of a bf16 row (16 columns), and the four waves' pieces of a
// 128-byte line must merge in L2 (with the streaming hint the bf16 forward ran 1.50 ms
// against 1.09).
__device__ inline void buf_store_bf16x2(float a, float b, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a, b), r, off, 0, 0);
}
// The value of lane l ^ 1 (the neighbouring column of an MFMA output tile).
__device__ inline float lane_pair_swap(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
}

__device__ inline bf16x8 cat_bf16(u32x2 a, u32x2 b) {
    const u32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
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

// Parts of a chunk's copy (issue_chunk).
constexpr int kCopyQ = 1, kCopyK = 2, kCopyV = 4;

template <int DK, int NW, int DS = 1>
struct Bf16Cfg {
    static constexpr int BV = 16 * NW;
    static constexpr int NWD = NW * DS;  // waves: DS of them share each 16-column block
    static constexpr int PP = DK / 8;    // 16-byte blocks per Q / K row
    static constexpr int PVB = BV / 8;   // 16-byte blocks per V row (this value block)
    static constexpr int Q_BYTES = kChunk * DK * 2;
    static constexpr int V_BYTES = kChunk * BV * 2;
    static constexpr int STAGE_BYTES = 2 * Q_BYTES + V_BYTES;
    // Masked intra-chunk matrix P, exchanged between waves in MFMA A-operand layout:
    // 6 operand blocks (row tile b, token block kb) x {hi, lo} x 64 lanes x 16 bytes.
    static constexpr int P_BYTES = 6 * 2 * 64 * 16;
    // With the dk split, each wave hands two row tiles of its partial Q S to its partner.
    static constexpr int X_BYTES = DS > 1 ? NWD * 2 * 64 * 16 : 0;
    static constexpr int FIT = (kLdsBudget - P_BYTES - X_BYTES) / STAGE_BYTES;
    static constexpr int STAGES = FIT >= 3 ? 3 : FIT;  // ring of chunk stages
    static constexpr int DEPTH = STAGES - 1;           // chunks copied ahead of the one computed
    // The state-only pass stages K and V only: three stages wherever they fit, and two
    // of its workgroups share a compute unit where their LDS allows.
    static constexpr int SO_STAGE_BYTES = Q_BYTES + V_BYTES;
    static constexpr int SO_STAGES = 3 * SO_STAGE_BYTES <= kLdsBudget ? 3 : 2;
    static constexpr int SO_PER_CU = 2 * SO_STAGES * SO_STAGE_BYTES <= kLdsBudget ? 2 : 1;
    static constexpr int QCOPIES = PP / NWD;           // copy instructions per wave per Q (or K) tile
    static constexpr int VCOPIES = PVB / NWD;          // ... per V tile
    static constexpr int NCOPY = 2 * QCOPIES + VCOPIES;
    static constexpr int NSTORE = 16 / DS;             // output stores per wave per chunk
    static constexpr int KB = DK / 32;                 // dk blocks of one MFMA
    static constexpr int MT = DK / 16;                 // state row tiles
    static_assert(DK % 32 == 0 && DK <= 256, "dk must be a multiple of 32 up to 256");
    static_assert(STAGES >= 2 && STAGES <= 3, "the chunk loop is unrolled over two or three stages");
    static_assert(PP % NWD == 0 && PVB % NWD == 0, "copies divide evenly between waves");
    static_assert(DS == 1 || (DS == 2 && KB % 2 == 0), "the dk split halves whole dk blocks");
    static_assert(STAGES * STAGE_BYTES + P_BYTES + X_BYTES <= kLdsBudget, "LDS budget");
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
// work_id: the workgroup's unit of work (its id for a single problem).
// OB16: o in bf16 (round to nearest even of the fp32 result) instead of fp32.
template <int DK, int NW, bool REV, bool SONLY, int DS = 1, bool OB16 = false>
__device__ __attribute__((always_inline)) inline void fwd_bf16_body(const FwdParams& p, int work_id) {
    using Cfg = Bf16Cfg<DK, NW, DS>;
    constexpr int BV = Cfg::BV, PP = Cfg::PP, PVB = Cfg::PVB, KB = Cfg::KB, MT = Cfg::MT;
    constexpr int NWD = Cfg::NWD, MTL = MT / DS, KBL = KB / DS;  // waves; state tiles, dk blocks per wave
    constexpr int NST = SONLY ? Cfg::SO_STAGES : Cfg::STAGES, DEPTH = NST - 1;
    constexpr int QROW = DK * 2, VROW = BV * 2;  // LDS row bytes
    // LDS: the Q tiles of every stage, then the K tiles, then the V tiles, then P and the
    // partial sums.  The state-only pass holds only the K and V tiles.
    constexpr int KREG = SONLY ? 0 : NST * Cfg::Q_BYTES;
    constexpr int VREG = KREG + NST * Cfg::Q_BYTES;
    constexpr int LDS_BYTES = SONLY ? VREG + NST * Cfg::V_BYTES : NST * Cfg::STAGE_BYTES + Cfg::P_BYTES + Cfg::X_BYTES;
    static_assert(LDS_BYTES <= kLdsBudget, "LDS budget");
    static_assert(!SONLY || Cfg::SO_PER_CU * LDS_BYTES <= kLdsBudget, "state-only workgroups per compute unit");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
    uint8_t* Pbuf = smem + NST * Cfg::STAGE_BYTES;
    uint8_t* Xbuf = Pbuf + Cfg::P_BYTES;

    Work wk;
    if (!decode_work(p, work_id, wk)) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    // Column block and dk half of this wave (the state rows of wave (wc, wd) are the
    // global tiles wd*MTL .. wd*MTL + MTL - 1).
    const int wc = DS == 1 ? wv : wv >> 1, wd = DS == 1 ? 0 : wv & 1;
    const float g2 = p.g_gamma[wk.h] * kLog2e;  // log2 of the per-step decay
    const int L = (int)wk.len;
    const int nch = (L + kChunk - 1) / kChunk;
    const int H = p.num_heads, dv = p.dv;
    const int col = 16 * wc + lr;  // this lane's value column inside the block
    // Operand heads: q at h and k, v at the kv head, or the other way round.
    const int qh = p.swap_heads ? wk.kvh : wk.h, kh = p.swap_heads ? wk.h : wk.kvh;
    const int QH = p.swap_heads ? p.num_kv_heads : H, KH = p.swap_heads ? H : p.num_kv_heads;
    const uint32_t qrow_b = (uint32_t)QH * DK * 2, krow_b = (uint32_t)KH * DK * 2;
    constexpr uint32_t ob = OB16 ? 2u : 4u;  // bytes per o element
    const uint32_t vrow_b = (uint32_t)KH * dv * 2, orow_b = (uint32_t)H * dv * ob;
    const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (int64_t)qh * DK;
    const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)kh * DK;
    const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)kh * dv + wk.vb * BV;
    const uint32_t smem_base = lds_addr(smem);

    // Tiles (1, 0) and (3, 2) lie above the diagonal: their halves of P stay zero.
    if (!SONLY && tid < 64) {
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
    f32x4 S[MTL];
    {
        // Without an initial state the descriptor is empty and every load returns 0.
        const auto ri = make_rsrc(wk.init_blk ? wk.init_blk : p.g_gamma, wk.init_blk ? (uint32_t)(DK * dv * 4) : 0u);
        const int rs = (int)p.init_rs, cs = (int)p.init_cs, gcol = wk.vb * BV + col;
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[mt][ii] = p.init_mul * buf_load_f32(ri, (dmap(wd * MTL + mt, 4 * lg + ii) * rs + gcol * cs) * 4);
        // Split without a scan: chain the earlier segments' own contributions into the
        // state entering this one (their slots hold [dk][dv] blocks, H heads apart).
        // Four slots' loads go out together before they are added in order.
        if (wk.chain > 0) {
            const float lam_seg = exp2f(g2 * (float)wk.chain_len);
            for (int j0 = 0; j0 < wk.chain; j0 += 4) {
                f32x4 blk4[4][MTL];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool real = j0 + u < wk.chain;
                    const auto rj = make_rsrc(real ? wk.chain_blk + (int64_t)(j0 + u) * H * DK * dv : wk.chain_blk,
                                              real ? (uint32_t)(DK * dv * 4) : 0u);
#pragma unroll
                    for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            blk4[u][mt][ii] = buf_load_f32(rj, (dmap(wd * MTL + mt, 4 * lg + ii) * dv + gcol) * 4);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (j0 + u < wk.chain) {
#pragma unroll
                        for (int mt = 0; mt < MTL; ++mt) S[mt] = lam_seg * S[mt] + blk4[u][mt];
                    }
            }
        }
    }
    bf16x8 Shi[KBL], Slo[KBL];
    split_state<KBL>(S, Shi, Slo);

    auto first_row = [&](int p0, int Lc) __attribute__((always_inline)) -> int64_t { return REV ? wk.start + L - p0 - Lc : wk.start + p0; };
    auto qk_off = [](int row, int blk) __attribute__((always_inline)) { return row * QROW + 16 * (blk ^ qk_swz<PP>(row)); };
    auto v_off = [](int row, int blk) __attribute__((always_inline)) { return row * VROW + 16 * (blk ^ v_swz<PVB>(row)); };

    // Copy the parts (Q, K, V) of chunk c into stage c % NST.  Past the last chunk the
    // descriptors are empty, so the copies only write zeros (keeping the per-chunk
    // operation count fixed for the waits below) into the stage the previous chunk
    // used.  While chunk c is computed, the copies of chunk c + DEPTH go out in three
    // parts (K at the start, V after the state update, Q after the Q S and tile
    // products), which spreads each workgroup's requests over the chunk.
    auto issue_chunk = [&](int c, int parts) __attribute__((always_inline)) {
        const uint32_t sidx = (uint32_t)(c % NST);
        const uint32_t qst = smem_base + sidx * Cfg::Q_BYTES, kst = smem_base + KREG + sidx * Cfg::Q_BYTES;
        const uint32_t vst = smem_base + VREG + sidx * Cfg::V_BYTES;
        const int p0 = c * kChunk;
        const bool real = c < nch;
        const int Lc = real ? min(kChunk, L - p0) : 1;
        const int64_t r0 = real ? first_row(p0, Lc) : 0;
        const RawBuf rq = raw_buf(qg + r0 * QH * DK, real ? (uint32_t)(Lc - 1) * qrow_b + DK * 2 : 0u);
        const RawBuf rk = raw_buf(kg + r0 * KH * DK, real ? (uint32_t)(Lc - 1) * krow_b + DK * 2 : 0u);
        const RawBuf rv = raw_buf(vg + r0 * KH * dv, real ? (uint32_t)(Lc - 1) * vrow_b + BV * 2 : 0u);
#pragma unroll
        for (int j = 0; j < Cfg::QCOPIES; ++j) {
            const int kbyte = j * NWD + wv;  // this wave's kilobyte of the tile
            const int B = kbyte * 64 + lane, row = B / PP;
            const int blk = (B % PP) ^ qk_swz<PP>(row);
            const int rs = REV ? Lc - 1 - row : row;  // out of range past the end
            if (!SONLY && (parts & kCopyQ)) copy16_to_lds(qst + kbyte * 1024, rq, rs * (int)qrow_b + blk * 16);
            if (parts & kCopyK) copy16_to_lds(kst + kbyte * 1024, rk, rs * (int)krow_b + blk * 16);
        }
#pragma unroll
        for (int j = 0; j < Cfg::VCOPIES; ++j) {
            const int kbyte = j * NWD + wv;
            const int B = kbyte * 64 + lane, row = B / PVB;
            const int blk = (B % PVB) ^ v_swz<PVB>(row);
            const int rs = REV ? Lc - 1 - row : row;
            if (parts & kCopyV) copy16_to_lds(vst + kbyte * 1024, rv, rs * (int)vrow_b + blk * 16);
        }
    };
    // Wait until this wave's copies of chunk c are in LDS.  Issued after them, in
    // order: the copies of DEPTH-1 later chunks and the output stores of the
    // min(c, DEPTH) chunks computed since.
    constexpr int NCOPY = SONLY ? Cfg::QCOPIES + Cfg::VCOPIES : Cfg::NCOPY;
    // bf16 o: two adjacent columns per dword, so half as many stores
    constexpr int NSTORE = SONLY ? 0 : (OB16 ? Cfg::NSTORE / 2 : Cfg::NSTORE);
    constexpr int W0 = (DEPTH - 1) * NCOPY;
    constexpr int WC = W0 + DEPTH * NSTORE;
    auto wait_chunk = [&](int c) __attribute__((always_inline)) {
        if (c >= DEPTH) {
            wait_vmem<(WC < 63 ? WC : 63)>();
        } else if (c == 0) {
            wait_vmem<(W0 < 63 ? W0 : 63)>();
        } else {
            constexpr int W1 = W0 + NSTORE;
            wait_vmem<(W1 < 63 ? W1 : 63)>();
        }
    };

    auto compute_chunk = [&](int c, const uint8_t* Qs, const uint8_t* Ks, const uint8_t* Vs)
                             __attribute__((always_inline)) {
        const int cn = c + DEPTH;  // the chunk whose copies go out during this one
        const int p0 = c * kChunk, Lc = min(kChunk, L - p0);
        const int vblk = 2 * wc + ((lr & 3) >> 1), vhalf = 8 * (lr & 1);  // this lane's V piece

        // S <- lam^Lc S + K^T (decayed V).  Operands by transposing reads: lane group
        // lg takes tokens 32kb + 8lg + 0..7; the A operand row of lane lr is dk
        // dmap(mt, lr); the B operand (column `col`) is decayed in registers.
        // A state handed in at the first processed position (gradient sweeps) reaches
        // the first chunk one decay step less far.
        const bool at_end = p.init_at_end && c == 0;
        float lamL = lamC;
        if (at_end || Lc != kChunk) {  // (uniform; a full chunk past the first keeps lamC)
            lamL = exp2f(g2 * (float)(at_end ? Lc - 1 : Lc));
            if (Lc != kChunk) {  // the last chunk of a sequence: decays to its own end
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = 32 * kb + 8 * lg + e;
                        vw[kb][e] = j < Lc ? exp2f(g2 * (float)(Lc - 1 - j)) : 0.f;
                    }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) S[mt] *= lamL;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int jr = 32 * kb + 8 * lg + (lr >> 2);  // token row this lane addresses
            u32x4 vw4 = __builtin_bit_cast(u32x4, cat_bf16(lds_tr16((const uint16_t*)(Vs + v_off(jr, vblk) + vhalf)),
                                                         lds_tr16((const uint16_t*)(Vs + v_off(jr + 4, vblk) + vhalf))));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                vw4[e] = pack_bf16x2(bf16_lo(vw4[e]) * vw[kb][2 * e], bf16_hi(vw4[e]) * vw[kb][2 * e + 1]);
            const bf16x8 vop = __builtin_bit_cast(bf16x8, vw4);
            bf16x8 kop[MTL];
#pragma unroll
            for (int mt = 0; mt < MTL; ++mt) {
                const int mg = wd * MTL + mt;  // global state tile
                const int kblk = 4 * (mg >> 1) + (lr & 3), khalf = 8 * (mg & 1);
                kop[mt] = cat_bf16(lds_tr16((const uint16_t*)(Ks + qk_off(jr, kblk) + khalf)),
                                   lds_tr16((const uint16_t*)(Ks + qk_off(jr + 4, kblk) + khalf)));
            }
#pragma unroll
            for (int mt = 0; mt < MTL; ++mt) S[mt] = mfma_bf16(kop[mt], vop, S[mt]);
            if constexpr (DK >= 192 && DS == 2) __builtin_amdgcn_sched_barrier(0);
        }
        issue_chunk(cn, kCopyV);
        if constexpr (SONLY) return;

        // Q S_prev for all 64 rows of this wave's columns (over its dk rows), and this
        // wave's share of the ten lower-triangle (K Q^T) tiles: tiles t = wv, wv + NWD,
        // ... (round robin).  Each wave masks its tiles and publishes P = scale (A .* M) in
        // bf16 hi + lo to LDS in A-operand layout; after a barrier each wave reads the
        // blocks of P for the row tiles it finishes.
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 O[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) O[b] = z;
        auto qs_and_tiles = [&](auto wconst) __attribute__((always_inline)) {
            constexpr int W = decltype(wconst)::value;
            constexpr int WD = DS == 1 ? 0 : (W & 1);  // dk half of wave W
            constexpr int NTILE = (10 - W + NWD - 1) / NWD;
            f32x4 At[NTILE];
#pragma unroll
            for (int s = 0; s < NTILE; ++s) At[s] = z;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bool own = kb / KBL == WD;  // a dk block of this wave's state rows
                bf16x8 qa[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) qa[r] = lds_load<bf16x8>(Qs + qk_off(16 * r + lr, 4 * kb + lg));
                if (own) {
                    const int kl = own ? kb - WD * KBL : 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        O[b] = mfma_bf16(qa[b], Shi[kl], O[b]);
                        O[b] = mfma_bf16(qa[b], Slo[kl], O[b]);
                    }
                }
#pragma unroll
                for (int s = 0; s < NTILE; ++s) {
                    const int t = W + s * NWD;
                    const int a = tile_a(t), b = tile_b(t);
                    const bf16x8 ka = lds_load<bf16x8>(Ks + qk_off(16 * a + lr, 4 * kb + lg));
                    At[s] = mfma_bf16(ka, qa[b], At[s]);
                }
                if constexpr (DK >= 192 && DS == 2) {
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int s = 0; s < NTILE; ++s) {
                const int t = W + s * NWD;
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
        if constexpr (NWD == 1) {
            qs_and_tiles(IntC<0>{});
        } else if constexpr (NWD == 2) {
            if (wv == 0) qs_and_tiles(IntC<0>{});
            else qs_and_tiles(IntC<1>{});
        } else if constexpr (NWD == 4) {
            switch (wv) {
                case 0: qs_and_tiles(IntC<0>{}); break;
                case 1: qs_and_tiles(IntC<1>{}); break;
                case 2: qs_and_tiles(IntC<2>{}); break;
                default: qs_and_tiles(IntC<3>{}); break;
            }
        } else {
            static_assert(NWD == 8, "2, 4 or 8 waves");
            switch (wv) {
                case 0: qs_and_tiles(IntC<0>{}); break;
                case 1: qs_and_tiles(IntC<1>{}); break;
                case 2: qs_and_tiles(IntC<2>{}); break;
                case 3: qs_and_tiles(IntC<3>{}); break;
                case 4: qs_and_tiles(IntC<4>{}); break;
                case 5: qs_and_tiles(IntC<5>{}); break;
                case 6: qs_and_tiles(IntC<6>{}); break;
                default: qs_and_tiles(IntC<7>{}); break;
            }
        }
        issue_chunk(cn, kCopyQ);
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
        // With the dk split, the two waves of a column block each hold Q S over half of
        // dk for all 64 rows; each finishes row tiles {0, 3} (wd 0) or {1, 2} (wd 1) and
        // hands the partner its partial sums for the other two.
        // The rest of the chunk is compiled once per dk half (WDC), so that the row tiles
        // a wave finishes, its hand-over slots and its store offsets are fixed in the code.
        auto finish = [&](auto wdconst) __attribute__((always_inline)) {
            constexpr int WDC = decltype(wdconst)::value;
            auto own_rows = [&](int b) __attribute__((always_inline)) { return DS == 1 || ((b == 0 || b == 3) ? 0 : 1) == WDC; };
            auto xslot = [&](int w, int b) __attribute__((always_inline)) {
                return Xbuf + ((w * 2 + (b < 2 ? 0 : 1)) * 64 + lane) * 16;
            };
            if constexpr (DS > 1) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (!own_rows(b)) lds_store<f32x4>(xslot(wv, b), O[b]);
            }
            lds_barrier();  // P complete (and the partial sums handed over)
            if constexpr (DS > 1) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (own_rows(b)) O[b] += lds_load<f32x4>(xslot(wv ^ 1, b));
            }

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
                    if (!own_rows(b)) continue;
                    const uint8_t* pp = Pbuf + (pidx(b, kb) * 2 * 64 + lane) * 16;
                    O[b] = mfma_bf16(lds_load<bf16x8>(pp), vop, O[b]);
                    O[b] = mfma_bf16(lds_load<bf16x8>(pp + 64 * 16), vop, O[b]);
                }
            }

            // Store the chunk's outputs; rows past the end fall outside the descriptor.
            const int64_t r0 = first_row(p0, Lc);
            const auto ro = make_rsrc(reinterpret_cast<char*>(p.o) + ((r0 * H + wk.h) * dv + wk.vb * BV) * ob,
                                      (uint32_t)(Lc - 1) * orow_b + BV * ob);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (!own_rows(b)) continue;
                if constexpr (OB16) {
                    // Lanes lr and lr ^ 1 hold neighbouring columns: the even lane writes
                    // both columns of rows ii = 0, 1, the odd lane those of rows 2, 3.
                    const bool odd = (lr & 1) != 0;
                    const float t0 = lane_pair_swap(O[b][0]), t1 = lane_pair_swap(O[b][1]);
                    const float t2 = lane_pair_swap(O[b][2]), t3 = lane_pair_swap(O[b][3]);
                    const float a0 = odd ? t2 : O[b][0], a1 = odd ? O[b][2] : t0;
                    const float b0 = odd ? t3 : O[b][1], b1 = odd ? O[b][3] : t1;
                    const int i0 = 16 * b + 4 * lg + (odd ? 2 : 0), cpair = (col & ~1) * 2;
                    const int r0s = REV ? Lc - 1 - i0 : i0, r1s = REV ? Lc - 2 - i0 : i0 + 1;
                    buf_store_bf16x2(a0, a1, ro, r0s * (int)orow_b + cpair);
                    buf_store_bf16x2(b0, b1, ro, r1s * (int)orow_b + cpair);
                } else {
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int i = 16 * b + 4 * lg + ii;
                        const int rs = REV ? Lc - 1 - i : i;
                        buf_store_f32(O[b][ii], ro, rs * (int)orow_b + col * 4);
                    }
                }
            }
        };
        if constexpr (DS == 1) finish(IntC<0>{});
        else if (wd == 0) finish(IntC<0>{});
        else finish(IntC<1>{});
        split_state<KBL>(S, Shi, Slo);
    };

    if (nch > 0) {
#pragma unroll
        for (int c = 0; c < DEPTH; ++c) issue_chunk(c, kCopyQ | kCopyK | kCopyV);
        // Unrolled over the ring, so that each stage's LDS addresses are a per-lane
        // base plus a constant offset.
        auto step = [&](int c, auto sconst) __attribute__((always_inline)) {
            constexpr int ST = decltype(sconst)::value;
            wait_chunk(c);
            lds_barrier();  // chunk c is in LDS; every wave is done with chunk c - 1
            issue_chunk(c + DEPTH, kCopyK);
            compute_chunk(c, smem + ST * Cfg::Q_BYTES, smem + KREG + ST * Cfg::Q_BYTES, smem + VREG + ST * Cfg::V_BYTES);
        };
        for (int c = 0; c < nch; c += NST) {
            step(c, IntC<0>{});
            if (c + 1 < nch) step(c + 1, IntC<1>{});
            if constexpr (NST > 2) {
                if (c + 2 < nch) step(c + 2, IntC<2>{});
            }
        }
        wait_vmem<0>();  // no copy may still be writing LDS when the workgroup ends
    }

    if (wk.fin_blk) {
        const float fm = (p.final_lam && nch > 0) ? p.final_mul * exp2f(g2) : p.final_mul;
        float* fb = wk.fin_blk + wk.vb * BV;
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) fb[(int64_t)dmap(wd * MTL + mt, 4 * lg + ii) * dv + col] = fm * S[mt][ii];
    }
}

// Workgroups per compute unit that the kernel is built for.
template <int DK, int NW, int DS, bool SONLY>
constexpr int bf16_wgs_per_cu() {
    return SONLY ? Bf16Cfg<DK, NW, DS>::SO_PER_CU : 1;
}

template <int DK, int NW, bool REV, bool SONLY, int DS = 1, bool OB16 = false>
__global__ __launch_bounds__(64 * NW * DS, (bf16_wgs_per_cu<DK, NW, DS, SONLY>())) void fwd_bf16_kernel(const FwdParams p) {
    fwd_bf16_body<DK, NW, REV, SONLY, DS, OB16>(p, blockIdx.x);
}

// Two problems of the same shape in one launch (a.p[0], a.p[1]: the dk and dv sweeps
// of the backward).  Workgroup ids alternate between them in runs of kNumXcd, so the
// two workgroups with the same work id share a die and run together.
template <int DK, int NW, bool REV, int DS = 1>
__global__ __launch_bounds__(64 * NW * DS, 1) void fwd_bf16_pair_kernel(const FwdArgs a) {
    const int bid = blockIdx.x;
    fwd_bf16_body<DK, NW, REV, false, DS>(a.p[(bid / kNumXcd) & 1], (bid / (2 * kNumXcd)) * kNumXcd + bid % kNumXcd);
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
    if (!decode_work(p, blockIdx.x, wk)) return;
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
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            S[mt][ii] = wk.init_blk ? p.init_mul * wk.init_blk[(int64_t)(16 * mt + 4 * lg + ii) * p.init_rs +
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

    if (wk.fin_blk) {
        const float fm = (p.final_lam && nch > 0) ? p.final_mul * exp2f(g2) : p.final_mul;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) wk.fin_blk[(int64_t)(16 * mt + 4 * lg + ii) * dv + vcol] = fm * S[mt][ii];
    }
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
// Intra-sequence split of fixed-length input, chaining step.  Row b (P segments of
// seg_len tokens, the last possibly shorter) owns state slots b (P - 1) + k, k < P - 1,
// which the state-only pass filled with segment k's own contribution dS_k (from a zero
// state).  In processing order, with S the state entering segment k (S_0 the row's
// initial state or zeros),
//     S_{k+1} = lam^{seg_len} S_k + dS_k,
// and slot k is overwritten by S_{k+1} (in place: each element is read before it is
// written).  One thread per 4 state elements; blockIdx.x = (row b * H + head h) *
// eblocks + eb, each block looping over every eblocks-th group of 256 float4.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void seg_scan_kernel(float* __restrict__ slots, const float* __restrict__ init,
                                                       const float* __restrict__ g_gamma, int H, int P, int seg_len,
                                                       int elems4, int eblocks) {
    const int eb = blockIdx.x % eblocks, row = blockIdx.x / eblocks;
    const int b = row / H, h = row % H;
    const int64_t elems = (int64_t)elems4 * 4;
    const float lam_seg = exp2f(g_gamma[h] * kLog2e * (float)seg_len);
    const float* ib = init ? init + ((int64_t)b * H + h) * elems : nullptr;
    const int64_t slot0 = (int64_t)b * (P - 1);
    for (int e4 = eb * blockDim.x + threadIdx.x; e4 < elems4; e4 += eblocks * blockDim.x) {
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
        if (ib) S = *reinterpret_cast<const f32x4*>(ib + 4 * e4);
        for (int k = 0; k + 1 < P; ++k) {
            f32x4* at = reinterpret_cast<f32x4*>(slots + ((slot0 + k) * H + h) * elems + 4 * e4);
            S = lam_seg * S + *at;
            *at = S;
        }
    }
}

// ---------------------------------------------------------------------------
// Packed-split planner (one workgroup, a thread per sequence): cut the packed
// sequences into segments so that the longest ones no longer set the length of the
// call.  With c_n the chunks of sequence n, J workgroups per segment and kNumCu
// compute units, the balanced load per compute unit is Lb = J * sum(c_n) / kNumCu
// chunks.  A sequence longer than 5/4 Lb (the state-only pass costs about a quarter
// of a segment) is cut into segments of S = max(min_seg, ceil(Lb / 2)) chunks; with
// `forced` > 1 every sequence of at least two chunks is cut into min(forced, c_n)
// segments.  Sequences whose slots would pass max_slots stay whole.  Writes the main
// pass's segments longest first (ties by sequence, then segment) and the state-only
// pass's segments (layout in lattn_launch.h).  Segments are numbered in processing
// order (mirrored positions in reverse), so only a sequence's last segment can be
// short.
// ---------------------------------------------------------------------------
// Exclusive prefix sum over the workgroup (one value per thread, buf of blockDim.x);
// total = the sum.
__device__ inline int block_exclusive_scan(int v, int32_t* buf, int& total) {
    const int tid = threadIdx.x, nt = blockDim.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {
        const int t = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += t;
        __syncthreads();
    }
    total = buf[nt - 1];
    const int incl = buf[tid];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(1024) void split_plan_kernel(const int32_t* __restrict__ cu, int num_seqs, int seqlen,
                                                          int wgs, int min_seg, int forced, int rev, int max_main,
                                                          int max_slots, int32_t* __restrict__ plan) {
    __shared__ int32_t s_start[kMaxPlanSeqs], s_len[kMaxPlanSeqs], s_P[kMaxPlanSeqs], s_S[kMaxPlanSeqs];
    __shared__ int32_t s_slot0[kMaxPlanSeqs], s_seg0[kMaxPlanSeqs], s_buf[1024];
    __shared__ int32_t g_len[kMaxPlanSegs], g_seq[kMaxPlanSegs], g_k[kMaxPlanSegs];
    __shared__ unsigned long long s_total;
    const int i = threadIdx.x;  // this thread's sequence (blockDim.x >= num_seqs, a power of two <= 1024)
    const bool mine = i < num_seqs;
    if (i == 0) s_total = 0;
    __syncthreads();
    int len = 0, start = 0;
    if (mine) {
        int64_t a = cu[i], e = cu[i + 1];
        a = min(max(a, (int64_t)0), (int64_t)seqlen);  // clamped as the work decode clamps
        e = min(max(e, a), (int64_t)seqlen);
        start = (int)a;
        len = (int)(e - a);
        atomicAdd(&s_total, (unsigned long long)((len + kChunk - 1) / kChunk));
    }
    __syncthreads();
    const int64_t lb = ((int64_t)s_total * wgs + kNumCu - 1) / kNumCu;  // balanced chunks per compute unit
    const int c = (len + kChunk - 1) / kChunk;
    int P = 1, S = c;
    if (mine) {
        if (forced > 1) {
            if (c >= 2) {
                const int f = min(forced, c);
                S = (c + f - 1) / f;
                P = (c + S - 1) / S;
            }
        } else if (4 * (int64_t)c > 5 * lb) {
            S = (int)max((int64_t)min_seg, (lb + 1) / 2);
            P = (c + S - 1) / S;
        }
    }
    // slots in sequence order; a sequence whose slots would pass the capacity stays whole
    int total;
    const int tent = P > 1 ? P - 1 : 0;
    if (block_exclusive_scan(tent, s_buf, total) + tent > max_slots) P = 1;
    const int slots = P > 1 ? P - 1 : 0;
    int n_slots, n_segs;
    const int slot0 = block_exclusive_scan(slots, s_buf, n_slots);
    const int seg0 = block_exclusive_scan(mine ? P : 0, s_buf, n_segs);
    if (i == 0) {
        plan[0] = n_segs;
        plan[1] = n_slots;
    }
    int32_t* mainl = plan + kPlanHeader;
    int32_t* sonly = mainl + kPlanEntry * max_main;
    if (mine) {
        s_start[i] = start;
        s_len[i] = len;
        s_P[i] = P;
        s_S[i] = S;
        s_slot0[i] = slot0;
        s_seg0[i] = seg0;
        const int64_t S64 = (int64_t)S * kChunk;
        for (int k = 0; k < P; ++k) {
            const int64_t a = (int64_t)k * S64;
            const int sl = (int)(P > 1 ? min(S64, (int64_t)len - a) : len);
            g_len[seg0 + k] = sl;
            g_seq[seg0 + k] = i;
            g_k[seg0 + k] = k;
            if (k < P - 1) {  // the state-only pass's segment (P > 1 here)
                int32_t* so = sonly + kPlanEntry * (slot0 + k);
                so[0] = start + (int)(rev ? (int64_t)len - a - sl : a);
                so[1] = sl;
                so[2] = i;
                so[3] = -1;
                so[4] = 0;
                so[5] = 0;
                so[6] = (int)S64;
                so[7] = slot0 + k;
            }
        }
    }
    __syncthreads();
    // Main pass: rank = longest first, then by (sequence, segment) = list order.
    for (int g = threadIdx.x; g < n_segs; g += blockDim.x) {
        const int sl = g_len[g];
        int rank = 0;
        for (int h = 0; h < n_segs; ++h) {
            const int lh = g_len[h];
            rank += (lh > sl) || (lh == sl && h < g);
        }
        const int n = g_seq[g], k = g_k[g], Pn = s_P[n];
        const int64_t S64 = (int64_t)s_S[n] * kChunk, a = (int64_t)k * S64;
        int32_t* e = mainl + kPlanEntry * rank;
        e[0] = s_start[n] + (int)(rev ? (int64_t)s_len[n] - a - sl : a);
        e[1] = sl;
        e[2] = n;
        e[3] = (Pn > 1 && k > 0) ? s_slot0[n] : -1;
        e[4] = Pn > 1 ? k : 0;
        e[5] = k == Pn - 1 ? 1 : 0;
        e[6] = (int)S64;
        e[7] = 0;
    }
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

// The dk split (two waves per 16-column block, eight waves per workgroup) for four
// column blocks at dk 64, 128 and 192; dk 256 leaves no LDS for the partial sums.
// The state-only pass keeps one wave per block (with the split it ran no faster).
template <int DK, int NW>
constexpr int bf16_dk_split() {
    return (NW == 4 && (DK == 64 || DK == 128 || DK == 192)) ? 2 : 1;
}

template <int DK, int NW>
hipError_t launch_bf16(const FwdParams& p, const FwdParams* p2, bool rev, bool sonly, hipStream_t s) {
    constexpr int DS = bf16_dk_split<DK, NW>();
    const dim3 block(64 * NW * DS);
    if (p2) {
        FwdArgs a;
        a.p[0] = p;
        a.p[1] = *p2;
        const dim3 grid(2 * fwd_grid_size(p));
        if (rev)
            hipLaunchKernelGGL((fwd_bf16_pair_kernel<DK, NW, true, DS>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((fwd_bf16_pair_kernel<DK, NW, false, DS>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(fwd_grid_size(p));
    if (sonly) {
        const dim3 block1(64 * NW);
        if (rev)
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, true, true>), grid, block1, 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, false, true>), grid, block1, 0, s, p);
    } else if (p.o_bf16) {
        if (rev)
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, true, false, DS, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, false, false, DS, true>), grid, block, 0, s, p);
    } else {
        if (rev)
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, true, false, DS>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<DK, NW, false, false, DS>), grid, block, 0, s, p);
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
hipError_t launch_bf16_nw(const FwdParams& p, const FwdParams* p2, int nw, bool rev, bool sonly, hipStream_t s) {
    if constexpr (bf16_variant(DK, 1)) {
        if (nw == 1) return launch_bf16<DK, 1>(p, p2, rev, sonly, s);
    }
    if constexpr (bf16_variant(DK, 2)) {
        if (nw == 2) return launch_bf16<DK, 2>(p, p2, rev, sonly, s);
    }
    if constexpr (bf16_variant(DK, 4)) {
        if (nw == 4) return launch_bf16<DK, 4>(p, p2, rev, sonly, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bf16_dk(const FwdParams& p, const FwdParams* p2, int nw, bool rev, bool sonly, hipStream_t s) {
    switch (p.dk) {
        case 32: return launch_bf16_nw<32>(p, p2, nw, rev, sonly, s);
        case 64: return launch_bf16_nw<64>(p, p2, nw, rev, sonly, s);
        case 128: return launch_bf16_nw<128>(p, p2, nw, rev, sonly, s);
        case 192: return launch_bf16_nw<192>(p, p2, nw, rev, sonly, s);
        case 256: return launch_bf16_nw<256>(p, p2, nw, rev, sonly, s);
        default: return hipErrorInvalidValue;
    }
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
    if (in_dtype == 0) return launch_bf16_dk(p, nullptr, nw, reverse, state_only, s);
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

hipError_t launch_fwd_pair(const FwdParams& a, const FwdParams& b, int nw, bool reverse, hipStream_t s) {
    if (a.dk != b.dk || a.dv != b.dv || a.nvb != b.nvb || a.group_size != b.group_size ||
        a.num_groups != b.num_groups)
        return hipErrorInvalidValue;
    return launch_bf16_dk(a, &b, nw, reverse, false, s);
}

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

hipError_t launch_seg_scan(float* slots, const float* init, const float* g_gamma, int B, int H, int P, int seg_len,
                           int64_t elems, hipStream_t s) {
    const int elems4 = (int)(elems / 4);
    if (B <= 0 || P < 2 || elems4 == 0) return hipSuccess;
    const int eblocks = std::max(1, std::min(64, (elems4 + 255) / 256));  // one block per 256 float4
    const dim3 grid((unsigned)B * (unsigned)H * (unsigned)eblocks);
    hipLaunchKernelGGL(seg_scan_kernel, grid, dim3(256), 0, s, slots, init, g_gamma, H, P, seg_len, elems4, eblocks);
    return hipGetLastError();
}

hipError_t launch_split_plan(const int32_t* cu, int num_seqs, int seqlen, int wgs_per_seq, int min_seg_chunks,
                             int forced, bool reverse, int max_main, int max_slots, int32_t* plan, hipStream_t s) {
    if (num_seqs < 1 || num_seqs > kMaxPlanSeqs || max_main > kMaxPlanSegs) return hipErrorInvalidValue;
    // a thread per sequence: the smallest power of two >= num_seqs, at least one wave
    int threads = 64;
    while (threads < num_seqs) threads *= 2;
    hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(threads), 0, s, cu, num_seqs, seqlen, wgs_per_seq,
                       min_seg_chunks, forced, reverse ? 1 : 0, max_main, max_slots, plan);
    return hipGetLastError();
}

hipError_t launch_seq_order(const int32_t* cu, int num_seqs, int seqlen, int32_t* order, hipStream_t s) {
    const int blocks = (num_seqs + 255) / 256;
    hipLaunchKernelGGL(seq_order_kernel, dim3(blocks), dim3(256), (size_t)num_seqs * sizeof(int32_t), s, cu,
                       num_seqs, seqlen, order);
    return hipGetLastError();
}

}  // namespace lattn
