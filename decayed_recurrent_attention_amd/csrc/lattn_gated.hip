// Gated recurrence kernels (GLA gates): per-token, per-channel log-decays on the key
// and value axes of the state.  The recurrence (ejkernel "recurrent" interface page,
// the g, gk and gv arguments) with every gate a log-decay:
//     S_t[a][c] = exp(g_gamma + g_t[a] + gk_t[a] + gv_t[c]) S_{t-1}[a][c] + k_t[a] v_t[c],
//     o_t = scale * q_t S_t.
#include <type_traits>

#include "lattn_device.h"

namespace lattn {
namespace {

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

// fp32 inputs.  One chunk per loop trip, two barriers: (1) the staged chunk is in LDS and the
// previous matrix phase is done; each thread then owns state channels (columns)
// and derives, from the decays summed over the chunk in registers, the decayed
// operands; (2) they are in LDS; the next chunk is staged from registers (its loads
// were issued a loop trip earlier; raw words are converted only here, so no load is
// waited for where it is issued) while the waves run the matrix phase.  The
// barriers wait for LDS operations only, so the prefetch loads stay in flight.
template <int DK, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gated_f32_kernel(const FwdParams p) {
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
    if (!decode_work(p, blockIdx.x, wk)) return;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.num_heads, dv = p.dv;
    const int64_t L = wk.len;
    const int nch = (int)((L + kGChunk - 1) / kGChunk);
    const bool rev = p.reverse != 0;
    const bool has_g = p.g != nullptr, has_gv = p.gv != nullptr;
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
            rq[s] = load4_raw<true>(p.q, row * qrow + qoff + 4 * c4);
            rk[s] = load4_raw<true>(p.k, row * krow + koff + 4 * c4);
            ra[s] = load4_raw<true>(gbase, row * qrow + qoff + 4 * c4);
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = tid + s * NT;
            const int t = item / (BV / 4), c4 = item % (BV / 4);
            const bool ok = item < Cfg::VITEMS && p0 + t < L;
            vok |= (ok ? 1u : 0u) << s;
            const int64_t row = tok_row(ok ? p0 + t : p0);
            rv[s] = load4_raw<true>(p.v, row * vrow + voff + 4 * c4);
            rb[s] = load4_raw<true>(gvbase, row * gvrow_r + gvoff_r + 4 * c4);
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
                const f32x4 a = has_g ? kLog2e * raw_to_f32(ra[s], true) : z;
                lds_store<f32x4>(Qs + t * KS + 4 * c4, ok ? raw_to_f32(rq[s], true) : z);
                lds_store<f32x4>(Ks + t * KS + 4 * c4, ok ? raw_to_f32(rk[s], true) : z);
                lds_store<f32x4>(As + t * KS + 4 * c4, ok ? a + gg2 : z);
            }
        }
#pragma unroll
        for (int s = 0; s < Cfg::VPER; ++s) {
            const int item = tid + s * NT;
            if (item < Cfg::VITEMS) {
                const int t = item / (BV / 4), c4 = item % (BV / 4);
                const bool ok = (vok >> s) & 1u;
                const f32x4 b = has_gv ? kLog2e * raw_to_f32(rb[s], true) : z;
                lds_store<f32x4>(Vs + t * VS + 4 * c4, ok ? raw_to_f32(rv[s], true) : z);
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
// Gated recurrence, bf16 inputs: the chunk algebra of gated_f32_kernel with every
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
// gated_f32_kernel for W and the intra term.
//
// Roles: a workgroup of NW blocks of 16 value columns.  Matrix waves come first: DS
// per block (GatedBCfg::DS), each holding the state of the block's columns over one
// half of the dk rows in accumulator registers; then two producer waves per block,
// which copy the raw chunks from global memory into a ring of LDS stages and derive
// the decayed operands.  The prep of chunk c+1 runs while the matrix waves compute
// chunk c; LDS holds the ring and two sets of decayed operands, and one barrier per
// chunk hands a set over.  With DS = 2 the two waves of a block each compute their
// half of the chunk's output tile; one hands its half to the other through LDS.
// Prep: one item (channel pair, quarter of the chunk) per producer lane, the four
// quarters of a pair in one lane quad; each quarter sums its four decays and the quad
// exchanges the partial sums (DPP), so every lane has its tokens' A_t and A_15.
// ---------------------------------------------------------------------------
template <int DK, int NW, bool GF32>
struct GatedBCfg {
    static constexpr int BV = 16 * NW;
    static constexpr int MT = DK / 16;
    static constexpr int KB = DK / 32;  // 32-deep blocks of the dk contraction
    // dk split: each 16-column block's state is held by DS matrix waves, one per half
    // of the dk rows (DS = 2 where the dk blocks split evenly), so two matrix waves
    // share each SIMD and hide each other's latencies.
    static constexpr int DS = KB % 2 == 0 ? 2 : 1;
    static constexpr int MTW = MT / DS, KBW = KB / DS;  // state tiles and dk blocks per matrix wave
    // Matrix waves first, then two producer waves per 16-column block.
    static constexpr int MW = NW * DS;       // matrix waves
    static constexpr int MTH = 64 * MW;      // matrix threads
    static constexpr int PW = 2;             // producer waves per column block
    static constexpr int PWAVES = NW * PW;   // producer waves
    static constexpr int PT = 64 * PWAVES;   // producer threads
    static constexpr int NT = MTH + PT;      // all threads
    // One staged raw chunk, filled by direct global-to-LDS copies of a kilobyte each:
    // rows of q, k and the key gate (bf16, or fp32 when two gates were summed) over DK
    // channels, then rows of v and the value gate over BV columns, each region rounded
    // up to whole kilobytes (dwords below).  Rows are unpadded; the 16-byte blocks of
    // token row t are XOR-swizzled (stage_dw, stage_fl) so that the prep's reads of a
    // half-wave (8 channel pairs x 4 quarters) hit distinct banks.
    static constexpr int QNB = DK / 8, GNB = GF32 ? DK / 4 : DK / 8, VNB = BV / 8;  // 16-byte blocks per row
    static constexpr int kib(int bytes) { return (bytes + 1023) / 1024; }
    static constexpr int NCQ = kib(kGChunk * DK * 2), NCG = kib(kGChunk * DK * (GF32 ? 4 : 2)),
                         NCV = kib(kGChunk * BV * 2);
    static constexpr int NCOPY = 2 * NCQ + NCG + 2 * NCV;  // copies per chunk
    // Copies per producer wave and chunk: copy i goes to wave i mod PWAVES; the slots
    // past NCOPY copy nothing into a sink kilobyte at the end of the stage, so every
    // wave issues the same count.
    static constexpr int CPW = (NCOPY + PWAVES - 1) / PWAVES;
    static constexpr bool SINK = CPW * PWAVES > NCOPY;
    static constexpr int ST_Q = 0;
    static constexpr int ST_K = ST_Q + 256 * NCQ;
    static constexpr int ST_G = ST_K + 256 * NCQ;
    static constexpr int ST_V = ST_G + 256 * NCG;
    static constexpr int ST_GV = ST_V + 256 * NCV;
    static constexpr int ST_SINK = ST_GV + 256 * NCV;
    static constexpr int ST_SIZE = ST_SINK + (SINK ? 256 : 0);
    // Decayed operands read along dk (token-major): bf16 hi half, lo half, 8 dwords
    // of pad (16-byte blocks per row = 2 mod 32: conflict-free operand reads).  The
    // state update reads the key rows transposed (lds_tr16).
    static constexpr int OPR = DK + 8;
    // Token-minor value rows (a row per column): four 16-byte blocks of four tokens,
    // [hi x4 | lo x4] in bf16 (raw v without a value gate: [v x4 | v x4]) or four
    // fp32, blocks swizzled (vblk).
    static constexpr int VMR = 16;
    // fp32 summed decays for the exact path (token-major).
    static constexpr int AR = DK + 4, BR = BV + 4;
    // One set of decayed operands.
    static constexpr int D_QH = 0;
    static constexpr int D_KP = D_QH + kGChunk * OPR;
    static constexpr int D_VP = D_KP + kGChunk * OPR;
    static constexpr int D_VT = D_VP + BV * VMR;
    static constexpr int D_BT = D_VT + BV * VMR;
    static constexpr int D_PRE = D_BT + BV * VMR;
    static constexpr int D_POST = D_PRE + DK;
    static constexpr int D_EB = D_POST + DK;
    static constexpr int D_SIZE = D_EB + BV;
    // The exact path's summed decays A and B and its W live in the set of decayed
    // operands that no wave uses at that point.
    static constexpr int X_A = 0, X_B = X_A + kGChunk * AR, X_W = X_B + kGChunk * BR, X_END = X_W + kGChunk * 17;
    // The partial outputs one wave of each pair hands to the other (DS = 2), per
    // chunk parity: a 16x16 fp32 tile per column block.
    static constexpr int XO_SIZE = DS == 2 ? 2 * NW * 256 : 0;
    // LDS: the staged ring (four chunks where they fit, else three), two sets of
    // decayed operands, the exact path's intra term OI and the partial outputs.
    static constexpr int FIXED = 2 * D_SIZE + kGChunk * BR + XO_SIZE;
    static constexpr int NST = (4 * ST_SIZE + FIXED) * 4 <= kLdsBudget ? 4 : 3;
    static constexpr int OFF_ST = 0;
    static constexpr int OFF_D = OFF_ST + NST * ST_SIZE;
    static constexpr int OFF_OI = OFF_D + 2 * D_SIZE;
    static constexpr int OFF_XO = OFF_OI + kGChunk * BR;
    static constexpr int DWORDS = OFF_XO + XO_SIZE;
    // Prep items: channel pairs x quarters.
    static constexpr int KPREP = 2 * DK, VPREP = 2 * BV;
    static_assert(DK % 32 == 0 && DK <= 128, "dk must be 32, 64 or 128");
    static_assert(X_END <= D_SIZE, "exact-path buffers fit a set of decayed operands");
    static_assert(CPW * 3 <= 63, "vmcnt range");
    static_assert(D_SIZE % 4 == 0 && OFF_D % 4 == 0 && OFF_OI % 4 == 0 && OFF_XO % 4 == 0 && D_PRE % 4 == 0,
                  "16-byte alignment");
    static_assert(DWORDS * 4 <= kLdsBudget, "LDS budget");
};

// A raw buffer descriptor whose words are read from the first lane: the values are
// workgroup-uniform, and the copy's inline assembly takes the descriptor in scalar
// registers even where the compiler kept a word in a vector register.
__device__ inline RawBuf uniform_buf(const void* base, uint32_t bytes) {
    RawBuf r = raw_buf(base, bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.d[i] = __builtin_amdgcn_readfirstlane(r.d[i]);
    return r;
}

// Swizzle of the 16-byte blocks of staged token row t in a region of nb blocks per
// row (step 2 for bf16 rows, 4 for fp32 rows): the four quarters of the chunk land
// on different bank groups.
__host__ __device__ constexpr int stage_swz(int t, int nb, int step) { return (step * (t >> 2)) & (nb - 1); }
// Dword index of dword w of token row t in a staged bf16 region of nb blocks per row.
__host__ __device__ constexpr int stage_dw(int t, int w, int nb) {
    return t * 4 * nb + (((w >> 2) ^ stage_swz(t, nb, 2)) << 2) + (w & 3);
}
// Index of float i of token row t in a staged fp32 region of nb blocks per row.
__host__ __device__ constexpr int stage_fl(int t, int i, int nb) {
    return t * 4 * nb + (((i >> 2) ^ stage_swz(t, nb, 4)) << 2) + (i & 3);
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
// s minus the bf16 value held in the low (high) half of w, as one v_dot2_f32_bf16 of w
// against the pair (-1, -0) (against (-0, -1)) accumulated onto s.  When w holds s
// truncated to bf16 the difference is exact in fp32, so this equals the mask and
// subtract it replaces, in one instruction instead of two.  The -0 keeps the pair a
// 32-bit literal: the compiler encodes the pair (-1, 0) as the inline constant -1.0,
// which the hardware reads as another value (checked on the GPU: wrong results).
__device__ inline float sub_bf16_lo(uint32_t w, float s) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x8000bf80u), s,
                                           false);
}
__device__ inline float sub_bf16_hi(uint32_t w, float s) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0xbf808000u), s,
                                           false);
}
// bf16 roundings of what the truncations h = hi_pack(a, b) leave (exact in fp32).
__device__ inline uint32_t lo_pack(uint32_t h, float a, float b) {
    return pack_bf16x2(sub_bf16_lo(h, a), sub_bf16_hi(h, b));
}
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
        float acc = la[0][x];
        cs[0] = acc;
#pragma unroll
        for (int tau = 1; tau < 4; ++tau) {
            acc += la[tau][x];
            cs[tau] = acc;
        }
        const float s0 = quad_get<0>(acc), s1 = quad_get<1>(acc), s2 = quad_get<2>(acc), s3 = quad_get<3>(acc);
        const float s01 = s0 + s1, s012 = s01 + s2;
        // sum of the earlier quarters (s012 for tq = 3, so that a = tot at the last token)
        const float pre = tq > 2 ? s012 : tq > 1 ? s01 : tq > 0 ? s0 : 0.f;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) a[tau][x] = pre + cs[tau];
        tot[x] = s012 + s3;
    }
}

template <int DK, int NW, bool GF32, bool GV>
__global__ __launch_bounds__((GatedBCfg<DK, NW, GF32>::NT), 1) void gated_bf16_kernel(const FwdParams p) {
    using Cfg = GatedBCfg<DK, NW, GF32>;
    constexpr int BV = Cfg::BV, PT = Cfg::PT;
    constexpr int DS = Cfg::DS, MW = Cfg::MW, MTW = Cfg::MTW, KBW = Cfg::KBW;
    constexpr int OPR = Cfg::OPR, AR = Cfg::AR, BR = Cfg::BR;
    constexpr int QNB = Cfg::QNB, GNB = Cfg::GNB, VNB = Cfg::VNB, NST = Cfg::NST, DEPTH = NST - 1, CPW = Cfg::CPW;
    __shared__ __attribute__((aligned(16))) uint32_t sm[Cfg::DWORDS];
    __shared__ int wide_flag[3];  // per chunk mod 3: take the exact VALU path
    float* OIf = reinterpret_cast<float*>(sm + Cfg::OFF_OI);
    auto staged = [&](int c) __attribute__((always_inline)) -> uint32_t* { return sm + Cfg::OFF_ST + (c % NST) * Cfg::ST_SIZE; };
    auto derived = [&](int c) __attribute__((always_inline)) -> uint32_t* { return sm + Cfg::OFF_D + (c & 1) * Cfg::D_SIZE; };

    Work wk;
    if (!decode_work(p, blockIdx.x, wk)) return;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wv >= MW;
    // Matrix waves: column block w, dk half h (rows 16 MTW h .. 16 MTW (h + 1) - 1).
    const int w = wv % NW, h = wv / NW;
    const int ptid = tid - Cfg::MTH;  // producer thread index
    const int H = p.num_heads, dv = p.dv;
    const int64_t L = wk.len;
    const int nch = (int)((L + kGChunk - 1) / kGChunk);
    const bool rev = p.reverse != 0;
    const bool has_g = p.g != nullptr;
    constexpr bool has_gv = GV;  // the launch picks the instance from p.gv
    const float gg2 = p.g_gamma ? p.g_gamma[wk.h] * kLog2e : 0.f;
    const int j = 16 * w + lr;        // matrix waves: this lane's column inside the block
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

    f32x4 S[MTW];  // this wave's state tiles: global tile h MTW + m
    const int64_t st_off = ((int64_t)wk.n * H + wk.h) * DK * dv;
    if (!producer) {
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[m][ii] = p.init ? p.init[st_off + (int64_t)(16 * (h * MTW + m) + 4 * lg + ii) * dv + vcol] : 0.f;
    }

    // Copies of chunk m into its stage (m mod NST), issued by the producer waves: copy
    // i of a chunk goes to producer wave i mod PWAVES, and the copies past NCOPY copy
    // nothing into the sink.  A descriptor covers exactly the chunk's valid token rows
    // of its tensor, so rows past the end of a sequence, and absent gates (empty
    // descriptors), arrive as zeros; past the last chunk every descriptor is empty,
    // so each step issues the same number of copies.
    //
    // Each producer wave's plan is fixed for the whole sequence: copy j has a region,
    // an LDS slot inside the stage, and a source offset per lane for full chunks.  A
    // full chunk then costs a pointer step of 16 rows and one descriptor per copy;
    // the last chunk, when partial, takes the general path (copy_general).
    const uint32_t sm_base = lds_addr(sm);
    const int pw = wv - MW;  // producer wave index (producer waves only)
    struct CopyRegion {
        const char* base;  // the tensor at the work's head and columns, token row 0
        uint32_t stride, rowb;  // row stride; valid bytes per row (0: absent, an empty descriptor)
        uint32_t dst;           // LDS byte offset of this copy's kilobyte inside a stage
        int first, lnb, sstep;  // the region's first copy; log2 blocks per row; swizzle step
    };
    auto copy_region = [&](int ci) __attribute__((always_inline)) -> CopyRegion {
        constexpr int gsz = GF32 ? 4 : 2;
        constexpr int LQ = __builtin_ctz(QNB), LG = __builtin_ctz(GNB), LV = __builtin_ctz(VNB);
        CopyRegion r{static_cast<const char*>(p.q), 0u, 0u, 4u * Cfg::ST_SINK, ci, 0, 2};
        if (ci < Cfg::NCQ) {
            r = {static_cast<const char*>(p.q) + qoff * 2, (uint32_t)qrow * 2, DK * 2, 4u * Cfg::ST_Q, 0, LQ, 2};
        } else if (ci < 2 * Cfg::NCQ) {
            r = {static_cast<const char*>(p.k) + koff * 2, (uint32_t)krow * 2, DK * 2, 4u * Cfg::ST_K, Cfg::NCQ, LQ, 2};
        } else if (ci < 2 * Cfg::NCQ + Cfg::NCG) {
            r = {has_g ? static_cast<const char*>(p.g) + qoff * gsz : static_cast<const char*>(p.q), (uint32_t)qrow * gsz,
                 has_g ? DK * gsz : 0u, 4u * Cfg::ST_G, 2 * Cfg::NCQ, LG, GF32 ? 4 : 2};
        } else if (ci < 2 * Cfg::NCQ + Cfg::NCG + Cfg::NCV) {
            r = {static_cast<const char*>(p.v) + voff * 2, (uint32_t)vrow * 2, BV * 2, 4u * Cfg::ST_V,
                 2 * Cfg::NCQ + Cfg::NCG, LV, 2};
        } else if (ci < Cfg::NCOPY) {
            r = {has_gv ? reinterpret_cast<const char*>(p.gv) + gvoff * 2 : static_cast<const char*>(p.q),
                 (uint32_t)gvrow * 2, has_gv ? BV * 2 : 0u, 4u * Cfg::ST_GV, 2 * Cfg::NCQ + Cfg::NCG + Cfg::NCV, LV, 2};
        }
        r.dst += 1024u * (uint32_t)(ci - r.first);
        return r;
    };
    // Source offset of this lane's 16-byte slot (token row, swizzled block) of copy ci
    // for a chunk of nv valid rows; past the chunk's rows it is out of range.
    auto lane_offset = [&](const CopyRegion& r, int ci, int nv) __attribute__((always_inline)) -> int {
        const int B = (ci - r.first) * 64 + lane, row = B >> r.lnb;
        const int blk = (B & ((1 << r.lnb) - 1)) ^ stage_swz(row, 1 << r.lnb, r.sstep);
        const int rs = rev ? nv - 1 - row : row;  // negative (out of range) past the end
        return row < kGChunk ? rs * (int)r.stride + blk * 16 : 0x7ffffff0;
    };
    // First token row of chunk m were it full (reverse: may lie before the sequence).
    auto full_low = [&](int m) __attribute__((always_inline)) -> int64_t {
        return rev ? wk.start + L - (int64_t)kGChunk * (m + 1) : wk.start + (int64_t)kGChunk * m;
    };
    const char* cur[CPW];  // copy j's source at the next chunk's first row, as if full
    uint32_t nrec_full[CPW], dst[CPW];
    int off_full[CPW], cpstep[CPW];
    if (producer) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int ci = j * Cfg::PWAVES + pw;
            const CopyRegion r = copy_region(ci);
            cur[j] = r.base + full_low(0) * (int64_t)r.stride;
            nrec_full[j] = r.rowb != 0 ? (uint32_t)(kGChunk - 1) * r.stride + r.rowb : 0u;
            dst[j] = r.dst;
            off_full[j] = lane_offset(r, ci, kGChunk);
            cpstep[j] = (rev ? -kGChunk : kGChunk) * (int)r.stride;
        }
    }
    auto copy_general = [&](int m, int j, uint32_t stage) __attribute__((always_inline)) {
        const int ci = j * Cfg::PWAVES + pw;
        const CopyRegion r = copy_region(ci);
        const int nv = chunk_nv(m);
        const char* src = r.base + chunk_low(m, nv) * (int64_t)r.stride;
        const uint32_t nrec = r.rowb != 0 ? (uint32_t)(nv - 1) * r.stride + r.rowb : 0u;
        copy16_to_lds(stage + r.dst, uniform_buf(src, nrec), lane_offset(r, ci, nv));
    };
    auto issue_chunk = [&](int m) __attribute__((always_inline)) {
        const uint32_t stage = sm_base + 4u * (uint32_t)(Cfg::OFF_ST + (m % NST) * Cfg::ST_SIZE);
        if (m == nch - 1 && chunk_nv(m) != kGChunk) {
#pragma unroll
            for (int j = 0; j < CPW; ++j) copy_general(m, j, stage);
        } else {
            const bool real = m < nch;
#pragma unroll
            for (int j = 0; j < CPW; ++j)
                copy16_to_lds(stage + __builtin_amdgcn_readfirstlane(dst[j]), uniform_buf(cur[j], real ? nrec_full[j] : 0u),
                              off_full[j]);
        }
#pragma unroll
        for (int j = 0; j < CPW; ++j) cur[j] += cpstep[j];
    };

    // Prep of chunk c (producer waves): staged(c) -> derived(c) and the chunk's flag.
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
                    const f32x2 g = lds_load<f32x2>(st + Cfg::ST_G + stage_fl(t, 2 * pp, GNB));
                    g0 = g[0];
                    g1 = g[1];
                } else {
                    const uint32_t w = st[Cfg::ST_G + stage_dw(t, pp, QNB)];
                    g0 = bf16_lo(w);
                    g1 = bf16_hi(w);
                }
                la[tau][0] = kLog2e * g0 + gg2;
                la[tau][1] = kLog2e * g1 + gg2;
            }
            if (nv < kGChunk) {  // a partial last chunk: tokens past its end add no decay
#pragma unroll
                for (int tau = 0; tau < 4; ++tau)
                    if (4 * tq + tau >= nv) la[tau][0] = la[tau][1] = 0.f;
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
            uint32_t kh[4];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const int t = 4 * tq + tau;
                const uint32_t qw = st[Cfg::ST_Q + stage_dw(t, pp, QNB)], kw = st[Cfg::ST_K + stage_dw(t, pp, QNB)];
                const float qv[2] = {bf16_lo(qw), bf16_hi(qw)}, kv[2] = {bf16_lo(kw), bf16_hi(kw)};
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    qh[tau][x] = qv[x] * hw_exp2(a[tau][x]);
                    kp[tau][x] = kv[x] * hw_exp2(off[x] - a[tau][x]);
                }
                kh[tau] = hi_pack(kp[tau][0], kp[tau][1]);
                kl[tau][0] = sub_bf16_lo(kh[tau], kp[tau][0]);
                kl[tau][1] = sub_bf16_hi(kh[tau], kp[tau][1]);
            }
            const int pd = gpos_dword(pp);
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                uint32_t* qr = d + Cfg::D_QH + (4 * tq + tau) * OPR + pd;
                uint32_t* kr = d + Cfg::D_KP + (4 * tq + tau) * OPR + pd;
                const uint32_t qhw = hi_pack(qh[tau][0], qh[tau][1]);
                qr[0] = qhw;
                qr[DK / 2] = lo_pack(qhw, qh[tau][0], qh[tau][1]);
                kr[0] = kh[tau];
                kr[DK / 2] = pack_bf16x2(kl[tau][0], kl[tau][1]);
            }
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
                    const uint32_t w = st[Cfg::ST_GV + stage_dw(t, qq, VNB)];
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
                    const uint32_t vw = st[Cfg::ST_V + stage_dw(t, qq, VNB)];
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
                    const uint32_t p0 = hi_pack(vp[0][x], vp[1][x]), p1 = hi_pack(vp[2][x], vp[3][x]);
                    const uint32_t t0 = hi_pack(vt[0][x], vt[1][x]), t1 = hi_pack(vt[2][x], vt[3][x]);
                    lds_store<u32x4>(d + Cfg::D_VP + row, u32x4{p0, p1, lo_pack(p0, vp[0][x], vp[1][x]),
                                                               lo_pack(p1, vp[2][x], vp[3][x])});
                    lds_store<u32x4>(d + Cfg::D_VT + row, u32x4{t0, t1, lo_pack(t0, vt[0][x], vt[1][x]),
                                                               lo_pack(t1, vt[2][x], vt[3][x])});
                }
            } else {  // v is exact in bf16: copy it token-minor, the four tokens twice
                // (the hi | lo k range of the intra term and of the state update meets
                // v's hi part twice, so the block is the MFMA operand as it stands)
                uint32_t w[4];
#pragma unroll
                for (int tau = 0; tau < 4; ++tau) w[tau] = st[Cfg::ST_V + stage_dw(4 * tq + tau, qq, VNB)];
                const uint32_t a0 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                               a1 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
                const uint32_t b0 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                               b1 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
                lds_store<u32x4>(d + Cfg::D_VT + vblk(2 * qq, tq), u32x4{a0, a1, a0, a1});
                lds_store<u32x4>(d + Cfg::D_VT + vblk(2 * qq + 1, tq), u32x4{b0, b1, b0, b1});
            }
        }
    };

    // Exact intra term of a wide chunk (producer waves; the matrix waves, which hold
    // the state in registers, only meet its three barriers in exact_wait): the summed
    // decays A and B of every channel from the staged gates (the prep keeps its own
    // only in registers, since few chunks come this way), then W, then
    // OI = W (v .* 2^{B_t - B_u}).  A, B and W live in derived(c + 1), which no wave
    // touches until the prep of chunk c + 1 starts after the last barrier here.
    auto exact_wait = [&]() __attribute__((always_inline)) {
        lds_barrier();
        lds_barrier();
        lds_barrier();
    };
    auto exact_chunk = [&](int c) __attribute__((always_inline)) {
        const uint32_t* st = staged(c);
        const int nv = chunk_nv(c);
        float* Af = reinterpret_cast<float*>(derived(c + 1) + Cfg::X_A);
        float* Bf = reinterpret_cast<float*>(derived(c + 1) + Cfg::X_B);
        float* Wf = reinterpret_cast<float*>(derived(c + 1) + Cfg::X_W);
        for (int i = ptid; i < DK + (has_gv ? BV : 0); i += PT) {
            float acc = 0.f;
            if (i < DK) {
                for (int t = 0; t < kGChunk; ++t) {
                    float gi;
                    if constexpr (GF32) gi = reinterpret_cast<const float*>(st + Cfg::ST_G)[stage_fl(t, i, GNB)];
                    else gi = bf16_half(st[Cfg::ST_G + stage_dw(t, i >> 1, QNB)], i & 1);
                    acc += t < nv ? kLog2e * gi + gg2 : 0.f;
                    Af[t * AR + i] = acc;
                }
            } else {
                const int j = i - DK;
                for (int t = 0; t < kGChunk; ++t) {
                    acc += t < nv ? kLog2e * bf16_half(st[Cfg::ST_GV + stage_dw(t, j >> 1, VNB)], j & 1) : 0.f;
                    Bf[t * BR + j] = acc;
                }
            }
        }
        lds_barrier();
        for (int e = ptid; e < kGChunk * kGChunk; e += PT) {
            const int t = e >> 4, u = e & 15;
            float w = 0.f;
            if (u <= t) {
                const float* at = Af + t * AR;
                const float* au = Af + u * AR;
#pragma unroll 2
                for (int i = 0; i < DK; i += 4) {  // dwords i/2, i/2 + 1 share a staged block
                    const u32x2 q2 = lds_load<u32x2>(st + Cfg::ST_Q + stage_dw(t, i / 2, QNB));
                    const u32x2 k2 = lds_load<u32x2>(st + Cfg::ST_K + stage_dw(u, i / 2, QNB));
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
        for (int e = ptid; e < kGChunk * BV; e += PT) {
            const int t = e / BV, jj = e % BV;
            const float bt = has_gv ? Bf[t * BR + jj] : 0.f;
            float acc = 0.f;
            for (int u = 0; u <= t; ++u) {
                const float vu = bf16_half(st[Cfg::ST_V + stage_dw(u, jj >> 1, VNB)], jj & 1);
                const float dd = has_gv ? hw_exp2(bt - Bf[u * BR + jj]) : 1.f;
                acc += Wf[t * 17 + u] * vu * dd;
            }
            OIf[t * BR + jj] = acc;
        }
        lds_barrier();
    };

    // Matrix phase of chunk c (matrix waves) over this wave's half of dk: returns its
    // share of the chunk's output tile (with DS = 2 the pair's shares add up to it;
    // the products are linear in the dk contraction, W's causal mask and bf16 split
    // included) and advances its state rows.
    auto matrix_chunk = [&](int c) __attribute__((always_inline)) -> f32x4 {
        const uint32_t* d = derived(c);
        const uint32_t* QHw = d + Cfg::D_QH + lr * OPR + 4 * lg + 16 * KBW * h;
        const uint32_t* KPw = d + Cfg::D_KP + lr * OPR + 4 * lg + 16 * KBW * h;
        const float* BTf = reinterpret_cast<const float*>(d + Cfg::D_BT);
        // Inter-chunk part (q .* 2^A) S: the state tile pair (2s, 2s+1), split into
        // bf16 hi + lo, is the B operand of dk block s.  W^T = (k ./ e) (q .* e)^T in
        // the same loop (q .* e is its B operand too); lane holds W[t = lr][u = 4lg + ii].
        // One accumulator per product: consecutive MFMAs accumulate in place.
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 O = z, W = z;
        const int vrow_j = vblk(j, lg);
#pragma unroll
        for (int s = 0; s < KBW; ++s) {
            const uint32_t* qr = QHw + 16 * s;
            const uint32_t* kr = KPw + 16 * s;
            const u32x4 qh = lds_load<u32x4>(qr), ql = lds_load<u32x4>(qr + DK / 2);
            const u32x4 kh = lds_load<u32x4>(kr), kl = lds_load<u32x4>(kr + DK / 2);
            const f32x4 s0 = S[2 * s], s1 = S[2 * s + 1];
            const u32x4 sh = {hi_pack(s0[0], s0[1]), hi_pack(s0[2], s0[3]), hi_pack(s1[0], s1[1]),
                              hi_pack(s1[2], s1[3])};
            const u32x4 sl = {lo_pack(sh[0], s0[0], s0[1]), lo_pack(sh[1], s0[2], s0[3]),
                              lo_pack(sh[2], s1[0], s1[1]), lo_pack(sh[3], s1[2], s1[3])};
            O = mfma_bf16_w(qh, sh, O);
            W = mfma_bf16_w(kh, qh, W);
            O = mfma_bf16_w(qh, sl, O);
            W = mfma_bf16_w(kh, ql, W);
            O = mfma_bf16_w(ql, sh, O);
            W = mfma_bf16_w(kl, qh, W);
        }
        // The chunk's path, read only now so that the products above do not wait for
        // it (W is wasted on a wide chunk; those are rare).  A wide chunk's exact intra
        // term comes from the producers, whose three barriers this wave meets here.
        const bool fast = wide_flag[c % 3] == 0;
        if (fast) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                if (4 * lg + ii > lr) W[ii] = 0.f;  // causal: u <= t
            // Intra term W (v .* 2^{-B}): k = 8lg + e covers the tokens 4lg + (e & 3)
            // with W's hi (e < 4) and lo (e >= 4) parts, against v's hi part twice.
            const u32x4 vpx = lds_load<u32x4>(d + (has_gv ? Cfg::D_VP : Cfg::D_VT) + vrow_j);
            const uint32_t w0 = hi_pack(W[0], W[1]), w1 = hi_pack(W[2], W[3]);
            const u32x4 wa = {w0, w1, lo_pack(w0, W[0], W[1]), lo_pack(w1, W[2], W[3])};
            f32x4 Oi = mfma_bf16_w(wa, has_gv ? u32x4{vpx[0], vpx[1], vpx[0], vpx[1]} : vpx, z);
            if (has_gv) Oi = mfma_bf16_half(wa[0], wa[1], vpx[2], vpx[3], Oi);
            O += Oi;
            if (has_gv) O *= lds_load<f32x4>(BTf + vrow_j);
        } else {
            exact_wait();
            if (has_gv) O *= lds_load<f32x4>(BTf + vrow_j);
            if (h == 0) {  // the exact intra term, once per pair
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) O[ii] += OIf[(4 * lg + ii) * BR + j];
            }
        }

        // State update of this wave's rows: S <- post .* (pre .* 2^{B_15}^T .* S +
        // kp^T vt), contracting over the 16 tokens with kp's hi and lo parts in one k
        // range.  kp^T comes from transposing reads of the token-major key rows: lane
        // group lg takes tokens 4lg .. 4lg+3; lane s of the group addresses token row
        // 4lg + (s >> 2) at the four positions of channels 16mt + 4(s & 3) .. +3, so
        // lane lr receives channel 16mt + lr (the position map of gpos_dword).
        const float* PREf = reinterpret_cast<const float*>(d + Cfg::D_PRE);
        const float* POSTf = reinterpret_cast<const float*>(d + Cfg::D_POST);
        const float eb = has_gv ? reinterpret_cast<const float*>(d + Cfg::D_EB)[j] : 1.f;
        if (!fast) {
#pragma unroll
            for (int m = 0; m < MTW; ++m) {
                const f32x4 pre = lds_load<f32x4>(PREf + 16 * (h * MTW + m) + 4 * lg);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) S[m][ii] *= pre[ii] * eb;
            }
        } else if (has_gv) {
#pragma unroll
            for (int m = 0; m < MTW; ++m) S[m] *= eb;
        }
        // Every operand is read first (the gated branch below would otherwise split
        // the reads into one wait per tile).
        const u32x4 vtx = lds_load<u32x4>(d + Cfg::D_VT + vrow_j);
        const u32x4 vt2 = has_gv ? u32x4{vtx[0], vtx[1], vtx[0], vtx[1]} : vtx;
        const uint16_t* ktr = reinterpret_cast<const uint16_t*>(d + Cfg::D_KP) + (4 * lg + (lr >> 2)) * (2 * OPR) +
                              8 * (lr & 3) + 32 * KBW * h;
        u32x4 ktx[MTW];
        f32x4 post[MTW];
#pragma unroll
        for (int m = 0; m < MTW; ++m) {
            const uint16_t* kt = ktr + 32 * (m >> 1) + 4 * (m & 1);  // tile h MTW + m (MTW is even)
            const u32x2 khi = lds_tr16(kt), klo = lds_tr16(kt + DK);
            ktx[m] = u32x4{khi[0], khi[1], klo[0], klo[1]};
            post[m] = lds_load<f32x4>(POSTf + 16 * (h * MTW + m) + 4 * lg);
        }
#pragma unroll
        for (int m = 0; m < MTW; ++m) S[m] = mfma_bf16_w(ktx[m], vt2, S[m]);
        if (has_gv) {
#pragma unroll
            for (int m = 0; m < MTW; ++m) S[m] = mfma_bf16_half(ktx[m][0], ktx[m][1], vtx[2], vtx[3], S[m]);
        }
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) S[m][ii] *= post[m][ii];
        return O;
    };
    // Output rows of chunk c from its finished tile.
    auto store_out = [&](int c, const f32x4& O) __attribute__((always_inline)) {
        const int nv = chunk_nv(c);
        const int64_t orow = (int64_t)H * dv;
        char* ob = reinterpret_cast<char*>(p.o + (chunk_low(c, nv) * orow + (int64_t)wk.h * dv + wk.vb * BV));
        if (nv == kGChunk) {  // (uniform) no row to skip
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                *reinterpret_cast<float*>(ob + 4 * (lrow(4 * lg + ii, kGChunk) * (uint32_t)orow + j)) = p.scale * O[ii];
        } else {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int t = 4 * lg + ii;
                if (t < nv) *reinterpret_cast<float*>(ob + 4 * (lrow(t, nv) * (uint32_t)orow + j)) = p.scale * O[ii];
            }
        }
    };
    // The partial output tile that wave h = 1 of column block w hands over for chunk c.
    auto xo = [&](int c) __attribute__((always_inline)) -> float* {
        return reinterpret_cast<float*>(sm + Cfg::OFF_XO + (((c & 1) * NW + w) * 64 + lane) * 4);
    };

    // Pipeline: before the barrier that opens step c, the producers have derived chunk
    // c and the copies of chunk c+1 have landed.  During step c the matrix waves
    // compute chunk c while the producers derive chunk c+1 and then issue the copies
    // of chunk c+NST into the stage chunk c used (chunks c+2 .. c+NST-1 are in
    // flight meanwhile).  A wide chunk first takes the exact path with all waves,
    // before its stage is reused.  Chunk flags cycle through three slots: slot
    // (c+2) mod 3 is cleared during step c, after every read of chunk c-1's flag and
    // before chunk c+2's prep.  The two roles run separate loops with the same
    // barriers in the same order.
    if (producer) {
        if (ptid == 0) wide_flag[0] = wide_flag[1] = wide_flag[2] = 0;
#pragma unroll
        for (int m = 0; m < NST; ++m) issue_chunk(m);
        wait_vmem<DEPTH * CPW>();  // this wave's copies of chunk 0 have landed
        lds_barrier();
        if (nch > 0) prep_chunk(0);
        for (int c = 0; c < nch; ++c) {
            wait_vmem<(DEPTH - 1) * CPW>();  // ... of chunk c+1
            lds_barrier();  // chunk c derived, chunk c+1 staged, chunk c's flag final
            if (wide_flag[c % 3] != 0) exact_chunk(c);
            if (c + 1 < nch) {
                if (ptid == 0) wide_flag[(c + 2) % 3] = 0;
                prep_chunk(c + 1);
            }
            issue_chunk(c + NST);
        }
        if constexpr (DS == 2) lds_barrier();  // the matrix waves' last hand-over
        wait_vmem<0>();  // no copy lands after the workgroup ends
    } else {
        // With DS = 2, wave h = 1 leaves its share of chunk c in LDS; after the next
        // barrier wave h = 0 adds it to its own and stores the chunk, one step later
        // (a last barrier after the loop hands over the final chunk).
        lds_barrier();
        f32x4 Oh = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < nch; ++c) {
            lds_barrier();
            // (DS = 2, h = 0) the partner's share of chunk c - 1 (at c = 0 the other
            // parity's slot, read but not used)
            f32x4 prev;
            if constexpr (DS == 2) {
                if (h == 0) prev = lds_load<f32x4>(xo(c - 1));
            }
            const f32x4 O = matrix_chunk(c);
            if constexpr (DS == 2) {
                if (h == 1) {
                    lds_store<f32x4>(xo(c), O);
                } else {
                    if (c > 0) store_out(c - 1, Oh + prev);
                    Oh = O;
                }
            } else {
                store_out(c, O);
            }
        }
        if constexpr (DS == 2) {
            lds_barrier();
            if (h == 0 && nch > 0) store_out(nch - 1, Oh + lds_load<f32x4>(xo(nch - 1)));
        }
    }

    if (!producer && p.final_state) {
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.final_state[st_off + (int64_t)(16 * (h * MTW + m) + 4 * lg + ii) * dv + vcol] = S[m][ii];
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

}  // namespace

namespace {
template <int DK, int NW>
hipError_t launch_gated_t(const FwdParams& p, bool bf16, hipStream_t s) {
    const dim3 grid(fwd_grid_size(p));
    // bf16: NW matrix waves plus 2 NW producer waves; fp32: NW waves
    const dim3 block_bf16(GatedBCfg<DK, NW, false>::NT), block_f32(64 * NW);
    const bool gv = p.gv != nullptr;
    if (bf16 && p.gk_is_f32 && gv)
        hipLaunchKernelGGL((gated_bf16_kernel<DK, NW, true, true>), grid, block_bf16, 0, s, p);
    else if (bf16 && p.gk_is_f32)
        hipLaunchKernelGGL((gated_bf16_kernel<DK, NW, true, false>), grid, block_bf16, 0, s, p);
    else if (bf16 && gv)
        hipLaunchKernelGGL((gated_bf16_kernel<DK, NW, false, true>), grid, block_bf16, 0, s, p);
    else if (bf16)
        hipLaunchKernelGGL((gated_bf16_kernel<DK, NW, false, false>), grid, block_bf16, 0, s, p);
    else
        hipLaunchKernelGGL((gated_f32_kernel<DK, NW>), grid, block_f32, 0, s, p);
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

}  // namespace lattn
