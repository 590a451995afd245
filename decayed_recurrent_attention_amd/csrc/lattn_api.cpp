// C ABI of liblattn.so: argument validation, kernel selection and launch.
// Every check that needs no GPU runs before the first HIP call, so argument
// errors are reported identically on machines without a device.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <initializer_list>
#include <climits>
#include <cstdint>
#include <cstring>

#include "lattn.h"
#include "lattn_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// Per device: 0 = not checked yet, 1 = gfx950, -1 = other.
std::atomic<int> g_device_ok[kMaxDevices];

// Forced kernel choices (lattn_set_knob); LATTN_KNOB_AUTO = the choice from the shape.
constexpr int kNumKnobs = 3;
std::atomic<int> g_knob[kNumKnobs] = {LATTN_KNOB_AUTO, LATTN_KNOB_AUTO, LATTN_KNOB_AUTO};
int knob(int which) { return g_knob[which].load(std::memory_order_relaxed); }

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

bool is_varlen(const lattn_problem& p) { return p.num_seqs > 0; }

int num_seqs_of(const lattn_problem& p) { return is_varlen(p) ? p.num_seqs : p.batch; }

// A kernel exists for head dims (dk, dv) of dtype `in_dtype` at some width.
bool have_dims(int in_dtype, int dk, int dv) {
    if (dv % 16 != 0 || dv > 256) return false;
    for (int nw : {1, 2, 4})
        if (lattn::have_fwd_kernel(in_dtype, dk, nw) && (dv / 16) % nw == 0) return true;
    return false;
}

// Shape/dtype checks that do not look at pointers.  A bf16 o is accepted where the
// caller allows it (the forward) and only for bf16 input.
int check_problem(const lattn_problem& p, bool bf16_out_ok = false) {
    if (p.batch < 1 || p.seqlen < 0 || p.num_heads < 1 || p.num_kv_heads < 1 || p.head_dim_qk < 1 ||
        p.head_dim_v < 1 || p.num_seqs < 0)
        return LATTN_ERR_INVALID_ARG;
    if (p.num_heads % p.num_kv_heads != 0) return LATTN_ERR_HEADS;
    if (is_varlen(p) && p.batch != 1) return LATTN_ERR_VARLEN_BATCH;
    if (p.in_dtype != LATTN_BF16 && p.in_dtype != LATTN_F32) return LATTN_ERR_UNSUPPORTED;
    const bool bf16_out = bf16_out_ok && p.in_dtype == LATTN_BF16 && p.out_dtype == LATTN_BF16;
    if (p.out_dtype != LATTN_F32 && !bf16_out) return LATTN_ERR_UNSUPPORTED;
    if (!have_dims(p.in_dtype, p.head_dim_qk, p.head_dim_v)) return LATTN_ERR_UNSUPPORTED;
    // The chunked kernels address the 64 token rows of a chunk with 32-bit signed byte
    // offsets from the chunk's first row: the widest row (an fp32 row of o, q, dq or dk
    // over all query heads) times 64 must stay below 2^31.
    if ((int64_t)p.num_heads * std::max(p.head_dim_qk, p.head_dim_v) * 4 * lattn::kChunk > INT32_MAX)
        return LATTN_ERR_UNSUPPORTED;
    return LATTN_OK;
}

// The gated recurrence: chunks of 16 tokens, dk 32, 64 or 128, value blocks of 64
// columns when dv allows, else 16.
int gated_nw(int dv) { return dv % 64 == 0 ? 4 : 1; }

int check_gated_problem(const lattn_problem& p) {
    if (p.batch < 1 || p.seqlen < 0 || p.num_heads < 1 || p.num_kv_heads < 1 || p.head_dim_qk < 1 ||
        p.head_dim_v < 1 || p.num_seqs < 0)
        return LATTN_ERR_INVALID_ARG;
    if (p.num_heads % p.num_kv_heads != 0) return LATTN_ERR_HEADS;
    if (is_varlen(p) && p.batch != 1) return LATTN_ERR_VARLEN_BATCH;
    if (p.in_dtype != LATTN_BF16 && p.in_dtype != LATTN_F32) return LATTN_ERR_UNSUPPORTED;
    if (p.out_dtype != LATTN_F32) return LATTN_ERR_UNSUPPORTED;
    if (p.head_dim_v % 16 != 0 || p.head_dim_v > 256) return LATTN_ERR_UNSUPPORTED;
    if (!lattn::have_gated_kernel(p.head_dim_qk, gated_nw(p.head_dim_v))) return LATTN_ERR_UNSUPPORTED;
    // the kernel addresses 16 token rows of any array with 32-bit byte offsets
    if ((int64_t)p.num_heads * std::max(p.head_dim_qk, p.head_dim_v) >= (int64_t(1) << 25))
        return LATTN_ERR_UNSUPPORTED;
    return LATTN_OK;
}

// The backward also runs the kernel with the head dims swapped.
int check_bwd_problem(const lattn_problem& p) {
    const int rc = check_problem(p);
    if (rc != LATTN_OK) return rc;
    if (!have_dims(p.in_dtype, p.head_dim_v, p.head_dim_qk)) return LATTN_ERR_UNSUPPORTED;
    return LATTN_OK;
}

// Workgroup width (waves) for a problem: the widest value block (fewer re-reads of
// Q and K) that still yields at least one workgroup per compute unit; small
// problems fall back to narrower blocks for more parallel workgroups.
int choose_nw(int in_dtype, int dk, int dv, int64_t heads) {
    const int units = dv / 16;
    auto usable = [&](int nw) { return units % nw == 0 && lattn::have_fwd_kernel(in_dtype, dk, nw); };
    if (const int want = knob(LATTN_KNOB_WAVES); want != LATTN_KNOB_AUTO) {
        if ((want == 1 || want == 2 || want == 4) && usable(want)) return want;
    }
    int narrowest = 0;
    for (int nw : {4, 2, 1}) {
        if (!usable(nw)) continue;
        if (heads * (units / nw) >= 256) return nw;
        narrowest = nw;
    }
    return narrowest;
}

int device_check() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LATTN_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known != 0) return known > 0 ? LATTN_OK : LATTN_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LATTN_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? LATTN_OK : LATTN_ERR_DEVICE;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch parameters for one run of the chunked kernel over problem p with head dims
// (dk, dv) of its operands (the forward's, or swapped for a gradient sweep).
// Returns false when the grid would not fit an int.
bool make_params(const lattn_problem& p, int dk, int dv, int nw, const float* g_gamma, float scale,
                 const int32_t* cu, const int32_t* order, lattn::FwdParams& fp, int num_seqs = -1) {
    fp = lattn::FwdParams{};
    fp.g_gamma = g_gamma;
    fp.cu = cu;
    fp.order = order;
    fp.batch = p.batch;
    fp.seqlen = p.seqlen;
    fp.num_heads = p.num_heads;
    fp.num_kv_heads = p.num_kv_heads;
    fp.dk = dk;
    fp.dv = dv;
    fp.num_seqs = num_seqs < 0 ? num_seqs_of(p) : num_seqs;
    fp.nvb = dv / (16 * nw);
    if ((int64_t)fp.num_seqs * p.num_kv_heads > INT_MAX) return false;
    fp.num_groups = fp.num_seqs * p.num_kv_heads;
    fp.group_size = (p.num_heads / p.num_kv_heads) * fp.nvb;
    fp.scale = scale;
    lattn::set_forward_defaults(fp);
    const int64_t grid = (int64_t)lattn::kNumXcd * ((fp.num_groups + lattn::kNumXcd - 1) / lattn::kNumXcd) *
                         fp.group_size;
    return grid <= INT_MAX;
}

int64_t heads_of(const lattn_problem& p) { return (int64_t)num_seqs_of(p) * p.num_heads; }

// Intra-sequence split of a bf16 forward: sequences are cut into segments (a multiple
// of the chunk) that run in parallel.  A state-only pass gives every segment but a
// sequence's last its own state contribution, a scan chains them into the state
// entering each segment, and the main pass runs every segment from that state.
//  - Fixed length: every batch row is cut into P segments of seg_len tokens when the
//    (row, head) pairs are too few to fill the GPU.
//  - Packed input: a planner kernel reads cu_seqlens on the device and cuts only the
//    sequences longer than the balanced load per compute unit (skewed lengths).
struct Split {
    int P = 0;            // fixed length: segments per row (0: no split)
    int seg_len = 0;      // fixed length: tokens per segment
    bool chain = false;   // fixed length: the main pass chains the slots (no scan)
    bool packed = false;  // packed input: the device-planned split runs
    int forced = 0;       // packed: segments per sequence forced by the knob (0: balance)
    int wgs = 0;          // packed: workgroups per segment (heads x value blocks)
    int min_seg = 0;      // packed: shortest segment in chunks
    int max_slots = 0;    // packed: capacity of the state slots and the state-only list
    int max_main = 0;     // packed: capacity of the main-pass list
};

// Shortest segment worth a state-only pass and a scan: 4 chunks up to dk 128, 8 above
// (those cost more at dk 192 and 256).
int min_seg_chunks(int dk) { return dk <= 128 ? 4 : 8; }

constexpr int kMaxMainChain = 15;

Split choose_split(const lattn_problem& p, int nw) {
    Split sp;
    if (is_varlen(p) || p.in_dtype != LATTN_BF16 || p.seqlen < 2 * lattn::kChunk) return sp;
    if ((int64_t)p.batch * p.num_heads * 64 > INT_MAX) return sp;  // the scan's grid
    const int64_t wgs = (int64_t)p.batch * p.num_heads * (p.head_dim_v / (16 * nw));
    int want;
    if (const int forced = knob(LATTN_KNOB_SPLIT); forced != LATTN_KNOB_AUTO) {  // forced segment count
        want = forced;
        if (want < 2) return sp;
    } else {
        if (wgs >= 128) return sp;  // at least half the compute units busy already
        // As many segments as keep the main pass to one workgroup per compute unit: a
        // second round costs more than the parallelism gains.  Measured (one box, us,
        // by segment count): B2 H12 d192 N2048 (72 workgroups) 93 / 75 / 60 / 75 for
        // 1 / 2 / 3 / 4; B2 H8 d256 N4096 (64) 206 / 153 / 114 / 94 / 100 for 1 / 2 / 3 /
        // 4 / 8; B2 H8 d64 N2048 (16) 58 / 42 / 25 / 26 for 1 / 2 / 8 / 16.
        want = (int)std::max<int64_t>(2, lattn::kNumCu / wgs);
        const int cap = p.seqlen / (min_seg_chunks(p.head_dim_qk) * lattn::kChunk);
        if (want > cap) want = cap;
        if (want < 2) return sp;
    }
    const int chunks = (p.seqlen + lattn::kChunk - 1) / lattn::kChunk;
    if (want > chunks) want = chunks;
    sp.seg_len = ((chunks + want - 1) / want) * lattn::kChunk;
    sp.P = (p.seqlen + sp.seg_len - 1) / sp.seg_len;
    if (sp.P < 2) return Split{};
    // Up to 15 earlier segments, the main pass chains the slots itself (four loads at a
    // time), which saves the scan launch: measured B2 H8 d64 N2048 (P 8) 24.5 -> 20.2 us,
    // B1 H8 d128 N32768 (P 16) 98.5 -> 96.0 us.  With more, every workgroup's start grows
    // and the slot reads grow with P^2, so the scan chains them in parallel instead.
    sp.chain = sp.P - 1 <= kMaxMainChain;
    return sp;
}

// Packed input: the planner's bounds.  Balanced mode cuts sequences longer than 5/4 of
// Lb = J * sum(chunks) / kNumCu into segments of at least Lb / 2 chunks, so at most
// 2 kNumCu / J + 1 state slots are used (J = workgroups per segment); forced mode
// cuts every sequence into at most `forced` segments.  The planner lists at most
// kMaxPlanSegs segments.
Split choose_packed_split(const lattn_problem& p, int nw) {
    Split sp;
    if (!is_varlen(p) || p.in_dtype != LATTN_BF16 || p.num_seqs > lattn::kMaxPlanSeqs) return sp;
    const int wgs = p.num_heads * (p.head_dim_v / (16 * nw));
    const int forced = knob(LATTN_KNOB_SPLIT);
    if (forced != LATTN_KNOB_AUTO && forced < 2) return sp;
    if (forced == LATTN_KNOB_AUTO && wgs >= lattn::kNumCu) return sp;  // Lb >= every sequence: nothing to cut
    sp.packed = true;
    sp.forced = forced == LATTN_KNOB_AUTO ? 0 : forced;
    sp.wgs = wgs;
    sp.min_seg = min_seg_chunks(p.head_dim_qk);
    const int64_t slots = sp.forced ? (int64_t)p.num_seqs * (sp.forced - 1)
                                    : 2 * ((lattn::kNumCu + wgs - 1) / wgs) + 2;
    if (slots < 1 || slots + p.num_seqs > lattn::kMaxPlanSegs) return Split{};  // the planner's segment table
    sp.max_slots = (int)slots;
    sp.max_main = p.num_seqs + sp.max_slots;
    return sp;
}

// Width and split of a forward launch: a split run uses the widest workgroups (most
// waves per compute unit) and makes up the count with segments.
int widest_nw(int in_dtype, int dk, int dv) {
    for (int nw : {4, 2, 1})
        if ((dv / 16) % nw == 0 && lattn::have_fwd_kernel(in_dtype, dk, nw)) return nw;
    return 0;
}

Split plan_forward(const lattn_problem& p, int& nw) {
    const int wide = widest_nw(p.in_dtype, p.head_dim_qk, p.head_dim_v);
    const Split sp = is_varlen(p) ? choose_packed_split(p, wide) : choose_split(p, wide);
    nw = (sp.P > 0 || sp.packed) ? wide : choose_nw(p.in_dtype, p.head_dim_qk, p.head_dim_v, heads_of(p));
    return sp;
}

size_t state_block_bytes(const lattn_problem& p) {
    return (size_t)p.num_heads * p.head_dim_qk * p.head_dim_v * sizeof(float);
}

// Workspace of a split forward: [plan (packed only)][state slots], each 256-byte aligned.
size_t split_plan_bytes(const Split& sp) {
    if (!sp.packed) return 0;
    const size_t words = lattn::kPlanHeader + (size_t)lattn::kPlanEntry * (sp.max_main + sp.max_slots);
    return round_up(words * sizeof(int32_t), 256);
}
size_t split_slot_count(const lattn_problem& p, const Split& sp) {
    return sp.packed ? (size_t)sp.max_slots : (size_t)p.batch * (sp.P - 1);
}
size_t split_workspace_bytes(const lattn_problem& p, const Split& sp) {
    return split_plan_bytes(sp) + round_up(split_slot_count(p, sp) * state_block_bytes(p), 256);
}

// Byte offsets of the backward workspace regions (each 256-byte aligned).
struct BwdLayout {
    size_t order = 0, part = 0, total = 0;
};
BwdLayout bwd_layout(const lattn_problem& p) {
    BwdLayout l;
    size_t off = 0;
    if (is_varlen(p) && p.num_seqs <= lattn::kMaxOrderedSeqs) {
        l.order = off;
        off += round_up((size_t)p.num_seqs * sizeof(int32_t), 256);
    }
    const size_t rows = (size_t)p.batch * (size_t)p.seqlen;
    if (p.num_heads > p.num_kv_heads) {
        l.part = off;
        const int d = p.head_dim_qk > p.head_dim_v ? p.head_dim_qk : p.head_dim_v;
        off += round_up(rows * p.num_heads * d * 4, 256);
    }
    l.total = off;
    return l;
}

}  // namespace

extern "C" {

int lattn_abi_version(void) { return 5; }

int lattn_set_knob(int which, int value, int* previous) {
    if (which < 0 || which >= kNumKnobs) return LATTN_ERR_INVALID_ARG;
    if (value != LATTN_KNOB_AUTO && value < 0) return LATTN_ERR_INVALID_ARG;
    const int old = g_knob[which].exchange(value, std::memory_order_relaxed);
    if (previous != nullptr) *previous = old;
    return LATTN_OK;
}

const char* lattn_status_string(int status) {
    switch (status) {
        case LATTN_OK: return "success";
        case LATTN_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or misaligned buffer)";
        case LATTN_ERR_VARLEN_BATCH: return "batch size must be 1 when cu_seqlens is given";
        case LATTN_ERR_HEADS: return "num_heads must be a multiple of num_kv_heads";
        case LATTN_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
        case LATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case LATTN_ERR_LAUNCH: return "kernel launch failed";
        case LATTN_ERR_DEVICE: return "no usable gfx950 device";
        default: return "unknown status";
    }
}

size_t lattn_fwd_workspace_size(const lattn_problem* p) {
    if (p == nullptr || check_problem(*p, true) != LATTN_OK) return 0;
    int nw = 0;
    const Split sp = plan_forward(*p, nw);
    if (sp.P > 0 || sp.packed) return split_workspace_bytes(*p, sp);
    if (!is_varlen(*p) || p->num_seqs > lattn::kMaxOrderedSeqs) return 0;
    return round_up((size_t)p->num_seqs * sizeof(int32_t), 256);
}

int lattn_lightning_g_gamma(int num_heads, int layer_idx, int num_layers, float* out_host) {
    if (num_heads < 1 || num_layers < 1 || layer_idx < 0 || layer_idx > num_layers || out_host == nullptr)
        return LATTN_ERR_INVALID_ARG;
    // Coefficient in double (a Python float on the page), rounded to float32; the
    // product with the float32 head index is a float32 product.
    const double coef = -(8.0 / (double)num_heads * (1.0 - (double)layer_idx / (double)num_layers));
    const float coef32 = (float)coef;
    for (int h = 0; h < num_heads; ++h) {
        volatile float hv = (float)h;
        out_host[h] = coef32 * hv;
    }
    return LATTN_OK;
}

int lattn_fwd(const lattn_problem* p, const void* q, const void* k, const void* v, const float* g_gamma,
              float scale, const float* initial_state, int reverse, const int32_t* cu_seqlens, void* o,
              float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    if (p == nullptr) return LATTN_ERR_INVALID_ARG;
    const int rc = check_problem(*p, true);
    if (rc != LATTN_OK) return rc;
    const int o_bf16 = p->out_dtype == LATTN_BF16 ? 1 : 0;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen != is_varlen(*p)) return LATTN_ERR_INVALID_ARG;
    const int64_t tokens = (int64_t)p->batch * p->seqlen;
    if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr))
        return LATTN_ERR_INVALID_ARG;
    if (g_gamma == nullptr || final_state == nullptr) return LATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(g_gamma, 4) ||
        !aligned(final_state, 16) || !aligned(initial_state, 16) || !aligned(cu_seqlens, 4) ||
        !aligned(workspace, 16))
        return LATTN_ERR_INVALID_ARG;
    const size_t need = lattn_fwd_workspace_size(p);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LATTN_ERR_WORKSPACE;

    int nw = 0;
    const Split sp = plan_forward(*p, nw);
    if (sp.P > 0 || sp.packed) {
        // state-only pass over every segment but each sequence's last -> slots; with
        // many segments of fixed length a scan -> the state entering each segment, in
        // place; main pass over every segment (chaining the slots itself otherwise).
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        int32_t* plan = sp.packed ? reinterpret_cast<int32_t*>(ws) : nullptr;
        float* slots = reinterpret_cast<float*>(ws + split_plan_bytes(sp));
        const int n_sonly = sp.packed ? sp.max_slots : p->batch * (sp.P - 1);
        const int n_main = sp.packed ? sp.max_main : p->batch * sp.P;
        lattn::FwdParams f1, f3;
        if (!make_params(*p, p->head_dim_qk, p->head_dim_v, nw, g_gamma, scale, nullptr, nullptr, f1, n_sonly) ||
            !make_params(*p, p->head_dim_qk, p->head_dim_v, nw, g_gamma, scale, nullptr, nullptr, f3, n_main))
            return LATTN_ERR_INVALID_ARG;
        for (lattn::FwdParams* f : {&f1, &f3}) {
            f->q = q;
            f->k = k;
            f->v = v;
            f->reverse = reverse != 0;
            f->slots = slots;
            f->plan = plan;
            f->plan_main = sp.max_main;
            f->plan_slots = sp.max_slots;
            f->seg_count = sp.P;
            f->seg_len = sp.seg_len;
            f->seg_chain = sp.chain ? 1 : 0;
        }
        f1.seg_phase = 1;
        f3.seg_phase = 2;
        f3.init = initial_state;
        f3.o = static_cast<float*>(o);
        f3.o_bf16 = o_bf16;
        f3.final_state = final_state;
        const int dc = device_check();
        if (dc != LATTN_OK) return dc;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (sp.packed &&
            lattn::launch_split_plan(cu_seqlens, p->num_seqs, p->seqlen, sp.wgs, sp.min_seg, sp.forced, reverse != 0,
                                     sp.max_main, sp.max_slots, plan, s) != hipSuccess)
            return LATTN_ERR_LAUNCH;
        if (n_sonly > 0 && lattn::launch_fwd(f1, p->in_dtype, nw, reverse != 0, s, true) != hipSuccess)
            return LATTN_ERR_LAUNCH;
        if (!sp.packed && !sp.chain && lattn::launch_seg_scan(slots, initial_state, g_gamma, p->batch, p->num_heads, sp.P,
                                                 sp.seg_len, (int64_t)p->head_dim_qk * p->head_dim_v, s) != hipSuccess)
            return LATTN_ERR_LAUNCH;
        if (lattn::launch_fwd(f3, p->in_dtype, nw, reverse != 0, s) != hipSuccess) return LATTN_ERR_LAUNCH;
        return LATTN_OK;
    }
    const int32_t* order = (varlen && need > 0) ? static_cast<const int32_t*>(workspace) : nullptr;
    lattn::FwdParams fp;
    if (!make_params(*p, p->head_dim_qk, p->head_dim_v, nw, g_gamma, scale, cu_seqlens, order, fp))
        return LATTN_ERR_INVALID_ARG;
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.init = initial_state;
    fp.o = static_cast<float*>(o);
    fp.o_bf16 = o_bf16;
    fp.final_state = final_state;

    const int dc = device_check();
    if (dc != LATTN_OK) return dc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fp.order != nullptr) {
        if (lattn::launch_seq_order(cu_seqlens, fp.num_seqs, p->seqlen, const_cast<int32_t*>(fp.order), s) !=
            hipSuccess)
            return LATTN_ERR_LAUNCH;
    }
    if (lattn::launch_fwd(fp, p->in_dtype, nw, reverse != 0, s) != hipSuccess) return LATTN_ERR_LAUNCH;
    return LATTN_OK;
}

size_t lattn_bwd_workspace_size(const lattn_problem* p) {
    if (p == nullptr || check_bwd_problem(*p) != LATTN_OK) return 0;
    return bwd_layout(*p).total;
}

int lattn_bwd(const lattn_problem* p, const void* q, const void* k, const void* v, const float* g_gamma,
              float scale, const float* initial_state, int reverse, const int32_t* cu_seqlens, const void* d_o,
              const float* d_final_state, float* dq, float* dk, float* dv, float* d_initial_state,
              void* workspace, size_t workspace_bytes, void* stream) {
    if (p == nullptr) return LATTN_ERR_INVALID_ARG;
    const int rc = check_bwd_problem(*p);
    if (rc != LATTN_OK) return rc;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen != is_varlen(*p)) return LATTN_ERR_INVALID_ARG;
    const int64_t tokens = (int64_t)p->batch * p->seqlen;
    if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || d_o == nullptr || dq == nullptr ||
                       dk == nullptr || dv == nullptr))
        return LATTN_ERR_INVALID_ARG;
    if (g_gamma == nullptr) return LATTN_ERR_INVALID_ARG;
    // The dk and dv sweeps carry D / scale, so scale must be finite, normal and nonzero.
    if (!(std::fabs(scale) >= 1.17549435e-38f && std::fabs(scale) <= 3.40282347e+38f)) return LATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) || !aligned(g_gamma, 4) ||
        !aligned(initial_state, 16) || !aligned(d_final_state, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(d_initial_state, 16) || !aligned(cu_seqlens, 4) || !aligned(workspace, 16))
        return LATTN_ERR_INVALID_ARG;
    const BwdLayout lay = bwd_layout(*p);
    if (lay.total > 0 && (workspace == nullptr || workspace_bytes < lay.total)) return LATTN_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const int32_t* order =
        (varlen && p->num_seqs <= lattn::kMaxOrderedSeqs) ? reinterpret_cast<const int32_t*>(ws + lay.order) : nullptr;
    const int dkd = p->head_dim_qk, dvd = p->head_dim_v;
    const bool grouped = p->num_heads > p->num_kv_heads;
    const void* dob = d_o;
    float* part = grouped ? reinterpret_cast<float*>(ws + lay.part) : nullptr;
    const float inv_scale = 1.0f / scale;
    const int64_t heads = heads_of(*p);

    // dq: the forward recurrence on (dO, V, K) with the transposed initial state.
    lattn::FwdParams pq, pk, pv;
    const int nw_q = choose_nw(p->in_dtype, dvd, dkd, heads);
    if (!make_params(*p, dvd, dkd, nw_q, g_gamma, scale, cu_seqlens, order, pq)) return LATTN_ERR_INVALID_ARG;
    pq.q = dob;
    pq.k = v;
    pq.v = k;
    pq.init = initial_state;
    pq.init_rs = 1;
    pq.init_cs = dvd;
    pq.o = dq;
    pq.final_state = nullptr;
    // dk: opposite direction on (V, dO, Q); the state is D^T / scale and d_final_state
    // enters at the first processed position.
    const int nw_k = nw_q;
    if (!make_params(*p, dvd, dkd, nw_k, g_gamma, scale, cu_seqlens, order, pk)) return LATTN_ERR_INVALID_ARG;
    pk.swap_heads = 1;
    pk.q = v;
    pk.k = dob;
    pk.v = q;
    pk.init = d_final_state;
    pk.init_rs = 1;
    pk.init_cs = dvd;
    pk.init_mul = inv_scale;
    pk.init_at_end = 1;
    pk.o = grouped ? part : dk;
    pk.final_state = nullptr;
    // dv: opposite direction on (K, Q, dO); the state is D / scale, and its final
    // value gives d_initial_state = lam * scale * state.
    const int nw_v = choose_nw(p->in_dtype, dkd, dvd, heads);
    if (!make_params(*p, dkd, dvd, nw_v, g_gamma, scale, cu_seqlens, order, pv)) return LATTN_ERR_INVALID_ARG;
    pv.swap_heads = 1;
    pv.q = k;
    pv.k = q;
    pv.v = dob;
    pv.init = d_final_state;
    pv.init_mul = inv_scale;
    pv.init_at_end = 1;
    pv.o = grouped ? part : dv;
    pv.final_state = d_initial_state;
    pv.final_mul = scale;
    pv.final_lam = 1;

    const int dc = device_check();
    if (dc != LATTN_OK) return dc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (order != nullptr &&
        lattn::launch_seq_order(cu_seqlens, p->num_seqs, p->seqlen, const_cast<int32_t*>(order), s) != hipSuccess)
        return LATTN_ERR_LAUNCH;
    const bool rev = reverse != 0;
    if (lattn::launch_fwd(pq, p->in_dtype, nw_q, rev, s) != hipSuccess) return LATTN_ERR_LAUNCH;
    // The dk and dv sweeps read the same Q and dO: with equal head dims (one kernel
    // shape) they run as one launch whose workgroups pair up per die, so the second
    // read of a tile mostly hits L2.  Knob LATTN_KNOB_BWD_PAIR = 0 keeps two launches.
    const bool pair = p->in_dtype == LATTN_BF16 && !grouped && dkd == dvd && nw_k == nw_v &&
                      knob(LATTN_KNOB_BWD_PAIR) != 0;
    if (pair) {
        if (lattn::launch_fwd_pair(pk, pv, nw_k, !rev, s) != hipSuccess) return LATTN_ERR_LAUNCH;
        return LATTN_OK;
    }
    if (lattn::launch_fwd(pk, p->in_dtype, nw_k, !rev, s) != hipSuccess) return LATTN_ERR_LAUNCH;
    if (grouped && lattn::launch_group_sum(part, dk, tokens, p->num_heads, p->num_kv_heads, dkd, s) != hipSuccess)
        return LATTN_ERR_LAUNCH;
    if (lattn::launch_fwd(pv, p->in_dtype, nw_v, !rev, s) != hipSuccess) return LATTN_ERR_LAUNCH;
    if (grouped && lattn::launch_group_sum(part, dv, tokens, p->num_heads, p->num_kv_heads, dvd, s) != hipSuccess)
        return LATTN_ERR_LAUNCH;
    return LATTN_OK;
}

int lattn_decode(const lattn_problem* p, const void* q, const void* k, const void* v, const float* g_gamma,
                 float scale, const float* state_in, float* state_out, void* o, void* stream) {
    if (p == nullptr) return LATTN_ERR_INVALID_ARG;
    if (p->batch < 1 || p->seqlen != 1 || p->num_seqs != 0 || p->num_heads < 1 || p->num_kv_heads < 1 ||
        p->head_dim_qk < 1 || p->head_dim_v < 1)
        return LATTN_ERR_INVALID_ARG;
    if (p->num_heads % p->num_kv_heads != 0) return LATTN_ERR_HEADS;
    if (p->in_dtype != LATTN_BF16 && p->in_dtype != LATTN_F32) return LATTN_ERR_UNSUPPORTED;
    if (p->out_dtype != LATTN_F32) return LATTN_ERR_UNSUPPORTED;
    if (p->head_dim_qk % 16 != 0 || p->head_dim_qk > 256 || p->head_dim_v % 16 != 0 || p->head_dim_v > 256)
        return LATTN_ERR_UNSUPPORTED;
    if (q == nullptr || k == nullptr || v == nullptr || g_gamma == nullptr || state_out == nullptr || o == nullptr)
        return LATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g_gamma, 4) || !aligned(state_in, 16) ||
        !aligned(state_out, 16) || !aligned(o, 16))
        return LATTN_ERR_INVALID_ARG;
    const int64_t blocks = (int64_t)p->batch * p->num_heads * (p->head_dim_v / lattn::decode_block(p->head_dim_v));
    if (blocks > INT_MAX) return LATTN_ERR_INVALID_ARG;
    lattn::DecodeParams dp;
    dp.q = q;
    dp.k = k;
    dp.v = v;
    dp.g_gamma = g_gamma;
    dp.state_in = state_in;
    dp.state_out = state_out;
    dp.o = static_cast<float*>(o);
    dp.batch = p->batch;
    dp.num_heads = p->num_heads;
    dp.num_kv_heads = p->num_kv_heads;
    dp.dk = p->head_dim_qk;
    dp.dv = p->head_dim_v;
    dp.scale = scale;
    const int dc = device_check();
    if (dc != LATTN_OK) return dc;
    if (lattn::launch_decode(dp, p->in_dtype, static_cast<hipStream_t>(stream)) != hipSuccess)
        return LATTN_ERR_LAUNCH;
    return LATTN_OK;
}

size_t lattn_fwd_gated_workspace_size(const lattn_problem* p, int gates) {
    if (p == nullptr || check_gated_problem(*p) != LATTN_OK) return 0;
    size_t bytes = 0;
    if (is_varlen(*p) && p->num_seqs <= lattn::kMaxOrderedSeqs) bytes += round_up((size_t)p->num_seqs * 4, 256);
    if ((gates & LATTN_GATE_G) && (gates & LATTN_GATE_GK))  // the two key gates are summed first
        bytes += round_up((size_t)p->batch * p->seqlen * p->num_heads * p->head_dim_qk * 4, 256);
    return bytes;
}

int lattn_fwd_gated(const lattn_problem* p, const void* q, const void* k, const void* v, const void* g,
                    const void* gk, const void* gv, const float* g_gamma, float scale, const float* initial_state,
                    int reverse, const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (p == nullptr) return LATTN_ERR_INVALID_ARG;
    const int rc = check_gated_problem(*p);
    if (rc != LATTN_OK) return rc;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen != is_varlen(*p)) return LATTN_ERR_INVALID_ARG;
    const int64_t tokens = (int64_t)p->batch * p->seqlen;
    if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr)) return LATTN_ERR_INVALID_ARG;
    if (final_state == nullptr) return LATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(gk, 16) ||
        !aligned(gv, 16) || !aligned(o, 16) || !aligned(g_gamma, 4) || !aligned(final_state, 16) ||
        !aligned(initial_state, 16) || !aligned(cu_seqlens, 4) || !aligned(workspace, 16))
        return LATTN_ERR_INVALID_ARG;
    const int gates = (g ? LATTN_GATE_G : 0) | (gk ? LATTN_GATE_GK : 0) | (gv ? LATTN_GATE_GV : 0);
    const size_t need = lattn_fwd_gated_workspace_size(p, gates);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LATTN_ERR_WORKSPACE;
    const int nw = gated_nw(p->head_dim_v);
    const bool ordered = varlen && p->num_seqs <= lattn::kMaxOrderedSeqs;
    const int32_t* order = ordered ? static_cast<const int32_t*>(workspace) : nullptr;
    float* gsum = (g && gk) ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                       (ordered ? round_up((size_t)p->num_seqs * 4, 256) : 0))
                            : nullptr;
    lattn::FwdParams fp;
    if (!make_params(*p, p->head_dim_qk, p->head_dim_v, nw, g_gamma, scale, cu_seqlens, order, fp))
        return LATTN_ERR_INVALID_ARG;
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.g = gsum ? static_cast<const void*>(gsum) : (g ? g : gk);
    fp.gk_is_f32 = gsum != nullptr;
    fp.gv = gv;
    fp.init = initial_state;
    fp.o = static_cast<float*>(o);
    fp.final_state = final_state;
    fp.reverse = reverse != 0;
    const int dc = device_check();
    if (dc != LATTN_OK) return dc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (order != nullptr &&
        lattn::launch_seq_order(cu_seqlens, fp.num_seqs, p->seqlen, const_cast<int32_t*>(order), s) != hipSuccess)
        return LATTN_ERR_LAUNCH;
    if (gsum != nullptr &&
        lattn::launch_gate_sum(g, gk, gsum, tokens * p->num_heads * p->head_dim_qk, p->in_dtype, s) != hipSuccess)
        return LATTN_ERR_LAUNCH;
    if (lattn::launch_gated(fp, p->in_dtype, nw, s) != hipSuccess) return LATTN_ERR_LAUNCH;
    return LATTN_OK;
}

}  // extern "C"
