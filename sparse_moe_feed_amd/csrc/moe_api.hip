// moe_api.hip -- the C ABI of libmoe: argument checks, workspace plan and
// the launch sequence of the sparse MoE feed-forward layer.
//
// Order of the layer (anatomy page on frontier-model-atlas, "Decoder
// microscope", Feed-forward panel): router logits, softmax, top-k routed
// experts, selected-weight normalisation; the shared expert runs alongside
// and is scaled by its own sigmoid gate.  moe_forward enqueues:
//   1. router logits + shared-gate column     (router.hip)
//   2. top-k, weights, gate                   (router.hip)
//   3. histogram / scan / permutation / tiles (permute.hip)
//   4. gate/up grouped GEMM -> h              (experts_*.hip)
//   5. down grouped GEMM -> weighted rows y, shared term -> out
//   6. combine: out[t] += sum_j y[row(t,j)]   (permute.hip)
#include "moe.h"
#include "moe_device.h"
#include "moe_kernels.h"

#include <algorithm>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

namespace {

thread_local std::string g_last_error;

// Events the next call on this thread records at its stage boundaries.
thread_local hipEvent_t g_stage_events[8];
thread_local int g_n_stage_events = 0;

// MOE_DEBUG_SYNC (environment, read at every stage boundary; unset, empty or
// "0" = off): the host waits for the stream after each stage, and the first
// stage whose kernels failed is named in moe_last_error (the call then
// returns MOE_ERR_HIP).  For finding a faulting kernel; not for streams under
// graph capture, and slow.
thread_local std::string g_debug_error;
thread_local const char *const *g_stage_names = nullptr;

const char *const kForwardStages[] = {
    "start", "router (RMSNorm if any, router logits, top-k selection, gate)",
    "permutation (histogram, scan, scatter, tile map)", "gate/up GEMM (h = silu(gate) * up)",
    "down GEMM (weighted rows y, shared term into out)", "combine (out += rows y)"};
const char *const kBackwardStages[] = {
    "start", "permutation and router logits", "gate/up recompute and G = W_dn^T dout",
    "SwiGLU and router backward", "dx of the routed rows", "dW_gate_up", "dW_down",
    "router GEMMs, dx combine and load-balancing loss"};

bool debug_sync_on() {
    const char *v = getenv("MOE_DEBUG_SYNC");
    return v && v[0] && strcmp(v, "0") != 0;
}

// Stage boundary i of the current call: its timing event, and under
// MOE_DEBUG_SYNC a wait that attributes any failure to stage i (the kernels
// enqueued since boundary i - 1).
void mark_stage(int i, hipStream_t s) {
    if (i < g_n_stage_events && g_stage_events[i]) (void)hipEventRecord(g_stage_events[i], s);
    if (i == 0) {
        g_debug_error.clear();
        return;
    }
    if (!g_debug_error.empty() || !debug_sync_on()) return;
    hipError_t err = hipStreamSynchronize(s);
    if (err == hipSuccess) err = hipPeekAtLastError();
    if (err != hipSuccess) {
        g_debug_error = std::string("MOE_DEBUG_SYNC: stage ") + std::to_string(i) + " failed";
        if (g_stage_names) g_debug_error += std::string(" (") + g_stage_names[i] + ")";
        g_debug_error += std::string(": ") + hipGetErrorString(err);
    }
}

// End of a call: forgets the stage events; a failure seen by MOE_DEBUG_SYNC
// outranks the launch status.
moe_status end_call(hipError_t err);

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_desc(const moe_desc *desc) {
    if (!desc) return MOE_ERR_INVALID_ARG;
    const moe_desc &d = *desc;
    if (d.d_model < 1 || d.n_experts < 1 || d.d_expert < 1 || d.d_shared < 0 || d.top_k < 1 ||
        d.top_k > d.n_experts)
        return MOE_ERR_INVALID_ARG;
    if (d.dtype != MOE_F32 && d.dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (d.flags != 0 && d.flags != MOE_FLAG_ROUTER_EXACT && d.flags != MOE_FLAG_ROUTER_SHORTLIST)
        return MOE_ERR_INVALID_ARG;
    if (d.flags == MOE_FLAG_ROUTER_SHORTLIST && d.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d.top_k > 32 || d.n_experts > 1024 || d.d_model > 16384) return MOE_ERR_UNSUPPORTED;
    if (d.dtype == MOE_BF16 &&
        (d.d_model % 64 != 0 || d.d_expert % 64 != 0 || d.d_shared % 64 != 0))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// T*(k+1) rows and T*(E+1) logits must stay within int32 indexing of rows.
moe_status check_T(const moe_desc *desc, int64_t T) {
    if (T < 0) return MOE_ERR_INVALID_ARG;
    const int64_t rows = T * (int64_t)(desc->top_k + 1);
    if (rows > (int64_t)0x7FFFFFFF / 2) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

struct Plan {
    size_t logits, wnorm, gate, counts, offsets, tile_start, tile_group, blk, rank, perm, h, h_shared, y,
        xnorm, total;
    int nblk;
    int max_tiles;
};

// The shortlist router serves bf16 layers of 128 tokens or more unless a
// flag picks a router.
bool uses_shortlist(const moe_desc &d, int64_t T) {
    return d.flags == MOE_FLAG_ROUTER_SHORTLIST || (d.flags == 0 && d.dtype == MOE_BF16 && T >= 128);
}

Plan make_plan(const moe_desc &d, int64_t T) {
    Plan p;
    const size_t esize = d.dtype == MOE_BF16 ? 2 : 4;
    const int64_t pairs = T * d.top_k;
    p.nblk = (int)((T + moe::kCountBlock - 1) / moe::kCountBlock);
    // tile map sized for the smaller of the two tile heights (the larger bound)
    p.max_tiles = (int)moe::max_gemm_tiles(T, d.top_k, d.n_experts, moe::kDecodeBM, d.d_shared > 0);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    p.logits = take((size_t)T * (d.n_experts + 1) * sizeof(float) *
                    (uses_shortlist(d, T) ? moe::shortlist_split(d.d_model) : 1));
    p.wnorm = take((size_t)d.n_experts * sizeof(float));
    p.gate = take((size_t)T * sizeof(float));
    p.counts = take((size_t)(d.n_experts + 1) * sizeof(int32_t));
    p.offsets = take((size_t)(d.n_experts + 1) * sizeof(int32_t));
    p.tile_start = take((size_t)(d.n_experts + 2) * sizeof(int32_t));
    p.tile_group = take((size_t)(p.max_tiles + 1) * sizeof(int32_t));
    p.blk = take((size_t)d.n_experts * p.nblk * sizeof(int32_t));
    p.rank = take((size_t)pairs * sizeof(int32_t));
    p.perm = take((size_t)pairs * sizeof(int32_t));
    p.h = take((size_t)pairs * d.d_expert * esize);
    p.h_shared = take((size_t)T * d.d_shared * esize);
    // binary32 rows where the weight-streaming path may serve the call (few
    // rows per expert) and for binary32 layers; 16-bit block floating point
    // rows from the grouped GEMMs otherwise
    const bool y_f32 = d.dtype != MOE_BF16 || pairs <= (int64_t)16 * d.n_experts;
    p.y = take((size_t)pairs * (y_f32 ? (size_t)d.d_model * sizeof(float)
                                      : (size_t)moe::y16_pitch(d.d_model)));
    p.xnorm = take((size_t)T * d.d_model * esize);
    p.total = off;
    return p;
}

moe::Problem make_problem(const moe_desc &d, int64_t T, const Plan &pl, void *ws) {
    moe::Problem p;
    memset(&p, 0, sizeof p);
    p.T = T;
    p.d = d.d_model;
    p.E = d.n_experts;
    p.k = d.top_k;
    p.F = d.d_expert;
    p.Fs = d.d_shared;
    p.bf16 = d.dtype == MOE_BF16;
    char *base = static_cast<char *>(ws);
    p.logits = reinterpret_cast<float *>(base + pl.logits);
    p.wnorm = reinterpret_cast<float *>(base + pl.wnorm);
    p.router = uses_shortlist(d, T);
    p.router_split = p.router ? moe::shortlist_split(d.d_model) : 1;
    p.gate = reinterpret_cast<float *>(base + pl.gate);
    p.counts = reinterpret_cast<int32_t *>(base + pl.counts);
    p.offsets = reinterpret_cast<int32_t *>(base + pl.offsets);
    p.tile_start = reinterpret_cast<int32_t *>(base + pl.tile_start);
    p.tile_group = reinterpret_cast<int32_t *>(base + pl.tile_group);
    p.blk = reinterpret_cast<int32_t *>(base + pl.blk);
    p.rank = reinterpret_cast<int32_t *>(base + pl.rank);
    p.perm = reinterpret_cast<int32_t *>(base + pl.perm);
    p.h = base + pl.h;
    p.h_shared = base + pl.h_shared;
    p.y = base + pl.y;
    p.nblk = pl.nblk;
    p.max_tiles = pl.max_tiles;
    return p;
}

// Workspace of moe_backward (regions as in moe::BwdArgs).
struct BwdPlan {
    size_t counts, offsets, tile_start, tile_group, blk, rank, perm, logits, au, au_sh, g, g_sh, dgu,
        dgu_sh, hh, hh_sh, dwp, gate, ds, q, dl, dxp, dxs, dxr, dob, part, total;
    int nblk, max_tiles, ldl, ldd, sh_split, sh_chunk, logit_split;
};

BwdPlan make_bwd_plan(const moe_desc &d, int64_t T) {
    BwdPlan p;
    const size_t es = d.dtype == MOE_BF16 ? 2 : 4;
    const int64_t pairs = T * d.top_k;
    const size_t F = (size_t)d.d_expert, Fs = (size_t)d.d_shared, dm = (size_t)d.d_model;
    p.nblk = (int)((T + moe::kCountBlock - 1) / moe::kCountBlock);
    p.max_tiles = (int)moe::max_gemm_tiles(T, d.top_k, d.n_experts, moe::kGemmBM, d.d_shared > 0);
    p.ldl = (d.n_experts + 1 + 3) / 4 * 4;  // 16-byte rows: the GEMM epilogue's vector stores
    p.ldd = (d.n_experts + 1 + 127) / 128 * 128;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    p.counts = take((size_t)(d.n_experts + 1) * 4);
    p.offsets = take((size_t)(d.n_experts + 1) * 4);
    p.tile_start = take((size_t)(d.n_experts + 2) * 4);
    p.tile_group = take((size_t)(p.max_tiles + 1) * 4);
    p.blk = take((size_t)d.n_experts * p.nblk * 4);
    p.rank = take((size_t)pairs * 4);
    p.perm = take((size_t)pairs * 4);
    // the router logits in two K slices at larger T (twice the blocks; the
    // consumers add the slices)
    p.logit_split = d.dtype == MOE_BF16 && T >= 1024 && d.d_model % 128 == 0 ? 2 : 1;
    p.logits = take((size_t)p.logit_split * T * p.ldl * 4);
    p.au = take((size_t)pairs * 2 * F * es);
    p.au_sh = take((size_t)T * 2 * Fs * es);
    p.g = take((size_t)pairs * F * 4);
    p.g_sh = take((size_t)T * Fs * 4);
    p.dgu = take((size_t)pairs * 2 * F * es);
    p.dgu_sh = take((size_t)T * 2 * Fs * es);
    p.hh = take((size_t)pairs * F * es);
    p.hh_sh = take((size_t)T * Fs * es);
    // G . h per row: one value, or one partial per 128 columns of G when the
    // SwiGLU backward runs in G's epilogue
    const size_t gparts = std::max<size_t>(1, (std::max(F, Fs) + 127) / 128);
    p.dwp = take((size_t)pairs * gparts * 4);
    p.gate = take((size_t)T * 4);
    p.ds = take((size_t)T * gparts * 4);
    p.q = take((size_t)T * 4);
    p.dl = take((size_t)T * p.ldd * es);
    p.dxp = take((size_t)pairs * dm * es);
    p.dxs = take((size_t)T * dm * es);
    p.dxr = take((size_t)T * dm * 4);
    p.dob = take(d.dtype == MOE_BF16 ? (size_t)T * dm * 2 : 0);  // dout rounded to bf16 once
    p.sh_split = moe::bwd_sh_split(T, d.dtype == MOE_BF16, d.d_shared);
    p.sh_chunk = moe::bwd_sh_chunk(T, p.sh_split);
    p.part = take((size_t)p.sh_split * 2 * Fs * dm * 4);
    p.total = off;
    return p;
}

moe_status hip_status(hipError_t err) {
    if (err == hipSuccess) return MOE_OK;
    g_last_error = hipGetErrorString(err);
    return MOE_ERR_HIP;
}

// A one-stage call (routing only, MXFP4 packing, RMSNorm alone): its launch
// status and, under MOE_DEBUG_SYNC, the failure of its kernels by name.
moe_status one_stage(hipError_t err, hipStream_t s, const char *name) {
    static thread_local const char *names[2] = {"start", nullptr};
    names[1] = name;
    g_stage_names = names;
    mark_stage(0, s);
    if (err == hipSuccess) mark_stage(1, s);
    return end_call(err);
}

moe_status end_call(hipError_t err) {
    g_n_stage_events = 0;
    if (!g_debug_error.empty()) {
        g_last_error = g_debug_error;
        g_debug_error.clear();
        return MOE_ERR_HIP;
    }
    return hip_status(err);
}

bool all_aligned(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return false;
    return true;
}

// Checks shared by the entry points, workspace aside.  Required pointers are
// listed in `req`.
moe_status check_args(const moe_desc *desc, int64_t T, std::initializer_list<const void *> req,
                      std::initializer_list<const void *> opt) {
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_T(desc, T);
    if (st != MOE_OK || T == 0) return st;
    for (const void *p : req)
        if (!p) return MOE_ERR_INVALID_ARG;
    if (!all_aligned(req) || !all_aligned(opt)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_common(const moe_desc *desc, int64_t T, std::initializer_list<const void *> req,
                        std::initializer_list<const void *> opt, void *ws, size_t ws_bytes) {
    moe_status st = check_args(desc, T, req, opt);
    if (st != MOE_OK || T == 0) return st;
    if (!ws || !aligned16(ws)) return MOE_ERR_WORKSPACE;
    if (ws_bytes < make_plan(*desc, T).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// Weight streaming (few rows per expert) or LDS-tiled MFMA GEMM (many).
bool use_decode_path(const moe::Problem &p) {
    if (!p.bf16 || p.d % 128 || p.F % 128 || p.Fs % 128) return false;
    return p.T * p.k <= (int64_t)16 * p.E;
}

// Tiles staged by direct global -> LDS loads need 128-column multiples and
// 32-bit row offsets (T*k*max(d, F) and T*(E+1) below 2^32).
bool use_dma_path(const moe::Problem &p) {
    if (!p.bf16 || p.F % 128 || p.Fs % 128) return false;
    const int64_t pairs = p.T * p.k;
    const int64_t widest = p.d > p.F ? p.d : p.F;
    return pairs * widest < ((int64_t)1 << 32) && p.T * (int64_t)(p.E + 1) < ((int64_t)1 << 32);
}

bool decode_regime(const moe::Problem &p) {
    return p.mx4 ? p.T * p.k <= (int64_t)16 * p.E : use_decode_path(p);
}

// The weight-streaming path skips the permutation step when an expert fits
// one tile (T <= kDecodeBM) and the exact router, run in the same call, lists
// the touched experts (its top-k experts of a token are distinct); the
// training forward keeps the permuted row order its saved tensors use.
bool direct_decode(const moe::Problem &p) {
    return decode_regime(p) && p.T <= moe::kDecodeBM && !p.au && p.router == 0;
}

// Stages 2..5 of a call: permutation (unless p.direct), gate/up, down, combine.
moe_status run_experts(moe::Problem p, hipStream_t s) {
    const bool decode = decode_regime(p);
    const bool dma = !decode && use_dma_path(p);
    // 256-row tiles once experts average 192+ rows
    const bool big = dma && !p.mx4 && p.T * p.k >= (int64_t)192 * p.E;  // MXFP4 GEMM: 128 rows
    const int bm = decode ? moe::kDecodeBM : big ? moe::kGemm256BM : moe::kGemmBM;
    p.y_f32 = !p.bf16 || decode;
    p.max_tiles = (int)moe::max_gemm_tiles(p.T, p.k, p.E, bm, p.Fs > 0);
    hipError_t err = p.direct ? hipSuccess : moe::launch_permute(p, bm, s);
    mark_stage(2, s);
    auto mark = [&](int i) { mark_stage(i, s); };
    if (err == hipSuccess)
        err = !p.bf16  ? moe::launch_experts_f32(p, s, mark)
              : p.mx4  ? (decode ? moe::launch_experts_decode_mx4(p, s, mark)
                                 : moe::launch_experts_mx4_gemm(p, s, mark))
              : decode ? moe::launch_experts_decode(p, s, mark)
              : dma    ? moe::launch_experts_dma(p, bm, s, mark)
                       : moe::launch_experts_bf16(p, s, mark);
    if (err == hipSuccess) err = moe::launch_combine(p, s);
    mark_stage(5, s);
    return end_call(err);
}

// MXFP4 expert weights: bf16 activations, 128-multiples (the packed tiles)
// and, for the GEMM path, 32-bit row offsets as use_dma_path.
moe_status check_mx4(const moe_desc *desc, int64_t T) {
    if (desc->dtype != MOE_BF16 || desc->d_model % 128 || desc->d_expert % 128 ||
        desc->d_shared % 128)
        return MOE_ERR_UNSUPPORTED;
    const int64_t pairs = T * desc->top_k;
    const int64_t widest = desc->d_model > desc->d_expert ? desc->d_model : desc->d_expert;
    if (pairs * widest >= ((int64_t)1 << 32) || T * (int64_t)desc->d_model >= ((int64_t)1 << 32))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.4e38f; }

// moe_forward / moe_forward_mx4 / moe_forward_prenorm: checks, then
// [RMSNorm into the workspace,] router, permutation, experts, combine.
// norm_weight != nullptr selects the pre-norm (x is then h).
// The training forward's saved buffer: the gate/up pre-activations, then
// (with the shortlist router) its logits, which the backward then reads
// instead of recomputing them: K-slice partials [split][T][E + 1] of
// x W_r^T, the shared gate's logit x . g in column E of slice 0 (zeros in
// the other slices' column E).
size_t saved_au_bytes(const moe_desc &d, int64_t T) {
    const size_t es = d.dtype == MOE_BF16 ? 2 : 4;
    return ((size_t)T * d.top_k * 2 * d.d_expert + (size_t)T * 2 * d.d_shared) * es;
}
size_t saved_logits_off(const moe_desc &d, int64_t T) { return align_up(saved_au_bytes(d, T)); }
size_t saved_logits_bytes(const moe_desc &d, int64_t T) {
    return (size_t)moe::shortlist_split(d.d_model) * T * (d.n_experts + 1) * sizeof(float);
}
// ... then (with more than one histogram block) the permutation: rank and
// perm [T k] and the counts [E + 1], int32.
int saved_nblk(int64_t T) { return (int)((T + moe::kCountBlock - 1) / moe::kCountBlock); }
bool saved_routing(const moe_desc &d, int64_t T) { return uses_shortlist(d, T) && saved_nblk(T) > 1; }
size_t saved_rank_off(const moe_desc &d, int64_t T) {
    return align_up(saved_logits_off(d, T) + saved_logits_bytes(d, T));
}
size_t saved_perm_off(const moe_desc &d, int64_t T) {
    return align_up(saved_rank_off(d, T) + (size_t)T * d.top_k * 4);
}
size_t saved_counts_off(const moe_desc &d, int64_t T) {
    return align_up(saved_perm_off(d, T) + (size_t)T * d.top_k * 4);
}
size_t saved_bytes_of(const moe_desc &d, int64_t T) {
    if (!uses_shortlist(d, T)) return saved_au_bytes(d, T);
    if (!saved_routing(d, T)) return saved_logits_off(d, T) + saved_logits_bytes(d, T);
    return saved_counts_off(d, T) + (size_t)(d.n_experts + 1) * 4;
}

moe_status forward_impl(const moe_desc *desc, int64_t T, const void *x, const void *norm_weight,
                        float eps, bool mx4, const void *w_router, const float *router_bias,
                        const void *w_gate_up, const void *w_down, const void *w_sh_gate_up,
                        const void *w_sh_down, const void *sh_gate, float *out,
                        int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                        void *stream, void *saved = nullptr, size_t saved_bytes = 0,
                        float *resid = nullptr) {
    moe_status st = check_common(desc, T, {x, w_router, w_gate_up, w_down, out, topk_idx, topk_w},
                                 {router_bias, w_sh_gate_up, w_sh_down, sh_gate, resid}, ws,
                                 ws_bytes);
    if (st != MOE_OK) return st;
    if (mx4) {
        st = check_mx4(desc, T);
        if (st != MOE_OK) return st;
    }
    if (T == 0) return MOE_OK;
    if (desc->d_shared > 0 && (!w_sh_gate_up || !w_sh_down || !sh_gate)) return MOE_ERR_INVALID_ARG;
    const Plan pl = make_plan(*desc, T);
    moe::Problem p = make_problem(*desc, T, pl, ws);
    if (saved) {
        p.au = saved;
        p.au_sh = static_cast<char *>(saved) + (size_t)T * desc->top_k * 2 * desc->d_expert *
                                                   (desc->dtype == MOE_BF16 ? 2 : 4);
        if (p.router == 1)  // the shortlist router's logits go straight into saved
            p.logits = reinterpret_cast<float *>(static_cast<char *>(saved) +
                                                 saved_logits_off(*desc, T));
        if (saved_routing(*desc, T)) {  // and the permutation
            char *sb = static_cast<char *>(saved);
            p.rank = reinterpret_cast<int32_t *>(sb + saved_rank_off(*desc, T));
            p.perm = reinterpret_cast<int32_t *>(sb + saved_perm_off(*desc, T));
            p.counts = reinterpret_cast<int32_t *>(sb + saved_counts_off(*desc, T));
        }
    }
    p.x = norm_weight ? static_cast<const void *>(static_cast<char *>(ws) + pl.xnorm) : x;
    p.w_router = w_router;
    p.router_bias = router_bias;
    p.mx4 = mx4;
    p.w_gate_up = w_gate_up;
    p.w_down = w_down;
    p.w_sh_gate_up = w_sh_gate_up;
    p.w_sh_down = w_sh_down;
    p.sh_gate = desc->d_shared > 0 ? sh_gate : nullptr;
    p.out = out;
    p.resid = resid;
    p.topk_idx = topk_idx;
    p.topk_w = topk_w;
    hipStream_t s = static_cast<hipStream_t>(stream);
    g_stage_names = kForwardStages;
    mark_stage(0, s);
    hipError_t err = hipSuccess;
    if (norm_weight)
        err = moe::launch_rmsnorm(x, norm_weight, eps, static_cast<char *>(ws) + pl.xnorm, T, p.d,
                                  p.bf16, s);
    p.direct = direct_decode(p);
    if (err == hipSuccess) err = moe::launch_router(p, nullptr, s);
    mark_stage(1, s);
    if (err != hipSuccess) return end_call(err);
    return run_experts(p, s);
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_desc *desc, int64_t T) {
    if (check_desc(desc) != MOE_OK || check_T(desc, T) != MOE_OK) return 0;
    return make_plan(*desc, T).total;
}

moe_status moe_workspace_query(const moe_desc *desc, int64_t T, moe_workspace_layout *layout) {
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_T(desc, T);
    if (st != MOE_OK) return st;
    if (!layout) return MOE_ERR_INVALID_ARG;
    const Plan p = make_plan(*desc, T);
    layout->logits = p.logits;
    layout->gate = p.gate;
    layout->counts = p.counts;
    layout->offsets = p.offsets;
    layout->perm = p.perm;
    layout->h = p.h;
    layout->h_shared = p.h_shared;
    layout->y = p.y;
    layout->xnorm = p.xnorm;
    layout->total = p.total;
    return MOE_OK;
}

moe_status moe_route(const moe_desc *desc, int64_t T, const void *x, const void *w_router,
                     const float *router_bias, const void *sh_gate, int32_t *topk_idx,
                     float *topk_w, float *sh_gate_out, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_common(desc, T, {x, w_router, topk_idx, topk_w},
                                 {router_bias, sh_gate, sh_gate_out}, ws, ws_bytes);
    if (st != MOE_OK || T == 0) return st;
    const Plan pl = make_plan(*desc, T);
    moe::Problem p = make_problem(*desc, T, pl, ws);
    p.x = x;
    p.w_router = w_router;
    p.router_bias = router_bias;
    // The gate column is computed only when both the vector and an output exist.
    p.sh_gate = (sh_gate && sh_gate_out) ? sh_gate : nullptr;
    p.topk_idx = topk_idx;
    p.topk_w = topk_w;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return one_stage(moe::launch_router(p, sh_gate_out, s), s,
                     "router (router logits, top-k selection, gate)");
}

moe_status moe_forward(const moe_desc *desc, int64_t T, const void *x, const void *w_router,
                       const float *router_bias, const void *w_gate_up, const void *w_down,
                       const void *w_sh_gate_up, const void *w_sh_down, const void *sh_gate,
                       float *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                       void *stream) {
    return forward_impl(desc, T, x, nullptr, 0.0f, false, w_router, router_bias, w_gate_up, w_down,
                        w_sh_gate_up, w_sh_down, sh_gate, out, topk_idx, topk_w, ws, ws_bytes,
                        stream);
}

size_t moe_saved_bytes(const moe_desc *desc, int64_t T) {
    if (check_desc(desc) != MOE_OK || check_T(desc, T) != MOE_OK) return 0;
    return saved_bytes_of(*desc, T);
}

moe_status moe_forward_train(const moe_desc *desc, int64_t T, const void *x, const void *w_router,
                             const float *router_bias, const void *w_gate_up, const void *w_down,
                             const void *w_sh_gate_up, const void *w_sh_down, const void *sh_gate,
                             float *out, int32_t *topk_idx, float *topk_w, void *saved,
                             size_t saved_bytes, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_T(desc, T);
    if (st != MOE_OK || T == 0) return st;
    if (!saved || !aligned16(saved) || saved_bytes < saved_bytes_of(*desc, T))
        return MOE_ERR_INVALID_ARG;
    return forward_impl(desc, T, x, nullptr, 0.0f, false, w_router, router_bias, w_gate_up, w_down,
                        w_sh_gate_up, w_sh_down, sh_gate, out, topk_idx, topk_w, ws, ws_bytes,
                        stream, saved, saved_bytes);
}

moe_status moe_experts(const moe_desc *desc, int64_t T, const void *x, const void *w_gate_up,
                       const void *w_down, const void *w_sh_gate_up, const void *w_sh_down,
                       const void *sh_gate, const int32_t *topk_idx, const float *topk_w,
                       float *out, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_common(desc, T, {x, w_gate_up, w_down, topk_idx, topk_w, out},
                                 {w_sh_gate_up, w_sh_down, sh_gate}, ws, ws_bytes);
    if (st != MOE_OK || T == 0) return st;
    if (desc->d_shared > 0 && (!w_sh_gate_up || !w_sh_down || !sh_gate)) return MOE_ERR_INVALID_ARG;
    const Plan pl = make_plan(*desc, T);
    moe::Problem p = make_problem(*desc, T, pl, ws);
    p.x = x;
    p.w_gate_up = w_gate_up;
    p.w_down = w_down;
    p.w_sh_gate_up = w_sh_gate_up;
    p.w_sh_down = w_sh_down;
    p.sh_gate = sh_gate;
    p.out = out;
    p.topk_idx = const_cast<int32_t *>(topk_idx);
    p.topk_w = const_cast<float *>(topk_w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    g_stage_names = kForwardStages;
    mark_stage(0, s);
    if (p.Fs > 0) {
        const hipError_t err = moe::launch_shared_gate(p, s);
        if (err != hipSuccess) {
            mark_stage(1, s);
            return end_call(err);
        }
    }
    mark_stage(1, s);
    return run_experts(p, s);
}

size_t moe_mx4_packed_bytes(int64_t rows, int64_t K) {
    if (rows <= 0 || K <= 0 || rows % 16 || K % 128) return 0;
    return (size_t)(rows / 16) * (size_t)(K / 128) * 1088;
}

moe_status moe_mx4_pack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                        void *packed, void *stream) {
    if (!codes || !scales || !packed || !aligned16(codes) || !aligned16(packed))
        return MOE_ERR_INVALID_ARG;
    if (moe_mx4_packed_bytes(rows, K) == 0) return MOE_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return one_stage(moe::launch_mx4_pack(codes, scales, rows, K, packed, s), s, "MXFP4 packing");
}

moe_status moe_forward_mx4(const moe_desc *desc, int64_t T, const void *x, const void *w_router,
                           const float *router_bias, const void *w_gate_up, const void *w_down,
                           const void *w_sh_gate_up, const void *w_sh_down, const void *sh_gate,
                           float *out, int32_t *topk_idx, float *topk_w, void *ws,
                           size_t ws_bytes, void *stream) {
    return forward_impl(desc, T, x, nullptr, 0.0f, true, w_router, router_bias, w_gate_up, w_down,
                        w_sh_gate_up, w_sh_down, sh_gate, out, topk_idx, topk_w, ws, ws_bytes,
                        stream);
}

moe_status moe_rmsnorm(const moe_desc *desc, int64_t T, const void *h, const void *norm_weight,
                       float eps, void *x_out, void *stream) {
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_T(desc, T);
    if (st != MOE_OK || T == 0) return st;
    if (!h || !norm_weight || !x_out || !all_aligned({h, norm_weight, x_out}) || !eps_ok(eps))
        return MOE_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return one_stage(moe::launch_rmsnorm(h, norm_weight, eps, x_out, T, desc->d_model,
                                         desc->dtype == MOE_BF16, s),
                     s, "RMSNorm");
}

moe_status moe_forward_prenorm(const moe_desc *desc, int64_t T, const void *h,
                               const void *norm_weight, float eps, int32_t weight_format,
                               const void *w_router, const float *router_bias,
                               const void *w_gate_up, const void *w_down,
                               const void *w_sh_gate_up, const void *w_sh_down, const void *sh_gate,
                               float *out, int32_t *topk_idx, float *topk_w, float *resid,
                               void *ws, size_t ws_bytes, void *stream) {
    if (weight_format != MOE_WEIGHTS_DTYPE && weight_format != MOE_WEIGHTS_MX4)
        return MOE_ERR_INVALID_ARG;
    if (resid && (resid == out || static_cast<const void *>(resid) == h))
        return check_desc(desc) != MOE_OK ? check_desc(desc) : MOE_ERR_INVALID_ARG;
    if (!norm_weight || !aligned16(norm_weight) || !eps_ok(eps)) {
        // a bad desc is reported first, as everywhere else
        moe_status st = check_desc(desc);
        return st != MOE_OK ? st : MOE_ERR_INVALID_ARG;
    }
    return forward_impl(desc, T, h, norm_weight, eps, weight_format == MOE_WEIGHTS_MX4, w_router,
                        router_bias, w_gate_up, w_down, w_sh_gate_up, w_sh_down, sh_gate, out,
                        topk_idx, topk_w, ws, ws_bytes, stream, nullptr, 0, resid);
}

moe_status moe_experts_mx4(const moe_desc *desc, int64_t T, const void *x, const void *w_gate_up,
                           const void *w_down, const void *w_sh_gate_up, const void *w_sh_down,
                           const void *sh_gate, const int32_t *topk_idx, const float *topk_w,
                           float *out, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_common(desc, T, {x, w_gate_up, w_down, topk_idx, topk_w, out},
                                 {w_sh_gate_up, w_sh_down, sh_gate}, ws, ws_bytes);
    if (st != MOE_OK) return st;
    st = check_mx4(desc, T);
    if (st != MOE_OK || T == 0) return st;
    if (desc->d_shared > 0 && (!w_sh_gate_up || !w_sh_down || !sh_gate)) return MOE_ERR_INVALID_ARG;
    const Plan pl = make_plan(*desc, T);
    moe::Problem p = make_problem(*desc, T, pl, ws);
    p.x = x;
    p.mx4 = true;
    p.w_gate_up = w_gate_up;
    p.w_down = w_down;
    p.w_sh_gate_up = w_sh_gate_up;
    p.w_sh_down = w_sh_down;
    p.sh_gate = sh_gate;
    p.out = out;
    p.topk_idx = const_cast<int32_t *>(topk_idx);
    p.topk_w = const_cast<float *>(topk_w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    g_stage_names = kForwardStages;
    mark_stage(0, s);
    if (p.Fs > 0) {
        const hipError_t err = moe::launch_shared_gate(p, s);
        if (err != hipSuccess) {
            mark_stage(1, s);
            return end_call(err);
        }
    }
    mark_stage(1, s);
    return run_experts(p, s);
}

const char *moe_status_string(moe_status status) {
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: layer shape not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    }
    return "unknown moe_status";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

void moe::set_last_error(const char *msg) { g_last_error = msg ? msg : ""; }

moe_status moe::check_forward_args(const moe_desc *desc, int64_t T, const void *x,
                                   const void *w_router, const float *router_bias,
                                   const void *w_gate_up, const void *w_down,
                                   const void *w_sh_gate_up, const void *w_sh_down,
                                   const void *sh_gate, const float *out,
                                   const int32_t *topk_idx, const float *topk_w) {
    moe_status st = check_args(desc, T, {x, w_router, w_gate_up, w_down, out, topk_idx, topk_w},
                               {router_bias, w_sh_gate_up, w_sh_down, sh_gate});
    if (st != MOE_OK || T == 0) return st;
    if (desc->d_shared > 0 && (!w_sh_gate_up || !w_sh_down || !sh_gate)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

extern "C" {

moe_status moe_stage_events(void *const *events, int n) {
    if (n < 0 || n > 8 || (n > 0 && !events)) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i) g_stage_events[i] = static_cast<hipEvent_t>(events[i]);
    g_n_stage_events = n;
    return MOE_OK;
}

}  // extern "C"

extern "C" {

size_t moe_backward_workspace_size(const moe_desc *desc, int64_t T) {
    if (check_desc(desc) != MOE_OK || check_T(desc, T) != MOE_OK) return 0;
    return make_bwd_plan(*desc, T).total;
}

moe_status moe_backward(const moe_desc *desc, int64_t T, const void *x, const void *w_router,
                        const float *router_bias, const void *w_gate_up, const void *w_down,
                        const void *w_sh_gate_up, const void *w_sh_down, const void *sh_gate,
                        const int32_t *topk_idx, const float *topk_w, const float *dout,
                        const void *saved, float aux_coef, float *dx, void *dw_router,
                        void *dw_gate_up,
                        void *dw_down, void *dw_sh_gate_up, void *dw_sh_down, void *dsh_gate,
                        float *aux_loss, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_T(desc, T);
    if (st != MOE_OK || T == 0) return st;
    const bool sh = desc->d_shared > 0;
    for (const void *q : std::initializer_list<const void *>{
             x, w_router, w_gate_up, w_down, topk_idx, topk_w, dout, dx, dw_router, dw_gate_up,
             dw_down})
        if (!q) return MOE_ERR_INVALID_ARG;
    if (sh && (!w_sh_gate_up || !w_sh_down || !sh_gate || !dw_sh_gate_up || !dw_sh_down ||
               !dsh_gate))
        return MOE_ERR_INVALID_ARG;
    if (!all_aligned({x, w_router, router_bias, w_gate_up, w_down, w_sh_gate_up, w_sh_down,
                      sh_gate, topk_idx, topk_w, dout, saved, dx, dw_router, dw_gate_up, dw_down,
                      dw_sh_gate_up, dw_sh_down, dsh_gate}))
        return MOE_ERR_INVALID_ARG;
    if (aux_loss && (reinterpret_cast<uintptr_t>(aux_loss) & 3u)) return MOE_ERR_INVALID_ARG;
    if (!(aux_coef >= -3.4e38f && aux_coef <= 3.4e38f)) return MOE_ERR_INVALID_ARG;
    const BwdPlan pl = make_bwd_plan(*desc, T);
    if (!ws || !aligned16(ws)) return MOE_ERR_WORKSPACE;
    if (ws_bytes < pl.total) return MOE_ERR_WORKSPACE;

    char *base = static_cast<char *>(ws);
    moe::Problem p;
    memset(&p, 0, sizeof p);
    p.T = T;
    p.d = desc->d_model;
    p.E = desc->n_experts;
    p.k = desc->top_k;
    p.F = desc->d_expert;
    p.Fs = desc->d_shared;
    p.bf16 = desc->dtype == MOE_BF16;
    p.topk_idx = const_cast<int32_t *>(topk_idx);
    p.counts = reinterpret_cast<int32_t *>(base + pl.counts);
    p.offsets = reinterpret_cast<int32_t *>(base + pl.offsets);
    p.tile_start = reinterpret_cast<int32_t *>(base + pl.tile_start);
    p.tile_group = reinterpret_cast<int32_t *>(base + pl.tile_group);
    p.blk = reinterpret_cast<int32_t *>(base + pl.blk);
    p.rank = reinterpret_cast<int32_t *>(base + pl.rank);
    p.perm = reinterpret_cast<int32_t *>(base + pl.perm);
    p.nblk = pl.nblk;
    p.max_tiles = pl.max_tiles;
    // with the training forward's permutation only the tile map is built
    const int32_t *counts_given = nullptr;
    if (saved && saved_routing(*desc, T)) {
        char *sb = static_cast<char *>(const_cast<void *>(saved));
        p.rank = reinterpret_cast<int32_t *>(sb + saved_rank_off(*desc, T));
        p.perm = reinterpret_cast<int32_t *>(sb + saved_perm_off(*desc, T));
        counts_given = reinterpret_cast<const int32_t *>(sb + saved_counts_off(*desc, T));
    }

    moe::BwdArgs a;
    memset(&a, 0, sizeof a);
    a.counts_given = counts_given;
    a.T = T;
    a.d = p.d;
    a.E = p.E;
    a.k = p.k;
    a.F = p.F;
    a.Fs = p.Fs;
    a.bf16 = p.bf16;
    a.x = x;
    a.w_router = w_router;
    a.w_gu = w_gate_up;
    a.w_dn = w_down;
    a.w_sgu = sh ? w_sh_gate_up : nullptr;
    a.w_sdn = sh ? w_sh_down : nullptr;
    a.sh_gate = sh ? sh_gate : nullptr;
    a.bias = router_bias;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.dout = dout;
    a.coef = aux_coef;
    a.dx = dx;
    a.dw_router = dw_router;
    a.dw_gu = dw_gate_up;
    a.dw_dn = dw_down;
    a.dw_sgu = sh ? dw_sh_gate_up : nullptr;
    a.dw_sdn = sh ? dw_sh_down : nullptr;
    a.dsh_gate = sh ? dsh_gate : nullptr;
    a.aux_loss = aux_loss;
    a.logits = reinterpret_cast<float *>(base + pl.logits);
    a.ldl = pl.ldl;
    a.logit_split = pl.logit_split;
    a.dwr_split = 1;
    a.counts = p.counts;
    a.offsets = p.offsets;
    a.tile_start = p.tile_start;
    a.tile_group = p.tile_group;
    a.perm = p.perm;
    a.rank = p.rank;
    a.logits_given = false;
    if (saved) {  // the training forward's pre-activations: no recompute
        a.au = const_cast<void *>(saved);
        a.au_sh = static_cast<char *>(const_cast<void *>(saved)) +
                  (size_t)T * p.k * 2 * p.F * (p.bf16 ? 2 : 4);
        a.au_given = true;
        if (uses_shortlist(*desc, T)) {  // and its router logits
            a.logits = reinterpret_cast<float *>(static_cast<char *>(const_cast<void *>(saved)) +
                                                 saved_logits_off(*desc, T));
            a.ldl = p.E + 1;
            a.logit_split = moe::shortlist_split(p.d);
            a.logits_given = true;
        }
    } else {
        a.au = base + pl.au;
        a.au_sh = base + pl.au_sh;
        a.au_given = false;
    }
    a.g = reinterpret_cast<float *>(base + pl.g);
    a.g_sh = reinterpret_cast<float *>(base + pl.g_sh);
    a.dgu = base + pl.dgu;
    a.dgu_sh = base + pl.dgu_sh;
    a.hh = base + pl.hh;
    a.hh_sh = base + pl.hh_sh;
    a.dwp = reinterpret_cast<float *>(base + pl.dwp);
    a.gate = reinterpret_cast<float *>(base + pl.gate);
    a.ds = reinterpret_cast<float *>(base + pl.ds);
    a.gtile = 0;
    a.q = reinterpret_cast<float *>(base + pl.q);
    a.dl = base + pl.dl;
    a.ldd = pl.ldd;
    a.dxp = base + pl.dxp;
    a.dxs = base + pl.dxs;
    a.dxr = reinterpret_cast<float *>(base + pl.dxr);
    a.dob = base + pl.dob;
    a.dw_kmin = -1;
    a.sh_split = pl.sh_split;
    a.sh_chunk = pl.sh_chunk;
    a.part = reinterpret_cast<float *>(base + pl.part);

    hipStream_t s = static_cast<hipStream_t>(stream);
    g_stage_names = kBackwardStages;
    mark_stage(0, s);
    const hipError_t err = moe::launch_backward(p, a, s, [&](int i) { mark_stage(i, s); });
    return end_call(err);
}

}  // extern "C"
