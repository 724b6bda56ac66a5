// moe_kernels.h -- host-side launchers of the libmoe kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <functional>

#include "moe.h"

namespace moe {

// Everything a launch needs to know about one call.  Pointers are device
// pointers; `esize` is the byte size of a weight/activation element.
struct Problem {
    int64_t T;
    int d, E, k, F, Fs;
    bool bf16;
    // inputs
    const void *x, *w_router, *w_gate_up, *w_down, *w_sh_gate_up, *w_sh_down, *sh_gate;
    const float *router_bias;
    // outputs / routing
    float *out;
    int32_t *topk_idx;
    float *topk_w;
    // workspace regions
    float *logits;      // [T, E+1]; shortlist router: [router_split, T, E+1]
    float *wnorm;       // [E] Euclidean norms of the router rows
    int router;         // 0: exact canonical logits for all experts; 1: MFMA shortlist
    int router_split;   // shortlist: K slices of the MFMA logits (partial sums)
    float *gate;        // [T]
    int32_t *counts;    // [E+1]
    int32_t *offsets;   // [E+1]
    int32_t *tile_start;// [E+2]
    int32_t *tile_group;// [max_tiles] group (expert, or E = shared) of each GEMM tile
    int max_tiles;      // upper bound on GEMM tiles for the tile height in use
    int32_t *blk;       // [E, nblk]
    int32_t *rank;      // [T*k] rank inside the histogram block, then the pair's row
    int32_t *perm;      // [T*k]
    void *y;            // [T*k] weighted down-projection of each routed row: rows of
                        // y16_pitch(d) bytes in 16-bit block floating point from
                        // the grouped GEMMs, binary32 [T*k, d] when y_f32
    bool y_f32;         // y in binary32: binary32 layers and the weight-streaming path
                        // (bf16 for bfloat16 layers, binary32 otherwise)
    void *h;            // [T*k, F]
    void *h_shared;     // [T, Fs]
    // training forward: the gate/up pre-activations [a | u] of every row
    // (routed rows in the permuted order, then the shared expert's), or null
    void *au;           // [T*k, 2F]
    void *au_sh;        // [T, 2Fs]
    int nblk;           // ceil(T / kCountBlock)
    // weight-streaming path without the permutation step (T <= kDecodeBM,
    // routing from this library's exact router): the router's select step
    // lists the touched experts (counts[e] = 1 once e is selected, counts[E]
    // = how many, tile_group[i] = the i-th in arrival order); block 0 serves
    // the shared expert (if any), the next blocks expert tile_group[x], each
    // finding its pairs in topk_idx, and h / y rows are indexed by pair id t*k+j
    bool direct;
    // MXFP4 expert weights: w_gate_up, w_down, w_sh_gate_up, w_sh_down are
    // then packed MXFP4 tensors (16 x 128 tiles of codes and scales)
    bool mx4;
    // residual stream [T, d] binary32 or null: the combine's store also does
    // resid[t] += out[t]
    float *resid;
};

// Sets the text moe_last_error returns on this thread.
void set_last_error(const char *msg);

// moe_forward's argument checks, the workspace aside (moe_status values).
moe_status check_forward_args(const moe_desc *desc, int64_t T, const void *x,
                              const void *w_router, const float *router_bias,
                              const void *w_gate_up, const void *w_down,
                              const void *w_sh_gate_up, const void *w_sh_down,
                              const void *sh_gate, const float *out, const int32_t *topk_idx,
                              const float *topk_w);

constexpr int kCountBlock = 256;     // tokens per histogram block
constexpr int kGemmBM = 128;         // rows per grouped-GEMM tile (MFMA paths)
constexpr int kDecodeBM = 32;        // rows per tile of the weight-streaming (decode) path
constexpr int kGemm256BM = 256;      // rows per tile for many tokens per expert

// Upper bound on sum_e ceil(c_e / bm) + ceil(T / bm) over any routing with
// sum_e c_e = T*k: each non-empty expert adds at most one partial tile.
inline int64_t max_gemm_tiles(int64_t T, int k, int E, int bm, bool shared) {
    const int64_t pairs = T * k;
    const int64_t routed = (pairs < E ? pairs : E) + pairs / bm;
    return routed + (shared ? (T + bm - 1) / bm : 0);
}

// Arguments of the LDS-tiled grouped GEMM kernels (bf16 in, fp32 accumulate).
struct GemmArgs {
    const uint16_t *x;
    const uint16_t *w;     // gate/up: [E, 2F, d]   down: [E, d, F]
    const uint16_t *w_sh;  // gate/up: [2Fs, d]     down: [d, Fs]
    uint16_t *h;           // [T*k, F]
    uint16_t *h_sh;        // [T, Fs]
    uint16_t *au, *au_sh;  // [T*k, 2F], [T, 2Fs] pre-activations [a | u] (training), or null
    float *out;            // [T, d]   shared expert's term (plain stores)
    uint8_t *y;            // [T*k] routed rows, weighted, y16 rows (plain stores)
    float *f;              // router logits [ksplit, T, ldf] (MODE 2): one partial per K slice
    float *wnorm;          // MODE 2: router row norms [E], from the blocks of slice ksplit (or null)
    int ldf, ksplit;
    const int32_t *perm, *counts, *offsets, *tile_start, *tile_group;
    const float *topk_w, *gate;
    int64_t T;
    int d, E, k, F, Fs;
    int nm, nn, gm;        // M-tiles, N-tiles and raster group height (raster_tile)
};

// Blocks of the 1-D grid that raster_tile maps onto nm x nn tiles.
inline unsigned raster_blocks(int nm, int nn, int gm) {
    return gm < 0 ? (unsigned)(8 * ((nm + 7) / 8) * nn) : (unsigned)(8 * ((nm * nn + 7) / 8));
}

// Router logits f = x W_r^T on MFMA (binary32 accumulate, any order), as
// p.router_split partial sums over consecutive slices of K.
hipError_t launch_router_gemm(const Problem &p, hipStream_t s);
// K slices of the shortlist router's MFMA logits for d (d % 64 == 0): twice
// the blocks for the short, wide GEMM; the select step adds them in order.
// At T = 4096, d = 2560 the route stage took 80 / 67 / 69 / 86 us with
// 1 / 2 / 4 / 8 slices.
inline int shortlist_split(int d) { return d % 128 == 0 ? 2 : 1; }
// Grouped GEMM expert stage with bm x 256 tiles (bm = 256 or 128) staged by
// direct global -> LDS loads; needs F, Fs % 128 == 0 and 32-bit offsets.
hipError_t launch_experts_dma(const Problem &p, int bm, hipStream_t s,
                              const std::function<void(int)> &mark);
// Router: logits (canonical binary32 order) then top-k / weights / gate.
hipError_t launch_router(const Problem &p, float *sh_gate_user, hipStream_t s);
// Pre-FFN RMSNorm of h [T, d] into x (bf16 or binary32), fixed binary32 order.
hipError_t launch_rmsnorm(const void *h, const void *gamma, float eps, void *x, int64_t T, int d,
                          bool bf16, hipStream_t s);
// Shared gate alone (used when the routing is given).
hipError_t launch_shared_gate(const Problem &p, hipStream_t s);
// Histogram, scan, stable permutation and GEMM tile map for tile height bm.
hipError_t launch_permute(const Problem &p, int bm, hipStream_t s);
// Counts (copied), offsets and the tile map of tile height bm from given
// per-expert counts, for a permutation whose rank and perm are there (E <= 1024).
hipError_t launch_permute_tiles(const Problem &p, const int32_t *counts_in, int bm, hipStream_t s);
// out[t] (= shared term, if any) += sum_j y[row(t, j)]
hipError_t launch_combine(const Problem &p, hipStream_t s);
// Expert stage for bfloat16 (MFMA) and binary32 (plain FMA) layers:
// gate/up then down.  mark(3) is called after gate/up, mark(4) after down.
hipError_t launch_experts_bf16(const Problem &p, hipStream_t s, const std::function<void(int)> &mark);
hipError_t launch_experts_f32(const Problem &p, hipStream_t s, const std::function<void(int)> &mark);
// Weight-streaming expert stage for few tokens per expert (tiles of kDecodeBM).
hipError_t launch_experts_decode(const Problem &p, hipStream_t s,
                                 const std::function<void(int)> &mark);
// The same with packed MXFP4 expert weights (p.mx4), decoded to bf16 in
// registers.
hipError_t launch_experts_decode_mx4(const Problem &p, hipStream_t s,
                                     const std::function<void(int)> &mark);
// Grouped GEMM expert stage with packed MXFP4 weights for many rows per expert
// (128 x 256 tiles, tile map for kGemmBM); d, F, Fs % 128 == 0, 32-bit offsets.
hipError_t launch_experts_mx4_gemm(const Problem &p, hipStream_t s,
                                   const std::function<void(int)> &mark);
// Backward pass of the layer for a given routing.  Weights, x and the
// activation intermediates are in the layer's dtype; dout, dx, logits, G and
// the per-row scalars are binary32.
struct BwdArgs {
    int64_t T;
    int d, E, k, F, Fs;
    bool bf16;
    const void *x, *w_router, *w_gu, *w_dn, *w_sgu, *w_sdn, *sh_gate;
    const float *bias;
    const int32_t *topk_idx;
    const float *topk_w;
    const float *dout;  // [T, d]
    float coef;         // load-balancing loss coefficient
    // outputs
    float *dx;          // [T, d]
    void *dw_router, *dw_gu, *dw_dn, *dw_sgu, *dw_sdn, *dsh_gate;
    float *aux_loss;    // [1] or null
    // workspace
    float *logits;      // [logit_split, T, ldl]  x . [W_r; g] (no bias) in logit_split K
                        // slices (partial sums; the logit is their sum); ldl = E + 1 rounded up to 4
    int ldl;
    int logit_split;
    bool logits_given;  // logits hold the training forward's router logits: not recomputed
    const int32_t *counts_given;  // non-null: rank / perm hold the training forward's
                                  // permutation, these its counts (only the tile map is built)
    int dwr_split;      // dW_router's reduction over the tokens in this many chunks (partials in part)
    const int32_t *counts, *offsets, *tile_start, *tile_group, *perm, *rank;
    void *au, *au_sh;   // [T*k, 2F], [T, 2Fs]  gate | up pre-activations
    bool au_given;      // au holds the training forward's values (no recompute)
    float *g, *g_sh;    // [T*k, F], [T, Fs]    W_dn^T dout of each row
    void *dgu, *dgu_sh; // [T*k, 2F], [T, 2Fs]  da | du
    void *hh, *hh_sh;   // [T*k, F], [T, Fs]    w h (h = silu(a) u; w the row's combine weight, s_t shared)
    float *dwp;         // [T*k, max(gtile, 1)] d/dw of each pair (pair order)
    float *gate, *ds;   // [T] s_t and [T, max(gtile, 1)] d/ds_t
    int gtile;          // 0: dwp / ds hold one value per row; > 0: per row, one partial
                        //   sum per 128 columns of G (G's direct-to-LDS tiles), gtile apart
    float *q;           // [T] f . p_t
    void *dl;           // [T, ldd] router-logit gradient, zero padded
    int ldd;
    void *dxp, *dxs;    // [T*k, d], [T, d]  dx of each routed row, of the shared expert
    float *dxr;         // [T, d]            dx of the router
    void *dob;          // [T, d] bf16       dout rounded once (bf16 layers on the direct-to-LDS tiles)
    int dw_kmin;        // weight-gradient launches skip groups with at most this many rows
    int sh_split;       // > 0: the shared expert's weight gradients reduce over the tokens
    int sh_chunk;       //   in sh_split chunks of sh_chunk rows, partials in part
    float *part;        // [sh_split, max(2 Fs d, d Fs)] binary32
};
// Chunks of the shared expert's weight-gradient reduction over T tokens
// (bfloat16 layers; 0: not split).
inline int bwd_sh_split(int64_t T, bool bf16, int Fs) {
    if (!bf16 || Fs == 0 || T <= 128) return 0;
    const int64_t s = (T + 511) / 512;
    return (int)(s < 16 ? s : 16);
}
inline int bwd_sh_chunk(int64_t T, int split) {
    return split ? (int)(((T + split - 1) / split + 63) / 64 * 64) : 0;
}
// p carries the routing and permutation buffers (tile map for kGemmBM rows).
// mark(i) after stage i: 1 logits, 2 gate/up and G (with the SwiGLU backward
// on the direct-to-LDS tiles), 3 SwiGLU (other paths) and router backward,
// 4 dX, 5 dW_gu, 6 dW_dn, 7 router GEMMs, combine and loss.
hipError_t launch_backward(const Problem &p, const BwdArgs &a, hipStream_t s,
                           const std::function<void(int)> &mark);
// dX of the routed and shared rows ([da | du] W_gu) and G (dOut W_dn) on
// direct-to-LDS tiles: bf16 layers with F, Fs and d multiples of 128 and
// 32-bit element offsets, router logits in at most two K slices.  G first
// rounds dOut to bf16 into dout_bf16 [T, d] (dob, which the down-projection
// weight gradients read later too); its epilogue runs the SwiGLU backward
// (dgu, hh, gate and the G . h partials in dwp / ds, a.gtile apart), so G is
// never stored.
bool bwd_dma_ok(const BwdArgs &a);
// Down-projection weight gradients of the routed experts with at most 128
// rows on streamed direct-to-LDS tiles (the shared expert's go to the tiled
// kernels): bf16 layers as bwd_dma_ok, the shared expert split (or absent);
// rounds dOut to bf16 into dob again first (fresh in the caches for its
// gathered reads and for the shared expert's gradient that follows).
bool bwd_dwdn_stream_ok(const BwdArgs &a);
hipError_t launch_bwd_dwdn_stream(const BwdArgs &a, hipStream_t s);
hipError_t launch_bwd_dx_dma(const BwdArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_bwd_g_dma(const BwdArgs &a, int max_tiles, void *dout_bf16, hipStream_t s);
// The shared expert's weight gradients (token chunks, binary32 partials into
// part) on the same tiles with both operands along the output axis; down
// reads dOut rounded to bf16 (dob) and s h (hh_sh).  The launch picks its own
// number of chunks (at most sh_split) for its gradient's shape and returns
// it in *split (the partials to sum).
bool bwd_wsh_dma_ok(const BwdArgs &a);
hipError_t launch_bwd_wsh_dma(const BwdArgs &a, bool down, hipStream_t s, int *split);
// dW_router and the shared gate's gradient (dL^T X) on the same tiles, split
// over token chunks into binary32 partials [*split, ldd, d] in part.
bool bwd_dwr_dma_ok(const BwdArgs &a);
hipError_t launch_bwd_dwr_dma(const BwdArgs &a, hipStream_t s, int *split);
// Row-major MXFP4 [rows, K] (codes, scales) -> packed tiles (rows % 16 == 0,
// K % 128 == 0).
hipError_t launch_mx4_pack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                           void *packed, hipStream_t s);

}  // namespace moe
